"""Pins for oracle.philox: published known-answer vectors and numpy's own Philox."""

import numpy as np
import pytest
from scipy import stats

from conftest import golden_rows
from oracle import philox


def test_known_answer_vectors():
    rows = golden_rows("philox4x64_10_kat.txt")
    assert len(rows) == 3
    for r in rows:
        ctr = [int(x, 16) for x in r[0:4]]
        key = [int(x, 16) for x in r[4:6]]
        want = tuple(int(x, 16) for x in r[6:10])
        assert philox.philox4x64_10(ctr, key) == want


def _numpy_philox(ctr, key):
    # numpy's Philox bumps the counter before producing a block, so start one below.
    c = list(ctr)
    i = 0
    while True:
        c[i] = (c[i] - 1) & philox.MASK64
        if c[i] != philox.MASK64:
            break
        i += 1
        if i == 4:
            break
    g = np.random.Philox(counter=np.array(c, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    return tuple(int(x) for x in g.random_raw(4))


def test_matches_numpy_philox_on_random_inputs():
    rng = np.random.default_rng(7)
    for _ in range(200):
        ctr = [int(x) for x in rng.integers(0, 2**64, size=4, dtype=np.uint64)]
        key = [int(x) for x in rng.integers(0, 2**64, size=2, dtype=np.uint64)]
        assert philox.philox4x64_10(ctr, key) == _numpy_philox(ctr, key)


def test_counter_layout_and_words():
    # u_acc / u_res of (b, v) come from words 0 / 1 of counter (v, b, offset, 0), key (seed, 0)
    seed, offset, b, v = 1234, 99, 5, 3
    w = _numpy_philox([v, b, offset, 0], [seed, 0])
    ua, ur = philox.node_uniforms(seed, offset, b, v)
    assert ua == philox.word_to_uniform(w[0])
    assert ur == philox.word_to_uniform(w[1])


def test_uniform_map_is_exact_and_open():
    assert philox.word_to_uniform(0) == 2.0 ** -53
    assert philox.word_to_uniform(2**64 - 1) == 1.0 - 2.0 ** -53
    assert 0.0 < philox.word_to_uniform(2**64 - 1) < 1.0
    u = philox.word_to_uniform(0x0123456789ABCDEF)
    # an odd multiple of 2**-53
    k = u * 2.0 ** 53
    assert k == int(k) and int(k) % 2 == 1


def test_uniforms_look_uniform():
    ua, ur = philox.uniforms(42, 0, 100, 50)
    u = np.array(ua + ur).ravel()
    assert u.min() > 0 and u.max() < 1
    assert abs(u.mean() - 0.5) < 4 * (1 / np.sqrt(12 * u.size))
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    # distinct offsets give distinct streams
    ub, _ = philox.uniforms(42, 1, 100, 50)
    assert not np.array_equal(np.array(ua), np.array(ub))
