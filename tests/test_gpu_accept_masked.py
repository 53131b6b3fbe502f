"""Accept / resample on rows with masked vocabulary entries, against the oracle.

A vocabulary is often masked (padding, constrained decoding) by -inf logits or by the dtype's
most negative finite value.  The second kind makes z / T overflow fp32 for T below about 1.4, so a
kernel that scales logits before taking differences must still give those entries no mass.  The
rows here carry both kinds: a band at the end of the vocabulary (a padded vocabulary), random
entries, and whole runs of 8192 entries -- one item of the statistics pass, so that every lane of
a wave and whole chunk statistics see only masked values.  Target and draft rows get independent
masks (p = 0 where q > 0 and the reverse); drafted tokens stay unmasked.
"""

import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_common import compare_accept, log, run_accept_gpu, run_accept_oracle

pytestmark = pytest.mark.gpu

# the most negative finite bf16 value (0xff7f), exactly representable in fp32
BF16_LOWEST = float(np.frombuffer(np.uint32(0xFF7F0000).tobytes(), dtype=np.float32)[0])
F32_LOWEST = float(np.finfo(np.float32).min)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _mask_rows(rows, keep, lowest, rng, run=8192):
    """Mask rows [n][V] in place: a band of the last 3% at `lowest`, 10% random entries at -inf,
    and on every other row a run of `run` entries at `lowest`; entries in `keep` are left alone."""
    n, V = rows.shape
    band = max(1, (3 * V) // 100)
    for i in range(n):
        m = np.zeros(V, dtype=bool)
        m[V - band:] = True
        lo_vals = m.copy()
        rnd = rng.random(V) < 0.10
        if i % 2 == 0 and V > run:
            s0 = int(rng.integers(0, (V - run) // run + 1)) * run
            m[s0:s0 + run] = True
            lo_vals[s0:s0 + run] = True
        m |= rnd
        m[keep] = False
        lo_vals[keep] = False
        rows[i, m & ~lo_vals] = -np.inf
        rows[i, m & lo_vals] = lowest


def _masked(w, seed):
    rng = np.random.default_rng(seed)
    lowest = BF16_LOWEST if w.dtype == "bf16" else F32_LOWEST
    tl = np.array(w.target_logits, copy=True)
    dl = np.array(w.draft_logits, copy=True) if w.draft_logits is not None else None
    for b in range(w.B):
        keep = np.unique(w.tokens[b, 1:])
        _mask_rows(tl[b], keep, lowest, rng)
        if dl is not None:
            _mask_rows(dl[b], keep, lowest, rng)
    return dataclasses.replace(w, name=w.name + "-masked", target_logits=tl, draft_logits=dl)


CASES = {
    # bf16 chain at T = 0.8: z / T of the lowest bf16 overflows fp32
    "chain-bf16": lambda: workloads.make_accept("chain", workloads.chain_parent(8, 5), 32000, 0.8, "bf16",
                                                3.0, 1.0, 8100),
    # trees of the EAGLE shape, V not a multiple of the item length (a partial last chunk)
    "tree-bf16": lambda: workloads.make_accept("tree", workloads.eagle_shaped_parents(4, seed_base=8200), 50000,
                                               0.7, "bf16", 3.0, 1.0, 8201),
    # fp32 chain at T = 0.5 (the lowest fp32 value times 1 / T overflows)
    "chain-f32": lambda: workloads.make_accept("chain32", workloads.chain_parent(8, 6), 40000, 0.5, "f32",
                                               3.0, 1.0, 8300),
    # greedy: the argmax ignores the masks
    "greedy-bf16": lambda: workloads.make_accept("greedy", workloads.chain_parent(8, 5), 32000, 0.0, "bf16",
                                                 3.0, 1.0, 8400, greedy_tokens=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_accept_masked_rows_match_oracle(name):
    w = _masked(CASES[name](), seed=8000 + list(CASES).index(name))
    log(f"accept on masked rows: {name}, B={w.B} N1={w.N1} V={w.V} T={w.T} {w.dtype}")
    got = run_accept_gpu(w)
    ora = run_accept_oracle(w)
    compare_accept(got, ora, check_probs=w.T > 0, name=f"masked-{name}")
    # probabilities of drafted tokens stay finite and in [0, 1]
    if w.T > 0:
        p = got["p_tok"][:, 1:]
        assert np.all((p >= 0) & (p <= 1)), f"[{name}] p_tok outside [0, 1]"
