"""Pins for oracle.kv_commit (CPU, float64).

* Attention after the commit: for every node n_d of an accepted path, plain
  causal attention of that node's query over the committed cache prefix
  (torch's scaled-dot-product attention, a library routine) equals the node's
  row of the tree-masked verify attention -- the commit keeps exactly what the
  node saw, in sequence order.  Paths are chosen so that some destinations are
  sources of shallower nodes, and longer than one 64-row chunk.
* A chain with every draft accepted, and a = 0, leave the cache unchanged.
* Invalid inputs leave the sequence untouched and report -1.
"""

import numpy as np
import torch
import torch.nn.functional as F

import workloads
from oracle import attention, kv_commit, tree


def _causal_last_row(q_rows, k, v, scale):
    """q_rows[H][D] attending to all of k/v[H][n][D]: the last row of causal attention."""
    q = torch.from_numpy(q_rows[:, None, :])
    return F.scaled_dot_product_attention(q, torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()[:, 0, :]


def _path_to(parent, v):
    """Accepted path ending at node v: n_1 .. n_depth(v) (root excluded)."""
    return tree.ancestors_or_self(parent, v)[::-1][1:]


def _ladder(m):
    """Tree of 2m+1 nodes whose deepest path is 1, 3, 5, ..., 2m-1 (each with a leaf sibling)."""
    parent = [-1, 0, 0]
    for k in range(1, m):
        parent += [2 * k - 1, 2 * k - 1]
    return np.asarray(parent, dtype=np.int32)


def test_committed_prefix_reproduces_tree_attention_rows():
    rng = np.random.default_rng(31)
    trees = [workloads.TREE6, workloads.random_tree(rng, 16, 3, 6), workloads.random_tree(rng, 39, 4, 8),
             _ladder(70)]
    for t, parent in enumerate(trees):
        parent = np.asarray(parent, dtype=np.int32)
        n1 = len(parent)
        hq, hkv, d = 4, 2, 8
        L = 5 + 3 * t
        a = workloads.make_attention("c", parent[None, :], [L], hq, hkv, d, "f32", 40 + t, extra_slack=3)
        mask, depth, st = tree.build_tree_mask_batch(parent[None, :])
        assert not st.any()
        ends = [int(np.argmax(depth[0]))] + [int(x) for x in rng.integers(0, n1, size=3)]
        for v in ends:
            path = _path_to(parent, v)
            nodes = np.full((1, n1), -1, dtype=np.int32)
            nodes[0, :len(path)] = path
            k_new, v_new, new_len = kv_commit.commit(a.k_cache, a.v_cache, [L], [len(path)], nodes)
            assert new_len[0] == L + 1 + len(path)
            rows = [(0, nd) for nd in [0] + path]
            ref, _ = attention.tree_attention(a.q, a.k_cache, a.v_cache, a.ctx_len, mask, a.scale, rows=rows)
            g = hq // hkv
            for dd, nd in enumerate([0] + path):
                n = L + 1 + dd                                    # context + root + n_1 .. n_dd
                k = np.repeat(k_new[0, :, :n, :].astype(np.float64), g, axis=0)
                vv = np.repeat(v_new[0, :, :n, :].astype(np.float64), g, axis=0)
                got = _causal_last_row(a.q[0, nd].astype(np.float64), k, vv, a.scale)
                np.testing.assert_allclose(got, ref[0, nd], rtol=0, atol=1e-12)


def test_destination_that_is_a_shallower_source():
    # path 3 -> 5 -> ... : the row of depth 3 goes to ctx + 3, which held node 3 (depth 1)
    parent = np.asarray([-1, 0, 0, 0, 3, 3, 5], dtype=np.int32)
    path = [3, 5, 6]
    rng = np.random.default_rng(2)
    L, Lmax = 4, 4 + 7 + 2
    kc = rng.normal(size=(1, 2, Lmax, 8))
    vc = rng.normal(size=(1, 2, Lmax, 8))
    nodes = np.asarray([path + [-1] * 4], dtype=np.int32)
    k_new, v_new, new_len = kv_commit.commit(kc, vc, [L], [3], nodes)
    assert new_len[0] == L + 4
    np.testing.assert_array_equal(k_new[0, :, :L + 1], kc[0, :, :L + 1])      # context and root
    for d, nd in enumerate(path, start=1):
        np.testing.assert_array_equal(k_new[0, :, L + d], kc[0, :, L + nd])
        np.testing.assert_array_equal(v_new[0, :, L + d], vc[0, :, L + nd])


def test_chain_all_accepted_and_nothing_accepted_are_identity():
    rng = np.random.default_rng(3)
    B, K, Lmax = 3, 5, 20
    kc, vc = rng.normal(size=(B, 2, Lmax, 4)), rng.normal(size=(B, 2, Lmax, 4))
    nodes = np.tile(np.arange(1, K + 2, dtype=np.int32), (B, 1))
    nodes[:, K:] = -1
    acc = np.asarray([K, 0, 2])
    nodes[1, :] = -1
    nodes[2, 2:] = -1
    k_new, v_new, new_len = kv_commit.commit(kc, vc, [3, 7, 0], acc, nodes)
    assert list(new_len) == [3 + 1 + K, 8, 3]
    np.testing.assert_array_equal(k_new, kc)
    np.testing.assert_array_equal(v_new, vc)


def test_invalid_sequences_are_untouched():
    rng = np.random.default_rng(4)
    B, n1, Lmax = 6, 7, 16
    kc, vc = rng.normal(size=(B, 1, Lmax, 4)), rng.normal(size=(B, 1, Lmax, 4))
    nodes = np.full((B, n1), -1, dtype=np.int32)
    nodes[:, :3] = [2, 4, 6]
    ctx = np.asarray([3, 3, 3, 3, 3, 10])
    acc = np.asarray([-1, -2, 3, 3, 3, 3])
    nodes[3, :3] = [2, 2, 6]          # not increasing
    nodes[4, :3] = [2, 4, 7]          # node outside the tree
    # sequence 2 is valid; sequence 5's context does not leave room for the tree
    k_new, v_new, new_len = kv_commit.commit(kc, vc, ctx, acc, nodes)
    assert list(new_len) == [-1, -1, 3 + 4, -1, -1, -1]
    for b in (0, 1, 3, 4, 5):
        np.testing.assert_array_equal(k_new[b], kc[b])
        np.testing.assert_array_equal(v_new[b], vc[b])
    bad = np.full((1, n1), -1, dtype=np.int32)
    bad[0, :2] = [1, 1]               # depth-2 node shallower than its depth allows
    assert kv_commit.commit(kc[:1], vc[:1], [3], [2], bad)[2][0] == -1
    bad[0, :2] = [0, 2]               # the root is not an accepted draft
    assert kv_commit.commit(kc[:1], vc[:1], [3], [2], bad)[2][0] == -1
