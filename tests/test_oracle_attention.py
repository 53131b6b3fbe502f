"""Pins for oracle.attention against torch's scaled-dot-product attention (CPU, float64).

* A chain-shaped tree must give plain causal attention over context + drafts.
* Every tree row must equal causal attention over the context followed by the
  root-to-node path alone (per-path brute force).
* The log-sum-exp output is checked through the effect of one extra key.
"""

import numpy as np
import torch
import torch.nn.functional as F

import workloads
from oracle import attention, tree


def _sdpa(q, k, v, mask, scale):
    """q[H][Nq][D], k/v[H][Nk][D] (float64), bool mask[Nq][Nk] (True = visible)."""
    return F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()


def _case(parent, ctx_len, hq, hkv, d, seed):
    parent = np.asarray(parent, dtype=np.int32)
    a = workloads.make_attention("t", parent, ctx_len, hq, hkv, d, "f32", seed)
    mask, depth, st = tree.build_tree_mask_batch(parent)
    assert not st.any()
    return a, mask


def test_chain_equals_causal_attention():
    B, K, hq, hkv, d = 3, 5, 6, 2, 16
    parent = workloads.chain_parent(B, K)
    a, mask = _case(parent, [24, 7, 1], hq, hkv, d, seed=11)
    out, lse = attention.tree_attention(a.q, a.k_cache, a.v_cache, a.ctx_len, mask, a.scale)
    g = hq // hkv
    for b in range(B):
        L = int(a.ctx_len[b])
        n = L + K + 1
        k = np.repeat(a.k_cache[b, :, :n, :].astype(np.float64), g, axis=0)   # head h -> kv h // g
        v = np.repeat(a.v_cache[b, :, :n, :].astype(np.float64), g, axis=0)
        q = a.q[b].astype(np.float64).transpose(1, 0, 2)                       # [H][N1][D]
        m = np.zeros((K + 1, n), dtype=bool)
        m[:, :L] = True
        m[:, L:] = np.tril(np.ones((K + 1, K + 1), dtype=bool))
        ref = _sdpa(q, k, v, m, a.scale).transpose(1, 0, 2)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_tree_rows_equal_per_path_causal_attention():
    rng = np.random.default_rng(5)
    parents = [workloads.TREE6] + [workloads.random_tree(rng, n - 1, 3, 5) for n in (9, 17, 40)]
    for t, parent in enumerate(parents):
        n1 = len(parent)
        a, mask = _case(parent[None, :], [13 + t], 4, 2, 8, seed=20 + t)
        out, _ = attention.tree_attention(a.q, a.k_cache, a.v_cache, a.ctx_len, mask, a.scale)
        L = int(a.ctx_len[0])
        for node in range(n1):
            path = tree.ancestors_or_self(parent, node)[::-1]               # root .. node
            pos = list(range(L)) + [L + j for j in path]
            for h in range(4):
                kv = h // 2
                k = a.k_cache[0, kv, pos, :].astype(np.float64)[None]
                v = a.v_cache[0, kv, pos, :].astype(np.float64)[None]
                q = a.q[0, node, h, :].astype(np.float64)[None, None, :]
                ref = _sdpa(q, k, v, np.ones((1, len(pos)), dtype=bool), a.scale)[0, 0]
                np.testing.assert_allclose(out[0, node, h], ref, rtol=0, atol=1e-12)


def test_lse_through_an_extra_key():
    # Add one key k0 = 0 (score 0) with value v0: SDPA output o' satisfies
    # o' = (Z o + v0) / (Z + 1) with Z = exp(lse), so Z = (v0 - o') / (o' - o).
    parent = workloads.TREE6[None, :]
    a, mask = _case(parent, [10], 2, 1, 8, seed=31)
    out, lse = attention.tree_attention(a.q, a.k_cache, a.v_cache, a.ctx_len, mask, a.scale)
    L = 10
    for node in range(7):
        path = tree.ancestors_or_self(workloads.TREE6, node)[::-1]
        pos = list(range(L)) + [L + j for j in path]
        for h in range(2):
            k = np.concatenate([a.k_cache[0, 0, pos, :], np.zeros((1, 8))]).astype(np.float64)[None]
            v0 = np.full((1, 8), 10.0)
            v = np.concatenate([a.v_cache[0, 0, pos, :], v0]).astype(np.float64)[None]
            q = a.q[0, node, h, :].astype(np.float64)[None, None, :]
            o2 = _sdpa(q, k, v, np.ones((1, len(pos) + 1), dtype=bool), a.scale)[0, 0]
            o = out[0, node, h]
            z = (v0[0] - o2) / (o2 - o)
            np.testing.assert_allclose(np.log(z), lse[0, node, h], rtol=0, atol=1e-9)


def test_selected_rows_match_full_output():
    parent = workloads.TREE6[None, :].repeat(2, axis=0)
    a, mask = _case(parent, [9, 4], 4, 4, 8, seed=41)
    out, lse = attention.tree_attention(a.q, a.k_cache, a.v_cache, a.ctx_len, mask, a.scale)
    rows = [(0, 3), (1, 6), (1, 0)]
    o2, l2 = attention.tree_attention(a.q, a.k_cache, a.v_cache, a.ctx_len, mask, a.scale, rows=rows)
    for b, i in rows:
        np.testing.assert_array_equal(o2[b, i], out[b, i])
        np.testing.assert_array_equal(l2[b, i], lse[b, i])


def test_short_context_parity_inputs_see_every_mask_bit():
    """The GPU parity cases with contexts of 0, 1 and 63 keys (the configurations' head layouts and
    trees) are built so that a wrong mask bit cannot hide under the 2e-2 bf16 tolerance: flipping
    any one bit (i, j), j < i, of a row moves that row of the oracle's output by more than twice
    the tolerance.  Checked on a seeded sample of 24 flips per sequence."""
    import workloads
    rng = np.random.default_rng(0)
    for shape in sorted(workloads.MASK_SENSITIVE_SHAPES):
        a = workloads.mask_sensitive_attention(shape)
        om, _, _ = tree.build_tree_mask_batch(a.parent)
        k64, v64 = a.k_cache.astype(np.float64), a.v_cache.astype(np.float64)
        B, n1 = a.parent.shape
        for b in range(B):
            for _ in range(24):
                i = int(rng.integers(1, n1))
                j = int(rng.integers(0, i))
                m = om.copy()
                m[b, i, j // 32] ^= np.uint32(1 << (j % 32))
                ref, _ = attention.tree_attention(a.q, k64, v64, a.ctx_len, om, a.scale, rows=[(b, i)])
                mut, _ = attention.tree_attention(a.q, k64, v64, a.ctx_len, m, a.scale, rows=[(b, i)])
                moved = np.abs(mut[b, i] - ref[b, i]).max()
                assert moved > 4e-2, (shape, int(a.ctx_len[b]), i, j, moved)
