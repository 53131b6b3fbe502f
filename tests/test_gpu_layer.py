"""GPU parity of specv_verify_layer against oracle.layer (through the C ABI).

Tolerance: |gpu - oracle| <= 2e-2 (1 + |oracle|) for outputs and for the cache rows the layer
writes.  The GPU stores every activation in bf16 between the steps (unit roundoff 2^-9 relative)
and rounds the output itself to bf16; replaying those roundings on the CPU against the float64
oracle gives at most 1e-2 (1 + |out|) on these workloads, so the bound leaves a factor of two.
Every other cache row must be untouched (bit-exact); a sequence without room in its cache or
with an invalid tree must give NaN and leave its cache alone.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from gpu_common import log
from oracle import layer as o_layer

pytestmark = pytest.mark.gpu

REL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _specv():
    import draft_verify_sampling_specv_amd as specv
    return specv


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)


def _run_gpu(li, parent=None):
    specv = _specv()
    parent = li.parent if parent is None else parent
    w = specv.LayerWeights(_bf(li.w_qkv), _bf(li.w_o), _bf(li.w_gate_up), _bf(li.w_down), _bf(li.attn_norm),
                           _bf(li.mlp_norm))
    kc, vc = _bf(li.k_cache), _bf(li.v_cache)
    mask, depth, _ = specv.build_tree_mask(torch.from_numpy(parent).cuda())
    out = specv.verify_layer(_bf(li.x), w, kc, vc, torch.from_numpy(li.ctx_len).cuda(), mask, depth, li.Hq)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), kc.float().cpu().numpy(), vc.float().cpu().numpy()


def _oracle(li, rows=None):
    w = o_layer.LayerWeights(li.w_qkv, li.w_o, li.w_gate_up, li.w_down, li.attn_norm, li.mlp_norm)
    return o_layer.verify_layer(li.x, w, li.k_cache, li.v_cache, li.ctx_len, li.parent, li.Hq, li.Hkv, rows=rows)


def _compare(li, gpu, ora, name, rows=None):
    out, kc, vc = gpu
    o_out, o_kc, o_vc = ora
    B, n1, _ = li.x.shape
    lmax = li.k_cache.shape[2]
    rows = rows or [(b, i) for b in range(B) for i in range(n1)]
    worst = 0.0
    for b, i in rows:
        ref = o_out[b, i]
        if np.isnan(ref).all():
            assert np.isnan(out[b, i]).all(), f"[{name}] ({b},{i}) should be NaN"
            continue
        err = np.abs(out[b, i] - ref) / (1.0 + np.abs(ref))
        worst = max(worst, float(err.max()))
        assert err.max() <= REL, f"[{name}] ({b},{i}) error {err.max():.4f}"
    for b in range(B):
        L = int(li.ctx_len[b])
        if 0 <= L and L + n1 <= lmax and not np.isnan(o_out[b]).all():
            for got, ref, src in ((kc, o_kc, li.k_cache), (vc, o_vc, li.v_cache)):
                err = np.abs(got[b, :, L:L + n1] - ref[b, :, L:L + n1]) / (1.0 + np.abs(ref[b, :, L:L + n1]))
                assert err.max() <= REL, f"[{name}] b={b} cache rows error {err.max():.4f}"
                assert np.array_equal(got[b, :, :L], src[b, :, :L]) and np.array_equal(got[b, :, L + n1:],
                                                                                        src[b, :, L + n1:])
        else:
            assert np.array_equal(kc[b], li.k_cache[b]) and np.array_equal(vc[b], li.v_cache[b]), \
                f"[{name}] b={b} cache touched"
    log(f"[{name}] rows {len(rows)}, worst error / (1 + |ref|) {worst:.4f}")


@pytest.mark.parametrize("shape", [
    # (B, n1, Hq, Hkv, D, inter, ctx): trees on the one-kernel attention path, ragged weight tiles
    # (N = 320 / 192 rows), a contraction of 3 steps, several activation launches (T = 280)
    (3, 7, 4, 2, 64, 384, 100),
    (3, 7, 3, 1, 64, 320, 90),
    (2, 13, 4, 2, 128, 256, 70),
    (40, 7, 4, 2, 64, 128, 40),
    # a tree on the MFMA tree-attention path (G n1 = 80 rows per KV head), with D = 128 and 64
    (2, 40, 4, 2, 128, 192, 150),
    (2, 37, 4, 2, 64, 128, 120),
    # the root alone (K = 0), and plain multi-head attention (Hq = Hkv)
    (5, 1, 4, 2, 64, 128, 30),
    (3, 9, 4, 4, 64, 192, 50),
])
def test_layer_random_trees(shape):
    B, n1, Hq, Hkv, D, inter, ctx = shape
    rng = np.random.default_rng(hash(shape) % 2**32)
    parent = np.stack([workloads.random_tree(rng, n1 - 1, 3, 6) for _ in range(B)]).reshape(B, n1)
    parent[0] = np.arange(-1, n1 - 1)                     # one chain
    ctxs = rng.integers(ctx // 2, ctx + 1, size=B)
    li = workloads.make_layer("layer", parent, ctxs, Hq, Hkv, D, inter, seed_base=int(rng.integers(1 << 30)),
                              extra_slack=3)
    log(f"verify_layer: B={B} N1={n1} Hq={Hq} Hkv={Hkv} D={D} inter={inter}")
    _compare(li, _run_gpu(li), _oracle(li), f"B={B} N1={n1} D={D}")


def test_layer_invalid_sequences():
    rng = np.random.default_rng(9)
    B, n1 = 5, 6
    parent = np.tile(np.arange(-1, n1 - 1), (B, 1)).astype(np.int32)
    parent[2, 4] = 4                                     # not a tree
    li = workloads.make_layer("layer-invalid", parent, [30, 40, 35, 20, 25], 4, 2, 64, 128, seed_base=77)
    lmax = li.k_cache.shape[2]
    li.ctx_len[1] = lmax - n1 + 1                        # no room for the nodes
    li.ctx_len[3] = -1
    li.ctx_len[4] = 2**31 - 2                            # ctx_len + K + 1 past the 32-bit range
    log("verify_layer: invalid sequences 1 (no room), 2 (bad tree), 3 (ctx -1), 4 (ctx 2^31 - 2)")
    _compare(li, _run_gpu(li), _oracle(li), "invalid")


def test_layer_chain_workload_sampled_rows():
    # the full chain workload (32 sequences x 6 nodes, hidden 4096, MLP 14336, context 2048); the
    # oracle computes q/k/v and the cache for every row and the rest for 24 sampled rows
    li = workloads.chain_layer()
    B, n1, _ = li.x.shape
    rng = np.random.default_rng(3)
    rows = sorted({(int(b), int(i)) for b, i in zip(rng.integers(0, B, 24), rng.integers(0, n1, 24))} |
                  {(0, 0), (B - 1, n1 - 1)})
    log(f"verify_layer: chain workload B={B} N1={n1} hidden 4096 inter 14336, {len(rows)} sampled rows")
    gpu = _run_gpu(li)
    _compare(li, gpu, _oracle(li, rows=rows), "chain layer", rows=rows)


def test_layer_output_may_overwrite_its_input():
    # out == x: the input is last read before the final residual product, so the result is the same
    specv = _specv()
    rng = np.random.default_rng(12)
    B, n1 = 3, 7
    parent = np.stack([workloads.random_tree(rng, n1 - 1, 3, 4) for _ in range(B)])
    li = workloads.make_layer("layer-inplace", parent, [40, 50, 60], 4, 2, 64, 192, seed_base=21)
    w = specv.LayerWeights(_bf(li.w_qkv), _bf(li.w_o), _bf(li.w_gate_up), _bf(li.w_down), _bf(li.attn_norm),
                           _bf(li.mlp_norm))
    mask, depth, _ = specv.build_tree_mask(torch.from_numpy(parent).cuda())
    ctx = torch.from_numpy(li.ctx_len).cuda()
    outs = []
    for inplace in (False, True):
        kc, vc = _bf(li.k_cache), _bf(li.v_cache)
        x = _bf(li.x)
        out = specv.verify_layer(x, w, kc, vc, ctx, mask, depth, li.Hq, out=x if inplace else None)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    log("verify_layer: in-place output matches")


def _pack_reference(w):
    """The tile order of specv_pack_weights written out in numpy: 16-byte unit
    ((rb (K/64) + s) 4 + j) 64 + l holds w[32 rb + l % 32][64 s + 32 (l / 32) + 8 j .. + 8]."""
    N, K = w.shape
    out = np.empty((N * K // 8, 8), dtype=w.dtype)
    u = 0
    for rb in range(N // 32):
        for s in range(K // 64):
            for j in range(4):
                for lane in range(64):
                    row, col = 32 * rb + lane % 32, 64 * s + 32 * (lane // 32) + 8 * j
                    out[u] = w[row, col:col + 8]
                    u += 1
    return out.reshape(N, K)


@pytest.mark.parametrize("N,K", [(32, 64), (64, 192), (320, 128)])
def test_pack_weights_tile_order(N, K):
    specv = _specv()
    rng = np.random.default_rng(N * 1000 + K)
    bits = rng.integers(0, 1 << 16, size=(N, K), dtype=np.uint16)       # every bf16 pattern, NaNs included
    w = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    packed = specv.pack_weights(w)
    torch.cuda.synchronize()
    got = packed.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _pack_reference(bits)), f"N={N} K={K}"
    log(f"pack_weights: N={N} K={K} matches the tile order")


@pytest.mark.parametrize("shape", [
    (3, 7, 4, 2, 64, 384, 100),
    (3, 7, 3, 1, 64, 320, 90),           # ragged weight tiles: rows past N clamped in both orders
    (2, 40, 4, 2, 128, 192, 150),
    (40, 7, 4, 2, 64, 128, 40),          # several activation launches
])
def test_packed_layer_is_bit_identical(shape):
    """The same products in the same order: outputs and cache rows equal to the row-major layer's."""
    specv = _specv()
    B, n1, Hq, Hkv, D, inter, ctx = shape
    rng = np.random.default_rng(sum(shape))
    parent = np.stack([workloads.random_tree(rng, n1 - 1, 3, 6) for _ in range(B)]).reshape(B, n1)
    li = workloads.make_layer("layer-packed", parent, rng.integers(ctx // 2, ctx + 1, size=B), Hq, Hkv, D, inter,
                              seed_base=int(rng.integers(1 << 30)), extra_slack=3)
    w = specv.LayerWeights(_bf(li.w_qkv), _bf(li.w_o), _bf(li.w_gate_up), _bf(li.w_down), _bf(li.attn_norm),
                           _bf(li.mlp_norm))
    wp = specv.pack_layer_weights(w)
    assert wp.packed and wp.attn_norm is w.attn_norm
    mask, depth, _ = specv.build_tree_mask(torch.from_numpy(parent).cuda())
    ctxt = torch.from_numpy(li.ctx_len).cuda()
    res = []
    for weights in (w, wp):
        kc, vc = _bf(li.k_cache), _bf(li.v_cache)
        out = specv.verify_layer(_bf(li.x), weights, kc, vc, ctxt, mask, depth, Hq)
        torch.cuda.synchronize()
        res.append([t.view(torch.int16).cpu().numpy() for t in (out, kc, vc)])
    for a, b, what in zip(res[0], res[1], ("out", "k_cache", "v_cache")):
        assert np.array_equal(a, b), f"{shape}: {what} differs between packed and row-major weights"
    log(f"verify_layer packed: B={B} N1={n1} Hq={Hq} Hkv={Hkv} D={D} inter={inter} bit-identical")


def test_packed_layer_chain_workload_bit_identical():
    specv = _specv()
    li = workloads.chain_layer()
    w = specv.LayerWeights(_bf(li.w_qkv), _bf(li.w_o), _bf(li.w_gate_up), _bf(li.w_down), _bf(li.attn_norm),
                           _bf(li.mlp_norm))
    wp = specv.pack_layer_weights(w)
    mask, depth, _ = specv.build_tree_mask(torch.from_numpy(li.parent).cuda())
    ctxt = torch.from_numpy(li.ctx_len).cuda()
    res = []
    for weights in (w, wp):
        kc, vc = _bf(li.k_cache), _bf(li.v_cache)
        out = specv.verify_layer(_bf(li.x), weights, kc, vc, ctxt, mask, depth, li.Hq)
        torch.cuda.synchronize()
        res.append([t.view(torch.int16).cpu().numpy() for t in (out, kc, vc)])
        del kc, vc
    for a, b, what in zip(res[0], res[1], ("out", "k_cache", "v_cache")):
        assert np.array_equal(a, b), f"chain workload: {what} differs between packed and row-major weights"
    log("verify_layer packed: chain workload bit-identical")
