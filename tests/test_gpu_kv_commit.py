"""GPU parity of specv_kv_commit against oracle.kv_commit (through the C ABI).

The committed cache prefix [0, new_ctx_len) and new_ctx_len are compared bit-exactly (the call
only moves rows); a sequence reported invalid (-1) must have its whole cache untouched.  Rows at
and after the new length are unspecified and not compared.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_common import dev, log, run_accept_gpu
from oracle import kv_commit as o_commit
from oracle import tree as o_tree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _specv():
    import draft_verify_sampling_specv_amd as specv
    return specv


def _ladder(m):
    parent = [-1, 0, 0]
    for k in range(1, m):
        parent += [2 * k - 1, 2 * k - 1]
    return np.asarray(parent, dtype=np.int32)


def _caches(rng, B, Hkv, Lmax, D, dtype):
    kc = rng.normal(size=(B, Hkv, Lmax, D)).astype(np.float32)
    vc = rng.normal(size=(B, Hkv, Lmax, D)).astype(np.float32)
    if dtype == "bf16":
        kc, vc = workloads.round_bf16(kc), workloads.round_bf16(vc)
    return kc, vc


def _run_and_compare(kc, vc, ctx, acc, nodes, dtype, name):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kg, vg = dev(kc, dt), dev(vc, dt)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    new = _specv().kv_commit(kg, vg, i32(ctx), i32(acc), i32(nodes))
    torch.cuda.synchronize()
    k_out, v_out = kg.float().cpu().numpy(), vg.float().cpu().numpy()
    new = new.cpu().numpy()
    ok, ov, onew = o_commit.commit(kc, vc, ctx, acc, nodes)
    assert list(new) == list(onew), f"[{name}] new_ctx_len {list(new)} vs {list(onew)}"
    for b in range(len(ctx)):
        n = int(onew[b])
        if n < 0:
            assert np.array_equal(k_out[b], kc[b]) and np.array_equal(v_out[b], vc[b]), f"[{name}] b={b} touched"
        else:
            assert np.array_equal(k_out[b, :, :n], ok[b, :, :n]), f"[{name}] b={b} K prefix differs"
            assert np.array_equal(v_out[b, :, :n], ov[b, :, :n]), f"[{name}] b={b} V prefix differs"
    moved = sum(int(sum(1 for d in range(1, a + 1) if nodes[b][d - 1] != d)) for b, a in enumerate(acc)
                if onew[b] >= 0)
    log(f"[{name}] sequences {len(ctx)}, invalid {int((onew < 0).sum())}, rows moved {moved}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_kv_commit_random_paths(dtype, D):
    rng = np.random.default_rng(7 + D + (1 if dtype == "f32" else 0))
    for n1, Hkv in ((6, 2), (61, 8), (65, 4), (130, 2)):
        B = 8
        parent = np.stack([workloads.random_tree(rng, n1 - 1, 4, 10) for _ in range(B)])
        ctx = rng.integers(0, 40, size=B)
        Lmax = int(ctx.max()) + n1 + 3
        kc, vc = _caches(rng, B, Hkv, Lmax, D, dtype)
        acc = np.zeros(B, dtype=np.int32)
        nodes = np.full((B, n1), -1, dtype=np.int32)
        for b in range(B):
            v = int(rng.integers(0, n1))
            path = o_tree.ancestors_or_self(parent[b], v)[::-1][1:]
            acc[b] = len(path)
            nodes[b, :len(path)] = path
        # invalid sequences: a failed accept, a non-increasing path, a context without room
        acc[1] = -1
        if acc[2] >= 2:
            nodes[2, 1] = nodes[2, 0]
        ctx[3] = Lmax - n1 + 1
        log(f"kv_commit: N1={n1} Hkv={Hkv} D={D} {dtype} paths {list(acc)}")
        _run_and_compare(kc, vc, ctx, acc, nodes, dtype, f"random N1={n1}")


def test_kv_commit_long_path_spans_chunks():
    rng = np.random.default_rng(11)
    parent = _ladder(150)                       # deepest path 1, 3, ..., 299: 150 rows, three chunks
    n1 = len(parent)
    B, Hkv, D = 2, 2, 128
    ctx = np.asarray([17, 0])
    Lmax = 17 + n1
    kc, vc = _caches(rng, B, Hkv, Lmax, D, "bf16")
    nodes = np.full((B, n1), -1, dtype=np.int32)
    nodes[:, :150] = np.arange(1, 300, 2)
    _run_and_compare(kc, vc, ctx, np.asarray([150, 97]), nodes, "bf16", "ladder")


def test_kv_commit_after_gpu_accept_on_eagle_trees():
    w = workloads.eagle_config()
    r = run_accept_gpu(w)
    B, n1 = w.parent.shape
    rng = np.random.default_rng(5)
    ctx = rng.integers(100, 300, size=B)
    Lmax = 300 + n1
    kc, vc = _caches(rng, B, 8, Lmax, 128, "bf16")
    _run_and_compare(kc, vc, ctx, r["accept_len"], r["out_nodes"], "bf16", "eagle accept")
