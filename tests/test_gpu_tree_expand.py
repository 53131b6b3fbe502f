"""GPU parity of specv_tree_expand against oracle.tree_expand (through the C ABI).

Tree arrays, node counts and new frontiers are compared exactly, scores within SCORE_ABS (the GPU
combines each row's log-sum-exp in fp64 from fp32 sums).  A sequence whose kept set was within
SCORE_TIE of changing (the oracle's margin at the cut) is a near tie: counted, not compared.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_common import log
from oracle import tree_expand as o_exp
from oracle import tree as o_tree

pytestmark = pytest.mark.gpu

SCORE_ABS = 1e-5       # per level
SCORE_TIE = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _specv():
    import draft_verify_sampling_specv_amd as specv
    return specv


def _gpu_level(logits, frontier, parent, tokens, score, n, k, T, keep, dtype):
    specv = _specv()
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tree = specv.DraftTree(torch.from_numpy(parent.astype(np.int32)).cuda(),
                           torch.from_numpy(tokens.astype(np.int32)).cuda(),
                           torch.from_numpy(score.astype(np.float64)).cuda(),
                           torch.from_numpy(n.astype(np.int32)).cuda())
    nf = specv.tree_expand(torch.from_numpy(logits).cuda().to(dt), torch.from_numpy(frontier.astype(np.int32)).cuda(),
                           tree, k, T, keep)
    torch.cuda.synchronize()
    return (tree.parent.cpu().numpy(), tree.tokens.cpu().numpy(), tree.score.cpu().numpy(),
            tree.n_nodes.cpu().numpy(), nf.cpu().numpy())


def _compare(gpu, ora, levels, name):
    gp, gt, gs, gn, gf = gpu
    op, ot, os_, on, of, margin = ora
    near, checked = 0, 0
    for b in range(len(gn)):
        if margin[b] < SCORE_TIE:
            near += 1
            continue
        checked += 1
        assert gn[b] == on[b], f"[{name}] b={b} n_nodes {gn[b]} vs {on[b]}"
        n = int(on[b])
        assert np.array_equal(gp[b, :n], op[b, :n]), f"[{name}] b={b} parent differs"
        assert np.array_equal(gt[b, :n], ot[b, :n]), f"[{name}] b={b} tokens differ"
        assert np.abs(gs[b, :n] - os_[b, :n]).max() <= SCORE_ABS * levels, f"[{name}] b={b} scores"
        assert np.array_equal(gf[b], of[b]), f"[{name}] b={b} new frontier differs"
    log(f"[{name}] sequences {len(gn)}, compared {checked}, near ties {near}")
    return checked


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tree_expand_random_levels(dtype):
    rng = np.random.default_rng(41 if dtype == "f32" else 42)
    compared = 0
    for case in range(20):
        B = int(rng.integers(1, 9))
        k = int(rng.choice([1, 2, 3, 4, 8, 16]))
        F = int(rng.integers(1, min(64, 1024 // k) + 1))
        V = int(rng.choice([5, 7, 64, 333, 1000, 4097, 32000]))
        T = float(rng.choice([0.5, 1.0, 1.7]))
        keep = int(rng.integers(1, F * k + 1))
        nmax = int(rng.integers(F + 1, F + 1 + 2 * keep))
        # an existing tree: the root plus F nodes under it with arbitrary (negative) scores
        parent = np.full((B, nmax), -1, dtype=np.int64)
        tokens = np.full((B, nmax), -1, dtype=np.int64)
        score = np.zeros((B, nmax))
        parent[:, 1:F + 1] = 0
        tokens[:, :F + 1] = rng.integers(0, V, (B, F + 1))
        score[:, 1:F + 1] = -rng.exponential(2.0, (B, F))
        n = np.full(B, F + 1, dtype=np.int64)
        frontier = np.tile(np.arange(1, F + 1), (B, 1))
        frontier[rng.random((B, F)) < 0.1] = -1                  # no row
        frontier[rng.random((B, F)) < 0.05] = nmax + 3           # not a node
        logits = rng.normal(0, 2.0, (B, F, V)).astype(np.float32)
        if dtype == "bf16":
            logits = workloads.round_bf16(logits)
        log(f"tree_expand case {case}: B={B} F={F} V={V} k={k} T={T} keep={keep} nmax={nmax} {dtype}")
        gpu = _gpu_level(logits, frontier, parent, tokens, score, n, k, T, keep, dtype)
        ora = o_exp.expand(logits.astype(np.float64), frontier, k, T, keep, parent, tokens, score, n)
        compared += _compare(gpu, ora, 1, f"case{case}")
    assert compared > 0


def test_tree_expand_ties():
    # identical rows: equal logits go to the lower token, equal scores to the earlier row
    z = np.array([0.0, 2.0, 2.0, 1.0, 2.0, -1.0], dtype=np.float32)
    logits = np.stack([z, z])[None]
    parent = np.full((1, 16), -1, dtype=np.int64)
    parent[0, 1:3] = 0
    tokens = np.zeros((1, 16), dtype=np.int64)
    score = np.zeros((1, 16))
    gp, gt, gs, gn, gf = _gpu_level(logits, np.array([[1, 2]]), parent, tokens, score, np.array([3]), 2, 1.0, 3,
                                    "f32")
    assert gn[0] == 6 and list(gp[0, 3:6]) == [1, 1, 2] and list(gt[0, 3:6]) == [1, 2, 1]
    assert list(gf[0]) == [3, 4, 5]


def test_tree_expand_builds_an_eagle_tree_level_by_level():
    # from the roots, four levels of top-3 expansion keeping 10 per level, V = 128256 bf16, the
    # draft rows a function of (sequence, node); then the tree is a valid parent array
    B, V, k, keep, T, nmax = 8, 128256, 3, 10, 0.7, 64
    specv = _specv()

    def rows_for(frontier):
        out = np.zeros((B, frontier.shape[1], V), dtype=np.float32)
        for b in range(B):
            for f, u in enumerate(frontier[b]):
                if u >= 0:
                    out[b, f] = np.random.default_rng(1_000_003 * b + int(u)).normal(0, 3.0, V)
        return workloads.round_bf16(out)

    roots = np.arange(B) * 11
    tree = specv.DraftTree.with_roots(torch.from_numpy(roots).cuda(), nmax)
    o_state = [np.full((B, nmax), -1, dtype=np.int64), np.full((B, nmax), -1, dtype=np.int64), np.zeros((B, nmax)),
               np.ones(B, dtype=np.int64)]
    o_state[1][:, 0] = roots
    frontier = np.zeros((B, 1), dtype=np.int64)
    o_frontier = frontier.copy()
    min_margin = np.full(B, np.inf)
    for level in range(4):
        logits = rows_for(frontier)
        nf = specv.tree_expand(torch.from_numpy(logits).cuda().to(torch.bfloat16),
                               torch.from_numpy(frontier.astype(np.int32)).cuda(), tree, k, T, keep)
        torch.cuda.synchronize()
        o_logits = rows_for(o_frontier).astype(np.float64)
        *o_state, o_nf, margin = o_exp.expand(o_logits, o_frontier, k, T, keep, *o_state)
        o_state = list(o_state)
        min_margin = np.minimum(min_margin, margin)
        frontier, o_frontier = nf.cpu().numpy().astype(np.int64), o_nf
    gpu = (tree.parent.cpu().numpy(), tree.tokens.cpu().numpy(), tree.score.cpu().numpy(),
           tree.n_nodes.cpu().numpy(), frontier)
    assert _compare(gpu, (*o_state, o_frontier, min_margin), 4, "eagle levels") > 0
    for b in range(B):
        n = int(gpu[3][b])
        assert n == 1 + 3 + 9 + keep + keep              # 3, then 9 (all), then 10 of 27, 10 of 30
        assert o_tree.validate_parent(gpu[0][b, :n]) == 0
