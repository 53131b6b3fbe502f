"""Pins for oracle.tree_expand (CPU, float64).

* Without pruning, L levels of top-3 expansion from the root give the complete 3-ary tree of
  depth L ([SD-EAGLE] exercise 4: the top 3 branches at every depth): (3^(L+1) - 1) / 2 nodes,
  children ordered by decreasing logit with no larger logit left out, and every node's score equal
  to the log of the product of the draft probabilities along its path (scipy's softmax, a product
  of probabilities rather than a sum of log-probabilities).
* With pruning, the survivors are exactly the `keep` best candidates (brute force over all of them),
  appended in frontier / rank order; the node capacity caps the count.
* Ties: equal logits -> lower token id; equal scores -> earlier frontier row.
* Frontier entries that are not nodes are ignored; child scores never exceed the parent's.
"""

import math

import numpy as np
from scipy.special import softmax

from oracle import tree_expand


def _rows(seed, V):
    """Draft logits as a function of the node id (a stand-in for the draft model)."""
    cache = {}

    def row(node):
        if node not in cache:
            cache[node] = np.random.default_rng(seed * 1000 + node).normal(0, 2.0, V)
        return cache[node]
    return row


def _tree(B, nmax, root_tokens):
    parent = np.full((B, nmax), -1, dtype=np.int64)
    tokens = np.full((B, nmax), -1, dtype=np.int64)
    score = np.zeros((B, nmax))
    tokens[:, 0] = root_tokens
    return parent, tokens, score, np.ones(B, dtype=np.int64)


def _grow(rows_b, frontier, k, T, keep, state):
    parent, tokens, score, n = state
    B, F = len(rows_b), max(len(f) for f in frontier)
    V = len(rows_b[0](0))
    logits = np.zeros((B, F, V))
    fr = np.full((B, F), -1, dtype=np.int64)
    for b in range(B):
        for i, u in enumerate(frontier[b]):
            fr[b, i] = u
            logits[b, i] = rows_b[b](u)
    out = tree_expand.expand(logits, fr, k, T, keep, parent, tokens, score, n)
    return out[:4], [list(x[x >= 0]) for x in out[4]], out[5]


def test_full_expansion_is_the_complete_top3_tree():
    V, T, L = 12, 0.8, 3
    rows = [_rows(1, V), _rows(2, V)]
    state = _tree(2, 64, [5, 7])
    frontier = [[0], [0]]
    for level in range(L):
        state, frontier, _ = _grow(rows, frontier, 3, T, 3 ** (level + 1), state)
    parent, tokens, score, n = state
    assert list(n) == [(3 ** (L + 1) - 1) // 2] * 2
    for b in range(2):
        for u in range(n[b]):
            kids = [c for c in range(n[b]) if parent[b, c] == u]
            if not kids:
                continue
            z = rows[b](u)
            kt = [int(tokens[b, c]) for c in kids]
            assert len(kids) == 3 and kids == sorted(kids)
            assert all(z[kt[i]] >= z[kt[i + 1]] for i in range(2))          # decreasing logit
            assert (z > z[kt[-1]]).sum() <= 2                                # nothing larger left out
            for c in kids:
                # score: log of the product of draft probabilities along the path
                prod, v = 1.0, c
                while parent[b, v] >= 0:
                    prod *= softmax(rows[b](int(parent[b, v])) / T)[int(tokens[b, v])]
                    v = int(parent[b, v])
                assert abs(score[b, c] - math.log(prod)) < 1e-12
                assert score[b, c] <= score[b, u]


def test_pruning_keeps_exactly_the_best_candidates():
    V, T, k = 20, 1.0, 4
    rng = np.random.default_rng(3)
    for trial in range(20):
        F = int(rng.integers(1, 7))
        nmax = 64
        parent, tokens, score, n = _tree(1, nmax, [0])
        # an existing tree of F nodes with arbitrary scores, all on the frontier
        n[0] = F + 1
        parent[0, 1:F + 1] = 0
        tokens[0, 1:F + 1] = rng.integers(0, V, F)
        score[0, 1:F + 1] = -rng.exponential(2.0, F)
        fr = np.arange(1, F + 1)[None, :]
        logits = rng.normal(0, 2, (1, F, V))
        keep = int(rng.integers(1, F * k + 2))
        p2, t2, s2, n2, nf, margin = tree_expand.expand(logits, fr, k, T, keep, parent, tokens, score, n)
        # brute force over every candidate: the survivors are the `keep` best
        cands = []
        for f in range(F):
            lq = logits[0, f] / T - np.log(np.exp(logits[0, f] / T).sum())
            for j, x in enumerate(np.argsort(-logits[0, f], kind="stable")[:k]):
                cands.append((score[0, f + 1] + lq[x], f, j, int(x)))
        m = min(keep, len(cands))
        best = sorted(cands, key=lambda c: (-c[0], c[1], c[2]))[:m]
        assert n2[0] == F + 1 + m
        kept = sorted(best, key=lambda c: (c[1], c[2]))
        for i, c in enumerate(kept):
            node = F + 1 + i
            assert parent[0, node] == -1 and p2[0, node] == c[1] + 1 and t2[0, node] == c[3]
            assert abs(s2[0, node] - c[0]) < 1e-12
        assert list(nf[0, :m]) == list(range(F + 1, F + 1 + m))
        dropped = [c[0] for c in cands if c not in best]
        if dropped:
            assert min(c[0] for c in best) >= max(dropped)
            assert abs(margin[0] - (min(c[0] for c in best) - max(dropped))) < 1e-12


def test_capacity_and_ignored_frontier_entries():
    V, T = 10, 1.0
    parent, tokens, score, n = _tree(1, 5, [0])
    n[0] = 2
    parent[0, 1] = 0
    logits = np.random.default_rng(4).normal(0, 1, (1, 3, V))
    fr = np.array([[1, -1, 7]])                          # -1 and a node id past the count: no rows
    p2, t2, s2, n2, nf, _ = tree_expand.expand(logits, fr, 3, T, 3, parent, tokens, score, n)
    assert n2[0] == 5                                    # capacity 5: three children of node 1
    assert list(p2[0, 2:5]) == [1, 1, 1]
    assert list(t2[0, 2:5]) == list(np.argsort(-logits[0, 0], kind="stable")[:3])
    p3, t3, s3, n3, nf3, _ = tree_expand.expand(logits, fr, 3, T, 3, p2, t2, s2, n2)
    assert n3[0] == 5 and list(nf3[0]) == [-1, -1, -1]   # full: nothing appended


def test_ties_go_to_lower_token_and_earlier_row():
    V, T = 6, 1.0
    parent, tokens, score, n = _tree(1, 16, [0])
    n[0] = 3
    parent[0, 1:3] = 0
    z = np.array([0.0, 2.0, 2.0, 1.0, 2.0, -1.0])
    logits = np.stack([z, z])[None]                      # two rows with equal scores everywhere
    p2, t2, s2, n2, nf, margin = tree_expand.expand(logits, np.array([[1, 2]]), 2, T, 3, parent, tokens,
                                                    score, n)
    # top-2 of each row: tokens 1, 2 (lowest ids among the three 2.0s); kept: row 0 both, row 1 first
    assert list(p2[0, 3:6]) == [1, 1, 2] and list(t2[0, 3:6]) == [1, 2, 1]
    assert margin[0] == 0.0
    # k larger than V proposes every token once
    p4, t4, _, n4, _, _ = tree_expand.expand(logits[:, :1], np.array([[1]]), 9, T, 9, parent, tokens, score, n)
    assert n4[0] == 3 + V and sorted(t4[0, 3:3 + V]) == list(range(V))
