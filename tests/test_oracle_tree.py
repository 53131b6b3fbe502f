"""Pins for oracle.tree: the six-node tree of the EAGLE lesson, chains, invariants."""

import numpy as np

from conftest import golden_rows
from oracle import tree
import workloads


def test_six_node_tree_from_the_lesson():
    rows = golden_rows("tree6_mask.txt")
    parent = [int(r[1]) for r in rows]
    mask, depth, status = tree.build_tree_mask(parent)
    assert status == 0
    assert mask.shape == (7, 1)
    assert [int(w) for w in mask[:, 0]] == [int(r[2], 16) for r in rows]
    assert list(depth) == [int(r[3]) for r in rows]
    assert parent == list(workloads.TREE6)


def test_chain_is_lower_triangular():
    for n1 in (1, 2, 6, 33, 70):
        parent = [-1] + list(range(n1 - 1))
        mask, depth, status = tree.build_tree_mask(parent)
        assert status == 0
        assert list(depth) == list(range(n1))
        for i in range(n1):
            for j in range(n1):
                assert tree.mask_bit(mask, i, j) == (j <= i)


def test_invariants_on_random_trees():
    rng = np.random.default_rng(3)
    for n1 in (2, 7, 31, 32, 33, 65, 130):
        parent = workloads.random_tree(rng, n1 - 1, 4, 9)
        mask, depth, status = tree.build_tree_mask(parent)
        assert status == 0
        for i in range(1, n1):
            expect = mask[parent[i]].copy()
            expect[i // 32] |= np.uint32(1 << (i % 32))
            assert np.array_equal(mask[i], expect)
            assert depth[i] == depth[parent[i]] + 1
        popcount = np.array([sum(bin(int(w)).count("1") for w in row) for row in mask])
        assert np.array_equal(popcount, depth + 1)


def test_invalid_parent_arrays():
    cases = [
        ([0, 0, 1], 1),          # root must be -1
        ([-1, 0, 2], 3),         # parent[2] == 2 (self / not earlier)
        ([-1, 0, 1, 5], 4),      # forward reference
        ([-1, -1, 0], 2),        # second root
        ([-1, 0, 0, 1, -7], 5),
    ]
    for parent, status in cases:
        mask, depth, st = tree.build_tree_mask(parent)
        assert st == status
        assert not mask.any()
        assert (depth == -1).all()
