"""Tree attention mask and node depth from a parent array.  Test infrastructure.

[SD-EAGLE] "Tree Attention Verification": the verify pass uses a causal mask
that encodes the tree topology -- every token attends only to its ancestors in
the tree -- so all draft nodes are verified in one forward pass.  [PTD]
Method 1, "Attention Masking", restructures the input and mask the same way.
Reading used here: "causal" includes the node itself, so bit (i, j) is set iff
j is i or an ancestor of i; a chain then gives the lower-triangular mask.

Parent array convention: node 0 is the root (the last committed token),
parent[0] = -1, and 0 <= parent[i] < i for i >= 1 (topological order).
"""

import numpy as np


def validate_parent(parent):
    """0 if the parent array is valid, else (index of the first bad entry) + 1."""
    parent = [int(x) for x in parent]
    if len(parent) == 0:
        return 1
    if parent[0] != -1:
        return 1
    for i in range(1, len(parent)):
        if not (0 <= parent[i] < i):
            return i + 1
    return 0


def ancestors_or_self(parent, i):
    """Node i followed by its ancestors up to the root (parent array must be valid)."""
    out = [i]
    while parent[out[-1]] >= 0:
        out.append(int(parent[out[-1]]))
    return out


def build_tree_mask(parent):
    """Return (mask, depth, status) for one sequence.

    mask[i][w]: bit (j % 32) of word w = j // 32 is set iff j is i or one of its
    ancestors; depth[i] = number of ancestors of i; status = validate_parent.
    An invalid parent array gives an all-zero mask and depth -1 everywhere.
    """
    parent = [int(x) for x in parent]
    n1 = len(parent)
    words = (n1 + 31) // 32
    mask = np.zeros((n1, words), dtype=np.uint32)
    depth = np.full(n1, -1, dtype=np.int32)
    status = validate_parent(parent)
    if status != 0:
        return mask, depth, status
    for i in range(n1):
        chain = ancestors_or_self(parent, i)
        depth[i] = len(chain) - 1
        for j in chain:
            mask[i, j // 32] |= np.uint32(1 << (j % 32))
    return mask, depth, status


def mask_bit(mask, i, j):
    return bool((int(mask[i, j // 32]) >> (j % 32)) & 1)


def build_tree_mask_batch(parent):
    """parent[B][N1] -> mask[B][N1][W], depth[B][N1], status[B]."""
    parent = np.asarray(parent)
    B, n1 = parent.shape
    words = (n1 + 31) // 32
    mask = np.zeros((B, n1, words), dtype=np.uint32)
    depth = np.zeros((B, n1), dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        mask[b], depth[b], status[b] = build_tree_mask(parent[b])
    return mask, depth, status
