"""Tree-masked attention of the draft nodes over a KV cache.  Test infrastructure.

[SD-EAGLE] "Tree Attention Verification": all tree nodes are verified in one
forward pass of the target; each node attends only to its ancestors through a
causal mask that encodes the tree, at the price of a few extra KV-cache
entries.  [PTD] Method 4, "Verification", verifies every node of the candidate
tree in one pass with the same attention mask.  [SD-review] §2 step 2: the
target sees the original context plus the drafted tokens at once.

Readings used (the pages are silent on these):
  * the committed context is fully visible to every node;
  * the tree's own K/V entries sit right after the context, node j at cache
    position ctx_len + j, and are visible to node i iff mask bit (i, j) is set
    (the mask comes from oracle.tree: ancestors and the node itself);
  * scores are scale * (q . k) with scale = 1/sqrt(D) unless given;
  * grouped-query attention maps query head h to KV head h // (Hq / Hkv).

Layouts: q[B][N1][Hq][D], k_cache / v_cache[B][Hkv][Lmax][D], ctx_len[B],
mask[B][N1][W].  Returns out[B][N1][Hq][D] and lse[B][N1][Hq] (natural-log
sum of exp of the visible scaled scores), both float64.
"""

import math

import numpy as np

from .tree import mask_bit


def visible_tree_nodes(mask_b, i, n1):
    """Tree nodes j whose K/V entry node i may attend to."""
    return [j for j in range(n1) if mask_bit(mask_b, i, j)]


def _attend(qs, k_ctx, v_ctx, k_tree, v_tree, scale):
    """Softmax attention of the query rows qs[G][D] over the given keys.

    Keys are the context block followed by the visible tree entries; the
    scores are plain dot products, the softmax is taken over all of them.
    """
    s = scale * np.concatenate([qs @ k_ctx.T, qs @ k_tree.T], axis=1)   # [G][n_keys]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    vals = np.concatenate([v_ctx, v_tree], axis=0)                       # [n_keys][D]
    out = (e / z) @ vals
    lse = (m + np.log(z))[:, 0]
    return out, lse


def tree_attention(q, k_cache, v_cache, ctx_len, mask, scale=None, rows=None):
    """Full output, or only the (b, i) pairs listed in `rows` (others stay 0)."""
    q = np.asarray(q, dtype=np.float64)
    B, n1, hq, d = q.shape
    hkv = k_cache.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, n1, hq, d), dtype=np.float64)
    lse = np.zeros((B, n1, hq), dtype=np.float64)
    if rows is None:
        rows = [(b, i) for b in range(B) for i in range(n1)]
    for b, i in rows:
        L = int(ctx_len[b])
        tree_pos = [L + j for j in visible_tree_nodes(mask[b], i, n1)]
        for kv in range(hkv):
            k_ctx = np.asarray(k_cache[b, kv, :L, :], dtype=np.float64)
            v_ctx = np.asarray(v_cache[b, kv, :L, :], dtype=np.float64)
            k_tree = np.asarray(k_cache[b, kv, tree_pos, :], dtype=np.float64)
            v_tree = np.asarray(v_cache[b, kv, tree_pos, :], dtype=np.float64)
            heads = slice(kv * group, (kv + 1) * group)
            o, l = _attend(q[b, i, heads, :], k_ctx, v_ctx, k_tree, v_tree, scale)
            out[b, i, heads, :] = o
            lse[b, i, heads] = l
    return out, lse
