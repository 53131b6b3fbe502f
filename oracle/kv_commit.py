"""KV-cache commit after a verify step.  Test infrastructure.

[SD-review] §4 (limitations): the KV-cache entries written for rejected draft
tokens have to be rolled back.  [SD-EAGLE] "Tree Attention Verification": the
verify pass costs a few extra KV-cache entries, one per tree node.

Readings used (the pages name the rollback but do not spell it out):
  * the verify pass wrote node j's K/V at cache position ctx_len + j (the same
    layout oracle.attention reads), node 0 being the root, i.e. the last
    committed token;
  * the accept rule returns the accepted nodes n_1, ..., n_a, one per depth;
    the committed sequence is then the context, the root and that path, so
    the entry of n_d belongs at position ctx_len + d and the new context
    length is ctx_len + 1 + a;
  * entries at and after the new length are free (the next verify pass writes
    its tree there); they are not part of the result;
  * a sequence whose inputs do not describe such a path (a < 0, which the
    accept rule uses for invalid trees, a path that is not increasing or has a
    node shallower than its depth allows, or a context that does not fit the
    tree) is left as it was and reported with new length -1.

Layouts: k_cache / v_cache[B][Hkv][Lmax][D], ctx_len[B], accept_len[B],
out_nodes[B][N1].
"""

import numpy as np


def commit_sequence(k_b, v_b, L, a, nodes, n1):
    """One sequence: returns (k, v, new_len) with the committed rows moved.

    k_b, v_b are [Hkv][Lmax][D]; the result is a new array, the input is not
    modified.  Every destination reads the cache as the verify pass left it.
    """
    Lmax = k_b.shape[1]
    ok = 0 <= a <= n1 - 1 and L >= 0 and L + n1 <= Lmax
    if ok:
        path = [int(x) for x in nodes[:a]]
        for d, nd in enumerate(path, start=1):
            if not (d <= nd < n1):
                ok = False
            if d > 1 and path[d - 2] >= nd:
                ok = False
    if not ok:
        return k_b.copy(), v_b.copy(), -1
    k_new, v_new = k_b.copy(), v_b.copy()
    for d, nd in enumerate(path, start=1):
        k_new[:, L + d, :] = k_b[:, L + nd, :]
        v_new[:, L + d, :] = v_b[:, L + nd, :]
    return k_new, v_new, L + 1 + a


def commit(k_cache, v_cache, ctx_len, accept_len, out_nodes):
    """Batch: returns (k_cache, v_cache, new_ctx_len) as new arrays."""
    B, n1 = np.asarray(out_nodes).shape
    k_out, v_out = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    new_len = np.empty(B, dtype=np.int64)
    for b in range(B):
        k_out[b], v_out[b], new_len[b] = commit_sequence(
            np.asarray(k_cache[b]), np.asarray(v_cache[b]), int(ctx_len[b]), int(accept_len[b]),
            out_nodes[b], n1)
    return k_out, v_out, new_len
