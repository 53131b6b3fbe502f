"""One transformer layer of the target model run over the draft nodes.  Test infrastructure.

[SD-EAGLE] "Two-Model Setup" (step 2): the target scores all K + 1 positions
of a step in one parallel forward pass.  [PTD] Method 4, "Verification": every
node of the candidate tree is verified in one forward pass that uses the tree
attention mask and the matching position encoding.  [SD-EAGLE] "Tree Attention
Verification": each node sees only its ancestors and adds one KV-cache entry.

The pages name no architecture.  Readings used:
  * a pre-norm decoder layer of the common open-model shape: RMS norm, a fused
    q/k/v projection, rotary position encoding of q and k, tree-masked
    attention (oracle.attention), an output projection added to the input,
    then RMS norm, a gated SiLU MLP (gate and up projections, silu(gate) * up,
    down projection) added to that;
  * rotary encoding pairs feature j with feature j + D/2 of a head and turns
    the pair by the angle pos * theta^(-2j/D) (theta = 10000 unless given);
  * a node's position is ctx_len + depth(node): the root (the last committed
    token, depth 0) sits at ctx_len and every node one past its parent, so all
    nodes of one depth share a position and a root-to-node path is numbered
    exactly as the same tokens would be in a plain causal forward;
  * the node's K/V entries are written at cache position ctx_len + node index,
    where the attention looks for them;
  * RMS norm: x / sqrt(mean(x^2) + eps) * g, eps = 1e-5 unless given.

Layouts (row-major, weights in the [out][in] layout of a linear map):
x[B][N1][Hd], Hd = Hq * D; w_qkv[(Hq + 2 Hkv) D][Hd] (rows: the Hq query
heads, then the Hkv key heads, then the Hkv value heads); w_o[Hd][Hq D];
w_gate_up[2 I][Hd] (rows: gate, then up); w_down[Hd][I]; norm gains [Hd];
caches [B][Hkv][Lmax][D].  Everything in float64.
"""

import math
from dataclasses import dataclass

import numpy as np

from . import attention, tree


@dataclass
class LayerWeights:
    w_qkv: np.ndarray
    w_o: np.ndarray
    w_gate_up: np.ndarray
    w_down: np.ndarray
    attn_norm: np.ndarray
    mlp_norm: np.ndarray


def rms_norm(x, g, eps=1e-5):
    """x / sqrt(mean over the last axis of x^2 + eps), times the gain g."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, dtype=np.float64)


def rope_angles(pos, D, theta=10000.0):
    """angle[..., j] = pos * theta^(-2j/D) for j < D/2."""
    j = np.arange(D // 2, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * j / D)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x, pos, theta=10000.0):
    """Rotate the pairs (x_j, x_{j + D/2}) of the last axis by rope_angles(pos); pos broadcasts
    against x's leading axes."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    ang = rope_angles(pos, D, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def verify_layer(x, w, k_cache, v_cache, ctx_len, parent, Hq, Hkv, eps=1e-5, theta=10000.0, rows=None):
    """Run the layer over every node of every sequence.

    Returns (out[B][N1][Hd], k_cache', v_cache') with the nodes' rotated keys and values written
    at ctx_len + node.  With `rows` (a list of (b, i)), the attention and everything after it is
    computed for those rows only (the others of `out` are 0); the caches are always complete.
    A sequence whose tree is invalid or whose context leaves no room for its nodes
    (ctx_len < 0 or ctx_len + N1 > Lmax) gets NaN outputs and an untouched cache.
    """
    x = np.asarray(x, dtype=np.float64)
    B, n1, hd = x.shape
    D = hd // Hq
    inter = w.w_down.shape[1]
    lmax = k_cache.shape[2]
    mask, depth, status = tree.build_tree_mask_batch(parent)
    ctx = np.asarray(ctx_len, dtype=np.int64)
    ok = (status == 0) & (ctx >= 0) & (ctx + n1 <= lmax)

    h = rms_norm(x, w.attn_norm, eps)
    qkv = h @ np.asarray(w.w_qkv, dtype=np.float64).T
    q = qkv[..., :Hq * D].reshape(B, n1, Hq, D)
    k = qkv[..., Hq * D:(Hq + Hkv) * D].reshape(B, n1, Hkv, D)
    v = qkv[..., (Hq + Hkv) * D:].reshape(B, n1, Hkv, D)
    pos = (ctx[:, None] + depth)[..., None]                         # [B][N1][1]
    q = rope(q, pos, theta)
    k = rope(k, pos, theta)

    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    for b in range(B):
        if ok[b]:
            L = int(ctx[b])
            kc[b, :, L:L + n1, :] = k[b].transpose(1, 0, 2)
            vc[b, :, L:L + n1, :] = v[b].transpose(1, 0, 2)

    if rows is None:
        rows = [(b, i) for b in range(B) for i in range(n1)]
    good = [(b, i) for b, i in rows if ok[b]]
    att, _ = attention.tree_attention(q, kc, vc, np.where(ok, ctx, 0), mask, 1.0 / math.sqrt(D), rows=good)
    out = np.zeros((B, n1, hd))
    bad = [(b, i) for b, i in rows if not ok[b]]
    for b, i in bad:
        out[b, i] = np.nan
    if good:
        gb, gi = np.array([r[0] for r in good]), np.array([r[1] for r in good])
        a = att[gb, gi].reshape(len(good), Hq * D)
        y = x[gb, gi] + a @ np.asarray(w.w_o, dtype=np.float64).T
        gu = rms_norm(y, w.mlp_norm, eps) @ np.asarray(w.w_gate_up, dtype=np.float64).T
        out[gb, gi] = y + (silu(gu[:, :inter]) * gu[:, inter:]) @ np.asarray(w.w_down, dtype=np.float64).T
    return out, kc, vc
