"""Pins for oracle.layer (CPU, float64).

* RMS norm and SiLU equal torch's library routines.
* Rotary encoding equals multiplication of the complex numbers x_j + i x_{j+D/2} by
  exp(i * angle) (torch.polar), is the identity at position 0, and composes: turning by m, then
  by n, is turning by m + n.
* Chain: the layer over a chain equals a plain causal decoder layer written independently with
  torch (rms_norm, linear, scaled_dot_product_attention with an explicit causal mask over the
  context plus the new tokens, silu), including the rotated keys and the values it appends to
  the cache.
* Tree: every node's output equals that plain causal layer run on the node's root-to-node path
  alone, at positions ctx_len .. ctx_len + depth; every node's cache entry equals the key/value of
  the path's last token.
* Invalid sequences get NaN outputs and an untouched cache.
* Planted mistakes (positions by node index instead of depth, a turned sign in the rotation,
  unrotated keys, gate and up swapped, the norm without eps) fail these checks.
"""

import inspect
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import layer, tree

TOL = 1e-10


def _weights(rng, Hq, Hkv, D, inter):
    hd = Hq * D
    g = lambda *s: rng.normal(size=s)
    return layer.LayerWeights(
        w_qkv=g((Hq + 2 * Hkv) * D, hd) / math.sqrt(hd), w_o=g(hd, Hq * D) / math.sqrt(Hq * D),
        w_gate_up=g(2 * inter, hd) / math.sqrt(hd), w_down=g(hd, inter) / math.sqrt(inter),
        attn_norm=1.0 + 0.2 * g(hd), mlp_norm=1.0 + 0.2 * g(hd))


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def _rope_complex(x, pos, theta):
    """x[n][H][D] turned by pos[n] as complex numbers x_j + i x_{j + D/2}."""
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / D)
    ang = pos[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def _plain_layer(x_seq, w, k_ctx, v_ctx, pos0, Hq, Hkv, eps=1e-5, theta=10000.0):
    """A plain causal decoder layer over tokens x_seq[n][Hd] at positions pos0 .. pos0 + n - 1 that
    follow a context with (already rotated) keys / values k_ctx, v_ctx[Hkv][L][D].
    Returns (out[n][Hd], k_new[Hkv][n][D], v_new[Hkv][n][D])."""
    X = _t(x_seq)
    n, hd = X.shape
    D = hd // Hq
    h = F.rms_norm(X, (hd,), weight=_t(w.attn_norm), eps=eps)
    qkv = F.linear(h, _t(w.w_qkv))
    q = qkv[:, :Hq * D].reshape(n, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(n, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(n, Hkv, D)
    pos = pos0 + torch.arange(n, dtype=torch.float64)
    q, k = _rope_complex(q, pos, theta), _rope_complex(k, pos, theta)
    L = k_ctx.shape[1]
    keys = torch.cat([_t(k_ctx), k.transpose(0, 1)], dim=1).repeat_interleave(Hq // Hkv, dim=0)
    vals = torch.cat([_t(v_ctx), v.transpose(0, 1)], dim=1).repeat_interleave(Hq // Hkv, dim=0)
    allowed = torch.ones(n, L + n, dtype=torch.bool)
    allowed[:, L:] = torch.tril(torch.ones(n, n, dtype=torch.bool))
    att = F.scaled_dot_product_attention(q.transpose(0, 1), keys, vals, attn_mask=allowed)   # [Hq][n][D]
    y = X + F.linear(att.transpose(0, 1).reshape(n, Hq * D), _t(w.w_o))
    gu = F.linear(F.rms_norm(y, (hd,), weight=_t(w.mlp_norm), eps=eps), _t(w.w_gate_up))
    inter = w.w_down.shape[1]
    out = y + F.linear(F.silu(gu[:, :inter]) * gu[:, inter:], _t(w.w_down))
    return out.numpy(), k.transpose(0, 1).numpy(), v.transpose(0, 1).numpy()


def _problem(rng, parent, Hq=4, Hkv=2, D=16, inter=96, lmax=40):
    parent = np.asarray(parent)
    B, n1 = parent.shape
    x = rng.normal(size=(B, n1, Hq * D))
    w = _weights(rng, Hq, Hkv, D, inter)
    kc = rng.normal(size=(B, Hkv, lmax, D))
    vc = rng.normal(size=(B, Hkv, lmax, D))
    ctx = rng.integers(0, lmax - n1 + 1, size=B)
    return x, w, kc, vc, ctx


# ----------------------------------------------------------------------------- pieces

def test_rms_norm_and_silu_match_torch():
    rng = np.random.default_rng(1)
    x, g = rng.normal(size=(5, 48)) * 3.0, rng.normal(size=48)
    ref = F.rms_norm(_t(x), (48,), weight=_t(g), eps=1e-5).numpy()
    assert np.abs(layer.rms_norm(x, g, 1e-5) - ref).max() < TOL
    z = rng.normal(size=1000) * 6.0
    assert np.abs(layer.silu(z) - F.silu(_t(z)).numpy()).max() < TOL


def test_rope_is_the_complex_rotation():
    rng = np.random.default_rng(2)
    for D, theta in ((4, 10000.0), (16, 500.0), (128, 10000.0)):
        x = rng.normal(size=(7, 3, D))
        pos = rng.integers(0, 40000, size=7).astype(np.float64)
        ref = _rope_complex(_t(x), _t(pos), theta).numpy()
        assert np.abs(layer.rope(x, pos[:, None], theta) - ref).max() < 1e-9
        assert np.abs(layer.rope(x, np.zeros((7, 1)), theta) - x).max() == 0.0
        two = layer.rope(layer.rope(x, pos[:, None], theta), 3.0 * np.ones((7, 1)), theta)
        assert np.abs(two - layer.rope(x, pos[:, None] + 3.0, theta)).max() < 1e-9


# ----------------------------------------------------------------------------- the layer

def _check_chain(run, seed=3, theta=10000.0):
    rng = np.random.default_rng(seed)
    n1, B, Hq, Hkv = 6, 3, 4, 2
    parent = np.tile(np.arange(-1, n1 - 1), (B, 1))
    x, w, kc, vc, ctx = _problem(rng, parent, Hq=Hq, Hkv=Hkv)
    out, ko, vo = run(x, w, kc, vc, ctx, parent, Hq, Hkv, theta=theta)
    for b in range(B):
        L = int(ctx[b])
        ref, kn, vn = _plain_layer(x[b], w, kc[b, :, :L], vc[b, :, :L], L, Hq, Hkv, theta=theta)
        assert np.abs(out[b] - ref).max() < TOL
        assert np.abs(ko[b, :, L:L + n1] - kn).max() < TOL and np.abs(vo[b, :, L:L + n1] - vn).max() < TOL
        assert np.array_equal(ko[b, :, :L], kc[b, :, :L]) and np.array_equal(ko[b, :, L + n1:], kc[b, :, L + n1:])


def _check_tree(run, seed=4):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv = 2, 4, 2
    parent = np.stack([workloads.random_tree(rng, 9, 3, 4) for _ in range(B)])
    x, w, kc, vc, ctx = _problem(rng, parent, Hq=Hq, Hkv=Hkv)
    out, ko, vo = run(x, w, kc, vc, ctx, parent, Hq, Hkv)
    for b in range(B):
        L = int(ctx[b])
        for i in range(parent.shape[1]):
            path = tree.ancestors_or_self(parent[b], i)[::-1]          # root .. i
            ref, kn, vn = _plain_layer(x[b, path], w, kc[b, :, :L], vc[b, :, :L], L, Hq, Hkv)
            assert np.abs(out[b, i] - ref[-1]).max() < TOL, (b, i)
            assert np.abs(ko[b, :, L + i] - kn[:, -1]).max() < TOL and np.abs(vo[b, :, L + i] - vn[:, -1]).max() < TOL


def test_chain_equals_plain_causal_layer():
    _check_chain(layer.verify_layer)
    _check_chain(layer.verify_layer, seed=5, theta=500.0)


def test_tree_node_equals_plain_layer_on_its_path():
    _check_tree(layer.verify_layer)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(6)
    parent = np.stack([workloads.random_tree(rng, 7, 3, 4) for _ in range(2)])
    x, w, kc, vc, ctx = _problem(rng, parent)
    full, _, _ = layer.verify_layer(x, w, kc, vc, ctx, parent, 4, 2)
    rows = [(0, 3), (1, 0), (1, 7)]
    part, _, _ = layer.verify_layer(x, w, kc, vc, ctx, parent, 4, 2, rows=rows)
    for b, i in rows:
        assert np.abs(part[b, i] - full[b, i]).max() < TOL


def test_invalid_sequences_give_nan_and_keep_the_cache():
    rng = np.random.default_rng(7)
    parent = np.tile(np.arange(-1, 5), (3, 1))
    parent[2, 3] = 3                                    # not a tree
    x, w, kc, vc, ctx = _problem(rng, parent, lmax=20)
    ctx[1] = 20 - 6 + 1                                 # no room for the nodes
    out, ko, vo = layer.verify_layer(x, w, kc, vc, ctx, parent, 4, 2)
    assert np.isfinite(out[0]).all()
    for b in (1, 2):
        assert np.isnan(out[b]).all()
        assert np.array_equal(ko[b], kc[b]) and np.array_equal(vo[b], vc[b])


# ----------------------------------------------------------------------------- planted mistakes

def _mutant(old, new):
    src = inspect.getsource(layer)
    assert old in src
    ns = {"__name__": "oracle._layer_mutant", "__package__": "oracle"}
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["verify_layer"]


@pytest.mark.parametrize("old,new,check", [
    # positions by node index instead of depth: right for chains only
    ("pos = (ctx[:, None] + depth)[..., None]", "pos = (ctx[:, None] + np.arange(n1)[None, :])[..., None]", "tree"),
    # the rotation turned the other way
    ("[a * c - b * s, b * c + a * s]", "[a * c + b * s, b * c - a * s]", "chain"),
    # keys left unrotated
    ("    k = rope(k, pos, theta)\n", "    k = k\n", "chain"),
    # gate and up halves swapped
    ("silu(gu[:, :inter]) * gu[:, inter:]", "silu(gu[:, inter:]) * gu[:, :inter]", "chain"),
    # eps dropped from the norm
    ("np.mean(x * x, axis=-1, keepdims=True) + eps", "np.mean(x * x, axis=-1, keepdims=True)", "chain"),
    # the node's entry written at ctx_len + depth instead of ctx_len + node
    ("kc[b, :, L:L + n1, :] = k[b].transpose(1, 0, 2)",
     "kc[b][:, L + depth[b], :] = k[b].transpose(1, 0, 2)", "tree"),
])
def test_pins_catch_planted_mistakes(old, new, check):
    run = _mutant(old, new)
    with pytest.raises(AssertionError):
        (_check_tree if check == "tree" else _check_chain)(run)
