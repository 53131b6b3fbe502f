"""Seeded synthetic inputs for the verify step (shared by the oracle tests and the GPU path).

This module only draws random numbers and arranges them in the layouts the
library takes; it holds none of the verify arithmetic (no softmax, no ratio
test, no residual).  Draft tokens are drawn from the draft distribution with
the Gumbel-max trick (argmax of logits / T plus Gumbel noise, top-k of the same
for k siblings drawn without replacement), which needs no normalisation.

The pages' workloads are models and datasets that are not available here (T5
on WMT / CNN-DM in the Leviathan et al. review; LLaMA / Qwen on MT-Bench, GSM,
HumanEval, MBPP in the PTD summary).  These synthetic inputs stand in for them
with the vocabulary sizes, draft shapes and acceptance-rate range the pages
quote (alpha 0.6-0.85, [SD-EAGLE] "Draft training: distillation"; 0.75 / 0.82,
[SD-EAGLE] "EAGLE").

Recipes (std-dev readings of N(0, s)):
  tiny   V=1000, chain K=4, fp32 target ~ N(0, 2), draft = target + N(0, 0.5),
         T=1; trials share the logits and differ in draft tokens and uniforms.
         Tree: root->{a,b}, a->{c,d}, b->{e,f}.  Attention: 4 heads (MHA),
         D=64, context 128, fp32 N(0, 1).
  chain  B=32, K=5, V=32000, bf16 target ~ N(0, 3), draft = target + N(0, 0.5285)
         (alpha ~ 0.8 at T=1), T=1 and a T=0 run; attention context 2048,
         Hq/Hkv = 32/8, D=128, bf16 N(0, 1).
  eagle  B=16, top-3 branching to depth 6 pruned to the 60 nodes of highest
         cumulative draft probability (best-first expansion), V=128256 bf16,
         N(0, 3) / draft noise 0.3845 (alpha ~ 0.8 at T=0.7), T=0.7; context 4096,
         64/8 heads.
  stress B=64, K=8, V=151936 fp32, target and draft independent N(0, 3), T=1.5;
         context 1024, 40/8 heads.
  ptd    B=4, 64-node tree grown at random under caps of 4 children and depth 8,
         V=128256 bf16, draft noise 0.6407 (alpha ~ 0.75), T=1; context 32768,
         64/8 heads.
  layer  the chain verify as one target layer: hidden 4096 (32/8 heads of 128),
         MLP width 14336, random-init bf16 weights N(0, 1/fan_in), norm gains
         1 + N(0, 0.2), hidden states N(0, 1); context 2048.
"""

from dataclasses import dataclass, field
import heapq
import math

import numpy as np
from scipy.special import logsumexp


# ----------------------------------------------------------------------------- dtype helpers

def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def as_dtype(x, dtype):
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------- containers

@dataclass
class AcceptInputs:
    name: str
    target_logits: np.ndarray      # [B][N1][V] float32 (bf16-representable if dtype == "bf16")
    draft_logits: np.ndarray       # [B][N1][V] float32, or None for a greedy-only call
    tokens: np.ndarray             # [B][N1] int32; tokens[b][0] is the committed root token
    parent: np.ndarray             # [B][N1] int32
    T: float
    dtype: str                     # "f32" or "bf16"
    seed: int
    offset: int

    @property
    def B(self):
        return self.tokens.shape[0]

    @property
    def N1(self):
        return self.tokens.shape[1]

    @property
    def V(self):
        return self.target_logits.shape[-1]


@dataclass
class AttnInputs:
    name: str
    q: np.ndarray                  # [B][N1][Hq][D] float32
    k_cache: np.ndarray            # [B][Hkv][Lmax][D]
    v_cache: np.ndarray
    ctx_len: np.ndarray            # [B] int32
    parent: np.ndarray             # [B][N1] int32
    dtype: str
    scale: float = field(default=0.0)

    def __post_init__(self):
        if not self.scale:
            self.scale = 1.0 / math.sqrt(self.q.shape[-1])


# ----------------------------------------------------------------------------- trees

def chain_parent(B, K):
    p = np.arange(-1, K, dtype=np.int32)
    return np.tile(p, (B, 1))


TREE6 = np.array([-1, 0, 0, 1, 1, 2, 2], dtype=np.int32)   # root->{a,b}, a->{c,d}, b->{e,f}


def random_tree(rng, n_draft, max_children, max_depth):
    """Grow a tree of n_draft nodes below the root: each new node hangs under a
    uniformly chosen node that still has fewer than max_children children and
    depth < max_depth.  Returns a BFS-numbered parent array of n_draft + 1."""
    parent = [-1]
    depth = [0]
    nkids = [0]
    for _ in range(n_draft):
        open_nodes = [v for v in range(len(parent)) if nkids[v] < max_children and depth[v] < max_depth]
        v = int(open_nodes[rng.integers(len(open_nodes))])
        parent.append(v)
        depth.append(depth[v] + 1)
        nkids.append(0)
        nkids[v] += 1
    return bfs_renumber(parent)


def bfs_renumber(parent):
    """Renumber a tree so that nodes appear level by level, children of an
    earlier node before children of a later one (keeps parent[i] < i)."""
    n = len(parent)
    kids = [[] for _ in range(n)]
    for c in range(1, n):
        kids[parent[c]].append(c)
    order = [0]
    for v in order:
        order.extend(kids[v])
    new_id = {old: i for i, old in enumerate(order)}
    out = np.empty(n, dtype=np.int32)
    for old in order:
        out[new_id[old]] = -1 if old == 0 else new_id[parent[old]]
    return out


def children_lists(parent):
    kids = [[] for _ in range(len(parent))]
    for c in range(1, len(parent)):
        kids[int(parent[c])].append(c)
    return kids


# ----------------------------------------------------------------------------- token draws

def gumbel(rng, shape):
    return -np.log(-np.log(rng.random(shape)))


def draw_children_tokens(rng, draft_row, T, k):
    """k distinct tokens drawn without replacement from softmax(draft_row / T)
    by Gumbel-top-k (at T == 0: the k largest logits)."""
    if T == 0:
        keys = np.asarray(draft_row, dtype=np.float64)
    else:
        keys = np.asarray(draft_row, dtype=np.float64) / T + gumbel(rng, draft_row.shape)
    top = np.argpartition(-keys, k - 1)[:k]
    return top[np.argsort(-keys[top], kind="stable")].astype(np.int32)


def draw_iid_tokens(rng, draft_row, T, k):
    """k tokens drawn independently (with replacement) from softmax(draft_row / T), each by
    Gumbel-max."""
    z = np.asarray(draft_row, dtype=np.float64) / T
    return np.array([int(np.argmax(z + gumbel(rng, z.shape))) for _ in range(k)], dtype=np.int32)


def draw_tree_tokens(rng, parent, draft_logits_b, T, V, siblings="without_replacement"):
    """Tokens for every node: the root token is uniform in [0, V); the children
    of v are drawn from draft row v -- without replacement (Gumbel-top-k),
    independently ("iid"), or as the row's top tokens ("deterministic")."""
    kids = children_lists(parent)
    tok = np.zeros(len(parent), dtype=np.int32)
    tok[0] = rng.integers(V)
    for v, ks in enumerate(kids):
        if ks:
            if siblings == "iid" and T > 0:
                tok[ks] = draw_iid_tokens(rng, draft_logits_b[v], T, len(ks))
            else:
                tok[ks] = draw_children_tokens(rng, draft_logits_b[v], 0 if siblings == "deterministic" else T,
                                               len(ks))
    return tok


# ----------------------------------------------------------------------------- logits

def draft_from_target(rng, target, sigma):
    return target + rng.normal(0.0, sigma, size=target.shape).astype(np.float32)


def make_accept(name, parent, V, T, dtype, target_std, draft_sigma, seed_base,
                independent_draft=False, tokens_T=None, greedy_tokens=False, siblings="without_replacement"):
    """Generic generator: per-node target rows ~ N(0, target_std), draft rows =
    target + N(0, draft_sigma) (or an independent N(0, target_std)), draft
    tokens drawn from the draft rows along the given parent arrays."""
    ss = np.random.SeedSequence(seed_base)
    r_t, r_d, r_tok = [np.random.default_rng(s) for s in ss.spawn(3)]
    B, n1 = parent.shape
    target = r_t.normal(0.0, target_std, size=(B, n1, V)).astype(np.float32)
    if independent_draft:
        draft = r_d.normal(0.0, target_std, size=(B, n1, V)).astype(np.float32)
    else:
        draft = draft_from_target(r_d, target, draft_sigma)
    target = as_dtype(target, dtype)
    draft = as_dtype(draft, dtype)
    tT = T if tokens_T is None else tokens_T
    tokens = np.stack([draw_tree_tokens(r_tok, parent[b], draft[b], 0 if greedy_tokens else tT, V, siblings)
                       for b in range(B)])
    return AcceptInputs(name, target, draft, tokens, np.ascontiguousarray(parent, dtype=np.int32),
                        float(T), dtype, seed=seed_base, offset=0)


def make_attention(name, parent, ctx_len, Hq, Hkv, D, dtype, seed_base, extra_slack=0):
    ss = np.random.SeedSequence(seed_base)
    r_q, r_k, r_v = [np.random.default_rng(s) for s in ss.spawn(3)]
    B, n1 = parent.shape
    ctx_len = np.asarray(ctx_len, dtype=np.int32)
    lmax = int(ctx_len.max()) + n1 + extra_slack
    q = as_dtype(r_q.standard_normal((B, n1, Hq, D), dtype=np.float32), dtype)
    k = as_dtype(r_k.standard_normal((B, Hkv, lmax, D), dtype=np.float32), dtype)
    v = as_dtype(r_v.standard_normal((B, Hkv, lmax, D), dtype=np.float32), dtype)
    return AttnInputs(name, q, k, v, ctx_len, np.ascontiguousarray(parent, dtype=np.int32), dtype)


@dataclass
class LayerInputs:
    name: str
    x: np.ndarray                  # [B][N1][Hq D] float32 (bf16 values)
    w_qkv: np.ndarray              # [(Hq + 2 Hkv) D][Hq D]
    w_o: np.ndarray                # [Hq D][Hq D]
    w_gate_up: np.ndarray          # [2 inter][Hq D]
    w_down: np.ndarray             # [Hq D][inter]
    attn_norm: np.ndarray          # [Hq D]
    mlp_norm: np.ndarray           # [Hq D]
    k_cache: np.ndarray            # [B][Hkv][Lmax][D]
    v_cache: np.ndarray
    ctx_len: np.ndarray            # [B] int32
    parent: np.ndarray             # [B][N1] int32
    Hq: int
    Hkv: int


def make_layer(name, parent, ctx_len, Hq, Hkv, D, inter, seed_base, extra_slack=0):
    """Random-init weights of a pre-norm decoder layer: projections ~ N(0, 1/fan_in), norm gains
    1 + N(0, 0.2); hidden states and cache entries ~ N(0, 1); all rounded to bf16."""
    ss = np.random.SeedSequence(seed_base)
    rs = [np.random.default_rng(s) for s in ss.spawn(9)]
    B, n1 = parent.shape
    hd = Hq * D
    ctx_len = np.asarray(ctx_len, dtype=np.int32)
    lmax = int(ctx_len.max()) + n1 + extra_slack

    def lin(r, rows, cols):
        return round_bf16(r.standard_normal((rows, cols), dtype=np.float32) / np.float32(math.sqrt(cols)))

    return LayerInputs(
        name, round_bf16(rs[0].standard_normal((B, n1, hd), dtype=np.float32)),
        lin(rs[1], (Hq + 2 * Hkv) * D, hd), lin(rs[2], hd, hd), lin(rs[3], 2 * inter, hd), lin(rs[4], hd, inter),
        round_bf16(1 + 0.2 * rs[5].standard_normal(hd, dtype=np.float32)),
        round_bf16(1 + 0.2 * rs[6].standard_normal(hd, dtype=np.float32)),
        round_bf16(rs[7].standard_normal((B, Hkv, lmax, D), dtype=np.float32)),
        round_bf16(rs[8].standard_normal((B, Hkv, lmax, D), dtype=np.float32)),
        ctx_len, np.ascontiguousarray(parent, dtype=np.int32), Hq, Hkv)


# ----------------------------------------------------------------------------- the configurations

SIGMA_CHAIN = 0.5285   # alpha ~ 0.80 at V=32000, N(0,3), T=1 (workloads/tune_sigma.py)
SIGMA_EAGLE = 0.3845   # alpha ~ 0.80 at V=128256, N(0,3), T=0.7
SIGMA_PTD = 0.6407     # alpha ~ 0.75 at V=128256, N(0,3), T=1


def tiny_chain_trials(trials=10_000, seed_base=1000):
    """One sequence's logits (V=1000, K=4) shared by `trials` rows, each with its
    own draft tokens (drawn from q) and its own uniforms (Philox counter b)."""
    ss = np.random.SeedSequence(seed_base)
    r_t, r_d, r_tok = [np.random.default_rng(s) for s in ss.spawn(3)]
    K, V = 4, 1000
    t1 = r_t.normal(0.0, 2.0, size=(K + 1, V)).astype(np.float32)
    d1 = draft_from_target(r_d, t1, 0.5)
    parent = chain_parent(trials, K)
    root = int(r_tok.integers(V))
    keys = d1[None, :K, :].astype(np.float64) + gumbel(r_tok, (trials, K, V))
    tokens = np.empty((trials, K + 1), dtype=np.int32)
    tokens[:, 0] = root
    tokens[:, 1:] = np.argmax(keys, axis=2)
    target = np.broadcast_to(t1, (trials, K + 1, V))
    draft = np.broadcast_to(d1, (trials, K + 1, V))
    return AcceptInputs("tiny-chain", target, draft, tokens, parent, 1.0, "f32", seed=seed_base, offset=0)


def tiny_tree(B=1, seed_base=1001):
    parent = np.tile(TREE6, (B, 1))
    return make_accept("tiny-tree", parent, 1000, 1.0, "f32", 2.0, 0.5, seed_base)


def tiny_tree_attention(seed_base=1002):
    parent = TREE6[None, :]
    return make_attention("tiny-tree-attn", parent, [128], 4, 4, 64, "f32", seed_base)


def chain_config(T=1.0, seed_base=2000):
    parent = chain_parent(32, 5)
    return make_accept("chain", parent, 32000, T, "bf16", 3.0, SIGMA_CHAIN, seed_base,
                       greedy_tokens=(T == 0))


def chain_attention(seed_base=2001, B=32):
    return make_attention("chain-attn", chain_parent(B, 5), [2048] * B, 32, 8, 128, "bf16", seed_base)


def chain_layer(seed_base=2002, B=32, inter=14336):
    """The chain verify as one layer of a 4096-wide model: 32/8 heads of 128 (the attention
    shape above), MLP width 14336 (the common open-model size at that width)."""
    return make_layer("chain-layer", chain_parent(B, 5), [2048] * B, 32, 8, 128, inter, seed_base)


def eagle_tree(rng, draft_rows_fn, T, n_keep=60, branch=3, max_depth=6):
    """Best-first expansion of the top-`branch` draft children (drawn without
    replacement) to depth `max_depth`, keeping the `n_keep` nodes of highest
    cumulative draft log-probability.  Since a child's cumulative probability
    never exceeds its parent's, the kept set is closed under ancestors.
    draft_rows_fn(node_id) returns the draft logit row of a node (rows are
    created on demand).  Returns (parent, tokens) in BFS order with the
    creation ids of the kept nodes."""
    heap = []          # (-cum_logq, creation id)
    nodes = {0: dict(parent=-1, depth=0, tok=None, cum=0.0)}
    kept = [0]
    next_id = 1

    def expand(v):
        nonlocal next_id
        row = draft_rows_fn(v).astype(np.float64)
        kids = draw_children_tokens(rng, row, T, branch)
        logq = row / T - logsumexp(row / T)
        for x in kids:
            nodes[next_id] = dict(parent=v, depth=nodes[v]["depth"] + 1, tok=int(x),
                                  cum=nodes[v]["cum"] + float(logq[x]))
            heapq.heappush(heap, (-nodes[next_id]["cum"], next_id))
            next_id += 1

    expand(0)
    while len(kept) < n_keep + 1 and heap:
        _, v = heapq.heappop(heap)
        kept.append(v)
        if nodes[v]["depth"] < max_depth:
            expand(v)
    kept_set = set(kept)
    # BFS order over the kept nodes (children in creation order)
    kids = {v: [] for v in kept}
    for v in sorted(kept):
        if v != 0 and nodes[v]["parent"] in kept_set:
            kids[nodes[v]["parent"]].append(v)
    order = [0]
    for v in order:
        order.extend(kids[v])
    new_id = {old: i for i, old in enumerate(order)}
    parent = np.array([-1] + [new_id[nodes[v]["parent"]] for v in order[1:]], dtype=np.int32)
    toks = [nodes[v]["tok"] for v in order]
    return parent, toks, order


def eagle_config(seed_base=3000, B=16, V=128256, n_keep=60):
    """Tree config: rows are drawn per created node; only the kept nodes' rows
    are stored."""
    ss = np.random.SeedSequence(seed_base)
    r_t, r_d, r_tok = [np.random.default_rng(s) for s in ss.spawn(3)]
    T = 0.7
    n1 = n_keep + 1
    target = np.empty((B, n1, V), dtype=np.float32)
    draft = np.empty((B, n1, V), dtype=np.float32)
    parent = np.empty((B, n1), dtype=np.int32)
    tokens = np.empty((B, n1), dtype=np.int32)
    for b in range(B):
        rows = {}

        def rows_fn(v):
            if v not in rows:
                t = as_dtype(r_t.normal(0.0, 3.0, size=V).astype(np.float32), "bf16")
                d = as_dtype(draft_from_target(r_d, t, SIGMA_EAGLE), "bf16")
                rows[v] = (t, d)
            return rows[v][1]

        p, toks, order = eagle_tree(r_tok, rows_fn, T, n_keep=n_keep)
        parent[b] = p
        tokens[b] = [int(r_tok.integers(V))] + toks[1:]
        for i, v in enumerate(order):
            rows_fn(v)
            target[b, i], draft[b, i] = rows[v]
    return AcceptInputs("eagle", target, draft, tokens, parent, T, "bf16", seed=seed_base, offset=0)


def eagle_attention(parent, seed_base=3001):
    B = parent.shape[0]
    return make_attention("eagle-attn", parent, [4096] * B, 64, 8, 128, "bf16", seed_base)


def stress_config(seed_base=4000, B=64):
    parent = chain_parent(B, 8)
    return make_accept("stress", parent, 151936, 1.5, "f32", 3.0, 0.0, seed_base, independent_draft=True)


def stress_attention(seed_base=4001, B=64):
    return make_attention("stress-attn", chain_parent(B, 8), [1024] * B, 40, 8, 128, "bf16", seed_base)


def ptd_parent(seed_base=5002, B=4):
    rng = np.random.default_rng(seed_base)
    return np.stack([random_tree(rng, 64, 4, 8) for _ in range(B)])


def ptd_config(seed_base=5000, B=4):
    parent = ptd_parent(B=B)
    return make_accept("ptd", parent, 128256, 1.0, "bf16", 3.0, SIGMA_PTD, seed_base)


def ptd_attention(parent, seed_base=5001):
    B = parent.shape[0]
    return make_attention("ptd-attn", parent, [32768] * B, 64, 8, 128, "bf16", seed_base)


def eagle_shaped_parents(B, seed_base=3200, V=512, T=0.7):
    """Trees of the EAGLE-style configuration's shape (top-3 children drawn without replacement,
    depth 6, the 60 nodes of highest cumulative draft probability kept) grown from cheap random
    draft rows (V = 512, N(0, 3)): for attention cases that need the shape, not the logits."""
    rng = np.random.default_rng(seed_base)
    out = []
    for _ in range(B):
        rows = {}

        def row(v):
            if v not in rows:
                rows[v] = 3.0 * rng.standard_normal(V)
            return rows[v]

        parent, _, _ = eagle_tree(rng, row, T)
        out.append(parent)
    return np.stack(out)


# Head layouts and trees of the four full-size configurations, for attention with very short
# contexts (0, 1 and 63 keys): there the tree's own keys carry much of the softmax weight.
MASK_SENSITIVE_SHAPES = {
    "chain": (32, 8),       # chain K=5
    "eagle": (64, 8),       # EAGLE-style tree, 61 nodes
    "stress": (40, 8),      # chain K=8
    "ptd": (64, 8),         # PTD-style random tree, 65 nodes
}
MASK_SENSITIVE_CONTEXTS = (0, 1, 63)


def mask_sensitive_attention(shape, seed_base=6000):
    hq, hkv = MASK_SENSITIVE_SHAPES[shape]
    B = len(MASK_SENSITIVE_CONTEXTS)
    if shape == "chain":
        parent = chain_parent(B, 5)
    elif shape == "stress":
        parent = chain_parent(B, 8)
    elif shape == "eagle":
        parent = eagle_shaped_parents(B)
    else:
        parent = ptd_parent(B=B)
    return make_attention(f"{shape}-short-ctx", parent, list(MASK_SENSITIVE_CONTEXTS), hq, hkv, 128, "bf16",
                          seed_base + sorted(MASK_SENSITIVE_SHAPES).index(shape))


def random_case(seed, B, n1, V, T, dtype="f32", max_children=3, max_depth=None,
                target_std=2.0, draft_sigma=0.7, siblings="without_replacement"):
    """Small random tree case for parity sweeps."""
    rng = np.random.default_rng(seed)
    md = n1 if max_depth is None else max_depth
    parent = np.stack([random_tree(rng, n1 - 1, max_children, md) for _ in range(B)])
    return make_accept(f"random-{seed}", parent, V, T, dtype, target_std, draft_sigma, seed + 7,
                       greedy_tokens=(T == 0), siblings=siblings)
