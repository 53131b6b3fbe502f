"""Exact accept / reject / resample rule of speculative decoding.  Test infrastructure.

Sources and the steps they fix:
  * [SD-EAGLE] "Two-Model Setup" and "Build it": the draft and the target
    distributions at temperature T are softmax(logits / T); the target is
    evaluated at all K + 1 positions in one pass.
  * [SD-EAGLE] "The Exactness Rule"; [SD-review] §2, algorithm step 3 and
    "Mathematical guarantee": for each drafted token x, left to right, draw
    r ~ U(0, 1) and accept x if r < p(x) / q(x); at the first rejection emit a
    replacement drawn from (p - q)+ / ||(p - q)+||_1 and stop.
  * [SD-EAGLE] "Two-Model Setup" step 4; [SD-review] §2 "Result": if all K are
    accepted, draw one bonus token from the target distribution of the last
    position.
  * [SD-EAGLE] "The Exactness Rule", greedy case: at T = 0 accept iff
    argmax(p) == x; otherwise emit argmax(p) and stop.
  * [PTD] Method 4, "Acceptance Logic": on a tree, greedy decoding accepts an
    edge when the verified token matches a child; sampling decoding decides by
    sampling without replacement over normalised probabilities, which keeps
    the target distribution.

Readings where the pages are silent, ambiguous or garbled:
  * The printed listing in "Build it" keeps only the scalar q(x) and subtracts
    it from the whole p vector when it forms the residual; that contradicts
    the rule stated in words and formulas on both pages, so the full q vector
    is used.
  * Tree sampling rule: at node v the children are tested in increasing node
    index.  After a child with token x is rejected, the target is replaced by
    its residual p' <- (p' - q')+ / sum (p' - q')+ and the draft by q without
    x, renormalised, q' <- q' [y != x] / (1 - q'(x)) -- the distribution the
    next sibling was drawn from when siblings are drawn without replacement.
    A child whose token repeats an earlier sibling's is skipped.  If every
    child is rejected the walk emits y ~ p'; at a leaf it emits the bonus
    y ~ p_v.  A chain (one child per node) is exactly the chain rule.
  * Greedy on a tree: the first child (by index) whose token equals the
    argmax is accepted; argmax ties go to the lowest token id.
  * "Sample from w" is inverse-CDF sampling: the smallest index i whose
    running sum (in index order) exceeds u * sum(w).
  * The acceptance test is the strict "<" of the pages; q'(x) == 0 counts as
    ratio +inf (accept); a residual of zero mass leaves p' unchanged.

Other ways the siblings may have been drafted ([PTD] Method 4 names sampling
without replacement; [SD-EAGLE] "EAGLE: tree drafting and feature reuse" has
the draft output K candidates per depth).  The walk is the same recursive
rejection rule with the proposal each sibling was actually drawn from:
  * "iid": siblings drawn independently from q_v (with replacement): the
    proposal stays q_v, so q' is not renormalised and a repeated token is
    tested like any other (after its first rejection p'(x) = 0, so it is
    rejected again, and the residual update still applies);
  * "deterministic": siblings are fixed candidates (for example the draft's
    top-k), i.e. each is proposed by a point mass at its token: accept x with
    probability p'(x); after a rejection p' <- (p' - delta_x)+ normalised, that
    is p' without x, renormalised; a repeated token has p'(x) = 0 and changes
    nothing, so it is skipped.  The draft logits are not used.

Decision margins: every uniform-driven decision records how far the uniform
was from flipping it (|u - ratio| for a ratio test; the distance of u * W from
the nearer boundary of the chosen token's CDF interval, divided by W, for a
draw).  Parity tests treat a sequence whose smallest margin is below 1e-6 as a
near tie.
"""

import math

import numpy as np

from .tree import validate_parent


def softmax_T(z, T):
    """softmax(z / T) in float64."""
    s = np.asarray(z, dtype=np.float64) / float(T)
    e = np.exp(s - s.max())
    return e / e.sum()


def inverse_cdf(w, u):
    """Smallest i with cumsum(w)[i] > u * sum(w); returns (i, margin).

    If rounding leaves u * W at or above every partial sum, the last index with
    positive weight is returned (margin 0).
    """
    w = np.asarray(w, dtype=np.float64)
    cdf = np.cumsum(w)
    total = cdf[-1]
    t = u * total
    hits = np.nonzero(cdf > t)[0]
    if hits.size == 0:
        return int(np.nonzero(w > 0)[0][-1]), 0.0
    i = int(hits[0])
    lower = cdf[i - 1] if i > 0 else 0.0
    margin = min(t - lower, cdf[i] - t) / total
    return i, float(margin)


def _ratio(p, q, x):
    if q[x] == 0.0:
        return math.inf
    return float(p[x] / q[x])


def chain_accept(zt, zd, tokens, T, u_acc, u_res):
    """The pages' chain step for one sequence with K = len(tokens) - 1 drafts.

    zt[K+1][V] target logits, zd[K][V] (or more rows) draft logits; tokens[0]
    is the last committed token and tokens[1..K] the drafts; u_acc[k] is the
    acceptance uniform of draft k, u_res[k] the draw uniform if the step ends
    at position k.  Returns (accepted drafts n, emitted tokens, min margin).
    """
    K = len(tokens) - 1
    emitted = []
    margin = math.inf
    for k in range(1, K + 1):
        x = int(tokens[k])
        if T == 0:
            y = int(np.argmax(zt[k - 1]))
            if y == x:
                emitted.append(x)
                continue
            emitted.append(y)
            return k - 1, emitted, margin
        p = softmax_T(zt[k - 1], T)
        q = softmax_T(zd[k - 1], T)
        ratio = _ratio(p, q, x)
        margin = min(margin, abs(u_acc[k] - ratio))
        if u_acc[k] < ratio:
            emitted.append(x)
            continue
        residual = np.maximum(p - q, 0.0)
        if residual.sum() <= 0.0:
            residual = p
        y, m = inverse_cdf(residual, u_res[k - 1])
        margin = min(margin, m)
        emitted.append(y)
        return k - 1, emitted, margin
    if T == 0:
        emitted.append(int(np.argmax(zt[K])))
        return K, emitted, margin
    y, m = inverse_cdf(softmax_T(zt[K], T), u_res[K])
    emitted.append(y)
    return K, emitted, min(margin, m)


def children_of(parent):
    kids = [[] for _ in range(len(parent))]
    for c in range(1, len(parent)):
        kids[int(parent[c])].append(c)
    return kids


SIBLING_RULES = ("without_replacement", "iid", "deterministic")


def tree_accept(zt, zd, tokens, parent, T, u_acc, u_res, trace=None, siblings="without_replacement"):
    """The tree walk for one sequence, for siblings drafted as `siblings` says.

    Returns (accept_len, out_nodes, out_tokens, margin).  out_nodes lists the
    accepted nodes from the first level down; out_tokens their tokens followed
    by the final (resampled, bonus or greedy) token.  If `trace` is a list, the
    walk appends ("test", node, ratio, accepted) for every ratio test and
    finally ("draw", node, weights) or ("greedy", node, token).
    """
    kids = children_of(parent)
    v = 0
    out_nodes = []
    out_tokens = []
    margin = math.inf
    while True:
        if T == 0:
            y = int(np.argmax(zt[v]))
            match = next((c for c in kids[v] if int(tokens[c]) == y), None)
            if match is not None:
                out_nodes.append(match)
                out_tokens.append(y)
                v = match
                continue
            out_tokens.append(y)
            if trace is not None:
                trace.append(("greedy", v, y))
            return len(out_nodes), out_nodes, out_tokens, margin
        p = softmax_T(zt[v], T)
        q = softmax_T(zd[v], T) if kids[v] and siblings != "deterministic" else None
        tried = set()
        accepted = None
        for c in kids[v]:
            x = int(tokens[c])
            if siblings != "iid":
                if x in tried:
                    continue
                tried.add(x)
            if siblings == "deterministic":
                q = np.zeros_like(p)
                q[x] = 1.0
            ratio = _ratio(p, q, x)
            margin = min(margin, abs(u_acc[c] - ratio))
            ok = u_acc[c] < ratio
            if trace is not None:
                trace.append(("test", c, ratio, ok))
            if ok:
                accepted = c
                break
            residual = np.maximum(p - q, 0.0)
            mass = residual.sum()
            if mass > 0.0:
                p = residual / mass
            if siblings == "without_replacement":
                qx = q[x]
                q = q.copy()
                q[x] = 0.0
                if qx < 1.0:
                    q = q / (1.0 - qx)
        if accepted is not None:
            out_nodes.append(accepted)
            out_tokens.append(int(tokens[accepted]))
            v = accepted
            continue
        y, m = inverse_cdf(p, u_res[v])
        margin = min(margin, m)
        out_tokens.append(y)
        if trace is not None:
            trace.append(("draw", v, p))
        return len(out_nodes), out_nodes, out_tokens, margin


def node_probs(zt, zd, tokens, parent, T, siblings="without_replacement"):
    """p_tok[v] = p_parent(v)(tokens[v]) and q_tok[v] likewise; NaN at v = 0 or T = 0, and q_tok
    NaN for deterministic siblings (no draft law)."""
    n1 = len(parent)
    p_tok = np.full(n1, np.nan)
    q_tok = np.full(n1, np.nan)
    if T == 0:
        return p_tok, q_tok
    kids = children_of(parent)
    for v in range(n1):
        if not kids[v]:
            continue
        p = softmax_T(zt[v], T)
        q = softmax_T(zd[v], T) if siblings != "deterministic" else None
        for c in kids[v]:
            p_tok[c] = p[int(tokens[c])]
            if q is not None:
                q_tok[c] = q[int(tokens[c])]
    return p_tok, q_tok


def accept_batch(target_logits, draft_logits, tokens, parent, T, u_acc, u_res, with_probs=True,
                 siblings="without_replacement"):
    """Batch driver: one tree walk per sequence.

    target_logits[B][N1][V], draft_logits[B][N1][V] (or None when T == 0),
    tokens[B][N1], parent[B][N1], u_acc / u_res [B][N1].  Returns a dict with
    accept_len[B], out_tokens[B][N1], out_nodes[B][N1] (-1 padded), p_tok,
    q_tok [B][N1] and margin[B].  A sequence whose parent array is invalid, or
    whose draft tokens fall outside [0, V), gets accept_len -1 and -1 / NaN
    outputs.
    """
    tokens = np.asarray(tokens)
    parent = np.asarray(parent)
    B, n1 = tokens.shape
    V = target_logits.shape[-1]
    accept_len = np.zeros(B, dtype=np.int32)
    out_tokens = np.full((B, n1), -1, dtype=np.int32)
    out_nodes = np.full((B, n1), -1, dtype=np.int32)
    p_tok = np.full((B, n1), np.nan)
    q_tok = np.full((B, n1), np.nan)
    margin = np.full(B, np.inf)
    for b in range(B):
        bad_tok = any(not (0 <= int(t) < V) for t in tokens[b, 1:])
        if validate_parent(parent[b]) != 0 or bad_tok:
            accept_len[b] = -1
            continue
        zt = target_logits[b]
        zd = draft_logits[b] if draft_logits is not None else None
        n, nodes, toks, m = tree_accept(zt, zd, tokens[b], parent[b], T, u_acc[b], u_res[b], siblings=siblings)
        accept_len[b] = n
        out_nodes[b, :len(nodes)] = nodes
        out_tokens[b, :len(toks)] = toks
        margin[b] = m
        if with_probs:
            p_tok[b], q_tok[b] = node_probs(zt, zd, tokens[b], parent[b], T, siblings)
    return dict(accept_len=accept_len, out_tokens=out_tokens, out_nodes=out_nodes,
                p_tok=p_tok, q_tok=q_tok, margin=margin)
