"""One level of draft-tree expansion.  Test infrastructure.

[SD-EAGLE] "EAGLE: tree drafting and feature reuse": the draft outputs a tree
of candidates, K per depth, 4-6 deep, and exercise 4 builds it from the top 3
branches at every depth; EAGLE-2 (same section) grows the tree dynamically,
wide where the draft is unsure and narrow where it is confident.  [PTD] Method
2, "Progressive Expansion & Pruning": every step drafts children for all
current leaves in one pass and appends them; width control caps the children
per parent.

Readings used (the pages give the ingredients, not an algorithm):
  * a level expands a frontier (the nodes added by the previous level, the
    root first): each frontier node proposes the k tokens of highest draft
    probability q = softmax(z / T) (k is the width cap; ties go to the lower
    token id, so the order is that of the raw logits);
  * a candidate's score is its path's cumulative draft log-probability,
    score(parent) + log q(token);
  * of all candidates of a sequence, the `keep` of highest score survive (the
    EAGLE-2 reading of "wide where unsure": a confident parent's children
    outscore an unsure parent's), fewer if the tree's node capacity is
    reached; ties go to the earlier frontier row, then the better rank;
  * survivors are appended in frontier order, then rank order, so node ids
    stay topological (a parent before its children) and breadth-first by
    level; they form the next frontier;
  * a frontier entry that is not a node of the tree (-1, or not below the
    node count and the capacity) has no row; k above V proposes all V tokens.

Layouts: draft_logits[B][F][V] (row f is frontier[b][f]'s draft logits; rows
with frontier -1 are unused), frontier[B][F], tree arrays parent / tokens /
score [B][Nmax] and n_nodes[B].  Everything in float64.
"""

import numpy as np


def row_topk(z, k, T):
    """The k largest logits of one row (ties: lower index first) and their log q under
    softmax(z / T).  Returns (tokens[k], log_q[k])."""
    z = np.asarray(z, dtype=np.float64)
    order = np.argsort(-z, kind="stable")[:k]
    s = z / T
    m = s.max()
    lse = m + np.log(np.exp(s - m).sum())
    return order.astype(np.int64), s[order] - lse


def expand_sequence(draft_rows, frontier, k, T, keep, parent, tokens, score, n, nmax):
    """One sequence.  Returns (parent, tokens, score, n, new_frontier, margin).

    margin is the score gap at the cut between the last survivor and the best
    candidate left out (inf when nothing was left out): how close the kept set
    was to changing.
    """
    parent, tokens, score = parent.copy(), tokens.copy(), score.copy()
    cands = []                       # (score, f, j, token, parent node)
    for f, u in enumerate(frontier):
        if not 0 <= u < min(n, nmax):    # not a node of the tree: the row is unused
            continue
        toks, lq = row_topk(draft_rows[f], k, T)
        for j in range(len(toks)):
            cands.append((score[u] + lq[j], f, j, int(toks[j]), int(u)))
    m = min(keep, len(cands), nmax - n)
    ranked = sorted(cands, key=lambda c: (-c[0], c[1], c[2]))
    margin = np.inf
    if 0 < m < len(ranked):
        margin = ranked[m - 1][0] - ranked[m][0]
    kept = sorted(ranked[:max(m, 0)], key=lambda c: (c[1], c[2]))
    new_frontier = []
    for c in kept:
        parent[n], tokens[n], score[n] = c[4], c[3], c[0]
        new_frontier.append(n)
        n += 1
    return parent, tokens, score, n, new_frontier, margin


def expand(draft_logits, frontier, k, T, keep, parent, tokens, score, n_nodes):
    """Batch: returns (parent, tokens, score, n_nodes, new_frontier[B][keep] (-1 padded), margin[B])."""
    B, nmax = np.asarray(parent).shape
    out_p, out_t = np.array(parent, copy=True), np.array(tokens, copy=True)
    out_s = np.array(score, dtype=np.float64, copy=True)
    out_n = np.array(n_nodes, copy=True)
    nf = np.full((B, keep), -1, dtype=np.int64)
    margin = np.full(B, np.inf)
    for b in range(B):
        out_p[b], out_t[b], out_s[b], out_n[b], fr, margin[b] = expand_sequence(
            draft_logits[b], [int(x) for x in frontier[b]], k, T, keep, out_p[b], out_t[b], out_s[b],
            int(n_nodes[b]), nmax)
        nf[b, :len(fr)] = fr
    return out_p, out_t, out_s, out_n, nf, margin
