"""Pins for oracle.accept.

What fixes the accept rule without any implementation to compare against:
  * exactness (Leviathan et al. review §2 "Mathematical guarantee"; EAGLE
    lesson "The Exactness Rule"): the emitted tokens follow the target law.
    Checked exactly (1e-12) by enumerating every draft draw and every
    accept/reject branch on tiny vocabularies, for chains and for trees whose
    siblings are drawn without replacement (PTD summary, "Acceptance Logic");
  * the closed form E[tokens] = (1 - a^(K+1)) / (1 - a) (EAGLE lesson,
    "Expected Speedup": 3.36 at a = 0.8, K = 4), exactly and empirically;
  * empirical distribution tests on the tiny configuration (10^4 trials);
  * the greedy rule and its special cases; identical draft and target;
  * the chain rule written as in the pages vs the tree walk on chains;
  * the scalar form of the sibling recursion used by the GPU kernel;
  * inverse-CDF sampling vs numpy.searchsorted.
Mutation tests plant plausible mistakes in a copy of the oracle (on the CPU)
and check that the exact-law pin catches each one.
"""

import inspect
import itertools
import math

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

from conftest import golden_rows
import workloads
from oracle import accept, philox

EPS_U = 2.0 ** -60            # forces an accept whenever the ratio is positive
TOP_U = 1.0 - 2.0 ** -53      # forces a reject whenever the ratio is below 1


# ----------------------------------------------------------------------------- exact law by enumeration

class PrefixModel:
    """Target / draft logits that depend on the token prefix, as a real model's do."""

    def __init__(self, V, seed, t_std=1.5, d_sigma=0.9, alpha=None, T=1.0):
        self.V, self.rng, self.t_std, self.d_sigma = V, np.random.default_rng(seed), t_std, d_sigma
        self.alpha, self.T = alpha, T
        self.rows = {}

    def get(self, prefix):
        if prefix not in self.rows:
            zt = self.rng.normal(0, self.t_std, self.V)
            noise = self.rng.normal(0, 1, self.V)
            if self.alpha is None:
                zd = zt + self.d_sigma * noise
            else:
                s = tune_scale(zt, noise, self.alpha, self.T)
                while s is None:                    # this noise cannot push alpha that low
                    noise = self.rng.normal(0, 1, self.V)
                    s = tune_scale(zt, noise, self.alpha, self.T)
                zd = zt + s * noise
            self.rows[prefix] = (zt, zd)
        return self.rows[prefix]


def alpha_of(zt, zd, T):
    return float(np.minimum(softmax(zt / T), softmax(zd / T)).sum())


def tune_scale(zt, noise, alpha, T):
    """Bisection on s so that sum(min(p, q)) == alpha for zd = zt + s * noise."""
    lo, hi = 0.0, 1.0
    while alpha_of(zt, zt + hi * noise, T) > alpha:
        hi *= 2
        if hi > 64:
            return None
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if alpha_of(zt, zt + mid * noise, T) > alpha:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def path_prefix(parent, tokens, v):
    out = []
    while v > 0:
        out.append(int(tokens[v]))
        v = int(parent[v])
    return tuple(out[::-1])


def enumerate_draws(parent, model, T):
    """All draft token assignments (siblings drawn without replacement from the
    draft law of their parent's prefix) with their probabilities."""
    n1 = len(parent)
    kids = accept.children_of(parent)
    internal = [v for v in range(n1) if kids[v]]
    tokens = np.zeros(n1, dtype=np.int64)

    def rec(idx, prob):
        if idx == len(internal):
            yield tokens.copy(), prob
            return
        v = internal[idx]
        q = softmax(model.get(path_prefix(parent, tokens, v))[1] / T)
        for tup in itertools.permutations(range(model.V), len(kids[v])):
            pr, mass = 1.0, 1.0
            for x in tup:
                pr *= q[x] / mass
                mass -= q[x]
            for c, x in zip(kids[v], tup):
                tokens[c] = x
            yield from rec(idx + 1, prob * pr)

    yield from rec(0, 1.0)


def walk_law(walk, parent, tokens, zt, zd, T):
    """Law of the emitted sequence for fixed draft tokens, integrating over the
    uniforms by exploring both outcomes of every ratio test (the trace gives the
    ratio the walk used) and weighting the final draw by the walk's weights."""
    n1 = len(parent)
    law = {}

    def explore(forced):
        u_acc = [EPS_U if forced.get(c, True) else TOP_U for c in range(n1)]
        trace = []
        n, nodes, toks, _ = walk(zt, zd, tokens, parent, T, u_acc, [0.5] * n1, trace=trace)
        tests = [t for t in trace if t[0] == "test"]
        prob = 1.0
        for _, c, ratio, ok in tests:
            if c in forced and forced[c] != ok:
                return                              # zero-probability branch
            a = min(1.0, ratio)
            prob *= a if ok else 1.0 - a
        free = [t for t in tests if t[1] not in forced]
        if free:
            c = free[0][1]
            explore({**forced, c: True})
            explore({**forced, c: False})
            return
        _, v, w = trace[-1]
        w = np.asarray(w)
        head = tuple(toks[:-1])
        for y in np.nonzero(w > 0)[0]:
            key = head + (int(y),)
            law[key] = law.get(key, 0.0) + prob * w[y] / w.sum()

    explore({})
    return law


def enumerate_iid_draws(parent, model, T):
    """All draft token assignments with siblings drawn independently (with replacement) from the
    draft law of their parent's prefix, with their probabilities."""
    n1 = len(parent)
    kids = accept.children_of(parent)
    internal = [v for v in range(n1) if kids[v]]
    tokens = np.zeros(n1, dtype=np.int64)

    def rec(idx, prob):
        if idx == len(internal):
            yield tokens.copy(), prob
            return
        v = internal[idx]
        q = softmax(model.get(path_prefix(parent, tokens, v))[1] / T)
        for tup in itertools.product(range(model.V), repeat=len(kids[v])):
            for c, x in zip(kids[v], tup):
                tokens[c] = x
            yield from rec(idx + 1, prob * float(np.prod([q[x] for x in tup])))

    yield from rec(0, 1.0)


def fixed_candidates(order):
    """Deterministic drafting: the children of a node get the first tokens of `order(zt, zd)`
    (distinct), a function of the prefix only; one assignment, probability 1."""
    def draws(parent, model, T):
        n1 = len(parent)
        kids = accept.children_of(parent)
        tokens = np.zeros(n1, dtype=np.int64)
        for v in range(n1):                      # parents come before children
            if kids[v]:
                zt, zd = model.get(path_prefix(parent, tokens, v))
                for c, x in zip(kids[v], order(zt, zd)):
                    tokens[c] = int(x)
        yield tokens, 1.0
    return draws


def full_law(parent, model, T, walk=None, draws=enumerate_draws):
    walk = walk or accept.tree_accept
    law = {}
    for tokens, p_draw in draws(parent, model, T):
        zt = np.stack([model.get(path_prefix(parent, tokens, v))[0] for v in range(len(parent))])
        zd = np.stack([model.get(path_prefix(parent, tokens, v))[1] for v in range(len(parent))])
        for seq, pr in walk_law(walk, parent, tokens, zt, zd, T).items():
            law[seq] = law.get(seq, 0.0) + p_draw * pr
    return law


def law_error(law, model, T):
    """max |P(s'+y...) - P(continue past s') * p(y | s')| over prefixes s'."""
    assert abs(sum(law.values()) - 1.0) < 1e-12
    prefixes = {s[:j] for s in law for j in range(len(s))}
    err = 0.0
    for pre in prefixes:
        cont = sum(pr for s, pr in law.items() if len(s) > len(pre) and s[:len(pre)] == pre)
        p = softmax(model.get(pre)[0] / T)
        for y in range(model.V):
            nxt = sum(pr for s, pr in law.items() if len(s) > len(pre) and s[:len(pre) + 1] == pre + (y,))
            err = max(err, abs(nxt - cont * p[y]))
    return err


CHAIN = lambda K: np.arange(-1, K, dtype=np.int64)


@pytest.mark.parametrize("K,V,T,seed", [(1, 5, 1.0, 1), (2, 4, 0.6, 2), (3, 4, 1.0, 3), (3, 3, 1.7, 4)])
def test_exact_law_chain(K, V, T, seed):
    model = PrefixModel(V, seed, T=T)
    assert law_error(full_law(CHAIN(K), model, T), model, T) < 1e-12


@pytest.mark.parametrize("parent,V,T,seed", [
    (workloads.TREE6, 3, 1.0, 5),
    (workloads.TREE6, 4, 0.8, 6),
    (np.array([-1, 0, 0, 0, 1, 2]), 4, 1.0, 7),          # three siblings at the root
    (np.array([-1, 0, 0, 0, 0]), 5, 1.3, 8),             # four siblings, no second level
    (np.array([-1, 0, 1, 1, 2]), 4, 1.0, 9),             # chain then a fork
])
def test_exact_law_tree(parent, V, T, seed):
    model = PrefixModel(V, seed, T=T)
    assert law_error(full_law(parent, model, T), model, T) < 1e-12


def _rule(name):
    return lambda *a, **kw: accept.tree_accept(*a, siblings=name, **kw)


# (vocabularies of 5-6: with fewer tokens the residual after one rejection is often a point mass,
# which makes several different rules agree)
SIBLING_TREES = [
    (workloads.TREE6, 4, 1.0, 21),
    (np.array([-1, 0, 0, 0]), 6, 0.8, 22),               # three siblings at the root
    (np.array([-1, 0, 0, 0, 0]), 5, 1.3, 23),            # four siblings
    (np.array([-1, 0, 0, 1]), 5, 1.0, 24),               # a fork, then one more level
]


@pytest.mark.parametrize("parent,V,T,seed", SIBLING_TREES)
def test_exact_law_iid_siblings(parent, V, T, seed):
    # siblings drawn independently from q (repeated tokens included): the walk with the
    # unrenormalised proposal keeps the target law
    model = PrefixModel(V, seed, T=T)
    assert law_error(full_law(parent, model, T, walk=_rule("iid"), draws=enumerate_iid_draws), model, T) < 1e-12
    # the without-replacement walk is exact for i.i.d. draws too: skipping a repeated token makes
    # the next test one whose proposal, given that its token is new, is q without the rejected ones
    assert law_error(full_law(parent, model, T, draws=enumerate_iid_draws), model, T) < 1e-12


@pytest.mark.parametrize("order", ["draft_top", "target_bottom"])
@pytest.mark.parametrize("parent,V,T,seed", SIBLING_TREES)
def test_exact_law_deterministic_siblings(parent, V, T, seed, order):
    # fixed candidates -- the draft's top tokens, or the target's least likely ones: either way
    # the emitted sequence follows the target law
    pick = {"draft_top": lambda zt, zd: np.argsort(-zd, kind="stable"),
            "target_bottom": lambda zt, zd: np.argsort(zt, kind="stable")}[order]
    model = PrefixModel(V + 1, seed, T=T)
    law = full_law(parent, model, T, walk=_rule("deterministic"), draws=fixed_candidates(pick))
    assert law_error(law, model, T) < 1e-12


def test_sibling_rules_are_not_interchangeable():
    # each rule is exact only for the drafting it describes
    model = PrefixModel(6, 25, T=1.0)
    tree = np.array([-1, 0, 0, 0])
    top = fixed_candidates(lambda zt, zd: np.argsort(-zd, kind="stable"))
    wrong = [
        (_rule("iid"), enumerate_draws),                  # without-replacement draws, proposal kept as q
        (accept.tree_accept, top),                        # fixed candidates treated as draws from q
        (_rule("iid"), top),
    ]
    for walk, draws in wrong:
        assert law_error(full_law(tree, model, 1.0, walk=walk, draws=draws), model, 1.0) > 1e-4


# ----------------------------------------------------------------------------- mutation tests

def _mutant(old, new):
    src = inspect.getsource(accept.tree_accept)
    assert old in src
    ns = dict(vars(accept))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["tree_accept"]


@pytest.mark.parametrize("old,new", [
    # the scalar-q residual of the printed listing
    ("residual = np.maximum(p - q, 0.0)", "residual = np.maximum(p - q[x], 0.0)"),
    # siblings treated as if drawn with replacement (q not renormalised)
    ("q = q / (1.0 - qx)", "pass"),
    # target row of the wrong node (off by one along the path)
    ("p = softmax_T(zt[v], T)", "p = softmax_T(zt[max(v - 1, 0)], T)"),
    # temperature dropped on the draft side
    ('q = softmax_T(zd[v], T) if kids[v] and siblings != "deterministic" else None',
     'q = softmax_T(zd[v], 1.0) if kids[v] and siblings != "deterministic" else None'),
    # residual taken against the original p instead of the running p'
    ("residual = np.maximum(p - q, 0.0)", "residual = np.maximum(softmax_T(zt[v], T) - q, 0.0)"),
])
def test_exact_law_catches_planted_mistakes(old, new):
    walk = _mutant(old, new)
    model = PrefixModel(4, 6, T=0.8)
    assert law_error(full_law(workloads.TREE6, model, 0.8, walk=walk), model, 0.8) > 1e-4


def test_iid_rule_catches_skipping_repeated_tokens():
    walk = _mutant('if siblings != "iid":', "if True:")
    model = PrefixModel(6, 26, T=1.0)
    law = full_law(np.array([-1, 0, 0, 0]), model, 1.0, walk=lambda *a, **kw: walk(*a, siblings="iid", **kw),
                   draws=enumerate_iid_draws)
    assert law_error(law, model, 1.0) > 1e-4


def test_deterministic_rule_catches_a_residual_against_the_draft_law():
    # the deterministic walk must subtract the point mass, not the draft's softmax
    walk = _mutant("""            if siblings == "deterministic":
                q = np.zeros_like(p)
                q[x] = 1.0""", """            if siblings == "deterministic":
                q = softmax_T(zd[v], T)""")
    model = PrefixModel(6, 27, T=1.0)
    law = full_law(np.array([-1, 0, 0, 0]), model, 1.0, walk=lambda *a, **kw: walk(*a, siblings="deterministic", **kw),
                   draws=fixed_candidates(lambda zt, zd: np.argsort(-zd, kind="stable")))
    assert law_error(law, model, 1.0) > 1e-4


# ----------------------------------------------------------------------------- E[tokens]

@pytest.mark.parametrize("alpha,K,V", [(0.8, 4, 4), (0.6, 3, 4), (0.9, 2, 6)])
def test_expected_tokens_closed_form_exact(alpha, K, V):
    model = PrefixModel(V, 11 + K, alpha=alpha, T=1.0)
    law = full_law(CHAIN(K), model, 1.0)
    dist = np.zeros(K + 1)
    for s, pr in law.items():
        dist[len(s) - 1] += pr
    want = np.array([alpha ** j * (1 - alpha) for j in range(K)] + [alpha ** K])
    np.testing.assert_allclose(dist, want, rtol=0, atol=1e-12)
    e = float(np.dot(np.arange(1, K + 2), dist))
    assert abs(e - (1 - alpha ** (K + 1)) / (1 - alpha)) < 1e-12
    for a, k, printed in golden_rows("expected_tokens.txt"):
        if float(a) == alpha and int(k) == K:
            assert round(e, 2) == float(printed)


# ----------------------------------------------------------------------------- empirical (tiny config, 10^4 trials)

@pytest.fixture(scope="module")
def tiny_trials():
    c = workloads.tiny_chain_trials(10_000)
    ua, ur = philox.uniforms(c.seed, c.offset, c.B, c.N1)
    r = accept.accept_batch(c.target_logits, c.draft_logits, c.tokens, c.parent, c.T, ua, ur,
                            with_probs=False)
    return c, r


def _tv(counts, p):
    return 0.5 * np.abs(counts / counts.sum() - p).sum()


def _chi2_pvalue(counts, p):
    exp = counts.sum() * p
    order = np.argsort(exp)
    obs_b, exp_b, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:                      # merge the smallest bins until each expects >= 5
        acc_o += counts[i]
        acc_e += exp[i]
        if acc_e >= 5:
            obs_b.append(acc_o)
            exp_b.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0:
        obs_b[-1] += acc_o
        exp_b[-1] += acc_e
    return stats.chisquare(obs_b, exp_b).pvalue


def test_empirical_tv_and_chi_square(tiny_trials):
    c, r = tiny_trials
    V = c.V
    p0 = softmax(c.target_logits[0, 0].astype(np.float64) / c.T)
    first = r["out_tokens"][:, 0]
    spec = np.bincount(first, minlength=V).astype(float)
    direct = np.bincount(np.random.default_rng(99).choice(V, size=first.size, p=p0), minlength=V).astype(float)
    # TV against p measured relative to the sampling-noise floor of 10^4 direct draws
    assert abs(_tv(spec, p0) - _tv(direct, p0)) < 0.01
    assert _chi2_pvalue(spec, p0) > 1e-3
    # every later position, conditioned on reaching it, follows that position's p
    for k in range(1, c.N1):
        reached = r["accept_len"] >= k
        pk = softmax(c.target_logits[0, k].astype(np.float64) / c.T)
        cnt = np.bincount(r["out_tokens"][reached, k], minlength=V).astype(float)
        assert _chi2_pvalue(cnt, pk) > 1e-3


def test_empirical_accept_length_law(tiny_trials):
    c, r = tiny_trials
    K = c.N1 - 1
    alphas = [alpha_of(c.target_logits[0, k].astype(np.float64), c.draft_logits[0, k].astype(np.float64), c.T)
              for k in range(K)]
    surv = np.cumprod([1.0] + alphas)                    # P(n >= j)
    law = np.append(surv[:-1] - surv[1:], surv[-1])      # P(n == j)
    counts = np.bincount(r["accept_len"], minlength=K + 1).astype(float)
    assert stats.chisquare(counts, law * counts.sum()).pvalue > 1e-3
    mean_tokens = (r["accept_len"] + 1).mean()
    se = (r["accept_len"] + 1).std() / math.sqrt(c.B)
    assert abs(mean_tokens - surv.sum()) < 4 * se


# ----------------------------------------------------------------------------- greedy

def test_greedy_chain_rule():
    rng = np.random.default_rng(1)
    K, V = 5, 50
    zt = rng.normal(0, 1, (K + 1, V))
    zt[2, 7] = zt[2].max() + 1.0
    zt[2, 3] = zt[2, 7]                                   # a tie: the lower index (3) wins
    am = [int(np.argmax(r)) for r in zt]
    assert am[2] == 3
    tokens = [0] + am[:K]
    parent = np.arange(-1, K)
    n, nodes, toks, m = accept.tree_accept(zt, None, tokens, parent, 0, [0.5] * 6, [0.5] * 6)
    assert n == K and nodes == [1, 2, 3, 4, 5] and toks == am[:K] + [am[K]]
    for j in range(1, K + 1):
        bad = list(tokens)
        bad[j] = (am[j - 1] + 1) % V
        n, nodes, toks, _ = accept.tree_accept(zt, None, bad, parent, 0, [0.5] * 6, [0.5] * 6)
        assert n == j - 1 and toks == am[:j - 1] + [am[j - 1]]


def test_greedy_tree_equals_brute_force_over_paths():
    rng = np.random.default_rng(2)
    for trial in range(200):
        n1 = int(rng.integers(2, 30))
        V = int(rng.integers(2, 6))
        parent = workloads.random_tree(rng, n1 - 1, min(3, V), 6)   # distinct sibling tokens
        zt = rng.integers(-3, 3, size=(n1, V)).astype(float)      # integer logits force ties
        kids = accept.children_of(parent)
        tokens = np.zeros(n1, dtype=int)
        for v in range(n1):
            if kids[v]:
                tokens[kids[v]] = rng.choice(V, size=len(kids[v]), replace=False)
        n, nodes, toks, _ = accept.tree_accept(zt, None, tokens, parent, 0, [0.5] * n1, [0.5] * n1)
        # brute force: the deepest node whose path tokens are each the argmax of the parent
        # row (with distinct sibling tokens at most one such path exists at every depth)
        best = [0]
        for v in range(1, n1):
            path, u = [], v
            while u > 0:
                path.append(u)
                u = parent[u]
            path = path[::-1]
            if all(int(tokens[w]) == int(np.argmax(zt[parent[w]])) for w in path):
                if len(path) > len(best) - 1 or (len(path) == len(best) - 1 and path < best[1:]):
                    best = [0] + path
        assert nodes == best[1:]
        assert toks[-1] == int(np.argmax(zt[best[-1]]))


# ----------------------------------------------------------------------------- special cases and equivalences

def test_identical_draft_and_target_accepts_everything():
    rng = np.random.default_rng(3)
    for T in (0.5, 1.0, 2.0):
        for parent in (np.arange(-1, 6), workloads.TREE6, workloads.random_tree(rng, 20, 3, 5)):
            n1 = len(parent)
            z = rng.normal(0, 2, (n1, 40))
            tokens = rng.integers(40, size=n1)
            kids = accept.children_of(parent)
            for v in range(n1):
                if kids[v]:
                    tokens[kids[v]] = rng.choice(40, size=len(kids[v]), replace=False)
            ua = list(rng.random(n1))
            n, nodes, _, _ = accept.tree_accept(z, z.copy(), tokens, parent, T, ua, list(rng.random(n1)))
            v, first_path = 0, []
            while kids[v]:
                v = kids[v][0]
                first_path.append(v)
            assert nodes == first_path


def test_chain_rule_equals_tree_walk_on_chains():
    rng = np.random.default_rng(4)
    for trial in range(300):
        K = int(rng.integers(0, 7))
        V = int(rng.integers(2, 30))
        T = [0, 0.5, 1.0, 1.5][trial % 4]
        zt = rng.normal(0, 2, (K + 1, V))
        zd = zt + rng.normal(0, 1.0, (K + 1, V))
        tokens = [int(rng.integers(V))] + [int(rng.integers(V)) for _ in range(K)]
        ua, ur = list(rng.random(K + 1)), list(rng.random(K + 1))
        n1, e1, m1 = accept.chain_accept(zt, zd, tokens, T, ua, ur)
        n2, nodes, e2, m2 = accept.tree_accept(zt, zd, tokens, np.arange(-1, K), T, ua, ur)
        assert (n1, e1) == (n2, e2) and nodes == list(range(1, n2 + 1))
        assert m1 == pytest.approx(m2, rel=1e-12, abs=1e-15)


def test_scalar_form_of_the_sibling_recursion():
    """After i rejections at a node the walk's target is (p - c_i q)+ / R_i with
    c_0 = 0, R_0 = Q_0 = 1, c_{i+1} = c_i + R_i / Q_i, Q_i = 1 - sum of the
    rejected q(x); the i+1-th ratio is (p/q - c_i)+ * Q_i / R_i."""
    rng = np.random.default_rng(5)
    seen_multi = 0
    for trial in range(400):
        V, nk = int(rng.integers(3, 40)), int(rng.integers(1, 5))
        nk = min(nk, V)
        T = float(rng.choice([0.7, 1.0, 1.4]))
        parent = np.array([-1] + [0] * nk)
        zt = rng.normal(0, 1.5, (nk + 1, V))
        zd = zt + rng.normal(0, 1.5, (nk + 1, V))
        tokens = np.array([0] + list(rng.choice(V, size=nk, replace=False)))
        trace = []
        accept.tree_accept(zt, zd, tokens, parent, T, [TOP_U] * (nk + 1), [0.5] * (nk + 1), trace=trace)
        p, q = softmax(zt[0] / T), softmax(zd[0] / T)
        c, R, Q = 0.0, 1.0, 1.0
        tests = [t for t in trace if t[0] == "test"]
        for i, (_, node, ratio, ok) in enumerate(tests):
            x = tokens[node]
            want = max(0.0, p[x] / q[x] - c) * Q / R
            assert abs(ratio - want) <= 1e-11 * max(1.0, want)
            if ok:
                break
            c = c + R / Q
            Q = Q - q[x]
            R = np.maximum(p - c * q, 0).sum()
        if trace[-1][0] == "draw" and trace[-1][1] == 0:
            w = trace[-1][2]
            np.testing.assert_allclose(w, np.maximum(p - c * q, 0) / R, rtol=0, atol=1e-12)
            if len(tests) >= 2:
                seen_multi += 1
    assert seen_multi > 20


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(6)
    for _ in range(2000):
        V = int(rng.integers(1, 60))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[rng.integers(V)] = 1.0
        u = float(rng.random())
        i, margin = accept.inverse_cdf(w, u)
        want = int(np.searchsorted(np.cumsum(w) / w.sum(), u, side="right"))
        if margin > 1e-12:
            assert i == want
        assert w[i] > 0


def test_invalid_inputs_give_minus_one():
    rng = np.random.default_rng(7)
    zt = rng.normal(size=(2, 4, 10))
    parent = np.array([[-1, 0, 1, 2], [-1, 0, 3, 1]])            # second: forward reference
    tokens = np.array([[0, 1, 2, 3], [0, 1, 2, 3]])
    ua, ur = philox.uniforms(1, 0, 2, 4)
    r = accept.accept_batch(zt, zt, tokens, parent, 1.0, ua, ur)
    assert r["accept_len"][0] >= 0 and r["accept_len"][1] == -1
    assert (r["out_tokens"][1] == -1).all() and np.isnan(r["p_tok"][1]).all()
    tokens[0, 2] = 10                                               # token out of range
    r = accept.accept_batch(zt, zt, tokens, np.array([[-1, 0, 1, 2]] * 2), 1.0, ua, ur)
    assert r["accept_len"][0] == -1 and r["accept_len"][1] >= 0


def test_node_probs():
    rng = np.random.default_rng(8)
    parent = workloads.TREE6
    zt, zd = rng.normal(size=(7, 12)), rng.normal(size=(7, 12))
    tokens = np.array([0, 1, 2, 3, 4, 5, 6])
    p_tok, q_tok = accept.node_probs(zt, zd, tokens, parent, 0.9)
    assert np.isnan(p_tok[0]) and np.isnan(q_tok[0])
    for v in range(1, 7):
        assert abs(p_tok[v] - softmax(zt[parent[v]] / 0.9)[tokens[v]]) < 1e-15
        assert abs(q_tok[v] - softmax(zd[parent[v]] / 0.9)[tokens[v]]) < 1e-15
    p0, q0 = accept.node_probs(zt, zd, tokens, parent, 0)
    assert np.isnan(p0).all() and np.isnan(q0).all()


def test_workload_alphas():
    """The recipes' draft noise gives the acceptance rates the configs name."""
    rng = np.random.default_rng(9)
    # tolerances cover the row-to-row spread of alpha over 16 rows
    for V, std, sigma, T, want, tol in [(32000, 3.0, workloads.SIGMA_CHAIN, 1.0, 0.80, 0.03),
                                        (128256, 3.0, workloads.SIGMA_EAGLE, 0.7, 0.80, 0.05),
                                        (128256, 3.0, workloads.SIGMA_PTD, 1.0, 0.75, 0.05),
                                        (1000, 2.0, 0.5, 1.0, 0.80, 0.04)]:
        a = []
        for _ in range(16):
            zt = workloads.round_bf16(rng.normal(0, std, V).astype(np.float32)).astype(np.float64)
            zd = workloads.round_bf16((zt + rng.normal(0, sigma, V)).astype(np.float32)).astype(np.float64)
            a.append(alpha_of(zt, zd, T))
        assert abs(np.mean(a) - want) < tol, (V, np.mean(a))
    zt, zd = rng.normal(0, 3, 151936), rng.normal(0, 3, 151936)
    assert 0.1 < alpha_of(zt, zd, 1.5) < 0.22
