"""Exact-enumeration machinery for the oracle's losslessness pins.

The draft-verification page (llm-infra-atlas "01 · Draft-then-verify", §2.1)
shows that one accept/residual step returns a token distributed exactly as p
for any p and q.  Repeating rounds therefore produces sequences distributed
exactly as the target's chain rule.  These helpers compute, with no sampling,
the probability of every output the oracle can produce: the oracle's output is
piecewise constant in its uniforms, so it is evaluated at the midpoint of
every cell of (r_1, r_2, ..., u) space and weighted by the cell's volume.

Cell edges in r come from the acceptance ratios the oracle reports for the
decisions it makes (a decision at position i accepts on [0, min(1, a_i))),
edges in u from the normalised weights of its final draw.  The outputs
themselves are always the oracle's answers at the midpoints, so a wrong
decision rule, a wrong residual, a wrong row index or an off-by-one in the
inverse CDF changes the resulting distribution.
"""
from __future__ import annotations

import itertools
import math
from collections import defaultdict

import numpy as np

import oracle


class Tables:
    """Deterministic random next-token tables p(.|ctx), q(.|ctx) over V tokens."""

    def __init__(self, V, seed, p_zero=0.0, q_zero=0.0):
        self.V, self.seed, self.p_zero, self.q_zero = V, seed, p_zero, q_zero
        self._cache = {}

    def _dist(self, ctx, which):
        key = (tuple(ctx), which)
        if key not in self._cache:
            h = self.seed * 1000003 + (1 if which == "p" else 2)
            for t in ctx:
                h = (h * 31 + t + 7) % (2 ** 61 - 1)
            rng = np.random.default_rng(h)
            d = rng.dirichlet(np.full(self.V, 0.7))
            zero = self.p_zero if which == "p" else self.q_zero
            if zero > 0:
                mask = rng.random(self.V) < zero
                mask[rng.integers(self.V)] = False  # keep at least one token
                d = np.where(mask, 0.0, d)
                d = d / d.sum()
            self._cache[key] = d
        return self._cache[key]

    def p(self, ctx):
        return self._dist(ctx, "p")

    def q(self, ctx):
        return self._dist(ctx, "q")

    def target_prob(self, seq, prefix=()):
        pr = 1.0
        ctx = list(prefix)
        for t in seq:
            pr *= self.p(ctx)[t]
            ctx.append(t)
        return pr


def logits_of(dist, T):
    with np.errstate(divide="ignore"):
        return T * np.log(dist)


def enumerate_cells(run, n_positions, V):
    """Exact output distribution of one oracle round.

    run(r [n_positions], u) -> (emitted tuple, a_trace [n_positions] (NaN where
    no decision was made), w [V] normalised weights of the final draw).
    Decisions are made in increasing position order.
    """
    out = defaultdict(float)

    def rec(fixed, prob):
        r = np.full(n_positions, 0.5)
        for i, v in fixed.items():
            r[i] = v
        _, a, w = run(r, 0.5)
        free = [i for i in range(n_positions) if not math.isnan(a[i]) and i not in fixed]
        if free:
            i = free[0]
            ai = min(1.0, a[i])
            if ai > 0.0:
                rec({**fixed, i: ai / 2.0}, prob * ai)
            if ai < 1.0:
                rec({**fixed, i: (1.0 + ai) / 2.0}, prob * (1.0 - ai))
            return
        C = 0.0
        for t in range(V):
            if w[t] <= 0.0:
                continue
            umid = C + w[t] / 2.0
            C += w[t]
            emitted, _, _ = run(r, umid)
            out[emitted] += prob * w[t]

    rec({}, 1.0)
    return out


def chain_sequence_distribution(tab: Tables, gamma, m, T=1.0, chain_core=None):
    """Distribution of the first m tokens produced by repeated chain rounds from an empty prefix."""
    V = tab.V
    core = chain_core or oracle.chain_core
    memo = {}

    def round_outcomes(prefix):
        res = defaultdict(float)
        for xs in itertools.product(range(V), repeat=gamma):
            wq = 1.0
            for j in range(gamma):
                wq *= tab.q(prefix + xs[:j])[xs[j]]
            if wq == 0.0:
                continue
            tgt = np.stack([logits_of(tab.p(prefix + xs[:j]), T) for j in range(gamma + 1)])
            drf = np.stack([logits_of(tab.q(prefix + xs[:j]), T) for j in range(gamma)])

            def run(r, u, tgt=tgt, drf=drf, xs=xs):
                o = core(tgt, drf, np.array(xs), T, r, u, dtype="f64")
                return tuple(xs[:o["n"]]) + (o["t"],), o["a"], o["w"]

            for e, pr in enumerate_cells(run, gamma, V).items():
                res[e] += wq * pr
        return res

    def dist(prefix):
        if len(prefix) >= m:
            return {prefix[:m]: 1.0}
        if prefix in memo:
            return memo[prefix]
        acc = defaultdict(float)
        for e, pr in round_outcomes(prefix).items():
            for s, pr2 in dist(prefix + e).items():
                acc[s] += pr * pr2
        memo[prefix] = acc
        return acc

    return dist(())


def tree_sequence_distribution(tab: Tables, parent, m, T=1.0):
    """Distribution of the first m tokens from repeated tree rounds whose
    siblings are drawn i.i.d. from the draft distribution of their parent's
    context (the tree shape is fixed by `parent`)."""
    V = tab.V
    N = len(parent)
    max_depth = N
    memo = {}

    def round_outcomes(prefix):
        res = defaultdict(float)
        for toks in itertools.product(range(V), repeat=N - 1):
            tok = (0,) + toks
            ctx = {0: prefix}
            wq = 1.0
            for i in range(1, N):
                ctx[i] = ctx[parent[i]] + (tok[i],)
                wq *= tab.q(ctx[parent[i]])[tok[i]]
            if wq == 0.0:
                continue
            tgt = np.stack([logits_of(tab.p(ctx[i]), T) for i in range(N)])[None]
            drf = np.stack([logits_of(tab.q(ctx[i]), T) for i in range(N)])[None]
            tok_a = np.array(tok, np.int32)[None]
            par_a = np.array(parent, np.int32)[None]

            def run(r, u, tgt=tgt, drf=drf, tok_a=tok_a, tok=tok):
                o = oracle.verify_tree(tgt, drf, tok_a, par_a, max_depth, T, 0, 0, "f64", r=r[None], u=np.array([u]),
                                       want_w=True)
                L = int(o["len"][0])
                emitted = tuple(tok[i] for i in o["path"][0][:L]) + (int(o["t"][0]),)
                return emitted, o["a"][0], o["w"][0]

            for e, pr in enumerate_cells(run, N, V).items():
                res[e] += wq * pr
        return res

    def dist(prefix):
        if len(prefix) >= m:
            return {prefix[:m]: 1.0}
        if prefix in memo:
            return memo[prefix]
        acc = defaultdict(float)
        for e, pr in round_outcomes(prefix).items():
            for s, pr2 in dist(prefix + e).items():
                acc[s] += pr * pr2
        memo[prefix] = acc
        return acc

    return dist(())


def _recurse(round_outcomes, m):
    memo = {}

    def dist(prefix):
        if len(prefix) >= m:
            return {prefix[:m]: 1.0}
        if prefix in memo:
            return memo[prefix]
        acc = defaultdict(float)
        for e, pr in round_outcomes(prefix).items():
            for s, pr2 in dist(prefix + e).items():
                acc[s] += pr * pr2
        memo[prefix] = acc
        return acc

    return dist(())


def chain_pm_sequence_distribution(tab: Tables, gamma, m, choose, T=1.0, verify=None):
    """Distribution of the first m tokens from repeated point-mass chain rounds
    whose drafts are chosen deterministically: x_j = choose(context)."""
    V = tab.V
    verify = verify or oracle.verify_chain_pm

    def round_outcomes(prefix):
        xs = []
        for _ in range(gamma):
            xs.append(int(choose(prefix + tuple(xs))))
        tgt = np.stack([logits_of(tab.p(prefix + tuple(xs[:j])), T) for j in range(gamma + 1)])[None]
        tok = np.array(xs, np.int32)[None]

        def run(r, u):
            o = verify(tgt, tok, T, 0, 0, "f64", r=r[None], u=np.array([u]), want_w=True)
            n = int(o["n"][0])
            return tuple(xs[:n]) + (int(o["t"][0]),), o["a"][0], o["w"][0]

        return enumerate_cells(run, gamma, V)

    return _recurse(round_outcomes, m)


def tree_pm_sequence_distribution(tab: Tables, parent, m, rank_source="q", T=1.0, pm=True):
    """Distribution of the first m tokens from repeated tree rounds whose
    siblings are deterministic: the k-th child (in index order) of a node is
    the k-th most likely token of the node's draft distribution (top-F
    siblings).  pm selects the point-mass rule, else the standard sibling
    rule with the node's draft q held fixed."""
    V = tab.V
    N = len(parent)
    max_depth = N

    def round_outcomes(prefix):
        ctx = {0: prefix}
        tok = [0] * N
        seen = defaultdict(int)
        for i in range(1, N):
            pu = parent[i]
            order = np.argsort(-(tab.q(ctx[pu]) if rank_source == "q" else tab.p(ctx[pu])), kind="stable")
            tok[i] = int(order[seen[pu]])
            seen[pu] += 1
            ctx[i] = ctx[pu] + (tok[i],)
        tgt = np.stack([logits_of(tab.p(ctx[i]), T) for i in range(N)])[None]
        drf = np.stack([logits_of(tab.q(ctx[i]), T) for i in range(N)])[None]
        tok_a = np.array(tok, np.int32)[None]
        par_a = np.array(parent, np.int32)[None]

        def run(r, u):
            if pm:
                o = oracle.verify_tree_pm(tgt, tok_a, par_a, max_depth, T, 0, 0, "f64", r=r[None],
                                          u=np.array([u]), want_w=True)
            else:
                o = oracle.verify_tree(tgt, drf, tok_a, par_a, max_depth, T, 0, 0, "f64", r=r[None],
                                       u=np.array([u]), want_w=True)
            L = int(o["len"][0])
            emitted = tuple(tok[i] for i in o["path"][0][:L]) + (int(o["t"][0]),)
            return emitted, o["a"][0], o["w"][0]

        return enumerate_cells(run, N, V)

    return _recurse(round_outcomes, m)


def max_marginal_error(tab: Tables, distr, m):
    err = 0.0
    total = 0.0
    for s in itertools.product(range(tab.V), repeat=m):
        want = tab.target_prob(s)
        got = distr.get(tuple(s), 0.0)
        total += got
        err = max(err, abs(want - got))
    return max(err, abs(total - 1.0))
