"""Exact-rational law of the accept-and-correct rule -- TEST INFRASTRUCTURE.

A third, independent statement of the rule in the encyclopedia entry
"Speculative decoding" (glopedia, 推测解码), section "Basic steps of proposal
and verification" (提议与核验的基本步骤), over ``fractions.Fraction`` for tiny
vocabularies.  Draft strings are enumerated with their proposal probability,
each position is accepted with probability min(1, p/q), the first rejected
position is redrawn from the normalised positive residual max(0, p - q), and a
bonus token is drawn from the target when every candidate passes.  Used only
to pin the fp64 oracle and the entry's worked example.

Distributions are given per position and do not depend on the prefix (the
one-step argument of the rule does not need prefix dependence).
"""
from __future__ import annotations

from fractions import Fraction
from itertools import product


def as_fractions(dist):
    return [Fraction(x) for x in dist]


def alpha(p_x: Fraction, q_x: Fraction) -> Fraction:
    """min(1, p/q); for q = 0: 1 if p > 0 else 0."""
    if q_x > 0:
        return min(Fraction(1), p_x / q_x)
    return Fraction(1) if p_x > 0 else Fraction(0)


def residual(p, q):
    """Normalised positive residual max(0, p - q); p itself if it has no mass."""
    r = [max(Fraction(0), a - b) for a, b in zip(p, q)]
    s = sum(r)
    if s == 0:
        return list(p)
    return [x / s for x in r]


def output_law(ps, qs):
    """Law of the emitted token string.  ``ps``: k+1 target distributions
    (position k is the bonus), ``qs``: k proposal distributions.  Returns a
    dict mapping the emitted tuple (accepted drafts + one corrected or bonus
    token) to its probability."""
    k = len(qs)
    assert len(ps) == k + 1
    ps = [as_fractions(p) for p in ps]
    qs = [as_fractions(q) for q in qs]
    law = {}

    def add(key, pr):
        if pr:
            law[key] = law.get(key, Fraction(0)) + pr

    def walk(j, prefix, pr):
        if j == k:
            for t, pt in enumerate(ps[k]):
                add(prefix + (t,), pr * pt)
            return
        res = residual(ps[j], qs[j])
        for x, qx in enumerate(qs[j]):
            if qx == 0:
                continue
            a = alpha(ps[j][x], qx)
            if a > 0:
                walk(j + 1, prefix + (x,), pr * qx * a)
            if a < 1:
                for t, rt in enumerate(res):
                    add(prefix + (t,), pr * qx * (1 - a) * rt)

    walk(0, (), Fraction(1))
    return law


def position_marginal(law, j, V):
    """P(the output has a token at position j and it equals t), t < V."""
    out = [Fraction(0)] * V
    for seq, pr in law.items():
        if len(seq) > j:
            out[seq[j]] += pr
    return out


def conditional_laws(law, j, V):
    """For every prefix of length j that the output can carry, the law of the
    token at position j given that prefix (and that position j exists)."""
    by_prefix = {}
    for seq, pr in law.items():
        if len(seq) > j:
            by_prefix.setdefault(seq[:j], [Fraction(0)] * V)[seq[j]] += pr
    out = {}
    for prefix, v in by_prefix.items():
        s = sum(v)
        out[prefix] = [x / s for x in v]
    return out


def acceptance_rate(p, q):
    """Probability that one position is accepted: sum over x of q(x) alpha(x)."""
    p, q = as_fractions(p), as_fractions(q)
    return sum((qx * alpha(px, qx) for px, qx in zip(p, q)), Fraction(0))


def all_strings(V, k):
    return product(range(V), repeat=k)
