"""Pins for the CPU oracle: facts fixed by the pages or by mathematics, not by
the oracle itself.  Each ``pin_*`` takes an ``oracle.Oracle`` handle and raises
AssertionError when the handle disagrees, so the same pins run against the
real oracle (test_oracle_pins.py) and against copies with planted mistakes
(test_oracle_mutations.py).

Sources: the encyclopedia entry "Speculative decoding" (glopedia, 推测解码),
section "Basic steps of proposal and verification" (提议与核验的基本步骤): the
ratio test, first-rejection stop, normalised positive residual, bonus token,
the three-token worked example, the greedy rule and the requirement that
temperature / top-k / nucleus settings apply to both distributions.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import scipy.special
import scipy.stats

from oracle import exact
from workloads import to_bf16_bits, worked_example

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ONE_BITS = 0x3F800000  # float32 1.0


def f32_of_bits(b: int) -> float:
    return float(np.array([b], np.uint32).view(np.float32)[0])


def first_true(pred) -> float:
    """Smallest float32 u in [0, 1) with pred(u) true (1.0 if none); pred must
    be monotone (false ... false true ... true) over [0, 1)."""
    lo, hi = 0, ONE_BITS
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(f32_of_bits(mid)):
            hi = mid
        else:
            lo = mid + 1
    return f32_of_bits(lo)


def _run(orc, target, draft, tokens, u):
    return orc.verify_stochastic(target, draft, np.array([tokens], np.int32),
                                 np.array([u], np.float32))


# ---------------------------------------------------------------------------
def pin_worked_example(orc):
    """The entry's example: p = (0.6, 0.3, 0.1), q = (0.5, 0.4, 0.1), B drafted
    with probability 0.4, accepted with probability 0.75, residual all on A,
    combined totals 0.6 / 0.3 / 0.1."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    target, draft, tokens = worked_example()
    ok, p, _ = orc.process_row(target[0, 0])
    assert ok and np.allclose(p, g["target"], atol=1e-7), p
    ok, q, _ = orc.process_row(draft[0, 0])
    assert ok and np.allclose(q, g["proposal"], atol=1e-7), q
    assert abs(q[g["drafted_token"]] - g["probability_of_drafting_it"]) < 1e-7
    r = orc.verify_stochastic(target, draft, tokens, np.array([[0.5, 0.5]], np.float32))
    assert abs(r["accept_prob"][0, 0] - g["accept_probability"]) < 1e-6, r["accept_prob"]
    # Accepted (u0 < 0.75): B kept, then the bonus drawn from the target.
    assert r["accepted_len"][0] == 1 and r["out_tokens"][0, 0] == 1
    for u1, want in ((0.0, 0), (0.59, 0), (0.61, 1), (0.89, 1), (0.91, 2), (0.999, 2)):
        r = orc.verify_stochastic(target, draft, tokens, np.array([[0.1, u1]], np.float32))
        assert list(r["out_tokens"][0]) == [1, want], (u1, r["out_tokens"])
    # Rejected (u0 >= 0.75): the residual holds only A's 0.1 gap -> always A.
    for u0 in (0.7500001, 0.8, 0.99):
        for u1 in (0.0, 0.25, 0.5, 0.75, 0.999):
            r = orc.verify_stochastic(target, draft, tokens, np.array([[u0, u1]], np.float32))
            assert r["accepted_len"][0] == 0 and r["out_tokens"][0, 0] == 0, (u0, u1, r)
    # Measured acceptance region of the decision map is [0, 0.75).
    a = first_true(lambda u0: _run(orc, target, draft, [1], [u0, 0.0])["accepted_len"][0] == 0)
    assert abs(a - 0.75) < 1e-6, a
    # Exact law of accept + correct equals the printed totals.
    law = exact.output_law([g["target"], g["target"]], [g["proposal"]])
    first = exact.position_marginal(law, 0, 3)
    assert [float(x) for x in first] == g["combined_law"]
    assert exact.alpha(Fraction(3, 10), Fraction(4, 10)) == Fraction(3, 4)
    assert exact.residual([Fraction(6, 10), Fraction(3, 10), Fraction(1, 10)],
                          [Fraction(5, 10), Fraction(4, 10), Fraction(1, 10)]) == \
        [Fraction(1), Fraction(0), Fraction(0)]


# ---------------------------------------------------------------------------
def map_law(orc, target, draft, T=1.0, top_k=0, top_p=1.0):
    """Law of the position-0 token and of the bonus token (given acceptance)
    of the oracle's decision map for k = 1, measured by bisection on the
    float32 uniforms (accept region and CDF breakpoints)."""
    V = target.shape[2]

    def run(x, u0, u1):
        return orc.verify_stochastic(target, draft, np.array([[x]], np.int32),
                                     np.array([[u0, u1]], np.float32), T, top_k, top_p)

    ok, q, _ = orc.process_row(draft[0, 0], T, top_k, top_p)
    assert ok
    law0 = np.zeros(V)
    bonus = None
    u_reject = f32_of_bits(ONE_BITS - 1)
    for x in range(V):
        if q[x] == 0:
            continue
        a = first_true(lambda u0: run(x, u0, 0.0)["accepted_len"][0] == 0)
        law0[x] += q[x] * a
        if a < 1.0:
            cuts = [0.0] + [first_true(lambda u1, t=t: run(x, u_reject, u1)["out_tokens"][0, 0] >= t)
                            for t in range(1, V)] + [1.0]
            law0 += q[x] * (1.0 - a) * np.diff(cuts)
        if a > 0.0 and bonus is None:
            cuts = [0.0] + [first_true(lambda u1, t=t: run(x, 0.0, u1)["out_tokens"][0, 1] >= t)
                            for t in range(1, V)] + [1.0]
            bonus = np.diff(cuts)
    return law0, bonus


def pin_law_of_decision_map(orc):
    """Accept + correct reproduces the target's law at the drafted position and
    the bonus is drawn from the target's next distribution (distribution
    preservation, 'Concept and scope' and 'Basic steps' sections)."""
    rs = np.random.default_rng(7)
    cases = [(3, 1.0, 0, 1.0), (4, 1.0, 0, 1.0), (5, 0.6, 0, 1.0), (4, 1.0, 2, 1.0),
             (5, 1.3, 0, 0.7), (5, 1.0, 3, 0.8)]
    for V, T, top_k, top_p in cases:
        t0 = rs.normal(0, 1.5, V).astype(np.float32)
        t1 = rs.normal(0, 1.5, V).astype(np.float32)
        d0 = (t0 + rs.normal(0, 1.0, V)).astype(np.float32)
        target = np.stack([t0, t1])[None]
        draft = d0[None, None]
        law0, bonus = map_law(orc, target, draft, T, top_k, top_p)
        _, p0, _ = orc.process_row(t0, T, top_k, top_p)
        _, p1, _ = orc.process_row(t1, T, top_k, top_p)
        assert np.allclose(law0, p0, atol=2e-6), (V, T, top_k, top_p, law0, p0)
        assert bonus is not None and np.allclose(bonus, p1, atol=2e-6), (bonus, p1)


# ---------------------------------------------------------------------------
def brute_force_probs(l: np.ndarray, T: float, top_k: int, top_p: float):
    """Temperature -> top-k -> top-p by a full sort (numpy), then softmax over
    the kept set.  Returns (probs, distance of the cut's cumulative masses to
    top_p, or inf when top-p is off)."""
    l = l.astype(np.float64)
    V = l.size
    keep = np.ones(V, bool)
    if 0 < top_k < V:
        tk = np.sort(l)[::-1][top_k - 1]
        keep &= l >= tk
    gap = np.inf
    if top_p < 1.0:
        vals = np.sort(l[keep])[::-1]
        w = scipy.special.softmax((vals - vals[0]) / T)
        c = np.cumsum(w)
        cut = int(np.argmax(c >= top_p)) if np.any(c >= top_p) else vals.size - 1
        tp = vals[cut]
        keep &= l >= tp
        gap = min(abs(w[vals > tp].sum() - top_p), abs(w[vals >= tp].sum() - top_p))
    z = np.where(keep, (l - l.max()) / T, -np.inf)
    return scipy.special.softmax(z), gap


def pin_softmax_and_filters(orc):
    """Processed probabilities equal a library softmax over the set a full
    sort keeps (temperature, top-k with ties kept, top-p over the top-k-
    renormalised probabilities), for fp32 and bf16 rows."""
    rs = np.random.default_rng(11)
    for trial in range(60):
        V = int(rs.integers(2, 400))
        l = rs.normal(0, rs.uniform(0.5, 4.0), V).astype(np.float32)
        if trial % 3 == 0:
            l = np.round(l * 2) / 2  # many ties
        if trial % 5 == 0:
            l[rs.integers(0, V, size=max(1, V // 10))] = -np.inf
        if not np.isfinite(l).any():
            l[0] = 0.0
        T = float(rs.choice([0.3, 0.7, 1.0, 1.9]))
        top_k = int(rs.choice([0, 1, 2, 5, 50, V, V + 3]))
        top_p = float(rs.choice([1.0, 0.95, 0.9, 0.5, 0.2]))
        for dtype in ("f32", "bf16"):
            row = to_bf16_bits(l) if dtype == "bf16" else l
            lf = (row.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else l
            want, gap = brute_force_probs(lf, T, top_k, top_p)
            if gap < 1e-9:
                continue
            ok, got, st = orc.process_row(row, T, top_k, top_p)
            assert ok
            assert np.allclose(got, want, rtol=1e-12, atol=1e-15), (trial, dtype, T, top_k, top_p)
            kept = want > 0
            zk = (lf.astype(np.float64) - lf.max()) / T
            assert abs(st["log_norm"] - scipy.special.logsumexp(zk[kept])) < 1e-12
            assert st["max_logit"] == lf.max()


# ---------------------------------------------------------------------------
def pin_acceptance_rate(orc):
    """The per-position acceptance probability sum_x q(x) min(1, p/q) equals
    sum_x min(p(x), q(x)) (one line from the ratio test)."""
    rs = np.random.default_rng(3)
    for _ in range(10):
        V = int(rs.integers(3, 60))
        t = rs.normal(0, 2, (1, 2, V)).astype(np.float32)
        d = (t[:, :1] + rs.normal(0, 1, (1, 1, V))).astype(np.float32)
        p = scipy.special.softmax(t[0, 0].astype(np.float64))
        q = scipy.special.softmax(d[0, 0].astype(np.float64))
        alphas = np.array([orc.verify_stochastic(t, d, np.array([[x]]),
                                                 np.array([[0.5, 0.5]], np.float32))
                           ["accept_prob"][0, 0] for x in range(V)])
        assert abs((q * alphas).sum() - np.minimum(p, q).sum()) < 1e-12


# ---------------------------------------------------------------------------
def inverse_cdf_numpy(w: np.ndarray, u: float) -> int:
    c = np.cumsum(w)
    return int(np.searchsorted(c, u * c[-1], side="right"))


def pin_special_cases(orc):
    """q = p always accepts and draws the bonus by inverse CDF; disjoint
    supports always reject at position 0 and draw from p_0; a rejected draft
    token is never redrawn; zero-mass tokens are never emitted; every
    position after the first rejection is discarded."""
    rs = np.random.default_rng(5)
    B, k, V = 40, 3, 50
    t = rs.normal(0, 2, (B, k + 1, V)).astype(np.float32)
    u = rs.random((B, k + 1)).astype(np.float32)
    # q = p: the draft logits are the target's.
    toks = np.array([[orc.sample_row(t[b, j], rs.random()) for j in range(k)] for b in range(B)])
    r = orc.verify_stochastic(t, t[:, :k].copy(), toks, u)
    assert (r["accepted_len"] == k).all()
    assert np.all(r["accept_prob"] == 1.0)
    for b in range(B):
        pk = scipy.special.softmax(t[b, k].astype(np.float64))
        assert r["out_tokens"][b, k] == inverse_cdf_numpy(pk, float(u[b, k]))
        assert list(r["out_tokens"][b, :k]) == list(toks[b])
    # Disjoint supports: target only on even ids, draft only on odd ids.
    te, do = t.copy(), rs.normal(0, 2, (B, k, V)).astype(np.float32)
    te[:, :, 1::2] = -np.inf
    do[:, :, 0::2] = -np.inf
    toks = np.array([[1 + 2 * int(rs.integers(0, V // 2)) for _ in range(k)] for _ in range(B)])
    u2 = u.copy()
    u2[:5, 0] = 0.0  # alpha = 0 must reject even for u = 0
    r = orc.verify_stochastic(te, do, toks, u2)
    assert (r["accepted_len"] == 0).all()
    for b in range(B):
        p0 = scipy.special.softmax(te[b, 0].astype(np.float64))
        assert r["out_tokens"][b, 0] == inverse_cdf_numpy(p0, float(u2[b, k]))
        assert (r["out_tokens"][b, 1:] == -1).all()
    # q(x) = 0 (draft logit -inf) takes the limit of min(1, p/q) as q -> 0+:
    # the same decision as a draft logit 80 below the rest (q ~ e^-80).
    for b in range(5):
        dz = (t[b:b + 1, :k] + rs.normal(0, 1, (1, k, V))).astype(np.float32)
        dlim = dz.copy()
        dz[0, 0, 7] = -np.inf
        dlim[0, 0, 7] = dz[0, 0].max() - 80.0
        tk = np.array([[7] + [0] * (k - 1)], np.int32)
        for uu in (0.0, 0.5, 0.999):
            uv = np.array([[uu] * (k + 1)], np.float32)
            r0 = orc.verify_stochastic(t[b:b + 1], dz, tk, uv)
            r1 = orc.verify_stochastic(t[b:b + 1], dlim, tk, uv)
            assert r0["accept_prob"][0, 0] == r1["accept_prob"][0, 0] == 1.0
            assert r0["accepted_len"][0] >= 1 and r1["accepted_len"][0] >= 1
    # A zero-mass token at index 0 is never drawn, even with u = 0.
    tz = t.copy()
    tz[:, :, 0] = -np.inf
    uz = u.copy()
    uz[:, k] = 0.0
    d = (tz[:, :k] + rs.normal(0, 1, (B, k, V))).astype(np.float32)
    toks = np.array([[orc.sample_row(d[b, j], rs.random()) for j in range(k)] for b in range(B)])
    r = orc.verify_stochastic(tz, d, toks, uz)
    n = r["accepted_len"]
    assert (r["out_tokens"][np.arange(B), n] != 0).all()
    # Rejected draft token never redrawn; first rejection ends the round.
    d = (t[:, :k] + rs.normal(0, 1.5, (B, k, V))).astype(np.float32)
    for trial in range(5):
        toks = np.array([[orc.sample_row(d[b, j], rs.random()) for j in range(k)]
                         for b in range(B)])
        uu = rs.random((B, k + 1)).astype(np.float32)
        r = orc.verify_stochastic(t, d, toks, uu)
        for b in range(B):
            nb = r["accepted_len"][b]
            a = r["accept_prob"][b]
            want_n = next((j for j in range(k) if not uu[b, j] < a[j]), k)
            assert nb == want_n, (b, nb, want_n, a, uu[b])
            if nb < k:
                assert r["out_tokens"][b, nb] != toks[b, nb]
            assert (r["out_tokens"][b, nb + 1:] == -1).all()


# ---------------------------------------------------------------------------
def pin_greedy(orc):
    """Greedy: compare with the target's most probable token (first maximum on
    ties), replace the first mismatch, bonus argmax when all match."""
    rs = np.random.default_rng(9)
    B, k, V = 30, 4, 64
    t = np.round(rs.normal(0, 1, (B, k + 1, V)) * 2).astype(np.float32) / 2  # ties
    am = t.argmax(axis=2)  # numpy returns the first maximum
    toks = am[:, :k].copy()
    flip = rs.random((B, k)) < 0.3
    toks[flip] = (toks[flip] + 1 + rs.integers(0, V - 1, flip.sum())) % V
    acc, out = orc.verify_greedy(t, toks)
    for b in range(B):
        n = next((j for j in range(k) if toks[b, j] != am[b, j]), k)
        assert acc[b] == n
        assert list(out[b, :n]) == list(toks[b, :n]) and out[b, n] == am[b, n]
        assert (out[b, n + 1:] == -1).all()
    for b in range(B):
        assert orc.argmax_row(t[b, 0]) == am[b, 0]
    # bf16 rows: the same first-maximum rule on the decoded values.
    tb = to_bf16_bits(t)
    acc2, out2 = orc.verify_greedy(tb, toks)
    assert (acc2 == acc).all() and (out2 == out).all()


# ---------------------------------------------------------------------------
def pin_bf16_decode(orc):
    """bf16 logits are decoded exactly: the same probabilities as the float32
    values torch's bfloat16 type decodes them to."""
    import torch
    rs = np.random.default_rng(13)
    x = rs.normal(0, 3, 997).astype(np.float32)
    bits = to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64), ref)
    ok, p_b, st = orc.process_row(bits, 0.7)
    ok2, p_f, st2 = orc.process_row(ref.astype(np.float32), 0.7)
    assert ok and ok2 and np.array_equal(p_b, p_f)
    assert st["max_logit"] == ref.max()
    assert np.allclose(p_b, scipy.special.softmax(ref / 0.7), rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------
def pin_invalid_inputs(orc):
    """NaN, +inf and rows without a finite logit make a row invalid, a draft
    token outside [0, V) makes its position ill-formed, and -inf is only a
    mask.  The walk over positions stops at the first rejection (the pages'
    first-rejection stop), so only what it consults before stopping can make
    the sequence invalid (accepted length -1)."""
    rs = np.random.default_rng(17)
    B, k, V = 10, 2, 16
    t = rs.normal(0, 1, (B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rs.normal(0, 1, (B, k, V))).astype(np.float32)
    # accept every consulted position (u = 0 and p(x) > 0 at the argmax) ...
    toks = np.argmax(t[:, :k], axis=2).astype(np.int32)
    u = np.zeros((B, k + 1), np.float32)
    u[:, k] = 0.5
    # ... except where a rejection at position 0 is forced: x masked in p
    reject0 = [1, 3, 7, 9]
    for b in reject0:
        t[b, 0, 0] = -np.inf
        toks[b, 0] = 0
    t[0, 1, 3] = np.nan          # consulted (position 0 passes): invalid
    t[1, 1, 3] = np.nan          # past the stop: valid, n = 0
    d[2, 0, :] = -np.inf         # draft row without a finite logit: invalid
    toks[3, 1] = V               # out of range past the stop: valid
    toks[4, 0] = -1              # out of range at position 0: invalid
    t[5, 0, 8:] = -np.inf        # masking only: valid
    toks[5, 0] = np.argmax(t[5, 0])
    t[6, k, 2] = np.inf          # bonus row consulted (all pass): invalid
    t[7, k, 2] = np.inf          # bonus row not consulted: valid
    d[8, 1, 5] = np.inf          # draft row at a consulted position: invalid
    d[9, 1, 5] = np.nan          # draft row past the stop: valid
    r = orc.verify_stochastic(t, d, toks, u)
    expect = [-1, 0, -1, 0, -1, k, -1, 0, -1, 0]
    assert list(r["accepted_len"]) == expect, list(r["accepted_len"])
    for b in range(B):
        if expect[b] < 0:
            assert (r["out_tokens"][b] == -1).all()
        else:
            n = expect[b]
            assert 0 <= r["out_tokens"][b, n] < V and (r["out_tokens"][b, n + 1:] == -1).all()
    # alpha is reported at every position, NaN exactly where it is ill-formed
    ap = r["accept_prob"]
    ill = np.zeros((B, k), bool)
    ill[0, 1] = ill[1, 1] = ill[2, 0] = ill[3, 1] = ill[4, 0] = ill[8, 1] = ill[9, 1] = True
    assert np.array_equal(np.isnan(ap), ill)
    assert (ap[reject0, 0] == 0).all()
    # a rejected position resamples from the residual, which here holds the
    # positive part of p - q over the unmasked tokens
    assert r["out_tokens"][1, 0] != 0
    # greedy walks the same way: mismatch at 0 where the token is not the argmax
    acc, out = orc.verify_greedy(t, toks)
    assert list(acc) == [-1, 0, k, 0, -1, k, -1, 0, k, 0], list(acc)
    assert out[2, k] == np.argmax(t[2, k]) and out[1, 0] == np.argmax(t[1, 0])
    ok, p, _ = orc.process_row(t[5, 0])
    assert ok and (p[8:] == 0).all() and abs(p.sum() - 1) < 1e-12
    ok, _, _ = orc.process_row(t[0, 1])
    assert not ok


# ---------------------------------------------------------------------------
def pin_boundary_flags(orc):
    """The boundary detector flags draws within 1e-6 of a decision and leaves
    draws far from every decision unflagged."""
    target, draft, tokens = worked_example()
    a = orc.verify_stochastic(target, draft, tokens, np.array([[0.5, 0.5]], np.float32))
    alpha = a["accept_prob"][0, 0]
    r = orc.verify_stochastic(target, draft, tokens, np.array([[alpha, 0.3]], np.float32))
    assert r["flags"][0] & 1
    r = orc.verify_stochastic(target, draft, tokens, np.array([[0.1, 0.6]], np.float32))
    assert r["flags"][0] & 2  # 0.6 is the first bonus breakpoint
    r = orc.verify_stochastic(target, draft, tokens, np.array([[0.1, 0.3]], np.float32))
    assert r["flags"][0] == 0


# ---------------------------------------------------------------------------
def cut_masses(l: np.ndarray, T: float, top_k: int, top_p: float):
    """Brute force of the top-p cut over distinct values (numpy): with pi the
    probabilities renormalised over the top-k set, M(v) = sum of pi over
    logits >= v.  The cut is the largest distinct value v with M(v) >= top_p
    (the shortest descending prefix that reaches top_p, ties kept; the lowest
    value if rounding leaves none).  Returns (mass strictly above the cut, mass
    at or above it)."""
    l = l.astype(np.float64)
    keep = np.ones(l.size, bool)
    if 0 < top_k < l.size:
        keep &= l >= np.sort(l)[::-1][top_k - 1]
    kept = l[keep]
    w = np.exp((kept - kept.max()) / T)
    w /= w.sum()
    vals = np.unique(kept)[::-1]  # distinct values, descending
    M = np.array([w[kept >= v].sum() for v in vals])
    reach = np.nonzero(M >= top_p)[0]
    i = int(reach[0]) if reach.size else vals.size - 1
    above = float(M[i - 1]) if i > 0 else 0.0
    return above, float(M[i])


def _near_cut(above, at, top_p):
    return abs(above - top_p) <= 1e-6 or abs(at - top_p) <= 1e-6


def pin_topp_boundary_flag(orc):
    """Flag bit 2 (a top-p cut mass within 1e-6 of top_p): the oracle's masses
    strictly above and at its cut equal the distinct-value brute force, and
    the flag of a sequence whose rows are all the given row is set exactly
    when one of those masses lies within 1e-6 of top_p.  Random rows (mostly
    far from a boundary), rows whose top_p is placed at a cumulative boundary
    plus an offset from -5e-6 to 5e-6, rows with ties at the cut, and top-k
    followed by top-p."""
    rs = np.random.default_rng(97)
    cases = []
    for trial in range(30):  # random rows
        V = int(rs.integers(3, 300))
        l = rs.normal(0, rs.choice([0.5, 1.0, 3.0]), V).astype(np.float32)
        cases.append((l, float(rs.choice([0.7, 1.0, 1.5])), int(rs.choice([0, 0, 5, 40])),
                      float(rs.uniform(0.3, 0.99))))
    for trial in range(36):  # top_p at a cumulative boundary plus an offset
        V = int(rs.integers(4, 200))
        l = rs.normal(0, 1.5, V).astype(np.float32)
        if trial % 3 == 0:
            l = np.round(l * 4) / 4  # ties at the cut
        T = float(rs.choice([0.8, 1.0]))
        top_k = int(rs.choice([0, 0, 10]))
        kept = l.astype(np.float64)
        if 0 < top_k < V:
            kept = kept[kept >= np.sort(kept)[::-1][top_k - 1]]
        w = np.exp((kept - kept.max()) / T)
        w /= w.sum()
        vals = np.unique(kept)[::-1]
        M = np.array([w[kept >= v].sum() for v in vals])
        inner = M[(M > 0.05) & (M < 0.95)]
        if inner.size == 0:
            continue
        off = [-5e-6, -1.5e-6, -8e-7, -3e-7, 0.0, 3e-7, 8e-7, 1.5e-6, 5e-6][trial % 9]
        cases.append((l, T, top_k, float(rs.choice(inner)) + off))
    n_near = n_far = 0
    for l, T, top_k, top_p in cases:
        above, at = cut_masses(l, T, top_k, top_p)
        d = min(abs(above - top_p), abs(at - top_p))
        if abs(d - 1e-6) < 1e-10:
            continue  # rounding could decide either way right at the bound
        ok, _, st = orc.process_row(l, T, top_k, top_p)
        assert ok
        if abs(at - top_p) > 1e-12:  # else either cut is right to the last bit (both near)
            assert abs(st["mass_above_cut"] - above) < 1e-12, (st, above, at, top_p)
            assert abs(st["mass_at_cut"] - at) < 1e-12, (st, above, at, top_p)
        # k = 1, every row the same row: q = p, so the draft is accepted and
        # the target rows 0 and 1 and the draft row 0 are all consulted
        tb = np.broadcast_to(l, (1, 2, l.size))
        db = np.broadcast_to(l, (1, 1, l.size))
        tok = int(np.argmax(l))
        r = orc.verify_stochastic(tb, db, np.array([[tok]], np.int32),
                                  np.array([[0.5, 0.5]], np.float32), T, top_k, top_p)
        assert r["accepted_len"][0] == 1
        near = _near_cut(above, at, top_p)
        assert bool(r["flags"][0] & 4) == near, (above, at, top_p, r["flags"][0])
        n_near += near
        n_far += not near
    assert n_near >= 15 and n_far >= 35, (n_near, n_far)
    # top-p off: no cut, no flag
    l = rs.normal(0, 1, 50).astype(np.float32)
    r = orc.verify_stochastic(np.broadcast_to(l, (1, 2, 50)), np.broadcast_to(l, (1, 1, 50)),
                              np.array([[0]], np.int32), np.array([[0.5, 0.5]], np.float32))
    assert r["flags"][0] & 4 == 0


# ---------------------------------------------------------------------------
def pin_chi_square(orc, n=1_000_000):
    """10^6 draws of the worked example: the emitted first token follows the
    target law (0.6, 0.3, 0.1) (chi-square, p-value >= 1e-3 at a fixed seed)."""
    target, draft, _ = worked_example()
    rs = np.random.default_rng(2024)
    ok, q, _ = orc.process_row(draft[0, 0])
    toks = rs.choice(3, size=(n, 1), p=q / q.sum()).astype(np.int32)
    u = rs.random((n, 2)).astype(np.float32)
    tb = np.broadcast_to(target, (n, 2, 3))
    db = np.broadcast_to(draft, (n, 1, 3))
    r = orc.verify_stochastic(tb, db, toks, u)
    counts = np.bincount(r["out_tokens"][:, 0], minlength=3)
    _, pval = scipy.stats.chisquare(counts, np.array([0.6, 0.3, 0.1]) * n)
    assert pval >= 1e-3, (counts, pval)
    acc = r["accepted_len"].mean()
    assert abs(acc - 0.9) < 0.003, acc  # P(accept) = sum min(p, q) = 0.5 + 0.3 + 0.1


# ---------------------------------------------------------------------------
def pin_pooled_rows(orc):
    """Pooled rows (sequences naming shared rows through maps).  The worked
    example's rows held once and shared by four branches give the outcomes
    the example fixes for each branch's draft and draws; out-of-range map
    entries count only where the walk consults them; relabelling the pool
    rows (with the maps) changes nothing."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    target, draft, _ = worked_example()
    tpool = np.ascontiguousarray(np.stack([target[0, 0], target[0, 0]]))  # row 1: bonus row (= p)
    dpool = np.ascontiguousarray(draft[0, :1])
    tmap = [[0, 1]] * 4 + [[0, 5], [0, 5], [0, 1], [7, 1]]
    dmap = [[0]] * 6 + [[-1], [0]]
    toks = [[1], [1], [0], [2], [1], [1], [1], [1]]
    u = [[0.7, 0.0], [0.8, 0.5], [0.99, 0.3], [0.999, 0.95],
         [0.7, 0.0], [0.8, 0.5], [0.1, 0.1], [0.1, 0.1]]
    r = orc.verify_stochastic_pooled(tpool, np.array(tmap), dpool, np.array(dmap),
                                     np.array(toks, np.int32), np.array(u, np.float32))
    # B: alpha 0.3 / 0.4 = 0.75 (accept at 0.7, reject at 0.8, residual all on
    # A); A: 0.6 / 0.5 >= 1; C: 0.1 / 0.1 = 1; bonus draws from p by inverse CDF
    assert abs(r["accept_prob"][0, 0] - g["accept_probability"]) < 1e-6
    assert list(r["accepted_len"]) == [1, 0, 1, 1, -1, 0, -1, -1], r["accepted_len"]
    assert [list(x) for x in r["out_tokens"][:4]] == [[1, 0], [0, -1], [0, 0], [2, 2]]
    assert list(r["out_tokens"][5]) == [0, -1]
    assert np.isnan(r["accept_prob"][6, 0]) and np.isnan(r["accept_prob"][7, 0])
    # relabelling: the same sequences through permuted pools and maps
    rs = np.random.default_rng(61)
    B, k, V, Pt, Pd = 12, 3, 7, 9, 8
    tp = rs.normal(0, 1.5, (Pt, V)).astype(np.float32)
    dp = rs.normal(0, 1.5, (Pd, V)).astype(np.float32)
    tm = rs.integers(0, Pt, (B, k + 1))
    dm = rs.integers(0, Pd, (B, k))
    toks = rs.integers(0, V, (B, k)).astype(np.int32)
    u = rs.random((B, k + 1)).astype(np.float32)
    a = orc.verify_stochastic_pooled(tp, tm, dp, dm, toks, u, 0.9, 0, 0.9)
    pt, pd = rs.permutation(Pt), rs.permutation(Pd)
    b = orc.verify_stochastic_pooled(tp[pt], np.argsort(pt)[tm], dp[pd], np.argsort(pd)[dm],
                                     toks, u, 0.9, 0, 0.9)
    for key in ("accepted_len", "out_tokens", "flags"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["accept_prob"], b["accept_prob"])
    # two sequences naming the same rows with the same tokens and draws agree,
    # and the draft map is not the target map
    tm[1], dm[1], toks[1], u[1] = tm[0], dm[0], toks[0], u[0]
    c = orc.verify_stochastic_pooled(tp, tm, dp, dm, toks, u, 0.9, 0, 0.9)
    assert np.array_equal(c["out_tokens"][0], c["out_tokens"][1])
    assert np.array_equal(c["accept_prob"][0], c["accept_prob"][1])
    # greedy over pooled one-hot rows: argmaxes 2, 0, 3, 1 for pool rows 0..3
    gp = np.full((4, 4), -1.0, np.float32)
    for i, x in enumerate([2, 0, 3, 1]):
        gp[i, x] = 2.0
    gm = [[0, 1, 2], [0, 3, 2], [1, 1, 1], [0, 1, 2], [0, 1, 9], [0, 1, 9]]
    gt = [[2, 0], [2, 1], [0, 0], [1, 0], [2, 0], [2, 1]]
    acc, out = orc.verify_greedy_pooled(gp, np.array(gm), np.array(gt, np.int32))
    assert list(acc) == [2, 2, 2, 0, -1, 1], acc
    assert [list(x) for x in out] == [[2, 0, 3], [2, 1, 3], [0, 0, 0], [2, -1, -1],
                                      [-1, -1, -1], [2, 0, -1]], out


# ---------------------------------------------------------------------------
def pin_outcome_lookup(orc, lookup=None):
    """Predicted-outcome lookup on the worked example's outcomes: drafting B
    and drawing u0 = 0.8 rejects it and emits A (outcome (0, A)); u0 = 0.7
    accepts it and the bonus draw u1 = 0 from p emits A (outcome (1, A)).
    First match wins, empty entries never match, an invalid sequence never
    hits."""
    import oracle as _oracle
    lookup = lookup or _oracle.outcome_lookup
    target, draft, _ = worked_example()
    tt = np.ascontiguousarray(np.broadcast_to(target, (3, 2, 3)))
    dd = np.ascontiguousarray(np.broadcast_to(draft, (3, 1, 3)))
    toks = np.array([[1], [1], [7]], np.int32)  # sequence 2: token out of range (invalid)
    u = np.array([[0.8, 0.5], [0.7, 0.0], [0.1, 0.1]], np.float32)
    r = orc.verify_stochastic(tt, dd, toks, u)
    assert list(r["accepted_len"]) == [0, 1, -1]
    assert [list(x) for x in r["out_tokens"][:2]] == [[0, -1], [1, 0]]
    pred_len = np.array([[1, 0, 0, -1], [0, 1, 1, 1], [-1, 0, 1, -1]], np.int32)
    pred_tok = np.array([[0, 1, 0, 0], [0, 2, 0, 0], [-1, 0, 0, -1]], np.int32)
    hits, count = lookup(r["accepted_len"], r["out_tokens"], pred_len, pred_tok)
    assert list(hits) == [2, 2, -1], hits
    assert count == 2
    # a miss, and an empty entry (length -1) that names the outcome's token
    hits, count = lookup(r["accepted_len"][:1], r["out_tokens"][:1], np.array([[-1, 1, 0]]),
                         np.array([[0, 0, 1]]))
    assert list(hits) == [-1] and count == 0


# ---------------------------------------------------------------------------
def pin_logits_processors(orc, apply=None):
    """Processors the rule requires to be in force on both sides: a masked
    token gets -inf (probability 0 after processing), a penalised token
    l / theta for l > 0 and l * theta otherwise (the repetition-penalty
    reading), NaN passes unchanged; bf16 output rounds to nearest even; no
    mask and theta = 1 change nothing."""
    import oracle as _oracle
    apply = apply or _oracle.apply_processors
    l = np.array([[[2.0, -2.0, 3.0, -1.5, 0.0, np.nan, 1.00390625, 5.0]]], np.float32)
    allow = np.array([[[0b11111011]]], np.uint32)   # token 2 masked
    pen = np.array([[[0b00110011]]], np.uint32)     # tokens 0, 1, 4, 5 penalised
    got = apply(l, allow, pen, 2.0)
    want = np.array([1.0, -4.0, -np.inf, -1.5, 0.0, np.nan, 1.00390625, 5.0], np.float32)
    assert np.array_equal(got[0, 0], want, equal_nan=True), got
    # ties to even: 1 + 2^-8 -> 1.0 (0x3F80); 1 + 3 * 2^-8 -> 1 + 2^-6 (0x3F82)
    b = apply(np.array([[[1.00390625, 1.01171875, -3.0]]], np.float32), None, None, 1.0, "bf16")
    assert list(b[0, 0]) == [0x3F80, 0x3F82, 0xC040], b
    rs = np.random.default_rng(5)
    x = rs.normal(0, 2, (2, 3, 70)).astype(np.float32)
    assert np.array_equal(apply(x, None, None, 1.0), x)
    # masked tokens get probability 0 after processing, and the rest renormalise
    m = np.zeros((1, 1, 3), np.uint32)
    m[0, 0, :] = 0xFFFFFFFF
    m[0, 0, 1] &= ~np.uint32(1 << 3)  # token 35 masked
    y = apply(x[:1, :1], m, None, 1.0)
    ok, p, _ = orc.process_row(y[0, 0])
    ok0, p0, _ = orc.process_row(x[0, 0])
    assert ok and ok0 and p[35] == 0.0
    keep = np.arange(70) != 35
    assert np.allclose(p[keep], p0[keep] / p0[keep].sum(), rtol=1e-12)


# ---------------------------------------------------------------------------
def _bf16_bits_exact(x):
    """bf16 bits of values exactly representable in bf16."""
    b = np.asarray(x, np.float32).view(np.uint32)
    assert ((b & 0xFFFF) == 0).all()
    return (b >> 16).astype(np.uint16)


def pin_lmhead_greedy(orc, greedy=None):
    """Greedy verify on LM-head logits: logits are the exact dot products of
    the bf16 inputs; the greedy rule takes the lowest index among equal
    maxima; a row with another logit within the fp32 summation bound of the
    largest is marked as a near tie, a clearly separated one is not."""
    import oracle as _oracle
    greedy = greedy or _oracle.lmhead_greedy
    d = 32
    w = np.zeros((4, d), np.float32)
    w[0, 0], w[1, 0], w[2, 0], w[3, 1] = 2.0, 3.0, 3.0, 1.0
    h = np.zeros((1, 3, d), np.float32)
    h[0, 0, 0] = 1.0            # logits 2, 3, 3, 0: tie between tokens 1 and 2
    h[0, 1, 1] = 5.0            # logits 0, 0, 0, 5
    h[0, 2, 0] = -1.0           # logits -2, -3, -3, 0
    hb, wb = _bf16_bits_exact(h), _bf16_bits_exact(w)
    L, S = _oracle.lmhead_logits(hb, wb)
    assert np.array_equal(L, [[2, 3, 3, 0], [0, 0, 0, 5], [-2, -3, -3, 0]])
    acc, out, near = greedy(hb, wb, np.array([[1, 3]], np.int32))
    assert list(acc) == [2] and list(out[0]) == [1, 3, 3], (acc, out)
    assert list(near[0]) == [True, False, False], near
    acc, out, near = greedy(hb, wb, np.array([[2, 3]], np.int32))  # 2 ties but 1 is first
    assert list(acc) == [0] and list(out[0]) == [1, -1, -1], (acc, out)
    acc, out, near = greedy(hb, wb, np.array([[1, 4]], np.int32))  # token outside V
    assert list(acc) == [-1]
    # near tie: the two logits differ by 2^-14 while large terms that cancel
    # in both make the sum of |products| ~3 x 10^4 (fp32 bound ~0.1); the
    # second row's gap of 2^-7 with |products| ~1 is clear
    w2 = np.ones((2, d), np.float32)
    w2[1, :2] = 1.0 + 2.0 ** -7
    h2 = np.zeros((1, 2, d), np.float32)
    h2[0, 0, 0], h2[0, 0, 1] = 1.0, -(1.0 - 2.0 ** -7)
    h2[0, 0, 2:] = np.tile([1024.0, -1024.0], (d - 2) // 2)
    h2[0, 1, 0] = 1.0
    acc, out, near = greedy(_bf16_bits_exact(h2), _bf16_bits_exact(w2), np.array([[1]], np.int32))
    assert list(near[0]) == [True, False], near
    assert list(out[0]) == [1, 1]


ALL_PINS = [pin_lmhead_greedy, pin_logits_processors, pin_outcome_lookup, pin_pooled_rows, pin_worked_example, pin_law_of_decision_map, pin_softmax_and_filters,
            pin_acceptance_rate, pin_special_cases, pin_greedy, pin_bf16_decode,
            pin_invalid_inputs, pin_boundary_flags, pin_topp_boundary_flag, pin_chi_square]
