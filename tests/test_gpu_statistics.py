"""Statistical checks of the GPU library over 10^6 draws, beyond its
element-by-element parity with the oracle.  With drafts drawn from q, the
token that accept-and-correct emits at a position follows the target law p
(the property the encyclopedia entry "Speculative decoding", section on the
basic steps of proposal and verification, states for the rule), and a
position is accepted with probability sum_x min(p(x), q(x)); with i.i.d.
positions the accepted length is geometric (truncated at k).  Checked on the
row-pass path (fp32 rows) and on the whole-sequence walk (bf16 batches),
with chi-square p-values >= 1e-3 at fixed seeds."""
from __future__ import annotations

import numpy as np
import pytest
import scipy.stats
import torch

import draft_token_verification_11_amd as sv
import oracle
import workloads
from tests.gpu_common import DEV, note, to_dev

pytestmark = pytest.mark.gpu

N = 1_000_000


def _verify(target, draft, toks, u, T=1.0, top_k=0, top_p=1.0):
    acc, out = sv.verify_stochastic(target, draft, torch.from_numpy(toks).to(DEV),
                                    torch.from_numpy(u).to(DEV), temperature=T, top_k=top_k,
                                    top_p=top_p)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def _chi(counts, probs):
    keep = probs > 0
    assert counts[~keep].sum() == 0, "a token of probability 0 was emitted"
    return scipy.stats.chisquare(counts[keep], probs[keep] / probs[keep].sum() * counts.sum())[1]


def test_worked_example_law_row_pass():
    """The three-token example (0.6, 0.3, 0.1) vs (0.5, 0.4, 0.1), one drafted
    position, fp32 logits broadcast to 10^6 sequences (seq_stride 0)."""
    target, draft, _ = workloads.worked_example()
    ok, p, _ = oracle.process_row(target[0, 0])
    ok2, q, _ = oracle.process_row(draft[0, 0])
    rs = np.random.default_rng(3001)
    toks = rs.choice(3, size=(N, 1), p=q / q.sum()).astype(np.int32)
    u = rs.random((N, 2)).astype(np.float32)
    tt = to_dev(target).expand(N, -1, -1)
    dd = to_dev(draft).expand(N, -1, -1)
    acc, out = _verify(tt, dd, toks, u)
    pval = _chi(np.bincount(out[:, 0], minlength=3), p)
    beta = float(np.minimum(p, q).sum())
    rate = float(acc.mean())
    note("row pass: emitted-token chi-square p=%.3g, acceptance %.5f vs %.5f" % (pval, rate, beta))
    assert pval >= 1e-3
    assert abs(rate - beta) <= 4 * np.sqrt(beta * (1 - beta) / N)


@pytest.mark.parametrize("top_p", [1.0, 0.85])
def test_walk_law_and_geometric_lengths(top_p):
    """bf16 rows of 16 tokens (4 live, 12 masked), k = 3 i.i.d. positions,
    10^6 sequences: the whole-sequence walk.  Emitted tokens follow p at
    every position; accepted lengths are geometric with ratio sum min(p, q)."""
    k, V = 3, 16
    lp = np.full(V, -np.inf, np.float32)
    lq = np.full(V, -np.inf, np.float32)
    lp[[2, 7, 11]] = np.log([0.55, 0.3, 0.15])
    lq[[2, 7, 11]] = np.log([0.35, 0.5, 0.15])
    lq[5] = np.log(0.05)  # a token only the draft proposes
    tb = workloads.to_bf16_bits(np.tile(lp, (1, k + 1, 1)))
    db = workloads.to_bf16_bits(np.tile(lq, (1, k, 1)))
    ok, p, _ = oracle.process_row(tb[0, 0], 1.0, 0, top_p)
    ok2, q, _ = oracle.process_row(db[0, 0], 1.0, 0, top_p)
    assert ok and ok2
    rs = np.random.default_rng(3002)
    toks = rs.choice(V, size=(N, k), p=q / q.sum()).astype(np.int32)
    u = rs.random((N, k + 1)).astype(np.float32)
    tt = to_dev(tb).expand(N, -1, -1)
    dd = to_dev(db).expand(N, -1, -1)
    acc, out = _verify(tt, dd, toks, u, top_p=top_p)
    assert (acc >= 0).all()
    # the token at position 0 (accepted draft or correction) follows p, and
    # so does the token at position 1 of the sequences that reach it
    p0 = _chi(np.bincount(out[:, 0], minlength=V), p)
    p1 = _chi(np.bincount(out[acc >= 1, 1], minlength=V), p)
    beta = float(np.minimum(p, q).sum())
    law = np.array([beta ** j * (1 - beta) for j in range(k)] + [beta ** k])
    pl = _chi(np.bincount(acc, minlength=k + 1), law)
    note("walk top_p=%g: position 0 chi-square p=%.3g, position 1 p=%.3g, length p=%.3g, beta %.4f"
         % (top_p, p0, p1, pl, beta))
    assert p0 >= 1e-3 and p1 >= 1e-3 and pl >= 1e-3


def _pooled_chi(counts, probs, min_expected=5.0):
    """Chi-square p-value with bins of expected count < min_expected pooled."""
    n = counts.sum()
    exp = probs / probs.sum() * n
    order = np.argsort(exp)
    c_s, e_s = counts[order].astype(np.float64), exp[order]
    small = e_s < min_expected
    cs = np.concatenate([c_s[~small], [c_s[small].sum()]]) if small.any() else c_s
    es = np.concatenate([e_s[~small], [e_s[small].sum()]]) if small.any() else e_s
    keep = es > 0
    return scipy.stats.chisquare(cs[keep], es[keep] * cs[keep].sum() / es[keep].sum())[1]


def test_config1_positions_follow_target_law():
    """Workload 1 (V = 1024, fp32, k = 4): its one sequence's rows broadcast to
    4 x 10^6 samples (four seeded batches of 10^6) with fresh draft tokens
    (from q) and uniforms.  The first emitted token follows p_0 and the token
    at position 1, given it exists, follows p_1 (chi-square over the pooled
    counts, small bins merged)."""
    w = workloads.generate(1, B=1)
    c = w.config
    k, V = c.k, c.V
    ps = [oracle.process_row(w.target[0, j], c.temperature, c.top_k, c.top_p)[1] for j in range(k + 1)]
    qs = [oracle.process_row(w.draft[0, j], c.temperature, c.top_k, c.top_p)[1] for j in range(k)]
    tt = to_dev(w.target).expand(N, -1, -1)
    dd = to_dev(w.draft).expand(N, -1, -1)
    c0 = np.zeros(V, np.int64)
    c1 = np.zeros(V, np.int64)
    accepted0 = 0
    for seed in (3003, 3004, 3005, 3006):
        rs = np.random.default_rng(seed)
        toks = np.stack([rs.choice(V, size=N, p=q / q.sum()) for q in qs], axis=1).astype(np.int32)
        u = rs.random((N, k + 1)).astype(np.float32)
        acc, out = _verify(tt, dd, toks, u, c.temperature, c.top_k, c.top_p)
        assert (acc >= 0).all()
        c0 += np.bincount(out[:, 0], minlength=V)
        c1 += np.bincount(out[acc >= 1, 1], minlength=V)
        accepted0 += int((acc >= 1).sum())
    p0 = _pooled_chi(c0, ps[0])
    p1 = _pooled_chi(c1, ps[1])
    beta0 = float(np.minimum(ps[0], qs[0]).sum())
    rate0 = accepted0 / (4 * N)
    note("config 1: position 0 chi-square p=%.3g, position 1 p=%.3g, P(accept 0) %.5f vs %.5f"
         % (p0, p1, rate0, beta0))
    assert p0 >= 1e-3 and p1 >= 1e-3
    assert abs(rate0 - beta0) <= 4 * np.sqrt(beta0 * (1 - beta0) / (4 * N))


def test_u_grid_law_walk():
    """Brute force on a tiny vocabulary (4 live tokens in bf16 rows of 8, k =
    2): every draft string, weighted by its proposal probability, against a
    midpoint grid of G = 64 points per uniform -- 4.2 M sequences through the
    whole-sequence walk.  The law of the emitted string matches the exact
    law of the rule (fractions) within 3 / G, the grid's resolution of the
    three decision breakpoints a string meets."""
    from fractions import Fraction
    from oracle import exact

    k, V, G = 2, 8, 64
    live = [0, 3, 5, 6]
    lp = np.full((k + 1, V), -np.inf, np.float32)
    lq = np.full((k, V), -np.inf, np.float32)
    lp[0, live] = np.log([0.4, 0.3, 0.2, 0.1])
    lp[1, live] = np.log([0.1, 0.2, 0.3, 0.4])
    lp[2, live] = np.log([0.25, 0.25, 0.25, 0.25])
    lq[0, live] = np.log([0.25, 0.25, 0.3, 0.2])
    lq[1, live] = np.log([0.4, 0.1, 0.1, 0.4])
    tb, db = workloads.to_bf16_bits(lp[None]), workloads.to_bf16_bits(lq[None])
    ps = [oracle.process_row(tb[0, j])[1] for j in range(k + 1)]
    qs = [oracle.process_row(db[0, j])[1] for j in range(k)]
    law = exact.output_law([[Fraction(float(x)) for x in p] for p in ps],
                           [[Fraction(float(x)) for x in q] for q in qs])
    strings = [(a, b) for a in live for b in live]
    g = (np.arange(G, dtype=np.float64) + 0.5) / G
    U = np.stack(np.meshgrid(g, g, g, indexing="ij"), axis=-1).reshape(-1, 3).astype(np.float32)
    n = len(strings) * len(U)
    toks = np.repeat(np.array(strings, np.int32), len(U), axis=0)
    u = np.tile(U, (len(strings), 1))
    tt = to_dev(tb).expand(n, -1, -1)
    dd = to_dev(db).expand(n, -1, -1)
    acc, out = _verify(tt, dd, toks, u)
    assert (acc >= 0).all()
    weight = np.repeat([qs[0][a] * qs[1][b] for a, b in strings], len(U)) / len(U)
    # emitted string (accepted drafts + one token) as one integer, base V + 1
    emitted = np.where(np.arange(k + 1)[None, :] <= acc[:, None], out + 1, 0).astype(np.int64)
    code = (emitted * (V + 1) ** np.arange(k + 1)[None, :]).sum(axis=1)
    keys, inv = np.unique(code, return_inverse=True)
    mass = np.bincount(inv, weights=weight)
    enc = lambda t: sum((x + 1) * (V + 1) ** j for j, x in enumerate(t))
    emp = dict(zip(keys.tolist(), mass.tolist()))
    err = max(abs(emp.get(enc(key), 0.0) - float(pr)) for key, pr in law.items())
    extra = sum(v for c, v in emp.items() if c not in {enc(key) for key in law})
    note("u-grid law: %d strings x %d^3 points, max |empirical - exact| = %.4f (bound %.4f), "
         "mass outside the exact support %.2g" % (len(strings), G, err, 3 / G, extra))
    assert err <= 3 / G and extra == 0.0
