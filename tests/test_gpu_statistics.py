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
