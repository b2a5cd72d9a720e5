"""Predicted-outcome lookup on the GPU against the oracle's plain loops:
random predicted sets (P from 1 to beyond a wave's 64 lanes) with the true
outcome planted in some, invalid sequences, duplicates; and the lookup
applied to a verify call's own outputs on the branch fan-out recipe."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import draft_token_verification_11_amd as sv
import oracle
import workloads
from tests.gpu_common import DEV, note, to_dev

pytestmark = pytest.mark.gpu


def _sets(rs, acc, out, P, plant=0.5, V=1000):
    B, k1 = out.shape
    pl = rs.integers(-1, k1, (B, P)).astype(np.int32)
    pt = rs.integers(0, V, (B, P)).astype(np.int32)
    for b in np.nonzero(rs.random(B) < plant)[0]:
        n = int(acc[b])
        if 0 <= n < k1:
            for _ in range(int(rs.integers(1, 3))):  # sometimes twice: the first counts
                i = int(rs.integers(0, P))
                pl[b, i], pt[b, i] = n, out[b, n]
    return pl, pt


def _gpu(acc, out, pl, pt):
    hit, cnt = sv.outcome_lookup(*(torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
                                   for x in (acc, out, pl, pt)))
    torch.cuda.synchronize()
    return hit.cpu().numpy(), int(cnt.cpu().item())


@pytest.mark.parametrize("P", [1, 16, 64, 65, 200, 4096])
def test_lookup_random_sets(P):
    rs = np.random.default_rng(90 + P)
    B, k, V = 3001 if P < 4096 else 97, 4, 1000
    acc = rs.integers(-1, k + 1, B).astype(np.int32)
    out = rs.integers(0, V, (B, k + 1)).astype(np.int32)
    for b in range(B):  # verify's layout: drafts, emitted, then -1
        if acc[b] < 0:
            out[b] = -1
        else:
            out[b, acc[b] + 1:] = -1
    pl, pt = _sets(rs, acc, out, P)
    ref_hit, ref_cnt = oracle.outcome_lookup(acc, out, pl, pt)
    hit, cnt = _gpu(acc, out, pl, pt)
    assert np.array_equal(hit, ref_hit)
    assert cnt == ref_cnt
    note("lookup P=%d: %d of %d sequences hit" % (P, cnt, B))


def test_lookup_after_verify_branch_fanout():
    """The fan-out recipe at V = 4096 (32 requests x 16 branches, k = 4,
    top-p 0.95): verify on the GPU, then look the outcomes up in sets that
    hold the true outcome for every other sequence."""
    rs = np.random.default_rng(99)
    c = workloads.CONFIGS[5]
    nreq, br, k, V = 32, 16, c.k, 4096
    B = nreq * br
    base = rs.normal(0, 2.0, (nreq, k + 1, V)).astype(np.float32)
    req = np.arange(B) // br
    t = workloads.to_bf16_bits(base[req])
    d = workloads.to_bf16_bits(base[req, :k] + rs.normal(0, 0.7, (B, k, V)).astype(np.float32))
    toks = oracle.sample_drafts(d, rs.random((B, k)), 1.0, 0, 0.95, threads=8)
    u = rs.random((B, k + 1)).astype(np.float32)
    acc, out = sv.verify_stochastic(to_dev(t), to_dev(d), torch.from_numpy(toks).to(DEV),
                                    torch.from_numpy(u).to(DEV), top_p=0.95)
    torch.cuda.synchronize()
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    pl, pt = _sets(rs, acc, out, 16, plant=0.0, V=V)
    for b in range(0, B, 2):
        pl[b, b % 16], pt[b, b % 16] = acc[b], out[b, acc[b]]
    ref_hit, ref_cnt = oracle.outcome_lookup(acc, out, pl, pt)
    hit, cnt = _gpu(acc, out, pl, pt)
    assert np.array_equal(hit, ref_hit) and cnt == ref_cnt
    assert cnt >= B // 2
    note("lookup after verify: %d of %d branches hit" % (cnt, B))
