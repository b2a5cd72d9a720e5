"""Fused LM head + greedy verify on the GPU against the oracle's fp64 logits
(exact products of the bf16 inputs): every sequence whose consulted rows have
no near tie (another logit within the fp32 summation bound of the largest)
must match exactly; at near ties every argmax the GPU acted on must be one of
the tied candidates, and its stop the first draft that differs from it.  Row counts cover the one, two and four 16-row blocks of the
kernel; vocabularies are ragged against its 256-wide tiles."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import draft_token_verification_11_amd as sv
import oracle
import workloads
from tests.gpu_common import DEV, note

pytestmark = pytest.mark.gpu


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _tokens(rs, best, V, p_random=0.25):
    B, k1 = best.shape
    toks = best[:, : k1 - 1].copy()
    rnd = rs.random(toks.shape) < p_random
    toks[rnd] = rs.integers(0, V, rnd.sum())
    return toks.astype(np.int32)


def _check(h, w, toks, label, hidden=None, weight=None, logits=None):
    acc, out = sv.verify_greedy_lmhead(hidden if hidden is not None else _dev_bf16(h),
                                       weight if weight is not None else _dev_bf16(w),
                                       torch.from_numpy(toks).to(DEV))
    torch.cuda.synchronize()
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    L, S = logits if logits is not None else oracle.lmhead_logits(h, w)
    racc, rout, near = oracle.lmhead_greedy(h, w, toks, logits=(L, S))
    B, k1 = near.shape
    k, V = k1 - 1, w.shape[0]
    consulted = np.zeros_like(near)
    for b in range(B):
        n = racc[b] if racc[b] >= 0 else k1 - 1
        consulted[b, : n + 1] = True
    clean = ~(near & consulted).any(axis=1)
    assert np.array_equal(acc[clean], racc[clean]), label
    assert np.array_equal(out[clean], rout[clean]), label
    # near ties: the GPU's argmax of every row it consulted is one of the
    # tied candidates, and its stop is the first draft that differs from it
    cand = None
    for b in np.nonzero(~clean)[0]:
        if cand is None:
            cand = oracle.lmhead_tie_candidates(L, S, h.shape[-1])
        n = int(acc[b])
        rows = [b * k1 + j for j in range(k1)]
        where = "%s: near-tie sequence %d gpu n=%d out=%s" % (label, b, n, list(out[b]))
        if n < 0:  # an out-of-range draft reached through tied matches
            j = next((j for j in range(k) if not 0 <= toks[b, j] < V), -1)
            assert j >= 0, where
            assert all(toks[b, i] in cand[rows[i]] for i in range(j)), where
            assert (out[b] == -1).all(), where
            continue
        assert all(0 <= toks[b, i] < V and toks[b, i] in cand[rows[i]] for i in range(n)), where
        assert np.array_equal(out[b, :n], toks[b, :n]) and (out[b, n + 1:] == -1).all(), where
        assert out[b, n] in cand[rows[n]], where
        if n < k:
            assert 0 <= toks[b, n] < V and out[b, n] != toks[b, n], where
    note("%s: %d sequences, %d with a near tie where consulted (each checked against its "
         "tied candidates)" % (label, B, int((~clean).sum())))
    return acc, out, racc, near


@pytest.mark.parametrize("B,k,d,V", [(1, 8, 256, 5000), (3, 9, 512, 4099), (16, 4, 256, 3000),
                                     (7, 3, 1024, 777), (13, 7, 256, 3001), (37, 7, 96, 3001),
                                     (40, 6, 96, 3001), (16, 8, 256, 5003)])
def test_lmhead_parity(B, k, d, V):
    rs = np.random.default_rng(B * 1000 + V)
    h, w, vs = workloads.lmhead(B, k, d, V, seed=B + V, boost=1.0)
    L, _ = oracle.lmhead_logits(h, w)
    best = np.argmax(L, axis=1).reshape(B, k + 1)
    _check(h, w, _tokens(rs, best, V), "lmhead B=%d k=%d d=%d V=%d" % (B, k, d, V))


def test_lmhead_strided_inputs():
    """hidden rows padded (pos stride d + 64, sequences apart by 2 extra rows)
    and weight rows padded (stride d + 32)."""
    rs = np.random.default_rng(5)
    B, k, d, V = 4, 4, 256, 2000
    h, w, vs = workloads.lmhead(B, k, d, V, seed=55, boost=1.0)
    hp = np.zeros((B, k + 3, d + 64), np.uint16)
    hp[:, : k + 1, :d] = h
    wp = np.zeros((V, d + 32), np.uint16)
    wp[:, :d] = w
    th = _dev_bf16(hp)[:, : k + 1, :d]
    tw = _dev_bf16(wp)[:, :d]
    assert th.stride(1) == d + 64 and tw.stride(0) == d + 32
    L, _ = oracle.lmhead_logits(h, w)
    best = np.argmax(L, axis=1).reshape(B, k + 1)
    _check(h, w, _tokens(rs, best, V), "lmhead strided", hidden=th, weight=tw)


def test_lmhead_full_size_greedy_shape():
    """B = 1, k = 8, d = 4096, V = 151936 (the greedy workload's shape), every
    row checked against fp64 logits; then 48 sequences (M = 432 rows)."""
    rs = np.random.default_rng(8)
    for B in (1, 48):
        h, w, vs = workloads.lmhead(B, 8, 4096, 151936, seed=3, boost=0.3)
        L, S = oracle.lmhead_logits(h, w)
        best = np.argmax(L, axis=1).reshape(B, 9)
        _check(h, w, _tokens(rs, best, 151936, 0.15), "lmhead full size B=%d" % B, logits=(L, S))
        del L, S


def test_lmhead_matches_unfused_gpu_path():
    """The same decisions as materialised fp32 logits (torch matmul in fp32 of
    the bf16 inputs) through spec_verify_greedy, away from near ties."""
    rs = np.random.default_rng(9)
    B, k, d, V = 8, 4, 512, 8192
    h, w, vs = workloads.lmhead(B, k, d, V, seed=9, boost=1.0)
    th, tw = _dev_bf16(h), _dev_bf16(w)
    logits = (th.float().reshape(-1, d) @ tw.float().t()).reshape(B, k + 1, V).contiguous()
    L, _ = oracle.lmhead_logits(h, w)
    toks = _tokens(rs, np.argmax(L, axis=1).reshape(B, k + 1), V)
    a1, o1 = sv.verify_greedy_lmhead(th, tw, torch.from_numpy(toks).to(DEV))
    a2, o2 = sv.verify_greedy(logits, torch.from_numpy(toks).to(DEV))
    torch.cuda.synchronize()
    _, _, racc, near = _check(h, w, toks, "lmhead vs unfused")
    clean = ~near.any(axis=1)
    assert torch.equal(a1[torch.from_numpy(clean).to(DEV)], a2[torch.from_numpy(clean).to(DEV)])
    assert torch.equal(o1[torch.from_numpy(clean).to(DEV)], o2[torch.from_numpy(clean).to(DEV)])


@pytest.mark.parametrize("d,V", [(256, 4000), (2048, 20000)])
def test_lmhead_every_row_argmax(d, V):
    """Unboosted rows (logits ~ N(0, 1): top-2 gaps ~0.2) with every draft
    equal to its row's argmax, so the walk consults every row (bonus
    included) and every argmax is compared."""
    rs = np.random.default_rng(d + V)
    B, k = 12, 5
    h, w, vs = workloads.lmhead(B, k, d, V, seed=d, boost=0.0)
    L, _ = oracle.lmhead_logits(h, w)
    best = np.argmax(L, axis=1).reshape(B, k + 1)
    acc, out, racc, near = _check(h, w, _tokens(rs, best, V, 0.0), "lmhead every row d=%d V=%d" % (d, V))
    assert (racc[~near.any(axis=1)] == k).all()


@pytest.mark.parametrize("d", [32, 96, 160])
def test_lmhead_k_tail(d):
    """d a multiple of 32 but not of the 64 the kernel loads per batch: the
    batch's second step lies past d and must add nothing."""
    rs = np.random.default_rng(d)
    B, k, V = 5, 3, 3001
    h, w, vs = workloads.lmhead(B, k, d, V, seed=d, boost=2.0)
    L, _ = oracle.lmhead_logits(h, w)
    best = np.argmax(L, axis=1).reshape(B, k + 1)
    acc, out, racc, near = _check(h, w, _tokens(rs, best, V, 0.0), "lmhead d=%d" % d)
    assert (acc[~near.any(axis=1)] == k).all()


@pytest.mark.parametrize("B,k", [(1, 1), (9, 7)])
def test_lmhead_largest_hidden_size(B, k):
    """d = 65536, the largest hidden size accepted: 2 rows on the direct-load
    kernel, 72 rows on the LDS-staged tiling; every consulted row compared
    away from near ties (their bound grows with d)."""
    rs = np.random.default_rng(65536 + B)
    d, V = 65536, 300
    h, w, vs = workloads.lmhead(B, k, d, V, seed=B, boost=0.5)
    L, _ = oracle.lmhead_logits(h, w)
    best = np.argmax(L, axis=1).reshape(B, k + 1)
    acc, out, racc, near = _check(h, w, _tokens(rs, best, V, 0.2), "lmhead d=65536 B=%d k=%d" % (B, k))
    assert (~near).any()
