"""Parity of the whole-sequence path: batches of aligned bf16 rows large
enough that every CU takes several sequences from the queue.  That path reads
each sequence's rows in walk order (target j, draft j, ratio test) and nothing
past the stop, so these tests check that every decision, correction and
reported alpha still equals the oracle's, with and without alpha requested,
for ragged vocabularies, strided rows, ill-formed positions and k from 1 to
the maximum."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import draft_token_verification_11_amd as sv
import oracle
import workloads
from tests.gpu_common import DEV, compare_stochastic, gpu_stochastic, note, to_dev

pytestmark = pytest.mark.gpu


def _batch() -> int:
    # at least two sequences per CU (the whole-sequence path), ragged against the grid
    return 2 * torch.cuda.get_device_properties(0).multi_processor_count + 37


def _case(rs, B, k, V, T, top_k, top_p, sigma=2.0, noise=0.7):
    t = rs.normal(0, sigma, (B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rs.normal(0, noise, (B, k, V))).astype(np.float32)
    tb, db = workloads.to_bf16_bits(t), workloads.to_bf16_bits(d)
    toks = oracle.sample_drafts(db, rs.random((B, k)), T, top_k, top_p)
    u = rs.random((B, k + 1)).astype(np.float32)
    return tb, db, toks, u


def _walk_only(target, draft, toks, u, T, top_k, top_p):
    """The same call without alpha (rows past the stop are not read)."""
    acc, out = sv.verify_stochastic(
        target if isinstance(target, torch.Tensor) else to_dev(target),
        draft if isinstance(draft, torch.Tensor) else to_dev(draft),
        torch.from_numpy(np.asarray(toks, np.int32)).to(DEV),
        torch.from_numpy(np.asarray(u, np.float32)).to(DEV),
        temperature=T, top_k=top_k, top_p=top_p)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def _path(tt, dd, T, top_k, top_p, alpha):
    return sv.verify_stochastic_path(tt, dd, temperature=T, top_k=top_k, top_p=top_p,
                                     return_accept_prob=alpha)


def _check(t, d, toks, u, T, top_k, top_p, label, tt=None, dd=None):
    ref = oracle.verify_stochastic(t, d, toks, u, T, top_k, top_p)
    tt = to_dev(t) if tt is None else tt
    dd = to_dev(d) if dd is None else dd
    assert _path(tt, dd, T, top_k, top_p, True) == sv.SPEC_PATH_SEQUENCE_WALK, label
    assert _path(tt, dd, T, top_k, top_p, False) == sv.SPEC_PATH_TASK_QUEUE, label
    acc, out, ap = gpu_stochastic(tt, dd, toks, u, T, top_k, top_p)
    compare_stochastic(ref, acc, out, ap, fp32=False, label=label + " alpha requested (walk)")
    acc2, out2 = _walk_only(tt, dd, toks, u, T, top_k, top_p)
    compare_stochastic(ref, acc2, out2, None, fp32=False, label=label + " task queue")
    # both modes take the same decisions (same statistics, same draws)
    assert np.array_equal(acc, acc2) and np.array_equal(out, out2), label
    return ref


@pytest.mark.parametrize("V", [1000, 4096, 8])
def test_walk_settings(V):
    rs = np.random.default_rng(31 + V)
    B = _batch()
    for T, top_k, top_p, k in [(1.0, 0, 0.95, 4), (0.8, 0, 1.0, 3), (1.0, 50, 0.9, 5),
                               (1.3, 5, 1.0, 1), (0.6, 0, 0.5, 2)]:
        t, d, toks, u = _case(rs, B, k, V, T, top_k, top_p)
        ref = _check(t, d, toks, u, T, top_k, top_p, "V=%d T=%g k=%d p=%g" % (V, T, top_k, top_p))
        note("  accepted-length histogram %s" % np.bincount(ref["accepted_len"], minlength=k + 1))


def test_walk_strided_and_ragged():
    """V = 777 at a padded row stride of 784 (16-byte aligned rows)."""
    rs = np.random.default_rng(41)
    B, k, V, S = _batch(), 4, 777, 784
    t, d, toks, u = _case(rs, B, k, V, 1.0, 0, 0.95)
    tp = np.zeros((B, k + 1, S), np.uint16)
    tp[:, :, :V] = t
    dp = np.zeros((B, k, S), np.uint16)
    dp[:, :, :V] = d
    _check(t, d, toks, u, 1.0, 0, 0.95, "stride 784", tt=to_dev(tp)[:, :, :V], dd=to_dev(dp)[:, :, :V])


def test_walk_extreme_k():
    rs = np.random.default_rng(43)
    B = _batch()
    for k, V in [(64, 64), (33, 136)]:
        # draft close to the target: long accepted runs reach deep positions
        t, d, toks, u = _case(rs, B, k, V, 1.0, 0, 0.9, noise=0.05)
        ref = _check(t, d, toks, u, 1.0, 0, 0.9, "k=%d V=%d" % (k, V))
        assert ref["accepted_len"].max() >= k // 2


def test_walk_window_edges():
    """Extreme bf16 codes in both whole-sequence kernels: many +-0 and top-k
    cuts that fall on 0, tiny and huge values among ordinary logits, rows
    whose finite values are all huge, and both ends of the row filter's
    exponent window [2^-31, 2^33) with their neighbours outside it."""
    rs = np.random.default_rng(53)
    B, k, V = _batch(), 3, 1000
    w_lo, w_hi = np.float32(2.0 ** -31), np.float32((2 - 2 ** -7) * 2.0 ** 32)
    below, above = np.float32((2 - 2 ** -7) * 2.0 ** -32), np.float32(2.0 ** 33)
    for T, top_k, top_p in [(1.0, 0, 0.9), (0.7, 20, 0.8), (1.0, 50, 1.0)]:
        t = rs.normal(0, 2, (B, k + 1, V)).astype(np.float32)
        d = (t[:, :k] + rs.normal(0, 0.7, (B, k, V))).astype(np.float32)
        for b in range(0, 20):  # many zeros
            t[b, :, ::3] = 0.0
            t[b, :, 1::6] = -0.0
        for b in range(20, 40):  # non-positive rows: top-k cuts on 0
            t[b] = -np.abs(t[b])
            t[b, :, :100] = 0.0
            d[b] = -np.abs(d[b])
            d[b, :, :60] = 0.0
        for b in range(40, 60):  # tiny values
            t[b, :, :5] = 1e-25
            d[b, 0, 7] = -3e-30
        for b in range(60, 80):  # huge values among ordinary ones
            t[b, 1, 3] = 1e25
            d[b, 0, 4] = -5e20
        for b in range(80, 100):  # every finite value huge, some -inf
            t[b, 0] = t[b, 0] * np.float32(2.0 ** 40)
            t[b, 0, ::7] = -np.inf
            if b < 90:
                d[b, 0] = d[b, 0] * np.float32(2.0 ** 40)
        for b in range(100, 120):  # the window's ends and their outside neighbours
            t[b, :, 0] = w_lo
            t[b, :, 1] = -w_lo
            t[b, :, 2] = below
            d[b, :, 3] = -below
            t[b, 1, 4] = w_hi
            d[b, 0, 5] = -w_hi
            t[b, 2, 6] = above
            d[b, 1, 7] = -above
        tb, db = workloads.to_bf16_bits(t), workloads.to_bf16_bits(d)
        toks = oracle.sample_drafts(db, rs.random((B, k)), T, top_k, top_p)
        u = rs.random((B, k + 1)).astype(np.float32)
        _check(tb, db, toks, u, T, top_k, top_p, "window edges T=%g k=%d p=%g" % (T, top_k, top_p))


def test_walk_ill_formed_positions():
    """Invalid rows and tokens count where the walk consults them."""
    rs = np.random.default_rng(47)
    B, k, V = _batch(), 3, 512
    for T, top_k, top_p in [(1.0, 0, 1.0), (1.0, 10, 0.8)]:
        t, d, toks, u = _case(rs, B, k, V, T, top_k, top_p)
        tf = workloads.bf16_bits_to_f32(t)
        nan, pinf, ninf = np.uint16(0x7FC0), np.uint16(0x7F80), np.uint16(0xFF80)
        toks[:8] = np.argmax(tf[:8, :k], axis=2)
        u[:8, :k] = 0.0
        t[0, 1, 5] = nan
        d[1, 2, 9] = pinf
        t[2, k, :] = ninf
        toks[3, 1] = V
        toks[4, 0] = -7
        d[5, 0, 100] = nan
        for b in (6, 7):
            t[b, 0, 0] = ninf
            toks[b, 0] = 0
        t[6, 2, 4] = nan
        toks[7, 2] = V
        t[7, k, :] = ninf
        # scattered damage over the rest of the batch
        for b in rs.choice(np.arange(8, B), size=40, replace=False):
            r = rs.integers(0, 2 * k + 1)
            (t[b, r] if r <= k else d[b, r - k - 1])[rs.integers(0, V)] = nan
        ref = _check(t, d, toks, u, T, top_k, top_p, "ill-formed T=%g k=%d p=%g" % (T, top_k, top_p))
        assert list(ref["accepted_len"][:8]) == [-1] * 6 + [0, 0]


def test_walk_queue_and_workspace():
    """Two calls in a row on one workspace: the sequence queue is left zero,
    so the second call takes every sequence again and agrees bit for bit."""
    rs = np.random.default_rng(53)
    B, k, V = _batch(), 4, 1000
    t, d, toks, u = _case(rs, B, k, V, 1.0, 0, 0.95)
    ws = torch.zeros(sv.workspace_size(sv.SPEC_OP_STOCHASTIC, B, k, V, 1.0, 0, 0.95),
                     dtype=torch.uint8, device=DEV)
    args = (to_dev(t), to_dev(d), torch.from_numpy(toks).to(DEV), torch.from_numpy(u).to(DEV))
    r1 = sv.verify_stochastic(*args, top_p=0.95, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    r2 = sv.verify_stochastic(*args, top_p=0.95, workspace=ws)
    r3 = sv.verify_stochastic(*args, top_p=0.95, return_accept_prob=True, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    assert torch.equal(r1[0], r3[0]) and torch.equal(r1[1], r3[1])
    assert int((r1[0] >= 0).sum()) == B


def test_walk_threshold_both_sides():
    """Two sequences per CU less one takes the row pass, exactly two per CU the
    position-task kernel: the same sequences, the oracle's results on both
    sides wherever its decisions are clear."""
    rs = np.random.default_rng(59)
    B, k, V = 2 * torch.cuda.get_device_properties(0).multi_processor_count, 3, 1000
    for T, top_k, top_p in [(1.0, 0, 0.95), (0.8, 20, 1.0)]:
        t, d, toks, u = _case(rs, B, k, V, T, top_k, top_p)
        ref = oracle.verify_stochastic(t, d, toks, u, T, top_k, top_p)
        ref1 = oracle.verify_stochastic(t[: B - 1], d[: B - 1], toks[: B - 1], u[: B - 1], T,
                                        top_k, top_p)
        assert _path(to_dev(t), to_dev(d), T, top_k, top_p, False) == sv.SPEC_PATH_TASK_QUEUE
        assert _path(to_dev(t[: B - 1]), to_dev(d[: B - 1]), T, top_k, top_p, False) == \
            sv.SPEC_PATH_ROW_PASS
        a_walk, o_walk = _walk_only(t, d, toks, u, T, top_k, top_p)
        a_rows, o_rows = _walk_only(t[: B - 1], d[: B - 1], toks[: B - 1], u[: B - 1], T, top_k, top_p)
        label = "threshold T=%g k=%d p=%g" % (T, top_k, top_p)
        compare_stochastic(ref, a_walk, o_walk, None, fp32=False, label=label + " B=%d task queue" % B)
        compare_stochastic(ref1, a_rows, o_rows, None, fp32=False, label=label + " B=%d row pass" % (B - 1))


@pytest.mark.parametrize("V", [40000, 40003])
def test_walk_count_tail_vectors(V):
    """Vocabularies whose rows leave each thread two or three full 16-byte
    vectors after the prefetched ones (loaded together at the end of the
    count), and at V = 40003 a partial last group: its rows sit at a padded
    stride of 40,008 elements, so that they stay 16-byte aligned and the
    position-task kernel (asserted) reads them."""
    from tests.test_gpu_parity import oracle_stochastic
    rs = np.random.default_rng(V)
    B, k = 2 * torch.cuda.get_device_properties(0).multi_processor_count, 2
    t, d, toks, u = _case(rs, B, k, V, 1.0, 0, 0.95)
    ref = oracle_stochastic(t, d, toks, u, 1.0, 0, 0.95)
    S = (V + 7) // 8 * 8
    tp = np.zeros((B, k + 1, S), np.uint16)
    tp[:, :, :V] = t
    dp = np.zeros((B, k, S), np.uint16)
    dp[:, :, :V] = d
    tt, dd = to_dev(tp)[:, :, :V], to_dev(dp)[:, :, :V]
    assert _path(tt, dd, 1.0, 0, 0.95, False) == sv.SPEC_PATH_TASK_QUEUE
    acc, out = _walk_only(tt, dd, toks, u, 1.0, 0, 0.95)
    compare_stochastic(ref, acc, out, None, fp32=False, label="count tail V=%d task queue" % V)
