"""Parity of the correction draw spread over the chip: small batches
(B at most half the CU count) of aligned rows spanning several 4,096-element
chunks take k_draw_split instead of one tail workgroup per
sequence.  Ragged vocabularies (last chunk partial, V not a multiple of 8
vectors), fp32 and bf16, filtered and unfiltered rows, rejections and bonus
draws, invalid sequences, and the workspace left zero."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import draft_token_verification_11_amd as sv
import oracle
import workloads
from tests.gpu_common import DEV, compare_stochastic, gpu_stochastic, note, to_dev

pytestmark = pytest.mark.gpu


def _case(rs, B, k, V, T, top_k, top_p, bf16, noise):
    t = rs.normal(0, 2.0, (B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rs.normal(0, noise, (B, k, V))).astype(np.float32)
    if bf16:
        t, d = workloads.to_bf16_bits(t), workloads.to_bf16_bits(d)
    toks = oracle.sample_drafts(d, rs.random((B, k)), T, top_k, top_p)
    u = rs.random((B, k + 1)).astype(np.float32)
    return t, d, toks, u


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("V", [20000, 16392, 65536, 8192, 4104])
def test_split_draw_parity(bf16, V):
    rs = np.random.default_rng(71 + V + bf16)
    B = 37
    for T, top_k, top_p, k, noise in [(1.0, 0, 1.0, 3, 0.7), (0.8, 0, 0.9, 2, 0.3),
                                      (1.0, 40, 0.95, 4, 0.05), (1.2, 0, 1.0, 1, 2.0)]:
        t, d, toks, u = _case(rs, B, k, V, T, top_k, top_p, bf16, noise)
        ref = oracle.verify_stochastic(t, d, toks, u, T, top_k, top_p)
        acc, out, ap = gpu_stochastic(t, d, toks, u, T, top_k, top_p)
        # fp32 rows of 16k-65k tokens put ~1e-5 of mass on each token, so
        # a top-p cut lands within 1e-6 of top_p in a large share of rows
        compare_stochastic(ref, acc, out, ap, fp32=not bf16,
                           label="split draw V=%d bf16=%s T=%g k=%d p=%g" % (V, bf16, T, top_k, top_p),
                           max_flag_frac=0.8 if (not bf16 and top_p < 1.0 and not top_k) else 0.15)
        note("  accepted-length histogram %s" % np.bincount(ref["accepted_len"][ref["accepted_len"] >= 0],
                                                             minlength=k + 1))


def test_split_draw_invalid_and_workspace():
    """Invalid sequences keep their outputs from the tail; two calls on one
    workspace agree and leave it zero."""
    rs = np.random.default_rng(79)
    B, k, V = 21, 3, 24576
    t, d, toks, u = _case(rs, B, k, V, 1.0, 0, 0.95, True, 0.7)
    t[0, 0, 7] = np.uint16(0x7FC0)  # NaN in target row 0: invalid at position 0
    toks[1, 0] = V                  # token out of range at position 0
    d[2, 0, 3] = np.uint16(0x7F80)  # +inf in draft row 0
    ref = oracle.verify_stochastic(t, d, toks, u, 1.0, 0, 0.95)
    assert list(ref["accepted_len"][:3]) == [-1, -1, -1]
    ws = torch.zeros(sv.workspace_size(sv.SPEC_OP_STOCHASTIC, B, k, V, 1.0, 0, 0.95),
                     dtype=torch.uint8, device=DEV)
    args = (to_dev(t), to_dev(d), torch.from_numpy(toks).to(DEV), torch.from_numpy(u).to(DEV))
    r1 = sv.verify_stochastic(*args, top_p=0.95, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    r2 = sv.verify_stochastic(*args, top_p=0.95, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    acc, out = r1[0].cpu().numpy(), r1[1].cpu().numpy()
    compare_stochastic(ref, acc, out, None, fp32=False, label="split draw invalid rows")
    assert (out[:3] == -1).all()


def test_split_draw_strided_ragged_and_batch_edges():
    """V = 20001 at a padded row stride of 20008 (aligned rows, a partial last
    vector), and batches on both sides of the spread draw's batch limit
    (B = 128 spreads its draws on a 256-CU part, B = 129 does not)."""
    rs = np.random.default_rng(83)
    k, V, Sd = 2, 20001, 20008
    for B in (128, 129):
        t, d, toks, u = _case(rs, B, k, V, 1.0, 0, 0.95, True, 0.7)
        tp = np.zeros((B, k + 1, Sd), np.uint16)
        tp[:, :, :V] = t
        dp = np.zeros((B, k, Sd), np.uint16)
        dp[:, :, :V] = d
        ref = oracle.verify_stochastic(t, d, toks, u, 1.0, 0, 0.95)
        acc, out, ap = gpu_stochastic(to_dev(tp)[:, :, :V], to_dev(dp)[:, :, :V], toks, u,
                                      1.0, 0, 0.95)
        compare_stochastic(ref, acc, out, ap, fp32=False, label="split draw strided B=%d" % B)
