"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Greedy must match bit for bit; stochastic must match on
every sequence the oracle does not flag as lying within 1e-6 of a decision
boundary; probabilities within 1e-6 absolute (fp32 inputs) or 2e-3 relative
(bf16 inputs)."""
from __future__ import annotations

import threading

import numpy as np
import pytest
import torch

import draft_token_verification_11_amd as sv
import oracle
import workloads
from tests.gpu_common import DEV, compare_stochastic, gpu_stochastic, note, to_dev

pytestmark = pytest.mark.gpu


def oracle_stochastic(target, draft, tokens, u, T, top_k, top_p, threads=8):
    """The oracle over slices of sequences in parallel threads (each call is
    the plain single-threaded oracle; ctypes releases the GIL)."""
    B = target.shape[0]
    parts = [None] * threads
    step = (B + threads - 1) // threads

    def work(i):
        lo, hi = i * step, min(B, (i + 1) * step)
        if lo < hi:
            parts[i] = oracle.verify_stochastic(target[lo:hi], draft[lo:hi], tokens[lo:hi],
                                                u[lo:hi], T, top_k, top_p)

    ths = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    parts = [p for p in parts if p is not None]
    ref = {k: np.concatenate([p[k] for p in parts]) for k in parts[0] if k != "inputs"}
    ref["inputs"] = {"target": target, "draft": draft, "tokens": np.asarray(tokens, np.int32),
                     "uniforms": np.asarray(u, np.float32), "temperature": float(T),
                     "top_k": int(top_k), "top_p": float(top_p)}
    return ref


def draft_tokens_from_oracle(w, threads=8):
    c = w.config
    return oracle.sample_drafts(w.draft, w.draft_u, c.temperature, c.top_k, c.top_p, threads)


def test_native_library_is_loaded():
    t, d, tok = workloads.worked_example()
    sv.verify_greedy(to_dev(t), torch.from_numpy(tok).to(DEV))
    torch.cuda.synchronize()
    maps = open("/proc/self/maps").read()
    assert sv.library_path() in maps


def test_worked_example_grid():
    """The entry's example on the GPU (V=3: the scalar, unaligned path), with
    one sequence per (u0, u1) grid point broadcast through seq_stride = 0."""
    t, d, tok = workloads.worked_example()
    u0s = [0.0, 0.1, 0.5, 0.7499, 0.7501, 0.8, 0.99, 0.9999999]
    u1s = [0.0, 0.3, 0.5999, 0.6001, 0.8999, 0.9001, 0.999]
    u = np.array([[a, b] for a in u0s for b in u1s], np.float32)
    B = len(u)
    tt = to_dev(t).expand(B, -1, -1)
    dd = to_dev(d).expand(B, -1, -1)
    assert tt.stride(0) == 0
    toks = np.ones((B, 1), np.int32)
    acc, out, ap = gpu_stochastic(tt, dd, toks, u, 1.0, 0, 1.0)
    ref = oracle.verify_stochastic(np.broadcast_to(t, (B, 2, 3)), np.broadcast_to(d, (B, 1, 3)),
                                   toks, u)
    assert abs(ap[0, 0] - 0.75) < 1e-6
    compare_stochastic(ref, acc, out, ap, label="worked example")
    rejected = acc == 0
    assert rejected.any() and (out[rejected, 0] == 0).all()  # the residual is all on A


def test_config1_parity():
    w = workloads.generate(1, B=512)
    c = w.config
    toks = draft_tokens_from_oracle(w)
    acc, out, ap = gpu_stochastic(w.target, w.draft, toks, w.uniforms, c.temperature, c.top_k,
                                  c.top_p)
    ref = oracle_stochastic(w.target, w.draft, toks, w.uniforms, c.temperature, c.top_k, c.top_p)
    nflag = compare_stochastic(ref, acc, out, ap, label="c1 x512")
    assert nflag <= 5


def test_config2_greedy_bit_exact():
    w = workloads.generate(2, B=4)
    toks = oracle.argmax_drafts(w.draft)
    rs = np.random.default_rng(0)
    toks2 = toks.copy()
    toks2[2:, rs.integers(0, 8)] = rs.integers(0, w.config.V)
    tgt = to_dev(w.target)
    for tk in (toks, toks2):
        acc, out = sv.verify_greedy(tgt, torch.from_numpy(tk).to(DEV))
        torch.cuda.synchronize()
        racc, rout = oracle.verify_greedy(w.target, tk)
        assert np.array_equal(acc.cpu().numpy(), racc)
        assert np.array_equal(out.cpu().numpy(), rout)
    # drafts equal to the target's argmax: every position accepted, bonus = argmax of row k
    am = np.stack([[oracle.argmax_row(w.target[b, j]) for j in range(9)] for b in range(4)])
    acc, out = sv.verify_greedy(tgt, torch.from_numpy(am[:, :8].astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    assert (acc.cpu().numpy() == 8).all() and np.array_equal(out.cpu().numpy(), am)


def test_config2_stochastic_parity():
    w = workloads.generate(2, B=16)
    c = w.config
    toks = draft_tokens_from_oracle(w)
    acc, out, ap = gpu_stochastic(w.target, w.draft, toks, w.uniforms, c.temperature, 0, 1.0)
    ref = oracle_stochastic(w.target, w.draft, toks, w.uniforms, c.temperature, 0, 1.0)
    compare_stochastic(ref, acc, out, ap, fp32=False, label="c2 x16")


def test_config3_parity_full():
    w = workloads.generate(3)
    c = w.config
    toks = draft_tokens_from_oracle(w)
    note("c3: drafts sampled")
    acc, out, ap = gpu_stochastic(w.target, w.draft, toks, w.uniforms, c.temperature, c.top_k,
                                  c.top_p)
    ref = oracle_stochastic(w.target, w.draft, toks, w.uniforms, c.temperature, c.top_k, c.top_p)
    compare_stochastic(ref, acc, out, ap, fp32=False, label="c3 full (B=64)")


def full_size_case(cfg, threads=16):
    """Every sequence of a workload at its full size, drafts drawn by the
    oracle's sampler from the processed q (the proposer's own draw), and the
    oracle's results for all of them."""
    c = workloads.CONFIGS[cfg]
    w = workloads.generate(cfg, threads=threads)
    note("c%d: inputs generated" % cfg)
    toks = draft_tokens_from_oracle(w, threads)
    note("c%d: drafts sampled" % cfg)
    ref = oracle_stochastic(w.target, w.draft, toks, w.uniforms, c.temperature, c.top_k, c.top_p,
                            threads)
    note("c%d: oracle done" % cfg)
    return w, toks, ref


def test_config4_parity_full_size():
    """Workload 4 at full size (256 x 8 positions, V = 262144, fp32): every
    sequence against the oracle."""
    w, toks, ref = full_size_case(4)
    c = w.config
    acc, out, ap = gpu_stochastic(w.target, w.draft, toks, w.uniforms, c.temperature, c.top_k,
                                  c.top_p)
    compare_stochastic(ref, acc, out, ap, fp32=True, label="c4 full size (B=256), all checked")


def test_config5_parity_full_size():
    """Workload 5 at full size (512 branch sequences x 4 positions,
    V = 151936, bf16, top-p 0.95): every sequence against the oracle, on the
    position-task kernel (the benchmarked call: no alpha) and on the
    whole-sequence walk (alpha requested)."""
    w, toks, ref = full_size_case(5)
    c = w.config
    tt, dd = to_dev(w.target), to_dev(w.draft)
    tk, uu = torch.from_numpy(toks).to(DEV), torch.from_numpy(w.uniforms).to(DEV)
    assert sv.verify_stochastic_path(tt, dd, top_p=c.top_p) == sv.SPEC_PATH_TASK_QUEUE
    acc, out = sv.verify_stochastic(tt, dd, tk, uu, temperature=c.temperature, top_k=c.top_k,
                                    top_p=c.top_p)
    torch.cuda.synchronize()
    compare_stochastic(ref, acc.cpu().numpy(), out.cpu().numpy(), None, fp32=False,
                       label="c5 full size (B=512) task queue, all checked")
    assert sv.verify_stochastic_path(tt, dd, top_p=c.top_p, return_accept_prob=True) == \
        sv.SPEC_PATH_SEQUENCE_WALK
    acc2, out2, ap2 = gpu_stochastic(tt, dd, toks, w.uniforms, c.temperature, c.top_k, c.top_p)
    compare_stochastic(ref, acc2, out2, ap2, fp32=False,
                       label="c5 full size (B=512) walk with alpha, all checked")


# ---------------------------------------------------------------------------
def _process_compare(rows_np, T, top_k, top_p, label, fp32):
    R, V = rows_np.shape
    res = sv.logits_process(to_dev(rows_np), temperature=T, top_k=top_k, top_p=top_p)
    torch.cuda.synchronize()
    probs = res["probs"].cpu().numpy().astype(np.float64)
    for r in range(R):
        ok, p, st = oracle.process_row(rows_np[r], T, top_k, top_p)
        assert bool(res["valid"][r]) == ok
        if not ok:
            continue
        near = (abs(st["mass_above_cut"] - top_p) <= 1e-6) or (abs(st["mass_at_cut"] - top_p) <= 1e-6)
        assert float(res["max_logit"][r]) == st["max_logit"], (label, r)
        if not near:
            assert float(res["threshold"][r]) == st["threshold"], (label, r, float(res["threshold"][r]), st["threshold"])
            assert abs(float(res["log_norm"][r]) - st["log_norm"]) <= 1e-6 * max(1.0, abs(st["log_norm"]))
            if fp32:
                assert np.abs(probs[r] - p).max() <= 1e-6, (label, r)
            else:
                big = p >= 1e-30
                assert (np.abs(probs[r][big] - p[big]) <= 2e-3 * p[big]).all(), (label, r)
                assert (probs[r][~big] <= 1e-29).all()
    note("%s: %d rows ok" % (label, R))


def test_logits_process_parity():
    w1 = workloads.generate(1, B=4)
    _process_compare(w1.target.reshape(-1, 1024), 1.0, 0, 1.0, "process c1 rows", True)
    _process_compare(w1.target.reshape(-1, 1024), 0.6, 17, 0.8, "process fp32 top-k/top-p (bisection)", True)
    w2 = workloads.generate(2, B=1)
    _process_compare(w2.target.reshape(-1, 151936), 0.7, 0, 1.0, "process c2 rows", False)
    w3 = workloads.generate(3, B=2)
    _process_compare(w3.draft.reshape(-1, 151936), 1.0, 50, 0.9, "process c3 rows (histogram)", False)
    w5 = workloads.generate(5, seqs=[0, 17])
    _process_compare(w5.draft.reshape(-1, 151936), 1.0, 0, 0.95, "process c5 rows (histogram)", False)


# ---------------------------------------------------------------------------
def _random_case(rs, B, k, V, dtype, T, top_k, top_p, mask_frac=0.0, sigma=2.0):
    t = rs.normal(0, sigma, (B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rs.normal(0, 1.0, (B, k, V))).astype(np.float32)
    if mask_frac:
        t[rs.random(t.shape) < mask_frac] = -np.inf
        d[rs.random(d.shape) < mask_frac] = -np.inf
        t[:, :, 0] = 0.0
        d[:, :, 0] = 0.0
    if dtype == "bf16":
        t, d = workloads.to_bf16_bits(t), workloads.to_bf16_bits(d)
    toks = oracle.sample_drafts(d, rs.random((B, k)), T, top_k, top_p)
    u = rs.random((B, k + 1)).astype(np.float32)
    return t, d, toks, u


@pytest.mark.parametrize("V", [1, 2, 7, 8, 9, 1000, 4097, 20001])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_vocabularies(V, dtype):
    rs = np.random.default_rng(V)
    for T, top_k, top_p in [(1.0, 0, 1.0), (0.5, 3, 1.0), (1.3, 0, 0.7), (1.0, 5, 0.9)]:
        t, d, toks, u = _random_case(rs, 6, 3, V, dtype, T, top_k, top_p)
        acc, out, ap = gpu_stochastic(t, d, toks, u, T, top_k, top_p)
        ref = oracle.verify_stochastic(t, d, toks, u, T, top_k, top_p)
        compare_stochastic(ref, acc, out, ap, fp32=(dtype == "f32"),
                           label="V=%d %s T=%g k=%d p=%g" % (V, dtype, T, top_k, top_p))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_strides_and_broadcast(dtype):
    """Rows at an odd element stride (scalar path) and a target broadcast to
    all sequences (seq_stride = 0) give the same result as packed copies."""
    rs = np.random.default_rng(5)
    B, k, V = 5, 4, 3001
    t, d, toks, u = _random_case(rs, B, k, V, dtype, 0.9, 0, 0.95)
    ref = oracle.verify_stochastic(t, d, toks, u, 0.9, 0, 0.95)
    pad = 3
    tp = np.zeros((B, k + 1, V + pad), t.dtype)
    tp[:, :, :V] = t
    dp = np.zeros((B, k, V + pad), d.dtype)
    dp[:, :, :V] = d
    tt = to_dev(tp)[:, :, :V]
    dd = to_dev(dp)[:, :, :V]
    acc, out, ap = gpu_stochastic(tt, dd, toks, u, 0.9, 0, 0.95)
    compare_stochastic(ref, acc, out, ap, fp32=(dtype == "f32"), label="odd stride " + dtype)
    tb = to_dev(t[:1]).expand(B, -1, -1)
    ref_b = oracle.verify_stochastic(np.broadcast_to(t[:1], t.shape), d, toks, u, 0.9, 0, 0.95)
    acc, out, ap = gpu_stochastic(tb, to_dev(d), toks, u, 0.9, 0, 0.95)
    compare_stochastic(ref_b, acc, out, ap, fp32=(dtype == "f32"), label="broadcast " + dtype)


@pytest.mark.parametrize("V", [777, 1024])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_masks_and_invalid_rows(dtype, V):
    """Invalid rows and tokens count only where the walk over positions
    consults them: before the first rejection, and the bonus row when every
    position passes."""
    rs = np.random.default_rng(8)
    B, k = 12, 3
    for T, top_k, top_p in [(1.0, 0, 1.0), (1.0, 10, 0.8)]:
        t, d, toks, u = _random_case(rs, B, k, V, dtype, T, top_k, top_p, mask_frac=0.5)
        tf = workloads.bf16_bits_to_f32(t) if dtype == "bf16" else t
        nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
        pinf = np.uint16(0x7F80) if dtype == "bf16" else np.float32(np.inf)
        ninf = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
        # sequences 0..7 pass every position they reach (token = argmax, u = 0)
        toks[:8] = np.argmax(tf[:8, :k], axis=2)
        u[:8, :k] = 0.0
        t[0, 1, 5] = nan           # consulted target row
        d[1, 2, 9] = pinf          # consulted draft row
        t[2, k, :] = ninf          # bonus row without a finite logit, all passed
        toks[3, 1] = V             # token out of range
        toks[4, 0] = -7
        d[5, 0, 100] = nan
        # sequences 6, 7 reject position 0 (its token masked in p); what lies
        # past the stop is never consulted
        for b in (6, 7):
            t[b, 0, 0] = ninf
            toks[b, 0] = 0
        t[6, 2, 4] = nan
        toks[7, 2] = V
        t[7, k, :] = ninf
        acc, out, ap = gpu_stochastic(t, d, toks, u, T, top_k, top_p)
        ref = oracle.verify_stochastic(t, d, toks, u, T, top_k, top_p)
        assert list(ref["accepted_len"][:8]) == [-1] * 6 + [0, 0]
        assert list(acc[:8]) == [-1] * 6 + [0, 0]
        assert (out[:6] == -1).all()
        compare_stochastic(ref, acc, out, ap, fp32=(dtype == "f32"), label="masks " + dtype)
        gacc, gout = sv.verify_greedy(to_dev(t), torch.from_numpy(toks).to(DEV))
        torch.cuda.synchronize()
        racc, rout = oracle.verify_greedy(t, toks)
        assert np.array_equal(gacc.cpu().numpy(), racc) and np.array_equal(gout.cpu().numpy(), rout)


def test_top_k_edge_values():
    rs = np.random.default_rng(12)
    B, k, V = 6, 3, 5000
    for top_k in (1, 2, V - 1, V, V + 10):
        for dtype in ("f32", "bf16"):
            t, d, toks, u = _random_case(rs, B, k, V, dtype, 1.0, top_k, 1.0)
            acc, out, ap = gpu_stochastic(t, d, toks, u, 1.0, top_k, 1.0)
            ref = oracle.verify_stochastic(t, d, toks, u, 1.0, top_k, 1.0)
            compare_stochastic(ref, acc, out, ap, fp32=(dtype == "f32"),
                               label="top_k=%d %s" % (top_k, dtype))


def test_ties_and_signed_zero():
    """Many equal logits (ties kept at top-k / top-p cuts) and -0 / +0 as one
    value."""
    rs = np.random.default_rng(13)
    B, k, V = 8, 3, 4096
    t = np.round(rs.normal(0, 1.5, (B, k + 1, V))).astype(np.float32)
    t[t == 0] = np.where(rs.random((t == 0).sum()) < 0.5, np.float32(-0.0), np.float32(0.0))
    d = np.round(t[:, :k] + rs.normal(0, 1, (B, k, V))).astype(np.float32)
    for dtype in ("f32", "bf16"):
        tt, dd = (t, d) if dtype == "f32" else (workloads.to_bf16_bits(t), workloads.to_bf16_bits(d))
        for top_k, top_p in [(3, 1.0), (40, 0.6), (0, 0.5), (0, 0.999)]:
            toks = oracle.sample_drafts(dd, rs.random((B, k)), 1.0, top_k, top_p)
            u = rs.random((B, k + 1)).astype(np.float32)
            acc, out, ap = gpu_stochastic(tt, dd, toks, u, 1.0, top_k, top_p)
            ref = oracle.verify_stochastic(tt, dd, toks, u, 1.0, top_k, top_p)
            compare_stochastic(ref, acc, out, ap, fp32=(dtype == "f32"),
                               label="ties %s k=%d p=%g" % (dtype, top_k, top_p))


def test_bf16_histogram_overflow_falls_back():
    """More than 65535 equal bf16 values in a row overflow a 16-bit counter;
    the kernel detects it and takes the bisection path."""
    rs = np.random.default_rng(21)
    B, k, V = 2, 2, 140000
    t = rs.normal(0, 2, (B, k + 1, V)).astype(np.float32)
    t[:, :, : 70000] = 0.5
    d = (t[:, :k] + rs.normal(0, 1, (B, k, V))).astype(np.float32)
    d[:, :, 10: 80000] = -1.0
    t, d = workloads.to_bf16_bits(t), workloads.to_bf16_bits(d)
    for top_k, top_p in [(0, 0.9), (100, 0.8), (0, 1.0)]:
        toks = oracle.sample_drafts(d, rs.random((B, k)), 1.0, top_k, top_p)
        u = rs.random((B, k + 1)).astype(np.float32)
        acc, out, ap = gpu_stochastic(t, d, toks, u, 1.0, top_k, top_p)
        ref = oracle.verify_stochastic(t, d, toks, u, 1.0, top_k, top_p)
        compare_stochastic(ref, acc, out, ap, fp32=False, label="overflow k=%d p=%g" % (top_k, top_p))
    _process_compare(t.reshape(-1, V), 1.0, 0, 0.9, "process overflow rows", False)


@pytest.mark.parametrize("case", ["tiny", "huge", "edges", "edges31", "zeros"])
def test_bf16_window_edges(case):
    """Extreme bf16 codes: many +-0 (and top-k cuts that fall on 0), non-zero
    magnitudes below 2^-63, values of 2^65 and above (one-hot rows), rows
    whose finite values all lie above the filter's exponent window, the codes
    2^-63 and (2 - 2^-7) 2^64 in rows of ordinary logits, and both ends of the
    row filter's exponent window [2^-31, 2^33) with their neighbours outside
    it (rows outside the window, or decisions among tiny values, take the
    exact bisection path)."""
    rs = np.random.default_rng(29)
    B, k, V = 6, 3, 3000
    t = rs.normal(0, 2, (B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rs.normal(0, 1, (B, k, V))).astype(np.float32)
    lo, hi = np.float32(2.0 ** -63), np.float32((2 - 2 ** -7) * 2.0 ** 64)
    if case == "tiny":
        t[0, :, :5] = 1e-25
        t[1, 0, 7] = -3e-30
        d[2, 1, 9] = 2e-22
    elif case == "huge":
        t[0, 1, 3] = 1e25
        d[1, 0, 4] = -5e20
        t[2, 2, 5] = np.float32(2.0 ** 65)
        t[3, 0, 6] = -np.float32(2.0 ** 65)
        # rows whose finite values all lie above the window, some -inf
        t[4, 1] = t[4, 1] * np.float32(2.0 ** 40)
        t[4, 1, ::7] = -np.inf
        d[5, 2] = d[5, 2] * np.float32(2.0 ** 36)
    elif case == "edges":
        t[:, :, 0] = lo
        t[:, :, 1] = -lo
        t[:, :, 2] = -hi
        d[:, :, 3] = -hi
        t[0, 1, 4] = hi
    elif case == "edges31":
        # both ends of the row filter's exponent window [2^-31, 2^33): the
        # smallest and largest codes inside it, and their neighbours outside
        w_lo, w_hi = np.float32(2.0 ** -31), np.float32((2 - 2 ** -7) * 2.0 ** 32)
        below, above = np.float32((2 - 2 ** -7) * 2.0 ** -32), np.float32(2.0 ** 33)
        t[:, :, 0] = w_lo
        t[:, :, 1] = -w_lo
        t[:, :, 2] = below
        d[:, :, 3] = -below
        t[1, :, 4] = w_hi
        d[2, 0, 5] = -w_hi
        t[3, 2, 6] = above
        d[4, 1, 7] = -above
    else:  # many +-0, and rows whose top-k cut falls on 0
        t[:, :, ::3] = 0.0
        t[:, :, 1::6] = -0.0
        t[3] = -np.abs(t[3])
        t[3, :, :100] = 0.0
    tb, db = workloads.to_bf16_bits(t), workloads.to_bf16_bits(d)
    settings = [(1.0, 0, 0.9), (1.0, 50, 1.0), (0.7, 20, 0.8), (1.0, 0, 1.0)]
    if case == "tiny":
        settings.append((0.05, 0, 0.9))  # a temperature at which tiny values' masses differ
    for T, top_k, top_p in settings:
        toks = oracle.sample_drafts(db, rs.random((B, k)), T, top_k, top_p)
        u = rs.random((B, k + 1)).astype(np.float32)
        acc, out, ap = gpu_stochastic(tb, db, toks, u, T, top_k, top_p)
        ref = oracle.verify_stochastic(tb, db, toks, u, T, top_k, top_p)
        compare_stochastic(ref, acc, out, ap, fp32=False,
                           label="window %s T=%g k=%d p=%g" % (case, T, top_k, top_p))
        _process_compare(tb.reshape(-1, V), T, top_k, top_p, "process window %s" % case, False)


def test_determinism_and_clean_workspace():
    w = workloads.generate(3, B=8)
    c = w.config
    toks = draft_tokens_from_oracle(w)
    ws = torch.zeros(sv.workspace_size(sv.SPEC_OP_STOCHASTIC, 8, 5, c.V, 1.0, 50, 0.9),
                     dtype=torch.uint8, device=DEV)
    args = (to_dev(w.target), to_dev(w.draft), torch.from_numpy(toks).to(DEV),
            torch.from_numpy(w.uniforms).to(DEV))
    r1 = sv.verify_stochastic(*args, top_k=50, top_p=0.9, return_accept_prob=True, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    r2 = sv.verify_stochastic(*args, top_k=50, top_p=0.9, return_accept_prob=True, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    wsg = torch.zeros(sv.workspace_size(sv.SPEC_OP_GREEDY, 8, 5, c.V), dtype=torch.uint8, device=DEV)
    sv.verify_greedy(args[0], args[2], workspace=wsg)
    wsp = torch.zeros(sv.workspace_size(sv.SPEC_OP_PROCESS, 40, 0, c.V), dtype=torch.uint8, device=DEV)
    sv.logits_process(args[1].reshape(-1, c.V), workspace=wsp)
    torch.cuda.synchronize()
    assert int(wsg.count_nonzero()) == 0 and int(wsp.count_nonzero()) == 0


@pytest.mark.parametrize("V", [300, 5000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_max_k_row_pass(V, dtype):
    """k = 64 (the largest) on the small-batch row pass: the draft a close copy
    of the target so that accepted runs reach deep positions and the bonus."""
    rs = np.random.default_rng(64 + V)
    B, k = 5, 64
    for T, top_k, top_p in [(1.0, 0, 1.0), (1.0, 20, 0.9)]:
        t = rs.normal(0, 2.0, (B, k + 1, V)).astype(np.float32)
        d = (t[:, :k] + rs.normal(0, 0.02, (B, k, V))).astype(np.float32)
        if dtype == "bf16":
            t, d = workloads.to_bf16_bits(t), workloads.to_bf16_bits(d)
        toks = oracle.sample_drafts(d, rs.random((B, k)), T, top_k, top_p)
        u = rs.random((B, k + 1)).astype(np.float32)
        acc, out, ap = gpu_stochastic(t, d, toks, u, T, top_k, top_p)
        ref = oracle.verify_stochastic(t, d, toks, u, T, top_k, top_p)
        compare_stochastic(ref, acc, out, ap, fp32=(dtype == "f32"),
                           label="k=64 V=%d %s T=%g k=%d p=%g" % (V, dtype, T, top_k, top_p))
        assert ref["accepted_len"].max() >= 32
    # greedy at k = 64: every draft the target's argmax, then one miss at 40
    am = oracle.argmax_drafts(t)
    full = am[:, :k].astype(np.int32)
    miss = full.copy()
    miss[1:, 40] = (am[1:, 40] + 1) % V
    tgt = to_dev(t)
    for tk in (full, miss):
        g_acc, g_out = sv.verify_greedy(tgt, torch.from_numpy(tk).to(DEV))
        torch.cuda.synchronize()
        racc, rout = oracle.verify_greedy(t, tk)
        assert np.array_equal(g_acc.cpu().numpy(), racc)
        assert np.array_equal(g_out.cpu().numpy(), rout)
    assert (racc[1:] == 40).all() and racc[0] == k
