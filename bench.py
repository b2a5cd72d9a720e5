"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = one spec_verify_stochastic call over one batch of synthetic inputs
already resident in HBM (every hot-path step: logits processing, ratio test,
first rejection, residual / bonus inverse-CDF draw).  The headline workload is
the branch-fanout verify: 32 requests x 16 branches = 512 sequences, k = 4
drafted positions each (2048 per call), V = 151936, bf16 logits, temperature 1,
top-p 0.95.  The default run also times workloads 1-4 (and workload 2's greedy
verify) and reports them under "workloads".

Per workload: HIP-event time per call, verified positions/s, the roofline
fraction of the dominant kernel and of the whole call, and the oracle leg
(the only part that runs the CPU oracle): the oracle on the timed call's own
inputs (its logits, draft tokens and uniforms) over every sequence on all of
the host's cores -- the parity check of the benchmarked call (mismatches,
boundary rows) and the all-core rate -- and on one core over a bounded
sample.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak), V=151936"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
HEADLINE = 5


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=0,
                    help="one workload (1-5) only; 0 = the headline workload 5 plus 1-4")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets cycled through (0 = enough to exceed the 256 MB MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="target time of each workload's one-core oracle sample (0 = skip the "
                         "oracle leg)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="0 = min(16, host cores)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the pooled-rows and next-row legs of workload 5")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for counter calibration)")
    ap.add_argument("--print-source-hash", action="store_true")
    return ap.parse_args()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_share(requested):
    """Worker threads for the host legs: the cores this process may run on,
    at most 16 (a one-GPU machine's share)."""
    if requested:
        return requested
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draft_tokens_on_gpu(sv, torch, draft, draft_u, T, top_k, top_p, chunk_rows=512):
    """The proposer's draw of each draft token from its processed q: the
    library's logits_process gives q, an inverse CDF (torch cumsum +
    searchsorted) with the seeded uniforms picks the token."""
    B, k, V = draft.shape
    rows = draft.contiguous().reshape(B * k, V)
    u = torch.from_numpy(draft_u.reshape(-1)).to(draft.device, torch.float64)
    out = torch.empty(B * k, dtype=torch.int64, device=draft.device)
    for lo in range(0, B * k, chunk_rows):
        hi = min(B * k, lo + chunk_rows)
        q = sv.logits_process(rows[lo:hi], temperature=T, top_k=top_k, top_p=top_p)["probs"]
        c = torch.cumsum(q.double(), dim=1)
        tgt = (u[lo:hi] * c[:, -1]).unsqueeze(1)
        idx = torch.searchsorted(c, tgt, right=True).squeeze(1)
        out[lo:hi] = idx.clamp_(max=V - 1)
        del q, c
    return out.view(B, k).to(torch.int32)


KERNEL_SOURCES = ["draft_token_verification_11_amd/csrc/sv_kernels.hpp",
                  "draft_token_verification_11_amd/csrc/sv_window.hpp",
                  "draft_token_verification_11_amd/csrc/sv_device.hpp",
                  "draft_token_verification_11_amd/csrc/sv_abi.hip"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg, kernel):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of
    known size), or None when no summary exists for this workload or the
    kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_workload%d.md" % cfg)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if not kernel.startswith(vals.get("kernel", "?")):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device copy of a known size (1 GiB read + 1 GiB written), for
    scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log("copy calibration: 3 copies of %d bytes" % n)


class Timer:
    """HIP events on the launch stream around a number of calls."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)

    def ms(self, fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        self.torch.cuda.synchronize()
        self.e0.record(self.stream)
        for i in range(steps):
            fn(i)
        self.e1.record(self.stream)
        self.torch.cuda.synchronize()
        return self.e0.elapsed_time(self.e1) / steps


# ---------------------------------------------------------------------------
# The oracle leg (the only code here that runs the CPU oracle).
def oracle_leg(c, host, toks, acc, out, threads, one_core_s):
    """The oracle on the timed call's own inputs: every sequence of input set
    0 on `threads` threads (parity of the benchmarked call and the all-core
    rate), then a bounded sample of sequences on one core."""
    import numpy as np

    import oracle
    from tests.gpu_common import parity_counts

    target, draft, uni = host
    B = target.shape[0]
    parts = [None] * threads
    step = (B + threads - 1) // threads

    def work(i):
        lo, hi = i * step, min(B, (i + 1) * step)
        if lo < hi:
            parts[i] = oracle.verify_stochastic(target[lo:hi], draft[lo:hi], toks[lo:hi],
                                                uni[lo:hi], c.temperature, c.top_k, c.top_p)

    def all_threads():
        ths = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
        for t in ths:
            t.start()
        for t in ths:
            t.join()

    t0 = time.perf_counter()
    all_threads()
    dt_all = time.perf_counter() - t0
    reps = 1
    while time.perf_counter() - t0 < 0.5:  # short runs (small batches) are repeated
        all_threads()
        reps += 1
    dt_all = (time.perf_counter() - t0) / reps
    parts = [p for p in parts if p is not None]
    used = len(parts)
    ref = {k: np.concatenate([p[k] for p in parts]) for k in parts[0] if k != "inputs"}
    ref["inputs"] = {"target": target, "draft": draft, "tokens": toks, "uniforms": uni,
                     "temperature": c.temperature, "top_k": c.top_k, "top_p": c.top_p}
    counts = parity_counts(ref, acc, out, fp32=(c.dtype == "f32"))
    res = {"all_cores": {"value": B * c.k / dt_all, "unit": "positions/s", "cores": used,
                         "sample": "all %d sequences of the timed input set, %.3f s wall on %d "
                                   "threads (mean of %d runs)" % (B, dt_all, used, reps)}}
    res.update(counts)
    if one_core_s > 0:
        try:
            mask = os.sched_getaffinity(0)
        except AttributeError:
            mask = None
        try:
            if mask:
                os.sched_setaffinity(0, {min(mask)})
            t0 = time.perf_counter()
            oracle.verify_stochastic(target[:1], draft[:1], toks[:1], uni[:1], c.temperature,
                                     c.top_k, c.top_p)
            per = max(time.perf_counter() - t0, 1e-5)
            n = int(max(1, min(B, one_core_s / per)))
            t0 = time.perf_counter()
            reps1 = 0
            while reps1 == 0 or time.perf_counter() - t0 < 0.5 * one_core_s:
                oracle.verify_stochastic(target[:n], draft[:n], toks[:n], uni[:n], c.temperature,
                                         c.top_k, c.top_p)
                reps1 += 1
            dt = (time.perf_counter() - t0) / reps1
        finally:
            if mask:
                os.sched_setaffinity(0, mask)
        res["one_core"] = {"value": n * c.k / dt, "unit": "positions/s", "cores": 1,
                           "sample": "%d of %d sequences, %.3f s on one core (mean of %d runs)"
                                     % (n, B, dt, reps1)}
    return res


# ---------------------------------------------------------------------------
def run_workload(cfg, args, sv, torch, dev, stream, threads, headline):
    """Times the verify call of one workload; returns its figures."""
    import numpy as np

    import workloads
    c = workloads.CONFIGS[cfg]
    esize = 2 if c.dtype == "bf16" else 4
    set_bytes = c.B * (2 * c.k + 1) * c.V * esize
    nsets = args.rotate or (1 if set_bytes >= 768e6 else min(4, int(np.ceil(768e6 / set_bytes))))
    log("workload %d: %s; %d input set(s) of %.1f MB" % (cfg, c.name, nsets, set_bytes / 1e6))

    def up(a):
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
        return t.view(torch.bfloat16) if a.dtype == np.uint16 else t

    sets, host = [], None
    for s in range(nsets):
        # set s holds sequences s*B .. s*B+B-1 of the same seeded recipe, in
        # one [B][2k+1][V] tensor: rows 0..k the target, rows k+1..2k the draft
        t0 = time.perf_counter()
        w = workloads.generate(cfg, seqs=np.arange(s * c.B, (s + 1) * c.B), threads=threads)
        tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        big = torch.empty((c.B, 2 * c.k + 1, c.V), dtype=tdt, device=dev)
        big[:, : c.k + 1] = up(w.target)
        big[:, c.k + 1:] = up(w.draft)
        uni = torch.from_numpy(w.uniforms).to(dev)
        tgt, drf = big[:, : c.k + 1], big[:, c.k + 1:]
        toks = draft_tokens_on_gpu(sv, torch, drf, w.draft_u, c.temperature, c.top_k, c.top_p)
        torch.cuda.synchronize()
        sets.append((tgt, drf, uni, toks, big))
        if s == 0:
            host = (w.target, w.draft, w.uniforms)
        del w
        log("  set %d ready in %.1f s" % (s, time.perf_counter() - t0))

    ws = torch.zeros(sv.workspace_size(sv.SPEC_OP_STOCHASTIC, c.B, c.k, c.V, c.temperature,
                                       c.top_k, c.top_p), dtype=torch.uint8, device=dev)
    acc = torch.empty(c.B, dtype=torch.int32, device=dev)
    out = torch.empty((c.B, c.k + 1), dtype=torch.int32, device=dev)
    timer = Timer(torch, stream)

    def step(i):
        tgt, drf, uni, toks, _ = sets[i % len(sets)]
        sv.verify_stochastic(tgt, drf, toks, uni, temperature=c.temperature, top_k=c.top_k,
                             top_p=c.top_p, out=(acc, out), workspace=ws, stream=stream)

    path = sv.verify_stochastic_path(sets[0][0], sets[0][1], temperature=c.temperature,
                                     top_k=c.top_k, top_p=c.top_p, stream=stream)
    # rows each input set's call reads: on the one-kernel paths the rows the
    # walk consults (target and draft up to the stop, the bonus row when all
    # pass), on the row pass every row; plus the draw's second pass over the
    # rows at the stop (t_n and d_n, or t_k)
    walk_rows, draw_rows, outs = [], [], []
    for i in range(len(sets)):
        step(i)
        torch.cuda.synchronize()
        n = acc.cpu().numpy()
        outs.append((n.copy(), out.cpu().numpy()))
        walk_rows.append(int(np.where(n < 0, 0, np.where(n < c.k, 2 * (n + 1), 2 * c.k + 1)).sum()))
        draw_rows.append(int(np.where(n < 0, 0, np.where(n < c.k, 2, 1)).sum()))
    mean_acc = float(outs[0][0][outs[0][0] >= 0].mean())
    t_wall = time.perf_counter()
    ms = timer.ms(step, args.steps, args.warmup)
    wall = time.perf_counter() - t_wall
    positions = c.B * c.k
    value = positions / (ms / 1e3)

    # the row pass over every target and draft row, launched alone through
    # spec_logits_process (statistics only): the dominant kernel of the
    # row-pass path, and context for the one-kernel paths
    rows_all = c.B * (2 * c.k + 1)
    proc_ws = torch.zeros(sv.workspace_size(sv.SPEC_OP_PROCESS, rows_all, 0, c.V, c.temperature,
                                            c.top_k, c.top_p), dtype=torch.uint8, device=dev)

    def row_pass(i):
        big = sets[i % len(sets)][4]
        sv.logits_process(big.view(-1, c.V), temperature=c.temperature, top_k=c.top_k,
                          top_p=c.top_p, return_probs=False, workspace=proc_ws, stream=stream)

    ms_rows = timer.ms(row_pass, args.steps, args.warmup)
    row_bytes = c.V * esize
    a1_bytes = rows_all * row_bytes  # every row once
    draw_bytes = float(np.mean([draw_rows[i % len(sets)] for i in range(args.steps)])) * row_bytes
    filtered = bool(c.top_k) or c.top_p < 1.0
    row_kernel = ("k_filter_win_persistent (exact bf16 window histogram, two workgroups per CU, top-k/top-p)"
                  if c.dtype == "bf16" and filtered else
                  "k_filter_bisect (fp32 top-k/top-p)" if filtered else
                  "k_row_partials (split-V max / sum of exponentials)")
    achieved_rows = a1_bytes / (ms_rows / 1e3) / 1e9
    direct = not filtered and c.V <= 4096  # the tail computes such rows' statistics itself
    if path != sv.SPEC_PATH_ROW_PASS:
        kernel = ("k_verify_pair_bf16 (position-task queue; a position's target and draft rows "
                  "counted at once into two exact bf16 window histograms)")
        alg_bytes = float(np.mean([walk_rows[i % len(sets)] for i in range(args.steps)])) * \
            row_bytes + draw_bytes
        kernel_ms = ms
        call_bytes = alg_bytes
    elif direct:
        kernel = "k_tail (rows of V <= 4096: statistics, tests and draw in one kernel per call)"
        alg_bytes = a1_bytes + draw_bytes
        kernel_ms = ms
        call_bytes = alg_bytes
    else:
        kernel = row_kernel
        alg_bytes = a1_bytes
        kernel_ms = ms_rows
        call_bytes = a1_bytes + draw_bytes
    achieved = alg_bytes / (kernel_ms / 1e3) / 1e9
    achieved_call = call_bytes / (ms / 1e3) / 1e9
    log("  %s path: %.4f ms/call (wall %.4f), %.4g positions/s; %s %.1f GB/s (%.1f%%); whole "
        "call %.1f%%; row pass over every row %.4f ms = %.1f GB/s (%.1f%%); mean accepted %.3f"
        % (sv.PATH_NAMES[path], ms, wall * 1e3 / args.steps, value, kernel.split()[0], achieved,
           100 * achieved / PEAK_HBM_GBPS, 100 * achieved_call / PEAK_HBM_GBPS, ms_rows,
           achieved_rows, 100 * achieved_rows / PEAK_HBM_GBPS, mean_acc))
    res = {
        "workload": c.name, "B": c.B, "k": c.k, "V": c.V, "logits_dtype": c.dtype,
        "temperature": c.temperature, "top_k": c.top_k, "top_p": c.top_p,
        "input_sets": len(sets), "path": sv.PATH_NAMES[path], "ms_per_call": ms,
        "positions_per_s": value, "mean_accepted": mean_acc,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": measured_traffic(cfg, kernel), "kernel": kernel,
                     "kernel_ms": kernel_ms, "algorithmic_bytes_per_launch": alg_bytes,
                     "whole_call": {"achieved": achieved_call,
                                    "frac": achieved_call / PEAK_HBM_GBPS,
                                    "algorithmic_bytes": call_bytes},
                     "row_pass_every_row": {"kernel": row_kernel, "ms": ms_rows, "bytes": a1_bytes,
                                            "achieved": achieved_rows,
                                            "frac": achieved_rows / PEAK_HBM_GBPS}},
    }
    del proc_ws

    if cfg == 2:
        # the greedy verify of the same rows: drafts are the argmax of the draft rows
        gtoks = [torch.argmax(s_[1].float(), dim=2).to(torch.int32) for s_ in sets]
        gacc = torch.empty(c.B, dtype=torch.int32, device=dev)
        gout = torch.empty((c.B, c.k + 1), dtype=torch.int32, device=dev)
        gws = torch.zeros(sv.workspace_size(sv.SPEC_OP_GREEDY, c.B, c.k, c.V), dtype=torch.uint8,
                          device=dev)

        def gstep(i):
            sv.verify_greedy(sets[i % len(sets)][0], gtoks[i % len(sets)], out=(gacc, gout),
                             workspace=gws, stream=stream)

        ms_g = timer.ms(gstep, args.steps, args.warmup)
        gstep(0)
        torch.cuda.synchronize()
        res["greedy"] = {"ms_per_call": ms_g, "positions_per_s": positions / (ms_g / 1e3),
                         "bytes": c.B * (c.k + 1) * row_bytes,
                         "achieved_GBps": c.B * (c.k + 1) * row_bytes / (ms_g / 1e3) / 1e9}
        res["greedy"]["_check"] = (gtoks[0].cpu().numpy(), gacc.cpu().numpy(), gout.cpu().numpy())
        log("  greedy: %.4f ms/call, %.4g positions/s" % (ms_g, positions / (ms_g / 1e3)))

    extras = {}
    if headline and not args.no_extras:
        extras = headline_extras(c, args, sv, torch, dev, stream, sets, step, acc, out, timer)

    # the oracle leg on input set 0: its own draft tokens and uniforms
    if args.cpu_seconds > 0:
        toks0 = sets[0][3].cpu().numpy()
        leg = oracle_leg(c, host, toks0, outs[0][0], outs[0][1], threads, args.cpu_seconds)
        res["oracle"] = leg
        log("  oracle: parity mismatches %d, boundary rows %d (inadmissible %d); %.4g positions/s "
            "on %d threads, %.4g on one core"
            % (leg["parity_mismatches"], leg["boundary_rows"], leg["boundary_inadmissible"],
               leg["all_cores"]["value"], leg["all_cores"]["cores"],
               leg.get("one_core", {}).get("value", float("nan"))))
        if cfg == 2:
            import oracle
            gt, ga, go = res["greedy"].pop("_check")
            racc, rout = oracle.verify_greedy(host[0], gt)
            res["greedy"]["bit_exact_vs_oracle"] = bool(np.array_equal(ga, racc) and
                                                        np.array_equal(go, rout))
    res.get("greedy", {}).pop("_check", None)
    del sets, ws, host
    torch.cuda.empty_cache()
    return res, extras


def headline_extras(c, args, sv, torch, dev, stream, sets, step, acc, out, timer):
    """Branch fan-out with pooled target rows, and the rows built beside the
    verify (processors pass, outcome lookup, fused LM head + greedy)."""
    extras = {}
    positions = c.B * c.k
    tgt0, drf0, uni0, toks0, big0 = sets[0]
    if c.branches > 1:
        # the same call with each request's target rows held once
        k1 = c.k + 1
        tpool = tgt0[::c.branches].contiguous().view(-1, c.V)
        dpool = big0.view(-1, c.V)
        bidx = torch.arange(c.B, device=dev, dtype=torch.int64)
        tmap = ((bidx // c.branches)[:, None] * k1 + torch.arange(k1, device=dev)[None, :]).to(torch.int32)
        dmap = (bidx[:, None] * (2 * c.k + 1) + k1 + torch.arange(c.k, device=dev)[None, :]).to(torch.int32)
        pws = torch.zeros(sv.workspace_size_pooled(sv.SPEC_OP_STOCHASTIC, tpool.shape[0],
                                                   dpool.shape[0], c.B, c.k, c.V, c.temperature,
                                                   c.top_k, c.top_p), dtype=torch.uint8, device=dev)
        pacc = torch.empty_like(acc)
        pout = torch.empty_like(out)

        def pstep(i):
            sv.verify_stochastic_pooled(tpool, dpool, toks0, uni0, target_map=tmap, draft_map=dmap,
                                        temperature=c.temperature, top_k=c.top_k, top_p=c.top_p,
                                        out=(pacc, pout), workspace=pws, stream=stream)

        step(0)
        pstep(0)
        torch.cuda.synchronize()
        same = bool(torch.equal(pacc, acc) and torch.equal(pout, out))
        ms_p = timer.ms(pstep, args.steps, args.warmup)
        extras["pooled_rows"] = {"target_rows": int(tpool.shape[0]), "ms_per_step": ms_p,
                                 "value": positions / (ms_p / 1e3), "unit": "positions/s",
                                 "same_outputs_as_dense": same}
        log("  pooled rows (%d target rows): %.4f ms, %.4g positions/s, outputs %s"
            % (tpool.shape[0], ms_p, positions / (ms_p / 1e3), "identical" if same else "DIFFER"))

    next_rows = {}
    W = (c.V + 31) // 32
    g = torch.Generator(device=dev).manual_seed(1234)
    allow = torch.randint(-2**31, 2**31 - 1, (c.B, 2 * c.k + 1, W), dtype=torch.int32,
                          device=dev, generator=g)
    pen = torch.randint(-2**31, 2**31 - 1, (c.B, 1, W), dtype=torch.int32, device=dev,
                        generator=g) & 0x01010101
    aout = torch.empty_like(big0)

    def apply_step(i):
        sv.logits_apply(big0, allow=allow, penalize=pen, theta=1.2, out=aout, stream=stream)

    ms_a = timer.ms(apply_step, args.steps, 1)
    a_bytes = big0.numel() * 2 * 2 + allow.numel() * 4 + pen.numel() * 4
    next_rows["logits_apply"] = {"kernel": "k_logits_apply", "ms": ms_a, "bytes": a_bytes,
                                 "achieved_GBps": a_bytes / (ms_a / 1e3) / 1e9,
                                 "frac": a_bytes / (ms_a / 1e3) / 1e9 / PEAK_HBM_GBPS,
                                 "rows": c.B * (2 * c.k + 1)}
    del aout, allow, pen
    # predicted-outcome lookup: 16 predictions per sequence that differ from
    # the call's outcome by construction, plus the true outcome planted at a
    # known slot in every fourth sequence; the hits must be exactly those
    step(0)
    torch.cuda.synchronize()
    P = 16
    n = acc.long().clamp(min=0)
    true_tok = out.gather(1, n.unsqueeze(1)).squeeze(1)
    pl = torch.randint(0, c.k + 1, (c.B, P), dtype=torch.int32, device=dev, generator=g)
    pt = torch.randint(0, c.V, (c.B, P), dtype=torch.int32, device=dev, generator=g)
    same_len = pl == acc[:, None]
    pt = torch.where(same_len & (pt == true_tok[:, None]), (pt + 1) % c.V, pt)
    planted = torch.zeros(c.B, dtype=torch.bool, device=dev)
    planted[::4] = True
    planted &= acc >= 0
    slot = torch.randint(0, P, (c.B,), device=dev, generator=g)
    rows = torch.nonzero(planted).squeeze(1)
    pl[rows, slot[rows]] = acc[rows]
    pt[rows, slot[rows]] = true_tok[rows].to(torch.int32)
    hits, cnt = sv.outcome_lookup(acc, out, pl, pt, stream=stream)
    torch.cuda.synchronize()
    want = torch.where(planted, slot, torch.full_like(slot, -1)).to(torch.int32)
    ms_l = timer.ms(lambda i: sv.outcome_lookup(acc, out, pl, pt, stream=stream), args.steps, 1)
    next_rows["outcome_lookup"] = {"kernels": "k_outcome_lookup + k_count_hits", "set_size": P,
                                   "us": ms_l * 1e3, "hits": int(cnt.item()),
                                   "planted": int(planted.sum().item()),
                                   "hits_at_planted_slots": bool(torch.equal(hits, want))}
    # fused LM head + greedy verify at the greedy workload's shape (k = 8,
    # V = 151936) with a synthetic head of d = 4096, at B = 1 and 48
    for Bl in (1, 48):
        d = 4096
        gh = torch.Generator(device=dev).manual_seed(77)
        Wh = (torch.randn((c.V, d), device=dev, generator=gh) / d ** 0.5).to(torch.bfloat16)
        Hd = torch.randn((Bl, 9, d), device=dev, generator=gh).to(torch.bfloat16)
        lt = torch.zeros((Bl, 8), dtype=torch.int32, device=dev)
        lws = torch.zeros(sv.workspace_size(sv.SPEC_OP_GREEDY_LMHEAD, Bl, 8, c.V),
                          dtype=torch.uint8, device=dev)
        la = torch.empty(Bl, dtype=torch.int32, device=dev)
        lo = torch.empty((Bl, 9), dtype=torch.int32, device=dev)
        Wt = Wh.t().contiguous()
        gws = torch.zeros(sv.workspace_size(sv.SPEC_OP_GREEDY, Bl, 8, c.V), dtype=torch.uint8,
                          device=dev)

        def fused(i):
            sv.verify_greedy_lmhead(Hd, Wh, lt, out=(la, lo), workspace=lws, stream=stream)

        def unfused(i):
            logits = torch.matmul(Hd.reshape(-1, d), Wt).view(Bl, 9, c.V)
            sv.verify_greedy(logits, lt, workspace=gws, stream=stream)

        r = {"fused_ms": timer.ms(fused, args.steps, 1),
             "unfused_bf16_matmul_then_verify_ms": timer.ms(unfused, args.steps, 1)}
        wbytes = c.V * d * 2 + Bl * 9 * d * 2
        r.update({"B": Bl, "k": 8, "d": d, "V": c.V, "rows": Bl * 9, "head_bytes": wbytes,
                  "fused_GBps": wbytes / (r["fused_ms"] / 1e3) / 1e9,
                  "fused_frac_hbm": wbytes / (r["fused_ms"] / 1e3) / 1e9 / PEAK_HBM_GBPS,
                  "fused_TFLOPs": 2.0 * Bl * 9 * c.V * d / (r["fused_ms"] / 1e3) / 1e12})
        next_rows["lmhead_greedy_B%d" % Bl] = r
        log("  fused LM head + greedy (B=%d, k=8, d=%d): %.4f ms, unfused %.4f ms"
            % (Bl, d, r["fused_ms"], r["unfused_bf16_matmul_then_verify_ms"]))
        # The stochastic rule has no fused kernel: what such a kernel would
        # have to beat is the two heads' products (target rows from the
        # target's head, draft rows from a head of the draft model's own)
        # followed by the stochastic verify over the logits they produce.
        Wd = (torch.randn((c.V, d), device=dev, generator=gh) / d ** 0.5).to(torch.bfloat16)
        Wdt = Wd.t().contiguous()
        Hq = torch.randn((Bl, 8, d), device=dev, generator=gh).to(torch.bfloat16)
        su = torch.rand((Bl, 9), device=dev, generator=gh)
        stok = torch.randint(0, c.V, (Bl, 8), device=dev, generator=gh, dtype=torch.int32)
        sws = torch.zeros(sv.workspace_size(sv.SPEC_OP_STOCHASTIC, Bl, 8, c.V, 0.7),
                          dtype=torch.uint8, device=dev)
        tl = torch.empty((Bl, 9, c.V), dtype=torch.bfloat16, device=dev)
        dl = torch.empty((Bl, 8, c.V), dtype=torch.bfloat16, device=dev)

        def products(i):
            torch.matmul(Hd.reshape(-1, d), Wt, out=tl.view(-1, c.V))
            torch.matmul(Hq.reshape(-1, d), Wdt, out=dl.view(-1, c.V))

        def verify_only(i):
            sv.verify_stochastic(tl, dl, stok, su, temperature=0.7, workspace=sws, stream=stream)

        def unfused_s(i):
            products(i)
            verify_only(i)

        rs_ = {"B": Bl, "k": 8, "d": d, "V": c.V, "temperature": 0.7,
               "two_bf16_matmuls_ms": timer.ms(products, args.steps, 1),
               "verify_stochastic_ms": timer.ms(verify_only, args.steps, 1),
               "unfused_total_ms": timer.ms(unfused_s, args.steps, 1)}
        # the bytes such a fused kernel could not avoid: both heads once
        rs_["heads_bytes"] = 2 * c.V * d * 2
        rs_["floor_ms_at_peak_hbm"] = rs_["heads_bytes"] / (PEAK_HBM_GBPS * 1e9) * 1e3
        next_rows["lmhead_stochastic_unfused_B%d" % Bl] = rs_
        log("  stochastic LM head, unfused (B=%d): products %.4f ms + verify %.4f ms = %.4f ms"
            % (Bl, rs_["two_bf16_matmuls_ms"], rs_["verify_stochastic_ms"], rs_["unfused_total_ms"]))
        del Wh, Wt, Hd, Wd, Wdt, Hq, tl, dl
    log("  logits_apply over %d rows: %.4f ms = %.0f GB/s; outcome lookup: %d hits of %d planted"
        % (c.B * (2 * c.k + 1), ms_a, next_rows["logits_apply"]["achieved_GBps"],
           next_rows["outcome_lookup"]["hits"], next_rows["outcome_lookup"]["planted"]))
    extras["next_rows"] = next_rows
    return extras


def main():
    args = parse()
    if args.print_source_hash:
        print(kernel_source_hash())
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (every sequence "
              "is independent, so G GPUs would each run this call on B/G sequences); run with "
              "--gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import draft_token_verification_11_amd as sv

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    threads = host_share(args.cpu_threads)
    head_cfg = args.config or HEADLINE
    head, extras = run_workload(head_cfg, args, sv, torch, dev, stream, threads, headline=True)
    others = {}
    if not args.config:
        for cfg in (1, 2, 3, 4):
            others[str(cfg)], _ = run_workload(cfg, args, sv, torch, dev, stream, threads, False)

    leg = head.get("oracle")
    cpu = None
    if leg:
        cpu = dict(leg["all_cores"], kind="oracle", cpu_model=cpu_model(),
                   one_core=leg.get("one_core"))
    line = {
        "metric": METRIC,
        "value": head["positions_per_s"],
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic of the path: per-element probabilities in fp32 (sums and
        # the ratio test in fp64); the logits themselves are config.logits_dtype
        "dtype": "fp32",
        "data": "synthetic (seeded generators, see workloads/)",
        "config": {k: head[k] for k in ("workload", "B", "k", "V", "logits_dtype", "temperature",
                                        "top_k", "top_p", "input_sets", "mean_accepted", "path")},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "parity": ({k: leg[k] for k in ("parity_mismatches", "boundary_rows",
                                        "boundary_inadmissible")} if leg else None),
    }
    line.update(extras)
    if others:
        line["workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
