"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = one spec_verify_stochastic call over one batch of synthetic inputs
already resident in HBM (every hot-path step: logits processing, ratio test,
first rejection, residual / bonus inverse-CDF draw).  The default workload is
the branch-fanout verify: 32 requests x 16 branches = 512 sequences, k = 4
drafted positions each (2048 per call), V = 151936, bf16 logits, temperature 1,
top-p 0.95.

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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, help="workload number (1-5)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets cycled through (0 = enough to exceed the 256 MB MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="0 = min(16, host cores)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for counter calibration)")
    ap.add_argument("--print-source-hash", action="store_true")
    return ap.parse_args()


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


def cpu_baseline(cfg, budget_s, threads):
    """The oracle, as it is, on a bounded sample of the same workload: whole
    sequences, drafts drawn by the oracle's own sampler, single-threaded calls
    spread over `threads` host threads."""
    import numpy as np

    import oracle
    import workloads
    c = workloads.CONFIGS[cfg]
    # calibrate on one sequence
    w1 = workloads.generate(cfg, seqs=[0])
    tok1 = oracle.sample_drafts(w1.draft, w1.draft_u, c.temperature, c.top_k, c.top_p)
    t0 = time.perf_counter()
    oracle.verify_stochastic(w1.target, w1.draft, tok1, w1.uniforms, c.temperature, c.top_k,
                             c.top_p)
    per_seq = max(time.perf_counter() - t0, 1e-4)
    n = int(max(1, min(c.B, budget_s * threads / per_seq)))
    seqs = np.linspace(0, c.B - 1, n).astype(np.int64)
    w = workloads.generate(cfg, seqs=seqs, threads=threads)
    toks = oracle.sample_drafts(w.draft, w.draft_u, c.temperature, c.top_k, c.top_p, threads)
    step = (n + threads - 1) // threads
    spans = [(lo, min(n, lo + step)) for lo in range(0, n, step)]

    def work(lo, hi):
        oracle.verify_stochastic(w.target[lo:hi], w.draft[lo:hi], toks[lo:hi], w.uniforms[lo:hi],
                                 c.temperature, c.top_k, c.top_p)

    ths = [threading.Thread(target=work, args=s) for s in spans]
    t0 = time.perf_counter()
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    dt = time.perf_counter() - t0
    return {"value": n * c.k / dt, "unit": "positions/s", "cores": len(spans), "kind": "oracle",
            "sample": "%d of %d sequences (k=%d, V=%d), %.1f s wall on %d threads"
                      % (n, c.B, c.k, c.V, dt, len(spans))}


def main():
    args = parse()
    if args.print_source_hash:
        print(kernel_source_hash())
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import draft_token_verification_11_amd as sv
    import workloads

    cfg = args.config
    c = workloads.CONFIGS[cfg]
    dev = torch.device("cuda:0")
    esize = 2 if c.dtype == "bf16" else 4
    host_threads = args.cpu_threads or min(16, os.cpu_count() or 1)
    set_bytes = c.B * (2 * c.k + 1) * c.V * esize
    nsets = args.rotate or max(1, int(np.ceil(3 * 256e6 / set_bytes)) if set_bytes < 768e6 else 1)
    log("workload %d: %s; %d input set(s) of %.1f MB" % (cfg, c.name, nsets, set_bytes / 1e6))

    def up(a):
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
        return t.view(torch.bfloat16) if a.dtype == np.uint16 else t

    sets = []
    for s in range(nsets):
        # set s holds sequences s*B .. s*B+B-1 of the same seeded recipe, in one
        # [B][2k+1][V] tensor: rows 0..k the target, rows k+1..2k the draft
        t0 = time.perf_counter()
        w = workloads.generate(cfg, seqs=np.arange(s * c.B, (s + 1) * c.B), threads=host_threads)
        tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        big = torch.empty((c.B, 2 * c.k + 1, c.V), dtype=tdt, device=dev)
        big[:, : c.k + 1] = up(w.target)
        big[:, c.k + 1:] = up(w.draft)
        uni = torch.from_numpy(w.uniforms).to(dev)
        draft_u = w.draft_u
        del w
        tgt, drf = big[:, : c.k + 1], big[:, c.k + 1:]
        toks = draft_tokens_on_gpu(sv, torch, drf, draft_u, c.temperature, c.top_k, c.top_p)
        torch.cuda.synchronize()
        sets.append((tgt, drf, uni, toks, big))
        log("  set %d ready in %.1f s" % (s, time.perf_counter() - t0))

    ws = torch.zeros(sv.workspace_size(sv.SPEC_OP_STOCHASTIC, c.B, c.k, c.V, c.temperature,
                                       c.top_k, c.top_p), dtype=torch.uint8, device=dev)
    acc = torch.empty(c.B, dtype=torch.int32, device=dev)
    out = torch.empty((c.B, c.k + 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        tgt, drf, uni, toks, _ = sets[i % len(sets)]
        sv.verify_stochastic(tgt, drf, toks, uni, temperature=c.temperature, top_k=c.top_k,
                             top_p=c.top_p, out=(acc, out, None), workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Large batches of aligned bf16 rows take the position-task kernel (one
    # kernel: rows in walk order, nothing past the first rejection); other
    # shapes a row pass over every row and a per-sequence tail kernel.
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    walk = c.dtype == "bf16" and (c.V * esize) % 16 == 0 and c.B >= 2 * cus
    # rows each input set's call reads: the rows the walk consults (target
    # and draft up to the stop, the bonus row when all pass) and the rows of
    # the second pass of the correction draw (t_n and d_n, or t_k)
    walk_rows, draw_rows = [], []
    for i in range(len(sets)):
        step(i)
        torch.cuda.synchronize()
        n = acc.cpu().numpy()
        walk_rows.append(int(np.where(n < 0, 0, np.where(n < c.k, 2 * (n + 1), 2 * c.k + 1)).sum()))
        draw_rows.append(int(np.where(n < 0, 0, np.where(n < c.k, 2, 1)).sum()))
        if i == 0:
            mean_acc = float(n.mean())
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    positions = c.B * c.k
    value = positions / (ms / 1e3)

    # The dominant kernel -- the per-row statistics pass over every target
    # and draft row -- timed alone: the same kernel on the same rows, launched
    # through spec_logits_process (statistics only, no dense output).
    proc_ws = torch.zeros(sv.workspace_size(sv.SPEC_OP_PROCESS, c.B * (2 * c.k + 1), 0, c.V,
                                            c.temperature, c.top_k, c.top_p),
                          dtype=torch.uint8, device=dev)

    def row_pass(i):
        big = sets[i % len(sets)][4]
        sv.logits_process(big.view(-1, c.V), temperature=c.temperature, top_k=c.top_k,
                          top_p=c.top_p, return_probs=False, workspace=proc_ws, stream=stream)

    for i in range(args.warmup):
        row_pass(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        row_pass(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_rows = ev0.elapsed_time(ev1) / args.steps

    row_bytes = c.V * esize
    a1_bytes = c.B * (2 * c.k + 1) * row_bytes  # every row once
    draw_bytes = np.mean([draw_rows[i % len(sets)] for i in range(args.steps)]) * row_bytes
    achieved_rows = a1_bytes / (ms_rows / 1e3) / 1e9
    row_kernel = ("k_filter_bf16_persistent (exact bf16 key histogram, top-k/top-p)"
                  if c.dtype == "bf16" and (c.top_k or c.top_p < 1.0) else
                  "k_filter_bisect (fp32 top-k/top-p)" if (c.top_k or c.top_p < 1.0) else
                  "k_row_partials (split-V max / sum of exponentials; rows of V <= 4096 get "
                  "their statistics in the tail instead, this line times the row pass alone)"
                  if c.V <= 4096 else
                  "k_row_partials (split-V max / sum of exponentials)")
    if walk:
        # the call is one kernel: its bytes are the rows it consults plus the
        # draw's second pass over the rows at the stop
        kernel = "k_verify_task_bf16 (position-task queue, exact bf16 key histogram)"
        alg_bytes = np.mean([walk_rows[i % len(sets)] for i in range(args.steps)]) * row_bytes + draw_bytes
        kernel_ms = ms
    else:
        kernel = row_kernel
        alg_bytes = a1_bytes
        kernel_ms = ms_rows
    achieved = alg_bytes / (kernel_ms / 1e3) / 1e9
    call_bytes = alg_bytes if walk else a1_bytes + draw_bytes
    achieved_call = call_bytes / (ms / 1e3) / 1e9
    traffic = measured_traffic(cfg, kernel)
    log("ms/step %.4f (wall %.4f), positions/s %.4g; %s: %.1f GB/s (%.1f%% of %g); "
        "row pass over every row (logits_process) %.4f ms = %.1f GB/s (%.1f%%); mean accepted %.3f"
        % (ms, wall * 1e3 / args.steps, value, kernel.split()[0], achieved,
           100 * achieved / PEAK_HBM_GBPS, PEAK_HBM_GBPS, ms_rows, achieved_rows,
           100 * achieved_rows / PEAK_HBM_GBPS, mean_acc))

    # Branch fan-out: the same call with each request's target rows held once
    # (pooled rows: 160 target rows for 32 requests instead of one copy per
    # branch); identical decisions and draws, fewer bytes.
    pooled = None
    if c.branches > 1:
        tgt0, drf0, uni0, toks0, big0 = sets[0]
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

        def pstep():
            sv.verify_stochastic_pooled(tpool, dpool, toks0, uni0, target_map=tmap, draft_map=dmap,
                                        temperature=c.temperature, top_k=c.top_k, top_p=c.top_p,
                                        out=(pacc, pout, None), workspace=pws, stream=stream)

        step(0)
        for _ in range(args.warmup):
            pstep()
        torch.cuda.synchronize()
        same = bool(torch.equal(pacc, acc) and torch.equal(pout, out))
        ev0.record(stream)
        for _ in range(args.steps):
            pstep()
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_p = ev0.elapsed_time(ev1) / args.steps
        pooled = {"target_rows": int(tpool.shape[0]), "ms_per_step": ms_p,
                  "value": positions / (ms_p / 1e3), "unit": "positions/s",
                  "same_outputs_as_dense": same}
        log("pooled rows (%d target rows): %.4f ms, %.4g positions/s, outputs %s"
            % (tpool.shape[0], ms_p, positions / (ms_p / 1e3), "identical" if same else "DIFFER"))

    # The next rows built beside the verify: logits processors over every row
    # of the input set (allow mask per position, repetition penalty per
    # sequence) and the predicted-outcome lookup on the call's outputs.
    next_rows = {}
    if c.dtype == "bf16":
        big0 = sets[0][4]
        W = (c.V + 31) // 32
        g = torch.Generator(device=dev).manual_seed(1234)
        allow = torch.randint(-2**31, 2**31 - 1, (c.B, 2 * c.k + 1, W), dtype=torch.int32,
                              device=dev, generator=g)
        pen = torch.randint(-2**31, 2**31 - 1, (c.B, 1, W), dtype=torch.int32, device=dev,
                            generator=g) & 0x01010101
        pout = torch.empty_like(big0)

        def apply_step():
            sv.logits_apply(big0, allow=allow, penalize=pen, theta=1.2, out=pout, stream=stream)

        apply_step()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            apply_step()
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_a = ev0.elapsed_time(ev1) / args.steps
        nelem = big0.numel()
        a_bytes = nelem * esize * 2 + allow.numel() * 4 + pen.numel() * 4
        next_rows["logits_apply"] = {
            "kernel": "k_logits_apply", "ms": ms_a, "bytes": a_bytes,
            "achieved_GBps": a_bytes / (ms_a / 1e3) / 1e9,
            "frac": a_bytes / (ms_a / 1e3) / 1e9 / PEAK_HBM_GBPS,
            "rows": c.B * (2 * c.k + 1)}
        P = 16
        pl = torch.randint(-1, c.k + 1, (c.B, P), dtype=torch.int32, device=dev, generator=g)
        pt = torch.randint(0, c.V, (c.B, P), dtype=torch.int32, device=dev, generator=g)
        step(0)
        pl[:, 0] = acc
        pt[:, 0] = out.gather(1, acc.clamp(min=0).long().unsqueeze(1)).squeeze(1)
        hits, cnt = sv.outcome_lookup(acc, out, pl, pt, stream=stream)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            sv.outcome_lookup(acc, out, pl, pt, stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        next_rows["outcome_lookup"] = {"kernels": "k_outcome_lookup + k_count_hits",
                                       "set_size": P, "us": ev0.elapsed_time(ev1) / args.steps * 1e3,
                                       "hits": int(cnt.item())}
        # fused LM head + greedy verify at the greedy workload's shape (B = 1,
        # k = 8, V = 151936) with a synthetic head of d = 4096: the logits are
        # never written; HBM-bound by the head (V d 2 bytes per call)
        for Bl in (1, 48):
            d = 4096
            gh = torch.Generator(device=dev).manual_seed(77)
            W = (torch.randn((c.V, d), device=dev, generator=gh) / d ** 0.5).to(torch.bfloat16)
            Hd = torch.randn((Bl, 9, d), device=dev, generator=gh).to(torch.bfloat16)
            lt = torch.zeros((Bl, 8), dtype=torch.int32, device=dev)
            lws = torch.zeros(sv.workspace_size(sv.SPEC_OP_GREEDY_LMHEAD, Bl, 8, c.V),
                              dtype=torch.uint8, device=dev)
            la = torch.empty(Bl, dtype=torch.int32, device=dev)
            lo = torch.empty((Bl, 9), dtype=torch.int32, device=dev)

            def fused():
                sv.verify_greedy_lmhead(Hd, W, lt, out=(la, lo), workspace=lws, stream=stream)

            Wt = W.t().contiguous()
            gws = torch.zeros(sv.workspace_size(sv.SPEC_OP_GREEDY, Bl, 8, c.V),
                              dtype=torch.uint8, device=dev)

            def unfused():
                logits = torch.matmul(Hd.reshape(-1, d), Wt).view(Bl, 9, c.V)
                sv.verify_greedy(logits, lt, workspace=gws, stream=stream)

            res = {}
            for name, f in (("fused", fused), ("unfused_bf16_matmul_then_verify", unfused)):
                f()
                torch.cuda.synchronize()
                ev0.record(stream)
                for _ in range(args.steps):
                    f()
                ev1.record(stream)
                torch.cuda.synchronize()
                res[name + "_ms"] = ev0.elapsed_time(ev1) / args.steps
            wbytes = c.V * d * 2 + Bl * 9 * d * 2
            res.update({"B": Bl, "k": 8, "d": d, "V": c.V, "rows": Bl * 9,
                        "head_bytes": wbytes,
                        "fused_GBps": wbytes / (res["fused_ms"] / 1e3) / 1e9,
                        "fused_frac_hbm": wbytes / (res["fused_ms"] / 1e3) / 1e9 / PEAK_HBM_GBPS,
                        "fused_TFLOPs": 2.0 * Bl * 9 * c.V * d / (res["fused_ms"] / 1e3) / 1e12})
            next_rows["lmhead_greedy_B%d" % Bl] = res
            log("fused LM head + greedy (B=%d, k=8, d=%d): %.4f ms (%.0f GB/s of head bytes), "
                "unfused %.4f ms" % (Bl, d, res["fused_ms"], res["fused_GBps"],
                                     res["unfused_bf16_matmul_then_verify_ms"]))
            del W, Wt, Hd
        log("logits_apply over %d rows: %.4f ms = %.0f GB/s; outcome lookup (P=%d): %.1f us"
            % (c.B * (2 * c.k + 1), ms_a, next_rows["logits_apply"]["achieved_GBps"], P,
               next_rows["outcome_lookup"]["us"]))
        del pout, allow, pen

    cpu = None
    if args.cpu_seconds > 0:
        log("cpu baseline: oracle on a bounded sample (~%.0f s of CPU work)" % args.cpu_seconds)
        cpu = cpu_baseline(cfg, args.cpu_seconds, host_threads)
        log("cpu baseline: %.4g positions/s (%s)" % (cpu["value"], cpu["sample"]))

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic of the path: per-element probabilities in fp32 (sums and
        # the ratio test in fp64); the logits themselves are config.logits_dtype
        "dtype": "fp32",
        "data": "synthetic (seeded generators, see workloads/)",
        "config": {"workload": c.name, "B": c.B, "k": c.k, "V": c.V, "logits_dtype": c.dtype,
                   "temperature": c.temperature, "top_k": c.top_k, "top_p": c.top_p,
                   "input_sets": len(sets), "mean_accepted": mean_acc},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "kernel": kernel, "kernel_ms": kernel_ms,
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "whole_call": {"achieved": achieved_call, "frac": achieved_call / PEAK_HBM_GBPS,
                                    "algorithmic_bytes": call_bytes},
                     "row_pass_every_row": {"kernel": row_kernel, "ms": ms_rows,
                                            "bytes": a1_bytes, "achieved": achieved_rows,
                                            "frac": achieved_rows / PEAK_HBM_GBPS}},
        "cpu_baseline": cpu,
    }
    if pooled is not None:
        line["pooled_rows"] = pooled
    if next_rows:
        line["next_rows"] = next_rows
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
