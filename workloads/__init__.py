"""Seeded synthetic inputs for the speculative-decoding verify step.

This module only draws random numbers and lays them out; it holds none of the
verify step's arithmetic (no softmax, no filtering, no accept test, no
sampling).  Both the GPU path's tests/benchmark and the CPU oracle consume the
arrays it returns, bit for bit.

Every array is drawn from ``numpy.random.default_rng([1000 + cfg, stream, i])``
where ``i`` is the sequence index (for the branch-fanout workload the target's
base draws use the request index), so any subset of sequences can be
regenerated on its own.  Streams:

  0  target logits noise      1  boost index (peaked workload)
  2  draft logits noise       3  proposer's sampling uniforms [k]
  4  verify uniforms [k+1]

Logits are generated in float32; bf16 workloads round them to bfloat16 with
round-to-nearest-even and return the raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import math
import threading
from dataclasses import dataclass, field

import numpy as np

STREAM_TARGET, STREAM_BOOST, STREAM_DRAFT, STREAM_DRAFT_U, STREAM_U = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Config:
    cfg: int
    name: str
    mode: str          # "stochastic", "greedy+stochastic"
    B: int
    k: int
    V: int
    dtype: str         # "f32" or "bf16"
    temperature: float
    top_k: int
    top_p: float
    branches: int = 1  # sequences per request sharing one target (fan-out workload)
    recipe: str = field(default="", compare=False)


CONFIGS = {
    1: Config(1, "stochastic B=1 k=4 V=1024 fp32", "stochastic", 1, 4, 1024, "f32",
              1.0, 0, 1.0,
              recipe="target ~ N(0, 2^2) iid; draft = target + N(0, 0.5^2); T=1, no filters"),
    2: Config(2, "greedy+stochastic B=1 k=8 V=151936 bf16 T=0.7", "greedy+stochastic", 1, 8,
              151936, "bf16", 0.7, 0, 1.0,
              recipe="target ~ N(0, 3^2) with +8 at one uniformly drawn index per row; "
                     "draft = target + N(0, 1); T=0.7"),
    3: Config(3, "stochastic B=64 k=5 V=151936 bf16 top-k 50 top-p 0.9", "stochastic", 64, 5,
              151936, "bf16", 1.0, 50, 0.9,
              recipe="target ~ N(0, 2.5^2); draft = 0.8 target + N(0, 1); T=1, top-k 50 "
                     "then top-p 0.9 on both sides"),
    4: Config(4, "stochastic B=256 k=8 V=262144 fp32 T=0.8", "stochastic", 256, 8, 262144,
              "f32", 0.8, 0, 1.0,
              recipe="target ~ N(0, 2^2) + Zipf-ranked bias -1.1 ln(v+1); "
                     "draft = target + N(0, 1.5^2); T=0.8, no filters"),
    5: Config(5, "branch-fanout 32x16 k=4 V=151936 bf16 top-p 0.95", "stochastic", 512, 4,
              151936, "bf16", 1.0, 0, 0.95, branches=16,
              recipe="per request a base ~ N(0, 2^2) of [k+1][V] shared by its 16 branches as "
                     "their target; each branch's draft = base[:k] + N(0, 0.7^2); T=1, top-p 0.95"),
}


def rng(cfg: int, stream: int, index: int) -> np.random.Generator:
    return np.random.default_rng([1000 + cfg, stream, index])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((bits >> 16) & 1) + np.uint32(0x7FFF)
    return ((bits + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(dst: np.ndarray, src: np.ndarray, dtype: str) -> None:
    if dtype == "bf16":
        dst[...] = to_bf16_bits(src)
    else:
        dst[...] = src


def _zipf_bias(V: int) -> np.ndarray:
    # Zipf(s=1.1)-ranked additive bias with rank = token id: -1.1 * ln(v + 1).
    return (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)


def _target_f32(c: Config, i: int) -> np.ndarray:
    k1, V = c.k + 1, c.V
    if c.cfg == 1:
        return (2.0 * rng(1, STREAM_TARGET, i).standard_normal((k1, V), np.float32))
    if c.cfg == 2:
        t = 3.0 * rng(2, STREAM_TARGET, i).standard_normal((k1, V), np.float32)
        idx = rng(2, STREAM_BOOST, i).integers(0, V, size=k1)
        t[np.arange(k1), idx] += np.float32(8.0)
        return t
    if c.cfg == 3:
        return 2.5 * rng(3, STREAM_TARGET, i).standard_normal((k1, V), np.float32)
    if c.cfg == 4:
        t = 2.0 * rng(4, STREAM_TARGET, i).standard_normal((k1, V), np.float32)
        return t + _zipf_bias(V)[None, :]
    if c.cfg == 5:
        request = i // c.branches
        return 2.0 * rng(5, STREAM_TARGET, request).standard_normal((k1, V), np.float32)
    raise ValueError(c.cfg)


def _draft_f32(c: Config, i: int, target: np.ndarray) -> np.ndarray:
    k, V = c.k, c.V
    noise = rng(c.cfg, STREAM_DRAFT, i).standard_normal((k, V), np.float32)
    sigma = {1: 0.5, 2: 1.0, 3: 1.0, 4: 1.5, 5: 0.7}[c.cfg]
    scale = 0.8 if c.cfg == 3 else 1.0
    return scale * target[:k] + np.float32(sigma) * noise


@dataclass
class Workload:
    config: Config
    seqs: np.ndarray        # indices of the generated sequences
    target: np.ndarray      # [n][k+1][V] float32 or uint16 (bf16 bits)
    draft: np.ndarray       # [n][k][V]
    uniforms: np.ndarray    # [n][k+1] float32 in [0,1): verify draws
    draft_u: np.ndarray     # [n][k] float64 in [0,1): proposer's sampling draws


def generate(cfg: int, seqs=None, threads: int = 8, B: int | None = None) -> Workload:
    """Generate the inputs of workload ``cfg`` for the given sequence indices
    (default: all B sequences; ``B`` overrides the batch size)."""
    c = CONFIGS[cfg]
    if B is not None:
        c = Config(**{**c.__dict__, "B": B})
    seqs = np.arange(c.B) if seqs is None else np.asarray(seqs, np.int64)
    n = len(seqs)
    npdt = np.uint16 if c.dtype == "bf16" else np.float32
    target = np.empty((n, c.k + 1, c.V), npdt)
    draft = np.empty((n, c.k, c.V), npdt)
    uniforms = np.empty((n, c.k + 1), np.float32)
    draft_u = np.empty((n, c.k), np.float64)

    def work(lo, hi):
        for a in range(lo, hi):
            i = int(seqs[a])
            t = _target_f32(c, i)
            _store(target[a], t, c.dtype)
            _store(draft[a], _draft_f32(c, i, t), c.dtype)
            uniforms[a] = rng(c.cfg, STREAM_U, i).random(c.k + 1, np.float32)
            draft_u[a] = rng(c.cfg, STREAM_DRAFT_U, i).random(c.k)

    threads = max(1, min(threads, n))
    step = int(math.ceil(n / threads))
    ths = [threading.Thread(target=work, args=(lo, min(n, lo + step)))
           for lo in range(0, n, step)]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    return Workload(c, seqs, target, draft, uniforms, draft_u)


def worked_example():
    """The three-token example of the encyclopedia entry "Speculative decoding"
    (glopedia), section "Basic steps of proposal and verification": target
    (A, B, C) = (0.6, 0.3, 0.1), proposal (0.5, 0.4, 0.1), drafted token B.
    Returned as fp32 logits ln(prob) for B=1, k=1, V=3: target rows 0 and 1
    (bonus) both hold the target distribution."""
    p = np.log(np.array([0.6, 0.3, 0.1], np.float64)).astype(np.float32)
    q = np.log(np.array([0.5, 0.4, 0.1], np.float64)).astype(np.float32)
    target = np.stack([p, p])[None]          # [1][2][3]
    draft = q[None, None, :].copy()          # [1][1][3]
    tokens = np.array([[1]], np.int32)       # B
    return target, draft, tokens


def lmhead(B: int, k: int, d: int, V: int, seed: int = 7, boost: float = 0.3,
           stream_base: int = 20):
    """Synthetic LM-head inputs (bf16 bits): weight W [V][d] ~ N(0, 1/d) and
    hidden [B][k+1][d] ~ N(0, 1) plus, per row, boost * sqrt(d) * W[v*] for a
    uniformly drawn token v* (peaked rows, as the greedy workload's +8 boost).
    Returns (hidden_bits, weight_bits, boosted token ids [B][k+1])."""
    rw = np.random.default_rng([9000 + seed, stream_base])
    w = (rw.standard_normal((V, d), np.float32) / np.float32(np.sqrt(d))).astype(np.float32)
    rh = np.random.default_rng([9000 + seed, stream_base + 1])
    h = rh.standard_normal((B, k + 1, d), np.float32)
    vs = rh.integers(0, V, size=(B, k + 1))
    if boost:
        h += np.float32(boost * np.sqrt(d)) * w[vs]
    return to_bf16_bits(h), to_bf16_bits(w), vs.astype(np.int32)
