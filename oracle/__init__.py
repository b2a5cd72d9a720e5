"""CPU oracle for the speculative-decoding verify step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library:
``oracle.c`` is a plain single-threaded fp64 implementation of the rule stated
in the encyclopedia entry "Speculative decoding" (glopedia, 推测解码), section
"Basic steps of proposal and verification" (提议与核验的基本步骤), and
``exact.py`` restates the same rule over exact rationals for tiny vocabularies.

Logits are passed as numpy arrays: ``float32`` for fp32 logits, ``uint16``
holding the raw bfloat16 bit patterns for bf16 logits.  Strides are taken from
the arrays themselves, so ``numpy.broadcast_to`` views (stride 0 over the
sequence axis) are accepted.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()

F32, BF16 = 0, 1
NEAR_ACCEPT, NEAR_SAMPLE, NEAR_TOPP = 1, 2, 4


def _compile(src: str, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` with gcc into ``liboracle.so`` (IEEE semantics, no
    FMA contraction, no fast-math)."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h")))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        _compile(_SRC, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_double
    lib.orc_process_row.argtypes = [vp, i32, i32, f64, i32, f64, vp, vp]
    lib.orc_process_row.restype = i32
    lib.orc_sample_row.argtypes = [vp, i32, i32, f64, i32, f64, f64]
    lib.orc_sample_row.restype = i32
    lib.orc_argmax_row.argtypes = [vp, i32, i32]
    lib.orc_argmax_row.restype = i32
    lib.orc_verify_stochastic.argtypes = [vp, i64, i64, vp, i64, i64, i32, vp, vp,
                                          i32, i32, i32, f64, i32, f64, vp, vp, vp, vp]
    lib.orc_verify_stochastic.restype = i32
    lib.orc_verify_greedy.argtypes = [vp, i64, i64, i32, vp, i32, i32, i32, vp, vp]
    lib.orc_verify_greedy.restype = i32
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("logits must be float32 or uint16 (bfloat16 bits), got %s" % a.dtype)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _row(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.ndim != 1:
        raise ValueError("expected one row")
    return a


def _strides(a: np.ndarray):
    if a.ndim != 3:
        raise ValueError("logits must be [B][rows][V]")
    if a.strides[2] != a.itemsize:
        raise ValueError("the vocabulary axis must be contiguous")
    return a.strides[0] // a.itemsize, a.strides[1] // a.itemsize


def _pool_map(m, B: int, rows: int) -> np.ndarray:
    if m is None:
        return np.arange(B * rows, dtype=np.int64).reshape(B, rows)
    m = np.asarray(m, dtype=np.int64)
    if m.shape != (B, rows):
        raise ValueError("row map must be [%d][%d]" % (B, rows))
    return m


def gather_rows(pool: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """The [B][r][V] logits that a row map names in a pool [P][V].  An index
    outside [0, P) gives a row of NaN (an ill-formed row under the rule)."""
    pool = np.asarray(pool)
    if pool.ndim != 2:
        raise ValueError("a row pool is [P][V]")
    P = pool.shape[0]
    ok = (rows >= 0) & (rows < P)
    out = pool[np.where(ok, rows, 0)]
    nan = np.float32(np.nan) if pool.dtype == np.float32 else np.uint16(0x7FC0)
    out[~ok] = nan
    return np.ascontiguousarray(out)


class Oracle:
    """The oracle's entry points bound to one compiled library."""

    # pooled rows -> [B][r][V] logits; an attribute so that tests can plant
    # mistakes in it
    gather = staticmethod(gather_rows)

    def __init__(self, lib):
        self.lib = lib

    @classmethod
    def from_source(cls, src_path: str, lib_path: str) -> "Oracle":
        """Compile another copy of the oracle source (used by tests that plant
        mistakes in a copy, on the CPU, to check that the pins catch them)."""
        _compile(src_path, lib_path)
        return cls(_bind(lib_path))

    def process_row(self, row, temperature=1.0, top_k=0, top_p=1.0):
        """Return (valid, probs[V] float64, stats) for one logits row."""
        row = _row(row)
        V = row.shape[0]
        probs = np.zeros(V, np.float64)
        stats = np.zeros(5, np.float64)
        valid = self.lib.orc_process_row(_ptr(row), _dtype_code(row), V, float(temperature),
                                         int(top_k), float(top_p), _ptr(probs), _ptr(stats))
        return bool(valid), probs, {"max_logit": stats[0], "threshold": stats[1],
                                    "log_norm": stats[2], "mass_above_cut": stats[3],
                                    "mass_at_cut": stats[4]}

    def sample_row(self, row, u, temperature=1.0, top_k=0, top_p=1.0) -> int:
        """Inverse-CDF draw (ascending vocabulary order) from the processed row."""
        row = _row(row)
        return int(self.lib.orc_sample_row(_ptr(row), _dtype_code(row), row.shape[0],
                                           float(temperature), int(top_k), float(top_p),
                                           float(u)))

    def argmax_row(self, row) -> int:
        row = _row(row)
        return int(self.lib.orc_argmax_row(_ptr(row), _dtype_code(row), row.shape[0]))

    def verify_stochastic(self, target, draft, tokens, uniforms, temperature=1.0, top_k=0,
                          top_p=1.0):
        """Stochastic verify of B sequences.  Returns a dict with ``accepted_len``
        [B], ``out_tokens`` [B][k+1], ``accept_prob`` [B][k] and ``flags`` [B]."""
        B, k1, V = target.shape
        k = k1 - 1
        if draft.shape != (B, k, V) or draft.dtype != target.dtype:
            raise ValueError("draft must be [B][k][V] with the target's dtype")
        tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, k)
        uniforms = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, k + 1)
        ts, tp = _strides(target)
        ds, dp = _strides(draft)
        acc = np.zeros(B, np.int32)
        out = np.zeros((B, k + 1), np.int32)
        ap = np.zeros((B, k), np.float64)
        flags = np.zeros(B, np.int32)
        rc = self.lib.orc_verify_stochastic(_ptr(target), ts, tp, _ptr(draft), ds, dp,
                                            _dtype_code(target), _ptr(tokens), _ptr(uniforms),
                                            B, k, V, float(temperature), int(top_k),
                                            float(top_p), _ptr(acc), _ptr(out), _ptr(ap),
                                            _ptr(flags))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
        # the inputs travel with the results, so that a check of a flagged
        # sequence can recompute its rows under either side of a decision
        inputs = {"target": target, "draft": draft, "tokens": tokens, "uniforms": uniforms,
                  "temperature": float(temperature), "top_k": int(top_k), "top_p": float(top_p)}
        return {"accepted_len": acc, "out_tokens": out, "accept_prob": ap, "flags": flags,
                "inputs": inputs}

    def verify_greedy(self, target, tokens):
        """Greedy verify.  Returns (accepted_len [B], out_tokens [B][k+1])."""
        B, k1, V = target.shape
        k = k1 - 1
        tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, k)
        ts, tp = _strides(target)
        acc = np.zeros(B, np.int32)
        out = np.zeros((B, k + 1), np.int32)
        rc = self.lib.orc_verify_greedy(_ptr(target), ts, tp, _dtype_code(target),
                                        _ptr(tokens), B, k, V, _ptr(acc), _ptr(out))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
        return acc, out

    def verify_stochastic_pooled(self, target_pool, target_map, draft_pool, draft_map, tokens,
                                 uniforms, temperature=1.0, top_k=0, top_p=1.0):
        """Stochastic verify over pooled rows: sequence b's target row j is
        target_pool[target_map[b][j]] and its draft row j draft_pool[
        draft_map[b][j]] (a map of None names rows b (k+1) + j and b k + j).
        Each sequence is verified on its own by the same rule; a map entry
        outside its pool stands for an ill-formed row."""
        B, k = np.asarray(tokens).reshape(len(tokens), -1).shape
        tm = _pool_map(target_map, B, k + 1)
        dm = _pool_map(draft_map, B, k)
        return self.verify_stochastic(self.gather(target_pool, tm), self.gather(draft_pool, dm),
                                      tokens, uniforms, temperature, top_k, top_p)

    def verify_greedy_pooled(self, target_pool, target_map, tokens):
        """Greedy verify over a pooled target (as verify_stochastic_pooled)."""
        B, k = np.asarray(tokens).reshape(len(tokens), -1).shape
        return self.verify_greedy(self.gather(target_pool, _pool_map(target_map, B, k + 1)),
                                  tokens)

    def sample_drafts(self, draft, u, temperature=1.0, top_k=0, top_p=1.0, threads=1):
        """Draw one token per draft row ([B][k][V]) from the processed q with the
        uniforms u [B][k] -- the proposer's own sampling, so that drafts meet the
        precondition that they come from the processed q."""
        B, k, V = draft.shape
        u = np.asarray(u, np.float64).reshape(B, k)
        out = np.zeros((B, k), np.int32)

        def work(lo, hi):
            for b in range(lo, hi):
                for j in range(k):
                    out[b, j] = self.sample_row(draft[b, j], u[b, j], temperature, top_k, top_p)

        if threads <= 1 or B == 1:
            work(0, B)
        else:
            step = (B + threads - 1) // threads
            ths = [threading.Thread(target=work, args=(i, min(B, i + step)))
                   for i in range(0, B, step)]
            for t in ths:
                t.start()
            for t in ths:
                t.join()
        return out

    def argmax_drafts(self, draft):
        B, k, V = draft.shape
        return np.array([[self.argmax_row(draft[b, j]) for j in range(k)] for b in range(B)],
                        np.int32)


_default = None


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(_bind(build()))
    return _default


def process_row(row, temperature=1.0, top_k=0, top_p=1.0):
    return default().process_row(row, temperature, top_k, top_p)


def sample_row(row, u, temperature=1.0, top_k=0, top_p=1.0):
    return default().sample_row(row, u, temperature, top_k, top_p)


def argmax_row(row):
    return default().argmax_row(row)


def verify_stochastic(target, draft, tokens, uniforms, temperature=1.0, top_k=0, top_p=1.0):
    return default().verify_stochastic(target, draft, tokens, uniforms, temperature, top_k,
                                       top_p)


def verify_greedy(target, tokens):
    return default().verify_greedy(target, tokens)


def sample_drafts(draft, u, temperature=1.0, top_k=0, top_p=1.0, threads=1):
    return default().sample_drafts(draft, u, temperature, top_k, top_p, threads)


def argmax_drafts(draft):
    return default().argmax_drafts(draft)


def verify_stochastic_pooled(target_pool, target_map, draft_pool, draft_map, tokens, uniforms,
                             temperature=1.0, top_k=0, top_p=1.0):
    return default().verify_stochastic_pooled(target_pool, target_map, draft_pool, draft_map,
                                              tokens, uniforms, temperature, top_k, top_p)


def verify_greedy_pooled(target_pool, target_map, tokens):
    return default().verify_greedy_pooled(target_pool, target_map, tokens)


def outcome_lookup(accepted_len, out_tokens, pred_len, pred_token):
    """Predicted-outcome lookup ("Speculative Speculative Decoding", ai-stack.site
    summary, sections 1 and 2: the proposer prepares drafts for a set of likely
    verification outcomes; the actual outcome either is in the set, a hit, or
    not).  The outcome of sequence b is (n, out_tokens[b][n]) with n =
    accepted_len[b]; returns (hit_index [B], hit count): the first matching
    entry of the sequence's set, or -1 (also for an invalid sequence).  Plain
    loops."""
    acc = [int(x) for x in np.asarray(accepted_len).reshape(-1)]
    out = np.asarray(out_tokens)
    pl = np.asarray(pred_len)
    pt = np.asarray(pred_token)
    k = out.shape[1] - 1
    hits = []
    for b, n in enumerate(acc):
        found = -1
        if 0 <= n <= k:
            t = int(out[b][n])
            for i in range(pl.shape[1]):
                if int(pl[b][i]) == n and int(pt[b][i]) == t:
                    found = i
                    break
        hits.append(found)
    hits = np.array(hits, np.int32)
    return hits, int((hits >= 0).sum())


def _bits(words, V):
    """Token bits of bitmask rows [..][ceil(V/32)] (uint32 words) -> bool [..][V]."""
    w = np.asarray(words).astype(np.uint32)
    x = np.arange(V)
    return ((w[..., x // 32] >> (x % 32).astype(np.uint32)) & 1).astype(bool)


def _bf16_decode(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def _bf16_round(f):
    """float32 -> bfloat16 bits, round to nearest even (NaN -> 0x7FC0)."""
    f = np.asarray(f, np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(f), np.uint16(0x7FC0), r)


def apply_processors(logits, allow=None, penalize=None, theta=1.0, out_dtype=None):
    """Logits processors in the order the verify step's rule requires them to
    be in force (the encyclopedia entry "Speculative decoding", section on
    the basic steps of proposal and verification, names repetition penalty,
    vocabulary masking and structured-output constraints): a token outside
    the allow mask gets -inf; a penalised token gets l / theta if l > 0, else
    l * theta, in float32.  logits: [S][rows][V] float32 or uint16 (bf16
    bits); masks: uint32 words [S][rows][W] (broadcastable).  Returns float32,
    or bf16 bits rounded to nearest even when out_dtype is "bf16"."""
    a = np.asarray(logits)
    V = a.shape[-1]
    f = _bf16_decode(a) if a.dtype == np.uint16 else a.astype(np.float32).copy()
    th = np.float32(theta)
    ok = np.ones(f.shape, bool) if allow is None else np.broadcast_to(_bits(allow, V), f.shape)
    pen = np.zeros(f.shape, bool) if penalize is None else np.broadcast_to(_bits(penalize, V), f.shape)
    out = f.copy()
    with np.errstate(invalid="ignore"):
        pos = f > 0
        out = np.where(pen & pos, (f / th).astype(np.float32), out)
        out = np.where(pen & ~pos, (f * th).astype(np.float32), out)
    out = np.where(ok, out, np.float32(-np.inf)).astype(np.float32)
    if out_dtype == "bf16":
        return _bf16_round(out)
    return out


def lmhead_logits(hidden_bits, weight_bits, rows=None, chunk=16384):
    """fp64 logits hidden @ weight^T of bf16 inputs (exact products, fp64
    sums) for the rows (flat indices into [B][k+1]) asked for, with, per
    logit, the sum of |products| (for rounding bounds).  numpy matmul."""
    H = _bf16_decode(hidden_bits).astype(np.float64)
    H = H.reshape(-1, H.shape[-1])
    if rows is not None:
        H = H[np.asarray(rows)]
    V = weight_bits.shape[0]
    L = np.empty((H.shape[0], V))
    S = np.empty((H.shape[0], V))
    for lo in range(0, V, chunk):
        W = _bf16_decode(weight_bits[lo:lo + chunk]).astype(np.float64)
        L[:, lo:lo + chunk] = H @ W.T
        S[:, lo:lo + chunk] = np.abs(H) @ np.abs(W).T
    return L, S


def lmhead_tie_candidates(L, S, d):
    """Per row of fp64 logits L (with S the sums of |products|, from
    lmhead_logits) the tokens whose logit lies within the fp32 summation
    bound gamma_d (S_top + S_x) of the largest: the argmaxes a kernel that
    accumulates in fp32 may report.  A list of index arrays, one per row."""
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    best = np.argmax(L, axis=1)
    top = L[np.arange(len(L)), best]
    stop = S[np.arange(len(L)), best]
    return [np.nonzero(L[r] >= top[r] - gamma * (stop[r] + S[r]))[0] for r in range(len(L))]


def lmhead_greedy(hidden_bits, weight_bits, tokens, logits=None):
    """Greedy verify on LM-head logits (the encyclopedia entry's greedy rule:
    compare each draft with the target's most probable token, replace the
    first mismatch; lowest index on ties).  Returns (accepted_len [B],
    out_tokens [B][k+1], near_tie [B][k+1]): near_tie marks rows where another
    token's logit lies within the fp32 summation bound gamma_d (|a| + |b|)
    of the largest (gamma_d = d u / (1 - d u), u = 2^-24), so that a kernel
    accumulating in fp32 may report either.  logits: (L, S) of lmhead_logits
    when already computed."""
    B, k1, d = hidden_bits.shape
    k = k1 - 1
    L, S = lmhead_logits(hidden_bits, weight_bits) if logits is None else logits
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    best = np.argmax(L, axis=1)  # first maximum
    top = L[np.arange(len(L)), best]
    stop = S[np.arange(len(L)), best]
    near = (L >= top[:, None] - gamma * (stop[:, None] + S)).sum(axis=1) > 1
    best = best.reshape(B, k1)
    near = near.reshape(B, k1)
    V = weight_bits.shape[0]
    toks = np.asarray(tokens, np.int64).reshape(B, k)
    acc = np.zeros(B, np.int32)
    out = np.full((B, k1), -1, np.int32)
    for b in range(B):
        n, valid = k, True
        for j in range(k):
            x = int(toks[b, j])
            if not 0 <= x < V:
                valid = False
                break
            if x != best[b, j]:
                n = j
                break
        if not valid:
            acc[b] = -1
            continue
        acc[b] = n
        out[b, :n] = toks[b, :n]
        out[b, n] = best[b, n]
    return acc, out, near
