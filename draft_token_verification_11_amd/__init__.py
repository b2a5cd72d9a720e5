"""libspecverify: the speculative-decoding verify step on one MI355X (gfx950).

This package is a thin binding over the C ABI declared in
``include/specverify.h``: it marshals torch tensors (device memory, strides,
the current HIP stream) into the C calls; every step of the verify runs in the
library's HIP kernels.  The raw C functions are reachable as
``lib().spec_verify_stochastic`` etc.; the wrappers below keep the same names
without the ``spec_`` prefix.

The rule (encyclopedia entry "Speculative decoding", glopedia, section "Basic
steps of proposal and verification"): accept each draft with probability
min(1, p/q), stop at the first rejection, redraw that position from the
normalised residual max(0, p - q), or draw a bonus token from the target when
every draft passes; greedy mode compares argmaxes.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["lib", "verify_stochastic", "verify_greedy", "logits_process", "workspace_size",
           "verify_stochastic_pooled", "verify_greedy_pooled", "workspace_size_pooled",
           "tree_branches", "outcome_lookup", "logits_apply", "verify_greedy_lmhead",
           "status_string", "SpecError", "verify_stochastic_path", "device_cu_count",
           "verify_stochastic_noalloc", "NOALLOC_SCRATCH_BYTES",
           "library_path"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SPEC_OK, SPEC_ERR_INVALID_ARG, SPEC_ERR_UNSUPPORTED, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP = range(5)
SPEC_DTYPE_F32, SPEC_DTYPE_BF16 = 0, 1
SPEC_OP_STOCHASTIC, SPEC_OP_GREEDY, SPEC_OP_PROCESS, SPEC_OP_GREEDY_LMHEAD = 0, 1, 2, 3
SPEC_PATH_ROW_PASS, SPEC_PATH_TASK_QUEUE, SPEC_PATH_SEQUENCE_WALK = 0, 1, 2
PATH_NAMES = {SPEC_PATH_ROW_PASS: "row pass", SPEC_PATH_TASK_QUEUE: "task queue",
              SPEC_PATH_SEQUENCE_WALK: "sequence walk"}


class spec_logits_t(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("seq_stride", ctypes.c_int64),
                ("pos_stride", ctypes.c_int64)]


class spec_sampling_t(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_float)]


class spec_processors_t(ctypes.Structure):
    _fields_ = [("allow", ctypes.c_void_p), ("allow_seq_stride", ctypes.c_int64),
                ("allow_pos_stride", ctypes.c_int64), ("penalize", ctypes.c_void_p),
                ("pen_seq_stride", ctypes.c_int64), ("pen_pos_stride", ctypes.c_int64),
                ("theta", ctypes.c_float)]


class SpecError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s" % (where, status_string(status)))
        self.status = status


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libspecverify.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    "libspecverify.so is missing at %s; build it with "
                    "`python -c 'import __graft_entry__ as g; g.build()'`" % _LIB_PATH)
            L = ctypes.CDLL(_LIB_PATH)
            vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
            P = ctypes.POINTER
            L.spec_workspace_size.argtypes = [i32, i32, i32, i32, P(spec_sampling_t)]
            L.spec_workspace_size.restype = sz
            L.spec_verify_stochastic.argtypes = [spec_logits_t, spec_logits_t, vp, vp, i32, i32,
                                                 i32, P(spec_sampling_t), vp, vp, vp, vp, sz, vp]
            L.spec_verify_stochastic.restype = ctypes.c_int
            L.spec_verify_stochastic_noalloc.argtypes = [spec_logits_t, spec_logits_t, vp, vp, i32,
                                                         i32, i32, P(spec_sampling_t), vp, vp, vp,
                                                         vp]
            L.spec_verify_stochastic_noalloc.restype = ctypes.c_int
            L.spec_verify_greedy.argtypes = [spec_logits_t, vp, i32, i32, i32, vp, vp, vp, sz, vp]
            L.spec_verify_greedy.restype = ctypes.c_int
            L.spec_logits_process.argtypes = [spec_logits_t, i32, i32, P(spec_sampling_t), vp, vp,
                                              vp, sz, vp]
            L.spec_logits_process.restype = ctypes.c_int
            L.spec_workspace_size_pooled.argtypes = [i32, i32, i32, i32, i32, i32,
                                                     P(spec_sampling_t)]
            L.spec_workspace_size_pooled.restype = sz
            L.spec_verify_stochastic_pooled.argtypes = [spec_logits_t, i32, vp, spec_logits_t, i32,
                                                        vp, vp, vp, i32, i32, i32,
                                                        P(spec_sampling_t), vp, vp, vp, vp, sz, vp]
            L.spec_verify_stochastic_pooled.restype = ctypes.c_int
            L.spec_verify_greedy_pooled.argtypes = [spec_logits_t, i32, vp, vp, i32, i32, i32, vp,
                                                    vp, vp, sz, vp]
            L.spec_verify_greedy_pooled.restype = ctypes.c_int
            i64 = ctypes.c_int64
            L.spec_verify_greedy_lmhead.argtypes = [vp, i64, i64, vp, i64, i32, vp, i32, i32, i32,
                                                    vp, vp, vp, sz, vp]
            L.spec_verify_greedy_lmhead.restype = ctypes.c_int
            L.spec_logits_apply.argtypes = [spec_logits_t, i32, i32, i32, P(spec_processors_t),
                                            spec_logits_t, vp]
            L.spec_logits_apply.restype = ctypes.c_int
            L.spec_outcome_lookup.argtypes = [vp, vp, i32, i32, vp, vp, i32, vp, vp, vp]
            L.spec_outcome_lookup.restype = ctypes.c_int
            L.spec_verify_stochastic_path.argtypes = [spec_logits_t, spec_logits_t, i32, i32, i32,
                                                      P(spec_sampling_t), i32, vp]
            L.spec_verify_stochastic_path.restype = ctypes.c_int
            L.spec_device_cu_count.argtypes = [vp]
            L.spec_device_cu_count.restype = ctypes.c_int
            L.spec_status_string.argtypes = [ctypes.c_int]
            L.spec_status_string.restype = ctypes.c_char_p
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().spec_status_string(int(status)).decode()


def _sampling(temperature: float, top_k: int, top_p: float) -> spec_sampling_t:
    return spec_sampling_t(float(temperature), int(top_k), float(top_p))


def workspace_size(op: int, B: int, k: int, V: int, temperature: float = 1.0, top_k: int = 0,
                   top_p: float = 1.0) -> int:
    s = _sampling(temperature, top_k, top_p)
    return int(lib().spec_workspace_size(int(op), int(B), int(k), int(V), ctypes.byref(s)))


# One zero-filled workspace per (device, stream), grown on demand.  The
# library leaves a workspace zero-filled after every call, so calls ordered on
# one stream can share it; calls on different streams get different buffers
# (the kernels' queue words must not be shared by calls that may overlap).  A
# buffer is zero-filled on the stream that uses it, and a grown buffer
# replaces the old one only on that stream, after the calls queued there.
_ws = {}


def _workspace(device: torch.device, nbytes: int, stream) -> torch.Tensor:
    dev = device.index if device.index is not None else torch.cuda.current_device()
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    key = (dev, st.cuda_stream)
    with _lock:
        buf = _ws.get(key)
        if buf is None or buf.numel() < nbytes:
            with torch.cuda.stream(st):
                buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            _ws[key] = buf
    return buf


def _out_tensor(t, shape, dtype, dev, what):
    """A caller's output tensor: on the logits' device, of the right dtype
    and shape, contiguous; anything else raises before any launch."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % what)
    if t.device != dev:
        raise ValueError("%s must live on %s, got %s" % (what, dev, t.device))
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s, got %s %s"
                         % (what, dtype, tuple(shape), t.dtype, tuple(t.shape)))
    return t


def _outputs(out, B, k, dev, with_ap):
    """(accepted_len, out_tokens[, accept_prob]) allocated, or the caller's
    checked."""
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
        ap = torch.empty((B, k), dtype=torch.float32, device=dev) if with_ap else None
        return acc, toks, ap
    acc = _out_tensor(out[0], (B,), torch.int32, dev, "accepted_len")
    toks = _out_tensor(out[1], (B, k + 1), torch.int32, dev, "out_tokens")
    ap = out[2] if len(out) > 2 else None
    if with_ap and ap is None:
        raise ValueError("return_accept_prob needs an accept_prob tensor in out")
    if ap is not None:
        ap = _out_tensor(ap, (B, k), torch.float32, dev, "accept_prob")
    return acc, toks, ap


def _workspace_arg(workspace, dev, need, stream):
    """The caller's workspace (checked: a contiguous byte tensor on the
    call's device holding at least `need` bytes), or the default one of the
    call's (device, stream)."""
    if workspace is None:
        return _workspace(dev, need, stream)
    if not isinstance(workspace, torch.Tensor) or workspace.device != dev or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % dev)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace holds %d bytes, the call needs %d"
                         % (workspace.numel() * workspace.element_size(), need))
    return workspace


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SPEC_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SPEC_DTYPE_BF16
    raise TypeError("logits must be float32 or bfloat16, got %s" % t.dtype)


def _logits(t: torch.Tensor, rows: int) -> spec_logits_t:
    if t.dim() != 3 or t.shape[1] != rows:
        raise ValueError("expected logits of shape [B][%d][V], got %s" % (rows, tuple(t.shape)))
    if not t.is_cuda:
        raise ValueError("logits must live in device memory")
    if t.stride(2) != 1:
        raise ValueError("the vocabulary axis must be contiguous")
    return spec_logits_t(t.data_ptr(), _dtype_code(t), 0, t.stride(0), t.stride(1))


def _stream(stream, dev=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream


def _check(rc: int, where: str) -> None:
    if rc != SPEC_OK:
        raise SpecError(rc, where)


def verify_stochastic(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                      uniforms: torch.Tensor, *, temperature: float = 1.0, top_k: int = 0,
                      top_p: float = 1.0, return_accept_prob: bool = False, out=None,
                      workspace: torch.Tensor | None = None, stream=None):
    """Stochastic verify.  target [B][k+1][V], draft [B][k][V] (same dtype,
    fp32 or bf16), draft_tokens [B][k] int32, uniforms [B][k+1] float32.
    Returns (accepted_len [B], out_tokens [B][k+1]) and, on request,
    accept_prob [B][k]."""
    B, k = draft_tokens.shape
    V = target.shape[2]
    tgt, drf = _logits(target, k + 1), _logits(draft, k)
    if draft.shape[0] != B or target.shape[0] != B or draft.shape[2] != V:
        raise ValueError("target, draft and draft_tokens disagree on B or V")
    dev = target.device
    if draft.device != dev:
        raise ValueError("target and draft must live on one device")
    tokens = draft_tokens.to(device=dev, dtype=torch.int32).contiguous()
    u = uniforms.to(device=dev, dtype=torch.float32).contiguous()
    if tuple(u.shape) != (B, k + 1):
        raise ValueError("uniforms must be [B][k+1]")
    acc, toks, ap = _outputs(out, B, k, dev, return_accept_prob)
    s = _sampling(temperature, top_k, top_p)
    need = lib().spec_workspace_size(SPEC_OP_STOCHASTIC, B, k, V, ctypes.byref(s))
    if need == 0:
        _check(SPEC_ERR_INVALID_ARG, "spec_workspace_size")
    ws = _workspace_arg(workspace, dev, need, stream)
    rc = lib().spec_verify_stochastic(tgt, drf, tokens.data_ptr(), u.data_ptr(), B, k, V,
                                      ctypes.byref(s), acc.data_ptr(), toks.data_ptr(),
                                      ap.data_ptr() if ap is not None else None,
                                      ws.data_ptr(), ws.numel() * ws.element_size(),
                                      _stream(stream, dev))
    _check(rc, "spec_verify_stochastic")
    return (acc, toks, ap) if return_accept_prob else (acc, toks)


NOALLOC_SCRATCH_BYTES = 16 << 20


def verify_stochastic_noalloc(target: torch.Tensor, draft: torch.Tensor,
                              draft_tokens: torch.Tensor, uniforms: torch.Tensor, *, out,
                              temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
                              stream=None):
    """verify_stochastic through spec_verify_stochastic_noalloc: no workspace,
    the library's per-GPU scratch array instead (calls that may overlap on
    one GPU race).  Every tensor must already be on the logits' device in
    its final dtype and layout -- draft_tokens int32 [B][k], uniforms
    float32 [B][k+1], out = (accepted_len, out_tokens[, accept_prob]) -- so
    that the call allocates nothing, here or in the library."""
    B, k = draft_tokens.shape
    V = target.shape[2]
    tgt, drf = _logits(target, k + 1), _logits(draft, k)
    dev = target.device
    if draft.device != dev or target.shape[0] != B or draft.shape[0] != B or draft.shape[2] != V:
        raise ValueError("target, draft and draft_tokens disagree on device, B or V")
    tokens = _out_tensor(draft_tokens, (B, k), torch.int32, dev, "draft_tokens")
    u = _out_tensor(uniforms, (B, k + 1), torch.float32, dev, "uniforms")
    acc, toks, ap = _outputs(out, B, k, dev, len(out) > 2 and out[2] is not None)
    s = _sampling(temperature, top_k, top_p)
    rc = lib().spec_verify_stochastic_noalloc(tgt, drf, tokens.data_ptr(), u.data_ptr(), B, k, V,
                                              ctypes.byref(s), acc.data_ptr(), toks.data_ptr(),
                                              ap.data_ptr() if ap is not None else None,
                                              _stream(stream, dev))
    _check(rc, "spec_verify_stochastic_noalloc")
    return (acc, toks, ap) if ap is not None else (acc, toks)


def verify_stochastic_path(target: torch.Tensor, draft: torch.Tensor, k: int | None = None, *,
                           temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
                           return_accept_prob: bool = False, stream=None) -> int:
    """The kernel path (SPEC_PATH_*) verify_stochastic takes for these logits
    and settings; nothing is launched."""
    k = draft.shape[1] if k is None else k
    tgt, drf = _logits(target, k + 1), _logits(draft, k)
    s = _sampling(temperature, top_k, top_p)
    rc = lib().spec_verify_stochastic_path(tgt, drf, target.shape[0], k, target.shape[2],
                                           ctypes.byref(s), int(bool(return_accept_prob)),
                                           _stream(stream, target.device))
    if rc < 0:
        _check(-rc, "spec_verify_stochastic_path")
    return rc


def device_cu_count(stream=None) -> int:
    """The compute-unit count the library sizes its grids by (cached once per
    device); the stream's device, or the current one."""
    return int(lib().spec_device_cu_count(stream.cuda_stream if stream is not None else None))


def verify_greedy(target: torch.Tensor, draft_tokens: torch.Tensor, *, out=None,
                  workspace: torch.Tensor | None = None, stream=None):
    """Greedy verify.  target [B][k+1][V], draft_tokens [B][k] int32.
    Returns (accepted_len [B], out_tokens [B][k+1])."""
    B, k = draft_tokens.shape
    V = target.shape[2]
    tgt = _logits(target, k + 1)
    if target.shape[0] != B:
        raise ValueError("target and draft_tokens disagree on B")
    dev = target.device
    tokens = draft_tokens.to(device=dev, dtype=torch.int32).contiguous()
    acc, toks, _ = _outputs(out, B, k, dev, False)
    need = lib().spec_workspace_size(SPEC_OP_GREEDY, B, k, V, None)
    if need == 0:
        _check(SPEC_ERR_INVALID_ARG, "spec_workspace_size")
    ws = _workspace_arg(workspace, dev, need, stream)
    rc = lib().spec_verify_greedy(tgt, tokens.data_ptr(), B, k, V, acc.data_ptr(), toks.data_ptr(),
                                  ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream, dev))
    _check(rc, "spec_verify_greedy")
    return acc, toks


def logits_process(logits: torch.Tensor, *, temperature: float = 1.0, top_k: int = 0,
                   top_p: float = 1.0, return_probs: bool = True,
                   workspace: torch.Tensor | None = None, stream=None):
    """Processes the rows of ``logits`` ([R][V] or [B][rows][V] with a
    contiguous vocabulary axis and uniformly strided rows).  Returns a dict
    with per-row ``max_logit``, ``threshold``, ``log_norm``, ``valid`` and,
    if requested, the dense fp32 ``probs`` [R][V]."""
    if logits.dim() == 3:
        if logits.stride(0) != logits.shape[1] * logits.stride(1):
            raise ValueError("rows must be uniformly strided")
        logits2 = logits.reshape(-1, logits.shape[2]) if logits.is_contiguous() else None
        if logits2 is None:
            raise ValueError("rows must be uniformly strided")
        logits = logits2
    if logits.dim() != 2 or logits.stride(1) != 1 or not logits.is_cuda:
        raise ValueError("logits must be a device tensor [R][V] with a contiguous last axis")
    R, V = logits.shape
    desc = spec_logits_t(logits.data_ptr(), _dtype_code(logits), 0, 0, logits.stride(0))
    s = _sampling(temperature, top_k, top_p)
    dev = logits.device
    stats = torch.empty((R, 4), dtype=torch.float32, device=dev)
    probs = torch.empty((R, V), dtype=torch.float32, device=dev) if return_probs else None
    need = lib().spec_workspace_size(SPEC_OP_PROCESS, R, 0, V, ctypes.byref(s))
    if need == 0:
        _check(SPEC_ERR_INVALID_ARG, "spec_workspace_size")
    ws = _workspace_arg(workspace, dev, need, stream)
    rc = lib().spec_logits_process(desc, R, V, ctypes.byref(s), stats.data_ptr(),
                                   probs.data_ptr() if probs is not None else None,
                                   ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream, dev))
    _check(rc, "spec_logits_process")
    out = {"max_logit": stats[:, 0], "threshold": stats[:, 1], "log_norm": stats[:, 2],
           "valid": stats[:, 3].view(torch.int32)}
    if probs is not None:
        out["probs"] = probs
    return out


# ---------------------------------------------------------------------------
# Pooled rows: sequences (the branches of one request, the root-to-leaf paths
# of a candidate tree) that share target or draft rows name them in a row pool
# through int32 maps; each shared row is stored and processed once.


def workspace_size_pooled(op: int, n_target_rows: int, n_draft_rows: int, B: int, k: int, V: int,
                          temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0) -> int:
    s = _sampling(temperature, top_k, top_p)
    return int(lib().spec_workspace_size_pooled(int(op), int(n_target_rows), int(n_draft_rows),
                                                int(B), int(k), int(V), ctypes.byref(s)))


def _pool(t: torch.Tensor) -> spec_logits_t:
    if t.dim() != 2 or not t.is_cuda or t.stride(1) != 1:
        raise ValueError("a row pool must be a device tensor [P][V] with a contiguous last axis")
    return spec_logits_t(t.data_ptr(), _dtype_code(t), 0, 0, t.stride(0))


def _row_map(m, shape, dev):
    if m is None:
        return None
    m = m.to(device=dev, dtype=torch.int32).contiguous()
    if tuple(m.shape) != shape:
        raise ValueError("row map must be %s, got %s" % (shape, tuple(m.shape)))
    return m


def verify_stochastic_pooled(target_pool: torch.Tensor, draft_pool: torch.Tensor,
                             draft_tokens: torch.Tensor, uniforms: torch.Tensor, *,
                             target_map: torch.Tensor | None = None,
                             draft_map: torch.Tensor | None = None, temperature: float = 1.0,
                             top_k: int = 0, top_p: float = 1.0,
                             return_accept_prob: bool = False, out=None,
                             workspace: torch.Tensor | None = None, stream=None):
    """Stochastic verify over pooled rows.  target_pool [Pt][V] and
    draft_pool [Pd][V] (same dtype); target_map [B][k+1] and draft_map [B][k]
    int32 name each sequence's rows in the pools (None: row b (k+1) + j, row
    b k + j).  A map entry outside its pool makes that row ill-formed.
    Otherwise as verify_stochastic."""
    B, k = draft_tokens.shape
    Pt, V = target_pool.shape
    Pd = draft_pool.shape[0]
    if draft_pool.shape[1] != V:
        raise ValueError("target and draft pools disagree on V")
    tgt, drf = _pool(target_pool), _pool(draft_pool)
    dev = target_pool.device
    tmap = _row_map(target_map, (B, k + 1), dev)
    dmap = _row_map(draft_map, (B, k), dev)
    tokens = draft_tokens.to(device=dev, dtype=torch.int32).contiguous()
    u = uniforms.to(device=dev, dtype=torch.float32).contiguous()
    if tuple(u.shape) != (B, k + 1):
        raise ValueError("uniforms must be [B][k+1]")
    if draft_pool.device != dev:
        raise ValueError("target and draft pools must live on one device")
    acc, toks, ap = _outputs(out, B, k, dev, return_accept_prob)
    s = _sampling(temperature, top_k, top_p)
    need = lib().spec_workspace_size_pooled(SPEC_OP_STOCHASTIC, Pt, Pd, B, k, V, ctypes.byref(s))
    if need == 0:
        _check(SPEC_ERR_INVALID_ARG, "spec_workspace_size_pooled")
    ws = _workspace_arg(workspace, dev, need, stream)
    rc = lib().spec_verify_stochastic_pooled(
        tgt, Pt, tmap.data_ptr() if tmap is not None else None, drf, Pd,
        dmap.data_ptr() if dmap is not None else None, tokens.data_ptr(), u.data_ptr(), B, k, V,
        ctypes.byref(s), acc.data_ptr(), toks.data_ptr(), ap.data_ptr() if ap is not None else None,
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream, dev))
    _check(rc, "spec_verify_stochastic_pooled")
    return (acc, toks, ap) if return_accept_prob else (acc, toks)


def verify_greedy_pooled(target_pool: torch.Tensor, draft_tokens: torch.Tensor, *,
                         target_map: torch.Tensor | None = None, out=None,
                         workspace: torch.Tensor | None = None, stream=None):
    """Greedy verify over a pooled target [Pt][V] with target_map [B][k+1]
    (None: row b (k+1) + j).  Returns (accepted_len [B], out_tokens [B][k+1])."""
    B, k = draft_tokens.shape
    Pt, V = target_pool.shape
    tgt = _pool(target_pool)
    dev = target_pool.device
    tmap = _row_map(target_map, (B, k + 1), dev)
    tokens = draft_tokens.to(device=dev, dtype=torch.int32).contiguous()
    acc, toks, _ = _outputs(out, B, k, dev, False)
    need = lib().spec_workspace_size_pooled(SPEC_OP_GREEDY, Pt, 0, B, k, V, None)
    if need == 0:
        _check(SPEC_ERR_INVALID_ARG, "spec_workspace_size_pooled")
    ws = _workspace_arg(workspace, dev, need, stream)
    rc = lib().spec_verify_greedy_pooled(tgt, Pt, tmap.data_ptr() if tmap is not None else None,
                                         tokens.data_ptr(), B, k, V, acc.data_ptr(),
                                         toks.data_ptr(), ws.data_ptr(),
                                         ws.numel() * ws.element_size(), _stream(stream, dev))
    _check(rc, "spec_verify_greedy_pooled")
    return acc, toks


def tree_branches(parents, tokens, leaves=None):
    """Branches of a parent-pointer candidate tree, for the pooled calls.

    Node 0 is the root (the last token already accepted); node i > 0 holds
    the drafted token ``tokens[i]`` and its parent ``parents[i] < i``.  Row i
    of the target pool (of the draft pool) holds the target's (the
    proposer's) logits for the token after the path root..i.  Every leaf (by
    default, every node without children) must lie at the same depth k >= 1.

    Returns (draft_tokens [B][k], target_map [B][k+1], draft_map [B][k]) as
    int32 CPU tensors, one row per leaf: the path root = n_0, n_1, .., n_k =
    leaf gives draft token j = tokens[n_{j+1}], target row j = n_j (row k the
    bonus row) and draft row j = n_j."""
    par = [int(x) for x in (parents.tolist() if hasattr(parents, "tolist") else parents)]
    tok = [int(x) for x in (tokens.tolist() if hasattr(tokens, "tolist") else tokens)]
    N = len(par)
    if N < 2 or len(tok) != N or par[0] != -1:
        raise ValueError("a tree needs a root (parent -1) and at least one child")
    for i in range(1, N):
        if not 0 <= par[i] < i:
            raise ValueError("node %d: parent must precede it" % i)
    if leaves is None:
        has_child = [False] * N
        for i in range(1, N):
            has_child[par[i]] = True
        leaves = [i for i in range(1, N) if not has_child[i]]
    paths = []
    for leaf in leaves:
        leaf = int(leaf)
        if not 0 < leaf < N:
            raise ValueError("leaf %d is not a node below the root" % leaf)
        path = [leaf]
        while path[-1] != 0:
            path.append(par[path[-1]])
        paths.append(path[::-1])
    k = len(paths[0]) - 1
    if any(len(p) - 1 != k for p in paths):
        raise ValueError("every leaf must lie at the same depth")
    node_map = torch.tensor(paths, dtype=torch.int32)
    draft_tokens = torch.tensor([[tok[n] for n in p[1:]] for p in paths], dtype=torch.int32)
    return draft_tokens, node_map, node_map[:, :k].contiguous()


def outcome_lookup(accepted_len: torch.Tensor, out_tokens: torch.Tensor, pred_len: torch.Tensor,
                   pred_token: torch.Tensor, *, return_count: bool = True, stream=None):
    """Predicted-outcome lookup after a verify call: for each sequence the
    index of the first entry of its predicted set ([B][P] lengths and tokens,
    a length < 0 is an empty entry) equal to its outcome (n, out_tokens[n]),
    or -1.  Returns hit_index [B] and, on request, the hit count [1]."""
    B = accepted_len.shape[0]
    k = out_tokens.shape[1] - 1
    P = pred_len.shape[1]
    if not accepted_len.is_cuda:
        raise ValueError("accepted_len must live in device memory")
    dev = accepted_len.device
    acc = accepted_len.to(torch.int32).contiguous()
    out = out_tokens.to(device=dev, dtype=torch.int32).contiguous()
    pl = pred_len.to(device=dev, dtype=torch.int32).contiguous()
    pt = pred_token.to(device=dev, dtype=torch.int32).contiguous()
    if tuple(out.shape) != (B, k + 1) or tuple(pl.shape) != (B, P) or tuple(pt.shape) != (B, P):
        raise ValueError("expected accepted_len [B], out_tokens [B][k+1], predicted sets [B][P]")
    hit = torch.empty(B, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev) if return_count else None
    rc = lib().spec_outcome_lookup(acc.data_ptr(), out.data_ptr(), B, k, pl.data_ptr(),
                                   pt.data_ptr(), P, hit.data_ptr(),
                                   cnt.data_ptr() if cnt is not None else None, _stream(stream, dev))
    _check(rc, "spec_outcome_lookup")
    return (hit, cnt) if return_count else hit


def _mask_rows(m, S, rows, W, dev):
    """(pointer, seq stride, pos stride) of bitmask rows [S|1][rows|1][W] (int32 words)."""
    if m is None:
        return None, 0, 0, None
    if m.dim() != 3 or m.shape[2] != W or m.dtype != torch.int32 or m.stride(2) != 1:
        raise ValueError("bitmask rows must be int32 [S|1][rows|1][%d] with contiguous words" % W)
    if m.device != dev:
        raise ValueError("bitmask rows must live on the logits' device")
    if m.shape[0] not in (1, S) or m.shape[1] not in (1, rows):
        raise ValueError("bitmask rows do not broadcast to [%d][%d]" % (S, rows))
    ss = m.stride(0) if m.shape[0] == S and S > 1 else 0
    ps = m.stride(1) if m.shape[1] == rows and rows > 1 else 0
    return m.data_ptr(), ss, ps, m


def logits_apply(logits: torch.Tensor, *, allow: torch.Tensor | None = None,
                 penalize: torch.Tensor | None = None, theta: float = 1.0,
                 out: torch.Tensor | None = None, out_dtype: torch.dtype | None = None,
                 stream=None) -> torch.Tensor:
    """Logits processors on [S][rows][V] logits: tokens outside the allow
    mask get -inf, penalised tokens l / theta (l > 0) or l * theta.  Masks
    are int32 words [S|1][rows|1][ceil(V/32)] (bit x % 32 of word x / 32).
    Writes `out` (default: a new tensor of out_dtype, default the input's;
    `out=logits` works in place) and returns it."""
    if logits.dim() != 3 or not logits.is_cuda or logits.stride(2) != 1:
        raise ValueError("logits must be a device tensor [S][rows][V] with a contiguous last axis")
    S, rows, V = logits.shape
    W = (V + 31) // 32
    dev = logits.device
    if out is None:
        out = torch.empty((S, rows, V), dtype=out_dtype or logits.dtype, device=dev)
    if tuple(out.shape) != (S, rows, V) or out.stride(2) != 1:
        raise ValueError("out must be [S][rows][V] with a contiguous last axis")
    ap, a_s, a_p, _a = _mask_rows(allow, S, rows, W, dev)
    pp, p_s, p_p, _p = _mask_rows(penalize, S, rows, W, dev)
    proc = spec_processors_t(ap, a_s, a_p, pp, p_s, p_p, float(theta))
    src = spec_logits_t(logits.data_ptr(), _dtype_code(logits), 0, logits.stride(0), logits.stride(1))
    dst = spec_logits_t(out.data_ptr(), _dtype_code(out), 0, out.stride(0), out.stride(1))
    rc = lib().spec_logits_apply(src, S, rows, V, ctypes.byref(proc), dst, _stream(stream, dev))
    _check(rc, "spec_logits_apply")
    return out


def verify_greedy_lmhead(hidden: torch.Tensor, weight: torch.Tensor, draft_tokens: torch.Tensor,
                         *, out=None, workspace: torch.Tensor | None = None, stream=None):
    """Fused LM head + greedy verify: hidden [B][k+1][d] and weight [V][d]
    (bf16, last axis contiguous, rows 16-byte aligned); the logits hidden @
    weight^T are reduced to per-row argmaxes on the matrix cores and never
    stored.  Returns (accepted_len [B], out_tokens [B][k+1])."""
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if hidden.dim() != 3 or weight.dim() != 2 or hidden.stride(2) != 1 or weight.stride(1) != 1:
        raise ValueError("expected hidden [B][k+1][d] and weight [V][d] with contiguous last axes")
    B, k = draft_tokens.shape
    V, d = weight.shape
    if tuple(hidden.shape) != (B, k + 1, d):
        raise ValueError("hidden must be [B][k+1][d] with the weight's d")
    dev = hidden.device
    tokens = draft_tokens.to(device=dev, dtype=torch.int32).contiguous()
    if weight.device != dev:
        raise ValueError("hidden and weight must live on one device")
    acc, toks, _ = _outputs(out, B, k, dev, False)
    need = lib().spec_workspace_size(SPEC_OP_GREEDY_LMHEAD, B, k, V, None)
    if need == 0:
        _check(SPEC_ERR_INVALID_ARG, "spec_workspace_size")
    ws = _workspace_arg(workspace, dev, need, stream)
    rc = lib().spec_verify_greedy_lmhead(hidden.data_ptr(), hidden.stride(0), hidden.stride(1),
                                         weight.data_ptr(), weight.stride(0), d, tokens.data_ptr(),
                                         B, k, V, acc.data_ptr(), toks.data_ptr(), ws.data_ptr(),
                                         ws.numel() * ws.element_size(), _stream(stream, dev))
    _check(rc, "spec_verify_greedy_lmhead")
    return acc, toks
