"""Parity of the pooled-row calls: sequences naming shared target and draft
rows through int32 maps (the branches of one request sharing its target rows,
the root-to-leaf paths of a candidate tree sharing its nodes' rows).  The
GPU results must equal the oracle's on the rows the maps name -- on the
whole-sequence walk (bf16, large batches; target statistics from a pass over
the target pool) and on the row-pass path (fp32, small batches) -- and equal
the dense call on the same rows materialised per sequence."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import draft_token_verification_11_amd as sv
import oracle
import workloads
from tests.gpu_common import DEV, compare_stochastic, note, to_dev

pytestmark = pytest.mark.gpu


def _cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def _walk_batch() -> int:
    return 2 * _cus() + 37


def _t(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def _gpu_pooled(tp, tm, dp, dm, toks, u, T, top_k, top_p, alpha=True, workspace=None):
    r = sv.verify_stochastic_pooled(
        to_dev(tp), to_dev(dp), _t(toks), torch.from_numpy(np.asarray(u, np.float32)).to(DEV),
        target_map=_t(tm), draft_map=_t(dm), temperature=T, top_k=top_k, top_p=top_p,
        return_accept_prob=alpha, workspace=workspace)
    torch.cuda.synchronize()
    return tuple(x.cpu().numpy() for x in r)


def _check(tp, tm, dp, dm, toks, u, T, top_k, top_p, label):
    fp32 = tp.dtype == np.float32
    ref = oracle.verify_stochastic_pooled(tp, tm, dp, dm, toks, u, T, top_k, top_p)
    acc, out, ap = _gpu_pooled(tp, tm, dp, dm, toks, u, T, top_k, top_p)
    # pooled rows are shared: a target row whose top-p cut lies near top_p
    # flags every branch (up to 16) that reads it, so flags come in groups
    compare_stochastic(ref, acc, out, ap, fp32=fp32, label=label, max_flag_frac=0.4)
    acc2, out2 = _gpu_pooled(tp, tm, dp, dm, toks, u, T, top_k, top_p, alpha=False)
    assert np.array_equal(acc, acc2) and np.array_equal(out, out2), label
    return ref, acc, out, ap


def _logits(x: np.ndarray, dtype: str) -> np.ndarray:
    return workloads.to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)


def _fanout(rs, nreq, branches, k, V, dtype, T, top_k, top_p, drop=3):
    """nreq requests x branches, the last request `drop` branches short;
    target rows per request, draft rows per branch (request's rows + noise)."""
    B = nreq * branches - drop
    base = rs.normal(0, 2.0, (nreq, k + 1, V)).astype(np.float32)
    req = np.arange(B) // branches
    drafts = base[req, :k] + rs.normal(0, 0.7, (B, k, V)).astype(np.float32)
    tp = _logits(base.reshape(-1, V), dtype)
    dp = _logits(drafts.reshape(-1, V), dtype)
    tm = req[:, None] * (k + 1) + np.arange(k + 1)[None, :]
    toks = oracle.sample_drafts(dp.reshape(B, k, V), rs.random((B, k)), T, top_k, top_p, threads=8)
    u = rs.random((B, k + 1)).astype(np.float32)
    return tp, tm, dp, toks, u


@pytest.mark.parametrize("path", ["walk", "row_pass"])
def test_branch_fanout(path):
    rs = np.random.default_rng(71 if path == "walk" else 72)
    k = 4
    if path == "walk":
        nreq, V, dtype = (_walk_batch() + 15) // 16 + 1, 1000, "bf16"
    else:
        nreq, V, dtype = 5, 777, "f32"
    for T, top_k, top_p in [(1.0, 0, 0.95), (0.8, 0, 1.0), (1.0, 50, 0.9)]:
        tp, tm, dp, toks, u = _fanout(rs, nreq, 16, k, V, dtype, T, top_k, top_p)
        ref, *_ = _check(tp, tm, dp, None, toks, u, T, top_k, top_p,
                         "fan-out %s %d x 16 V=%d T=%g top_k=%d top_p=%g"
                         % (path, nreq, V, T, top_k, top_p))
        note("  accepted-length histogram %s" % np.bincount(ref["accepted_len"][ref["accepted_len"] >= 0],
                                                           minlength=k + 1))


def _tree(rs, branching, V, dtype, T, top_k, top_p):
    """A candidate tree with the given fan-out per level; node rows of the
    target N(0, 2^2), of the proposer target + N(0, 0.7^2); each child's token
    drawn from its parent's processed proposer row."""
    parents = [-1]
    level = [0]
    for f in branching:
        nxt = []
        for p in level:
            for _ in range(f):
                parents.append(p)
                nxt.append(len(parents) - 1)
        level = nxt
    N = len(parents)
    t = rs.normal(0, 2.0, (N, V)).astype(np.float32)
    d = t + rs.normal(0, 0.7, (N, V)).astype(np.float32)
    tp, dp = _logits(t, dtype), _logits(d, dtype)
    tokens = [0] + [oracle.sample_row(dp[parents[i]], rs.random(), T, top_k, top_p)
                    for i in range(1, N)]
    toks, tm, dm = sv.tree_branches(parents, tokens)
    B, k = toks.shape
    u = rs.random((B, k + 1)).astype(np.float32)
    return tp, tm.numpy(), dp, dm.numpy(), toks.numpy(), u


@pytest.mark.parametrize("path", ["walk", "row_pass"])
def test_tree_paths(path):
    rs = np.random.default_rng(73 if path == "walk" else 74)
    if path == "walk":
        branching, V, dtype = [(_walk_batch() + 63) // 64, 8, 8], 1024, "bf16"
    else:
        branching, V, dtype = [3, 3, 2], 513, "f32"
    for T, top_k, top_p in [(1.0, 0, 1.0), (0.7, 20, 0.9)]:
        tp, tm, dp, dm, toks, u = _tree(rs, branching, V, dtype, T, top_k, top_p)
        _check(tp, tm, dp, dm, toks, u, T, top_k, top_p,
               "tree %s %s (%d nodes, %d paths) T=%g top_k=%d top_p=%g"
               % (path, branching, len(tp), len(toks), T, top_k, top_p))


@pytest.mark.parametrize("path", ["walk", "row_pass"])
def test_bad_map_entries(path):
    """Out-of-range map entries count only at the positions the walk
    consults: before the first rejection, or the bonus row after k passes."""
    rs = np.random.default_rng(75)
    k = 3
    if path == "walk":
        B, V, dtype = _walk_batch(), 512, "bf16"
    else:
        B, V, dtype = 40, 300, "f32"
    t = rs.normal(0, 2.0, (B * (k + 1), V)).astype(np.float32)
    d = rs.normal(0, 2.0, (B * k, V)).astype(np.float32)
    tm = np.arange(B * (k + 1)).reshape(B, k + 1)
    dm = np.arange(B * k).reshape(B, k)
    toks = rs.integers(0, V, (B, k)).astype(np.int32)
    u = rs.random((B, k + 1)).astype(np.float32)
    nt, nd = len(t), len(d)
    # sequences 0-2 accept every position (u = 0, tokens the target's argmax
    # with a draft that supports them); 3-5 reject at position 0 (p(x) = 0)
    for b in range(6):
        for j in range(k):
            x = int(np.argmax(t[tm[b, j]]))
            toks[b, j] = x
            d[dm[b, j], x] = t[tm[b, j], x]
        u[b, :k] = 0.0
    for b in (3, 4, 5):
        t[tm[b, 0], toks[b, 0]] = -np.inf
    tm[0, 1] = -1        # consulted: invalid
    dm[1, 2] = nd        # consulted: invalid
    tm[2, k] = nt + 5    # bonus row, consulted: invalid
    tm[3, 2] = -1        # past the stop: ignored
    tm[4, k] = -1        # bonus row not consulted: ignored
    dm[5, 1] = -7        # past the stop: ignored
    for b in rs.choice(np.arange(6, B), size=min(20, B - 6), replace=False):
        if rs.random() < 0.5:
            tm[b, rs.integers(0, k + 1)] = rs.choice([-3, nt, 1 << 30])
        else:
            dm[b, rs.integers(0, k)] = rs.choice([-1, nd, nd + 1000])
    tp, dp = _logits(t, dtype), _logits(d, dtype)
    ref, acc, out, ap = _check(tp, tm, dp, dm, toks, u, 1.0, 0, 1.0, "bad map entries " + path)
    assert list(acc[:6]) == [-1, -1, -1, 0, 0, 0], acc[:6]


@pytest.mark.parametrize("path", ["walk", "row_pass"])
def test_pooled_equals_dense(path):
    """The pooled call and the dense call on the same rows materialised per
    sequence take identical decisions and draws, bit for bit."""
    rs = np.random.default_rng(76)
    k = 4
    if path == "walk":
        nreq, V, dtype = (_walk_batch() + 15) // 16 + 1, 2048, "bf16"
    else:
        nreq, V, dtype = 4, 1000, "f32"
    T, top_k, top_p = 1.0, 0, 0.95
    tp, tm, dp, toks, u = _fanout(rs, nreq, 16, k, V, dtype, T, top_k, top_p)
    B = len(toks)
    acc, out, ap = _gpu_pooled(tp, tm, dp, None, toks, u, T, top_k, top_p)
    tgt = tp[tm]                      # [B][k+1][V]
    drf = dp.reshape(B, k, V)
    r = sv.verify_stochastic(to_dev(tgt), to_dev(drf), _t(toks),
                             torch.from_numpy(u).to(DEV), temperature=T, top_k=top_k,
                             top_p=top_p, return_accept_prob=True)
    torch.cuda.synchronize()
    acc_d, out_d, ap_d = (x.cpu().numpy() for x in r)
    assert np.array_equal(acc, acc_d) and np.array_equal(out, out_d)
    assert np.array_equal(ap, ap_d, equal_nan=True)


def test_greedy_pooled():
    rs = np.random.default_rng(77)
    for dtype, branching, V in [("bf16", [6, 5, 4], 4096), ("f32", [3, 2, 2, 2], 777)]:
        parents = [-1]
        level = [0]
        for f in branching:
            nxt = []
            for p in level:
                for _ in range(f):
                    parents.append(p)
                    nxt.append(len(parents) - 1)
            level = nxt
        N = len(parents)
        t = rs.normal(0, 3.0, (N, V)).astype(np.float32)
        t[np.arange(N), rs.integers(0, V, N)] += 8.0
        tp = _logits(t, dtype)
        best = np.array([oracle.argmax_row(tp[i]) for i in range(N)])
        # tokens: the parent's argmax most of the time, so paths run deep
        tokens = [0] + [int(best[parents[i]]) if rs.random() < 0.8 else int(rs.integers(0, V))
                        for i in range(1, N)]
        toks, tm, _ = sv.tree_branches(parents, tokens)
        toks, tm = toks.numpy(), tm.numpy()
        B = len(toks)
        tm[rs.choice(B, size=4, replace=False), rs.integers(0, tm.shape[1], 4)] = -1
        racc, rout = oracle.verify_greedy_pooled(tp, tm, toks)
        acc, out = sv.verify_greedy_pooled(to_dev(tp), _t(toks), target_map=_t(tm))
        torch.cuda.synchronize()
        acc, out = acc.cpu().numpy(), out.cpu().numpy()
        assert np.array_equal(acc, racc) and np.array_equal(out, rout), dtype
        note("greedy pooled %s %d paths: accepted-length histogram %s, %d invalid"
             % (dtype, B, np.bincount(racc[racc >= 0], minlength=tm.shape[1]),
                int((racc < 0).sum())))


@pytest.mark.parametrize("path", ["walk", "row_pass"])
def test_pooled_workspace_left_zero(path):
    rs = np.random.default_rng(78)
    k = 4
    if path == "walk":
        nreq, V, dtype = (_walk_batch() + 15) // 16 + 1, 1000, "bf16"
    else:
        nreq, V, dtype = 3, 600, "f32"
    for T, top_k, top_p in [(1.0, 0, 0.95), (1.0, 0, 1.0)]:
        tp, tm, dp, toks, u = _fanout(rs, nreq, 16, k, V, dtype, T, top_k, top_p)
        B = len(toks)
        need = sv.workspace_size_pooled(sv.SPEC_OP_STOCHASTIC, len(tp), len(dp), B, k, V, T,
                                        top_k, top_p)
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        r1 = _gpu_pooled(tp, tm, dp, None, toks, u, T, top_k, top_p, workspace=ws)
        assert int(ws.count_nonzero()) == 0
        r2 = _gpu_pooled(tp, tm, dp, None, toks, u, T, top_k, top_p, workspace=ws)
        assert int(ws.count_nonzero()) == 0
        for a, b in zip(r1, r2):
            assert np.array_equal(a, b, equal_nan=True)
    need = sv.workspace_size_pooled(sv.SPEC_OP_GREEDY, len(tp), 0, B, k, V)
    wsg = torch.zeros(need, dtype=torch.uint8, device=DEV)
    sv.verify_greedy_pooled(to_dev(tp), _t(toks), target_map=_t(tm), workspace=wsg)
    torch.cuda.synchronize()
    assert int(wsg.count_nonzero()) == 0


def test_config5_pooled_full_size():
    """The branch fan-out workload (32 requests x 16 branches, k = 4,
    V = 151936, bf16, top-p 0.95) with each request's target rows held once:
    160 target rows instead of 2,560.  Every sequence equals the dense call
    on the materialised rows and is checked against the oracle."""
    from tests.test_gpu_parity import full_size_case
    w, toks, ref = full_size_case(5)
    c = w.config
    k1 = c.k + 1
    tp = np.ascontiguousarray(w.target[::c.branches].reshape(-1, c.V))
    tm = (np.arange(c.B) // c.branches)[:, None] * k1 + np.arange(k1)[None, :]
    dp = w.draft.reshape(-1, c.V)
    acc, out, ap = _gpu_pooled(tp, tm, dp, None, toks, w.uniforms, c.temperature, c.top_k, c.top_p)
    note("c5 pooled: gpu done (%d target rows)" % len(tp))
    r = sv.verify_stochastic(to_dev(w.target), to_dev(w.draft), _t(toks),
                             torch.from_numpy(w.uniforms).to(DEV), temperature=c.temperature,
                             top_k=c.top_k, top_p=c.top_p, return_accept_prob=True)
    torch.cuda.synchronize()
    acc_d, out_d, ap_d = (x.cpu().numpy() for x in r)
    assert np.array_equal(acc, acc_d) and np.array_equal(out, out_d)
    assert np.array_equal(ap, ap_d, equal_nan=True)
    compare_stochastic(ref, acc, out, ap, fp32=False, label="c5 pooled (B=512), all checked")


def test_pooled_walk_max_k():
    """k = 64 (the maximum) on the pooled walk: 64 draft steps per sequence,
    target statistics for 65 rows per sequence from the pool pass."""
    rs = np.random.default_rng(79)
    k, V = 64, 64
    nreq = (_walk_batch() + 3) // 4 + 1
    tp, tm, dp, toks, u = _fanout(rs, nreq, 4, k, V, "bf16", 1.0, 0, 0.9, drop=1)
    ref, *_ = _check(tp, tm, dp, None, toks, u, 1.0, 0, 0.9, "pooled walk k=64")
    note("  deepest accepted length %d" % ref["accepted_len"].max())


def test_pooled_unaligned_rows():
    """Pools whose rows are not 16-byte aligned (V = 777 at stride 777, bf16
    and fp32): the scalar-load row pass."""
    rs = np.random.default_rng(80)
    for dtype in ("bf16", "f32"):
        tp, tm, dp, toks, u = _fanout(rs, 3, 8, 3, 777, dtype, 1.0, 0, 0.95)
        _check(tp, tm, dp, None, toks, u, 1.0, 0, 0.95, "pooled unaligned %s" % dtype)


def test_pooled_walk_single_request():
    """One request, every branch sharing its five target rows (a pool of 5
    rows: the pre-pass has fewer rows than XCD ranges), enough branches for
    the walk."""
    rs = np.random.default_rng(81)
    k, V = 4, 2000
    nb = _walk_batch() + 20
    tp, tm, dp, toks, u = _fanout(rs, 1, nb, k, V, "bf16", 1.0, 0, 0.95, drop=0)
    assert len(tp) == k + 1
    _check(tp, tm, dp, None, toks, u, 1.0, 0, 0.95, "pooled walk, one request x %d branches" % nb)
