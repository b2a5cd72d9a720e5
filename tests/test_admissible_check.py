"""The checker that GPU parity applies to boundary-flagged sequences, run on
the CPU with the oracle standing in for the GPU: the oracle's own results
pass; results computed under the neighbouring top-p cut (the other side of
a flagged cut) or with a near accept draw decided the other way pass; a
wrong emitted token, a wrong stop, a broken prefix or a wrong alpha fail."""
import numpy as np
import pytest

import oracle
from tests.gpu_common import check_admissible, compare_stochastic
from tests.oracle_pins import cut_masses


def _near_cut_case():
    """Sequences whose every row is one fp32 row with top_p placed 3e-7 above
    a cumulative boundary (the cut is near: flag bit 2), k = 2."""
    rs = np.random.default_rng(5)
    V, k, B = 40, 2, 24
    l = rs.normal(0, 1.5, V).astype(np.float32)
    w = np.exp(l.astype(np.float64) - l.max())
    w /= w.sum()
    vals = np.sort(l.astype(np.float64))[::-1]
    M = np.array([w[l >= v].sum() for v in vals])
    top_p = float(M[6]) + 3e-7
    t = np.ascontiguousarray(np.broadcast_to(l, (B, k + 1, V)))
    d = (t[:, :k] + rs.normal(0, 0.4, (B, k, V))).astype(np.float32)
    toks = oracle.sample_drafts(d, rs.random((B, k)), 1.0, 0, top_p)
    u = rs.random((B, k + 1)).astype(np.float32)
    return t, d, toks, u, top_p, M[6]


def test_oracle_results_pass_and_neighbour_cut_passes():
    t, d, toks, u, top_p, boundary = _near_cut_case()
    ref = oracle.verify_stochastic(t, d, toks, u, 1.0, 0, top_p)
    above, at = cut_masses(t[0, 0], 1.0, 0, top_p)
    assert abs(above - top_p) <= 1e-6  # the mass above the cut is near
    assert (ref["flags"] & 4).all()
    # the oracle's own outputs are admissible
    compare_stochastic(ref, ref["accepted_len"], ref["out_tokens"],
                       ref["accept_prob"].astype(np.float32), label="self", max_flag_frac=1.0)
    # results under the cut one value up (top_p just below the boundary)
    alt = oracle.verify_stochastic(t, d, toks, u, 1.0, 0, float(boundary) - 1e-12)
    assert (alt["out_tokens"] != ref["out_tokens"]).any() or \
        (np.abs(alt["accept_prob"] - ref["accept_prob"]) > 1e-6).any()
    compare_stochastic(ref, alt["accepted_len"], alt["out_tokens"],
                       alt["accept_prob"].astype(np.float32), label="neighbour cut",
                       max_flag_frac=1.0)


def test_wrong_results_fail():
    t, d, toks, u, top_p, _ = _near_cut_case()
    ref = oracle.verify_stochastic(t, d, toks, u, 1.0, 0, top_p)
    inp = ref["inputs"]
    acc, out, ap = ref["accepted_len"], ref["out_tokens"], ref["accept_prob"]
    i = int(np.nonzero(acc == 0)[0][0])  # a sequence rejected at position 0
    # the emitted token moved to a token outside every admissible interval
    bad = out[i].copy()
    V = t.shape[-1]
    _, p, _ = oracle.process_row(t[i, 0], 1.0, 0, top_p)
    bad[0] = int(np.argmin(np.where(p > 0, p, np.inf)))
    if bad[0] == out[i, 0]:
        bad[0] = (out[i, 0] + V // 2) % V
    with pytest.raises(AssertionError):
        check_admissible(inp, i, 0, bad, ap[i], True, "wrong token")
    # a stop moved past a clearly rejecting position
    a0 = ap[i, 0]
    if u[i, 0] - a0 > 1e-3:
        long = np.array(list(toks[i]) + [out[i, 0]], np.int32)
        with pytest.raises(AssertionError):
            check_admissible(inp, i, 2, long, ap[i], True, "wrong stop")
    # the prefix broken
    j = int(np.nonzero(acc >= 1)[0][0])
    brk = out[j].copy()
    brk[0] = (brk[0] + 1) % V
    with pytest.raises(AssertionError):
        check_admissible(inp, j, int(acc[j]), brk, ap[j], True, "prefix")
    # alpha off by 1e-3
    with pytest.raises(AssertionError):
        check_admissible(inp, j, int(acc[j]), out[j], ap[j] + 1e-3, True, "alpha")
    # too many flagged sequences for the bound
    with pytest.raises(AssertionError):
        compare_stochastic(ref, acc, out, ap.astype(np.float32), label="bound", max_flag_frac=0.5)


def test_near_accept_either_way():
    """The worked example with u_0 equal to alpha: accepting (then a bonus
    draw) and rejecting (then the residual's A) are both admissible."""
    import workloads
    t, d, tok = workloads.worked_example()
    a = oracle.verify_stochastic(t, d, tok, np.array([[0.5, 0.5]], np.float32))["accept_prob"][0, 0]
    u = np.array([[a, 0.3]], np.float32)
    ref = oracle.verify_stochastic(t, d, tok, u)
    assert ref["flags"][0] & 1
    inp = ref["inputs"]
    ap = ref["accept_prob"][0]
    check_admissible(inp, 0, 0, np.array([0, -1], np.int32), ap, True, "reject")  # residual: A
    check_admissible(inp, 0, 1, np.array([1, 0], np.int32), ap, True, "accept")   # bonus at 0.3: A
    with pytest.raises(AssertionError):
        check_admissible(inp, 0, 0, np.array([1, -1], np.int32), ap, True, "residual B")
    with pytest.raises(AssertionError):
        check_admissible(inp, 0, 1, np.array([1, 2], np.int32), ap, True, "bonus C")
