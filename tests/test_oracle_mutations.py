"""Plant plausible mistakes in copies of the oracle source (on the CPU) and
check that the pins catch every one of them.  The real oracle is untouched;
each mutant is compiled into a temporary library of its own."""
import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "ratio inverted (q/p)": ("double a = p / q;", "double a = q / p;", 1),
    "residual sign flipped (q - p)": ("double d = pn[i] - qn[i];", "double d = qn[i] - pn[i];", 1),
    "residual not clipped at zero": ("r[i] = d > 0.0 ? d : 0.0;", "r[i] = d;", 1),
    "resample from p instead of the residual": ("if (S == 0.0)\n        for", "if (1)\n        for", 1),
    "no stop at first rejection": ("alpha[j])) {\n        n = j;\n        break;",
                                   "alpha[j])) {\n        n = j;", 1),
    "non-strict accept (u <= alpha)": ("!((double)ub[j] < alpha[j])", "!((double)ub[j] <= alpha[j])", 1),
    "bonus from the last drafted row": ("} else {\n      for (int i = 0; i < V; i++) r[i] = pn[i];",
                                        "} else {\n      for (int i = 0; i < V; i++) r[i] = P[(size_t)(k - 1) * V + i];", 1),
    "temperature multiplies": ("(l[i] - m) / T", "(l[i] - m) * T", None),
    "top-k off by one": ("t_k = scratch[top_k - 1];", "t_k = scratch[top_k];", 1),
    "top-p not renormalised after top-k": ("cum += exp((scratch[j] - m) / T) / z_k;",
                                           "cum += exp((scratch[j] - m) / T) / (z_k * 1.5);", 1),
    "inverse CDF uses >=": ("if (run > target) {", "if (run >= target) {", 1),
    "greedy keeps the last maximum": ("l[i] > l[best]", "l[i] >= l[best]", 1),
    "bf16 decoded with the wrong shift": ("((uint32_t)half) << 16", "((uint32_t)half) << 15", 1),
    "max logit ignored in the exponent": ("if (l[i] >= thr) z += exp((l[i] - m) / T);",
                                          "if (l[i] >= thr) z += exp((l[i] - m + 0.25) / T);", 1),
    "q = 0 rejects a token p supports": ("return p > 0.0 ? 1.0 : 0.0;", "return 0.0;", 1),
    "bonus row consulted after a rejection": ("if (valid && n == k && !pres[k].valid) valid = 0;",
                                              "if (!pres[k].valid) valid = 0;", 1),
    "ill-formed position past the stop invalidates": ("if (isnan(alpha[j])) {\n        valid = 0;\n        break;\n      }\n      if (!((double)ub[j] < alpha[j])) {\n        n = j;\n        break;\n      }",
                                                      "if (isnan(alpha[j])) {\n        valid = 0;\n        break;\n      }\n      if (!((double)ub[j] < alpha[j]) && n == k) {\n        n = j;\n      }", 1),
    "top-p boundary flag never set": ("f |= ORC_NEAR_TOPP;", "(void)0;", 2),
    "top-p boundary flag always set": ("flags[b] = f;", "flags[b] = f | (top_p < 1.0 ? ORC_NEAR_TOPP : 0);", 1),
    "mass above the cut counts its ties": ("if (scratch[j] > t_p) above += pi;",
                                           "if (scratch[j] >= t_p) above += pi;", 1),
    "boundary distance 1e-3 instead of 1e-6": ("return fabs(a - b) <= 1e-6;",
                                               "return fabs(a - b) <= 1e-3;", 1),
}

FAST_PINS = [p for p in pins.ALL_PINS if p is not pins.pin_chi_square]


def _mutant(tmp_path, name, old, new, count):
    src = open(SRC).read()
    assert old in src, name
    if count is not None:
        assert src.count(old) == count, (name, src.count(old))
    mutated = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    return oracle.Oracle.from_source(str(path), str(tmp_path / "libmutant.so"))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(tmp_path, name):
    old, new, count = MUTATIONS[name]
    orc = _mutant(tmp_path, name, old, new, count)
    caught = []
    for pin in FAST_PINS + [lambda o: pins.pin_chi_square(o, n=200_000)]:
        try:
            pin(orc)
        except AssertionError:
            caught.append(getattr(pin, "__name__", "chi_square"))
        except Exception as e:  # a crash or a NaN path also counts as caught
            caught.append("%s raised %s" % (getattr(pin, "__name__", "?"), type(e).__name__))
    assert caught, "no pin caught the planted mistake: %s" % name


# Mistakes planted in the pooled-row gather (Python), one subclass each.
def _gather_ignoring_map(pool, rows):
    flat = np.arange(rows.size).reshape(rows.shape) % len(pool)
    return oracle.gather_rows(pool, flat)


def _gather_clamping(pool, rows):
    return oracle.gather_rows(pool, np.clip(rows, 0, len(pool) - 1))


def _gather_off_by_one(pool, rows):
    return oracle.gather_rows(pool, np.where(rows > 0, rows - 1, rows))


class _TargetMapForDrafts(oracle.Oracle):
    def verify_stochastic_pooled(self, tp, tm, dp, dm, toks, u, *args):
        k = np.asarray(toks).shape[1]
        return super().verify_stochastic_pooled(tp, tm, dp, np.asarray(tm)[:, :k], toks, u, *args)


POOL_MUTATIONS = {
    "pool map ignored": lambda lib: type("M", (oracle.Oracle,), {"gather": staticmethod(_gather_ignoring_map)})(lib),
    "out-of-range map entry clamped": lambda lib: type("M", (oracle.Oracle,), {"gather": staticmethod(_gather_clamping)})(lib),
    "map entries off by one": lambda lib: type("M", (oracle.Oracle,), {"gather": staticmethod(_gather_off_by_one)})(lib),
    "target map used for the drafts": lambda lib: _TargetMapForDrafts(lib),
}


@pytest.mark.parametrize("name", sorted(POOL_MUTATIONS))
def test_pins_catch_pool_mutation(name):
    orc = POOL_MUTATIONS[name](oracle.default().lib)
    with pytest.raises(AssertionError):
        pins.pin_pooled_rows(orc)


# Mistakes planted in the predicted-outcome lookup.
def _lookup_last(acc, out, pl, pt):
    acc, out, pl, pt = (np.asarray(x) for x in (acc, out, pl, pt))
    hits = []
    for b, n in enumerate(acc.reshape(-1)):
        m = [i for i in range(pl.shape[1]) if 0 <= n < out.shape[1] and pl[b][i] == n and pt[b][i] == out[b][n]]
        hits.append(m[-1] if m else -1)
    hits = np.array(hits)
    return hits, int((hits >= 0).sum())


def _lookup_token_ignored(acc, out, pl, pt):
    acc, pl = np.asarray(acc).reshape(-1), np.asarray(pl)
    hits = np.array([next((i for i in range(pl.shape[1]) if n >= 0 and pl[b][i] == n), -1)
                     for b, n in enumerate(acc)])
    return hits, int((hits >= 0).sum())


def _lookup_empty_matches(acc, out, pl, pt):
    acc, out, pl, pt = (np.asarray(x) for x in (acc, out, pl, pt))
    hits = []
    for b, n in enumerate(acc.reshape(-1)):
        t = out[b][n] if 0 <= n < out.shape[1] else None
        hits.append(next((i for i in range(pl.shape[1]) if t is not None and (pl[b][i] == n or pl[b][i] < 0) and pt[b][i] == t), -1))
    hits = np.array(hits)
    return hits, int((hits >= 0).sum())


@pytest.mark.parametrize("mutant", [_lookup_last, _lookup_token_ignored, _lookup_empty_matches],
                         ids=lambda f: f.__name__)
def test_pins_catch_lookup_mutation(mutant):
    with pytest.raises(AssertionError):
        pins.pin_outcome_lookup(oracle.default(), lookup=mutant)


# Mistakes planted in the logits processors.
def _apply_penalty_sign_blind(logits, allow=None, penalize=None, theta=1.0, out_dtype=None):
    out = oracle.apply_processors(logits, allow, None, 1.0)
    if penalize is not None:
        pen = np.broadcast_to(oracle._bits(penalize, out.shape[-1]), out.shape)
        out = np.where(pen & np.isfinite(out), (out / np.float32(theta)).astype(np.float32), out)
    return oracle._bf16_round(out) if out_dtype == "bf16" else out


def _apply_mask_inverted(logits, allow=None, penalize=None, theta=1.0, out_dtype=None):
    inv = None if allow is None else ~np.asarray(allow, np.uint32)
    return oracle.apply_processors(logits, inv, penalize, theta, out_dtype)


def _apply_truncating_bf16(logits, allow=None, penalize=None, theta=1.0, out_dtype=None):
    out = oracle.apply_processors(logits, allow, penalize, theta)
    if out_dtype == "bf16":
        return (out.view(np.uint32) >> 16).astype(np.uint16)
    return out


@pytest.mark.parametrize("mutant", [_apply_penalty_sign_blind, _apply_mask_inverted,
                                    _apply_truncating_bf16], ids=lambda f: f.__name__)
def test_pins_catch_processor_mutation(mutant):
    with pytest.raises(AssertionError):
        pins.pin_logits_processors(oracle.default(), apply=mutant)


# Mistakes planted in the LM-head greedy oracle.
def _lm_last_max(hidden, weight, tokens):
    import oracle as o
    L, S = o.lmhead_logits(hidden, weight)
    V = L.shape[1]
    best = V - 1 - np.argmax(L[:, ::-1], axis=1)  # last maximum
    B, k1, _ = hidden.shape
    acc, out, near = o.lmhead_greedy(hidden, weight, tokens)
    best = best.reshape(B, k1)
    toks = np.asarray(tokens).reshape(B, k1 - 1)
    for b in range(B):
        if acc[b] < 0:
            continue
        n = next((j for j in range(k1 - 1) if toks[b, j] != best[b, j]), k1 - 1)
        acc[b] = n
        out[b] = -1
        out[b, :n] = toks[b, :n]
        out[b, n] = best[b, n]
    return acc, out, near


def _lm_no_bound(hidden, weight, tokens):
    acc, out, near = oracle.lmhead_greedy(hidden, weight, tokens)
    return acc, out, np.zeros_like(near)


@pytest.mark.parametrize("mutant", [_lm_last_max, _lm_no_bound], ids=lambda f: f.__name__)
def test_pins_catch_lmhead_mutation(mutant):
    with pytest.raises(AssertionError):
        pins.pin_lmhead_greedy(oracle.default(), greedy=mutant)
