"""The fp64 oracle against its pins (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
from tests import oracle_pins as pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def _random_dist(rs, V, zero_prob=0.2):
    w = [Fraction(int(rs.integers(0, 7))) if rs.random() < zero_prob else
         Fraction(int(rs.integers(1, 9))) for _ in range(V)]
    if sum(w) == 0:
        w[0] = Fraction(1)
    s = sum(w)
    return [x / s for x in w]


def test_exact_law_preserves_target():
    """Exact rationals: for tiny vocabularies and k <= 3, the token at every
    position, given any prefix, follows that position's target law, and the
    acceptance probability is sum min(p, q)."""
    rs = np.random.default_rng(1)
    for trial in range(25):
        V = int(rs.integers(2, 5))
        k = int(rs.integers(1, 4))
        ps = [_random_dist(rs, V) for _ in range(k + 1)]
        qs = [_random_dist(rs, V) for _ in range(k)]
        law = exact.output_law(ps, qs)
        assert sum(law.values()) == 1
        for j in range(k + 1):
            for prefix, cond in exact.conditional_laws(law, j, V).items():
                assert cond == ps[j], (trial, j, prefix)
        # acceptance at position 0 = sum min(p, q)
        acc0 = sum(pr for seq, pr in law.items() if len(seq) > 1)
        assert acc0 == sum(min(a, b) for a, b in zip(ps[0], qs[0]))
        assert exact.acceptance_rate(ps[0], qs[0]) == acc0


def test_exact_law_rejects_wrong_rules():
    """The exact law distinguishes the rule from plausible wrong ones (sanity
    of the exact module itself)."""
    p = [Fraction(6, 10), Fraction(3, 10), Fraction(1, 10)]
    q = [Fraction(5, 10), Fraction(4, 10), Fraction(1, 10)]
    law = exact.output_law([p, p], [q])
    assert exact.position_marginal(law, 0, 3) == p
    # Resampling from p instead of the residual does not preserve the law.
    wrong = [sum(qx * exact.alpha(px, qx) * (1 if t == x else 0) +
                 qx * (1 - exact.alpha(px, qx)) * p[t] for x, (px, qx) in enumerate(zip(p, q)))
             for t in range(3)]
    assert wrong != p


def test_oracle_matches_exact_law_numerically(orc):
    """Oracle probabilities fed into the exact module give the oracle's own
    accept probabilities (alpha) within rounding."""
    rs = np.random.default_rng(21)
    for _ in range(10):
        V = 4
        t = rs.normal(0, 1, (1, 2, V)).astype(np.float32)
        d = (t[:, :1] + rs.normal(0, 1, (1, 1, V))).astype(np.float32)
        _, p, _ = orc.process_row(t[0, 0])
        _, q, _ = orc.process_row(d[0, 0])
        for x in range(V):
            r = orc.verify_stochastic(t, d, np.array([[x]]), np.array([[0.5, 0.5]], np.float32))
            a = exact.alpha(Fraction(p[x]), Fraction(q[x]))
            assert abs(float(a) - r["accept_prob"][0, 0]) < 1e-15
