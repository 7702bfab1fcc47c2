"""Pins for oracle.model against the figures printed in "LLM Primer VI —
Chapitre 9 — Décodage spéculatif" §9.1 and §9.3 (tests/golden/primer_ch9_claims.json).

The page prints ranges, not a worked example, so the pins check that the
closed forms reproduce them for α in the page's own typical range, and that
they reproduce them only with the bonus token counted (the reading taken).
"""
import json
import os

import numpy as np
import pytest

from oracle import model

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "primer_ch9_claims.json")))


def test_expected_tokens_closed_form():
    for a in (0.5, 0.8, 0.9):
        for N in range(0, 12):
            assert model.expected_tokens(a, N) == pytest.approx((1 - a ** (N + 1)) / (1 - a))
    assert model.expected_tokens_rows([0.8] * 5) == pytest.approx(model.expected_tokens(0.8, 5))
    assert model.expected_tokens_rows([]) == 1.0


def test_best_n_reproduces_the_page():
    # α between 0.06 and 0.10 lies inside the page's typical 0.05-0.15
    for alpha in (0.06, 0.07, 0.08, 0.09, 0.10):
        for case in GOLDEN["best_n"]["cases"]:
            n = model.best_n(case["acceptance"], alpha)
            assert case["low"] <= n <= case["high"], (alpha, case, n)


def test_without_the_bonus_token_the_page_is_not_reproduced():
    def best_without_bonus(a, alpha):
        vals = [(model.expected_tokens(a, n) - 1) / (1 + alpha * n) for n in range(65)]
        return int(np.argmax(vals))
    hits = 0
    for alpha in (0.06, 0.07, 0.08, 0.09, 0.10):
        ok = all(c["low"] <= best_without_bonus(c["acceptance"], alpha) <= c["high"]
                 for c in GOLDEN["best_n"]["cases"])
        hits += ok
    assert hits < 5


def test_asymptotic_speedup_is_one_over_alpha():
    for case in GOLDEN["asymptote"]["cases"]:
        s = model.speedup(1.0 - 1e-12, 20000, case["alpha"])
        assert s == pytest.approx(case["speedup"], rel=1e-3)


def test_verify_cost_at_n4_matches_alpha_range():
    g = GOLDEN["verify_cost_at_n4"]
    lo, hi = GOLDEN["alpha_typical"]["low"], GOLDEN["alpha_typical"]["high"]
    assert model.verify_cost_ratio(lo, g["N"]) == pytest.approx(g["low"])
    assert model.verify_cost_ratio(0.125, g["N"]) == pytest.approx(g["high"])
    assert model.verify_cost_ratio(hi, g["N"]) > g["high"]   # the two ranges overlap only up to 0.125


def test_alpha_from_times_inverts_the_cost_model():
    for alpha in (0.01, 0.05, 0.15):
        for N in (1, 4, 8):
            t0 = 3.7
            assert model.alpha_from_times(t0 * model.verify_cost_ratio(alpha, N), t0, N) \
                == pytest.approx(alpha)
