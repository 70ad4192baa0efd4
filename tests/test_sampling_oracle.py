"""Pins of the sampling oracle (oracle/sampling.py) against closed forms.

Each case is worked out by hand from the chain temperature -> top-k -> top-p
-> renormalise -> draw ("Coming back to Failed Star", section "Next: one
complete deterministic generation arc") and the readings in the oracle
header; none re-runs the oracle's own formulas.
"""
import math

import numpy as np
import pytest

import synth
from oracle import greedy_argmax
from oracle import sampling as smp


def L(*probs):
    """Logits whose softmax is the given (normalised) probabilities."""
    return np.log(np.asarray(probs, dtype=np.float64))


def test_temperature_zero_is_greedy():
    rows = synth.logit_rows(7, 6, 300)
    rows[0, 17] = rows[0].max()          # exact tie: lowest ID wins
    for r in rows:
        assert smp.sample(r, 0.0, 0, 1.0, 0.5) == greedy_argmax(r)


def test_top_k_one_is_argmax_for_any_draw():
    r = synth.logit_rows(8, 1, 500)[0]
    for u in (0.0, 0.3, 0.999):
        for t in (0.5, 1.0, 3.0):
            assert smp.sample(r, t, 1, 1.0, u) == int(np.argmax(r))


def test_two_tokens_closed_form():
    # p = [3/4, 1/4]; cumulative in ID order: 0.75, 1.0
    x = L(0.75, 0.25)
    assert smp.sample(x, 1.0, 0, 1.0, 0.74) == 0
    assert smp.sample(x, 1.0, 0, 1.0, 0.76) == 1


def test_temperature_reshapes_before_filters():
    # logits [0, ln 2]: p ∝ exp(x / T)
    x = np.array([0.0, math.log(2.0)])
    # T = 1: p = [1/3, 2/3]
    assert smp.sample(x, 1.0, 0, 1.0, 0.33) == 0
    assert smp.sample(x, 1.0, 0, 1.0, 0.34) == 1
    # T = 1/2: p ∝ [1, 4] -> [0.2, 0.8]
    assert smp.sample(x, 0.5, 0, 1.0, 0.19) == 0
    assert smp.sample(x, 0.5, 0, 1.0, 0.21) == 1
    # T large: p -> [1/2, 1/2]
    assert smp.sample(x, 1e9, 0, 1.0, 0.49) == 0
    assert smp.sample(x, 1e9, 0, 1.0, 0.51) == 1


def test_uniform_logits_map_u_to_floor():
    x = np.zeros(10)
    for u in (0.0, 0.05, 0.31, 0.57, 0.999):
        assert smp.sample(x, 1.0, 0, 1.0, u) == int(math.floor(u * 10))


def test_top_p_cut_and_renormalisation():
    x = L(0.5, 0.3, 0.2)
    ids, q = smp.kept_tokens(x, 1.0, 0, 0.75)          # 0.5 < 0.75 <= 0.8 -> {0, 1}
    assert list(ids) == [0, 1]
    assert np.allclose(q, [0.625, 0.375])
    assert list(smp.kept_tokens(x, 1.0, 0, 0.45)[0]) == [0]          # 0.45 <= 0.5
    assert list(smp.kept_tokens(x, 1.0, 0, 0.85)[0]) == [0, 1, 2]
    # draw after renormalisation: cumulative 0.625, 1.0
    assert smp.sample(x, 1.0, 0, 0.75, 0.62) == 0
    assert smp.sample(x, 1.0, 0, 0.75, 0.63) == 1


def test_filter_order_top_k_before_top_p():
    # top-k (2) first renormalises [0.5, 0.3] -> [0.625, 0.375]; p = 0.6 then keeps {0}.
    # (Top-p first would see 0.5 < 0.6 and keep {0, 1}.)
    x = L(0.5, 0.3, 0.2)
    assert list(smp.kept_tokens(x, 1.0, 2, 0.6)[0]) == [0]


def test_filter_order_temperature_before_top_p():
    # T = 2 flattens [0.5, 0.3, 0.2] to ∝ sqrt: [0.4155, 0.3218, 0.2627]; p = 0.45 keeps {0, 1}.
    # (Top-p at T = 1 would keep {0} since 0.5 >= 0.45.)
    x = L(0.5, 0.3, 0.2)
    assert list(smp.kept_tokens(x, 2.0, 0, 0.45)[0]) == [0, 1]


def test_top_k_ties_are_kept():
    x = np.array([3.0, 2.0, 2.0, 2.0, 1.0])
    assert list(smp.kept_tokens(x, 1.0, 2, 1.0)[0]) == [0, 1, 2, 3]
    assert list(smp.kept_tokens(x, 1.0, 1, 1.0)[0]) == [0]
    assert list(smp.kept_tokens(x, 1.0, 5, 1.0)[0]) == [0, 1, 2, 3, 4]


def test_non_finite_never_drawn():
    x = np.array([np.nan, 0.0, np.inf, 0.0, -np.inf])
    got = {smp.sample(x, 1.0, 0, 1.0, u) for u in np.linspace(0, 0.999, 50)}
    assert got == {1, 3}
    assert smp.sample(np.array([np.nan, np.inf]), 1.0, 0, 1.0, 0.3) == -1


def test_empirical_frequencies_match_probabilities():
    p = np.array([0.05, 0.3, 0.1, 0.25, 0.02, 0.18, 0.07, 0.03])
    x = np.log(p)
    us = synth.uniforms(11, 20000)
    cnt = np.bincount([smp.sample(x, 1.0, 0, 1.0, float(u)) for u in us], minlength=8)
    assert np.max(np.abs(cnt / us.size - p)) < 0.015      # > 4 standard deviations of each frequency


def test_acceptable_is_unique_away_from_boundaries():
    x = L(0.5, 0.3, 0.2)
    assert smp.acceptable(x, 1.0, 0, 0.75, 0.3) == [0]
    # draw within eps of the 0.625 boundary admits both neighbours
    assert smp.acceptable(x, 1.0, 0, 0.75, 0.625, eps=1e-6) == [0, 1]
