"""The attention-score bound the prefill attention uses as a fixed softmax shift.

With the per-head q/k RMSNorm of the pass ("Coming back to Failed Star",
Second sitting; the norm is applied per head before RoPE), every normalised
row has length at most sqrt(d), the norm weight scales each element by at most
max|g|, and RoPE rotates pairs, so a base-2 score obeys

    |q'.k'| / sqrt(d) * log2(e)  <=  log2(e) * sqrt(d) * max|g_q| * max|g_k|.

These checks use the oracle's own RMSNorm and RoPE on rows built to sit at the
bound (k parallel to q, all the weight on the largest gain) and on random
rows, so a bound that forgot the sqrt(d), a gain or the RoPE step fails.
"""
import numpy as np
import pytest

from oracle import oracle as O

LOG2E = 1.4426950408889634


def bound(gq, gk, d):
    return LOG2E * np.sqrt(d) * np.max(np.abs(gq)) * np.max(np.abs(gk))


def score2(q, k, gq, gk, pos, d, eps=1e-6, theta=1e6):
    qn = O.rope(O.rms_norm(q, gq, eps)[None, None, :], np.array([pos]), theta)[0, 0]
    kn = O.rope(O.rms_norm(k, gk, eps)[None, None, :], np.array([pos]), theta)[0, 0]
    return float(qn @ kn) / np.sqrt(d) * LOG2E


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bound_holds_on_random_rows(d):
    rng = np.random.default_rng(d)
    for _ in range(200):
        gq = 1 + 0.1 * rng.standard_normal(d)
        gk = 1 + 0.1 * rng.standard_normal(d)
        q = rng.standard_normal(d) * rng.uniform(0.01, 100)
        k = rng.standard_normal(d) * rng.uniform(0.01, 100)
        pos = int(rng.integers(0, 40960))
        assert abs(score2(q, k, gq, gk, pos, d)) <= bound(gq, gk, d)


@pytest.mark.parametrize("d", [64, 128])
def test_bound_is_reached_by_a_one_hot_pair(d):
    # all of q and k on the dim with the largest gains: after the norm the row is
    # sqrt(d) e_i, so q'.k' = d g_q,i g_k,i at position 0 (RoPE is the identity)
    rng = np.random.default_rng(7)
    gq = 1 + 0.1 * rng.standard_normal(d)
    gk = gq.copy()
    i = int(np.argmax(np.abs(gq)))
    q = np.zeros(d)
    q[i] = 3.0
    s = score2(q, q.copy(), gq, gk, 0, d, eps=0.0)
    assert s == pytest.approx(bound(gq, gk, d), rel=1e-12)
    # a bound without sqrt(d), or with only one gain, is exceeded
    assert s > LOG2E * np.max(np.abs(gq)) * np.max(np.abs(gk))
    assert s > LOG2E * np.sqrt(d) * np.max(np.abs(gq))


def test_bound_survives_rotation():
    # the same pair at any position (both rotated by the same angles) keeps the
    # score; q and k at different rotations never exceed the bound either
    d = 128
    rng = np.random.default_rng(3)
    gq = 1 + 0.1 * rng.standard_normal(d)
    gk = 1 + 0.1 * rng.standard_normal(d)
    q = rng.standard_normal(d)
    s0 = score2(q, q.copy(), gq, gq, 0, d)
    for pos in (1, 17, 4095):
        assert score2(q, q.copy(), gq, gq, pos, d) == pytest.approx(s0, rel=1e-9)
    b = bound(gq, gk, d)
    for pa, pb in ((0, 5), (100, 3), (4000, 1)):
        qn = O.rope(O.rms_norm(q, gq, 1e-6)[None, None, :], np.array([pa]), 1e6)[0, 0]
        kn = O.rope(O.rms_norm(q, gk, 1e-6)[None, None, :], np.array([pb]), 1e6)[0, 0]
        assert abs(float(qn @ kn) / np.sqrt(d) * LOG2E) <= b
