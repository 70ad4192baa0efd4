"""Pins of the fp8 (e4m3) weight and activation option in the oracle
(oracle/fp8.py; the reading is in its header).

Checked against the format's definition rather than against the module
itself: known codes of the format (1.0 = 0x38, 448 = 0x7e, 2^-9 = 0x01, the
NaN codes), brute-force nearest-value search over the whole grid with the
tie rule checked on the code's parity, saturation, closed forms (rows already
on the grid times a power of two quantize losslessly; a row's maximum maps
to 448), the error bound of a rounding, and the places where the forward
pass applies the activation rule (exactly the 2L + 1 RMSNorm outputs, the
values the norms produce).
"""
import math

import numpy as np
import pytest

import synth
from oracle import fp8 as F
from oracle import oracle as O


def test_known_codes_of_the_format():
    assert F.e4m3_decode(0x38) == 1.0
    assert F.e4m3_decode(0x7E) == 448.0
    assert F.e4m3_decode(0x01) == 2.0 ** -9                  # smallest subnormal
    assert F.e4m3_decode(0x08) == 2.0 ** -6                  # smallest normal
    assert F.e4m3_decode(0x07) == 7 / 8 * 2.0 ** -6          # largest subnormal
    assert F.e4m3_decode(0x30) == 0.5
    assert F.e4m3_decode(0xC0) == -2.0
    assert F.e4m3_decode(0x3C) == 1.5
    assert math.isnan(F.e4m3_decode(0x7F)) and math.isnan(F.e4m3_decode(0xFF))
    assert F.e4m3_decode(0x80) == 0.0 and math.copysign(1, F.e4m3_decode(0x80)) < 0


def test_grid_is_the_format():
    g = F.e4m3_grid()
    assert len(g) == 127 and g[0] == 0 and g[-1] == 448
    assert np.all(np.diff(g) > 0)
    # every finite positive value is an integer 1..15 (subnormal: 1..7) times a power of two,
    # with 8 values per binade above 2^-6 and spacing 2^-9 below it
    for v in g[1:]:
        e = math.floor(math.log2(v))
        if v < 2 ** -6:
            assert (v / 2 ** -9).is_integer()
        else:
            assert ((v / 2 ** e) * 8).is_integer() and 8 <= (v / 2 ** e) * 8 < 16
    assert F.e4m3_code(g).tolist() == list(range(127))
    assert F.e4m3_code(-g[1:]).tolist() == [0x80 | c for c in range(1, 127)]


def test_rounding_is_nearest_with_ties_to_even_code():
    rng = np.random.default_rng(21)
    g = F.e4m3_grid()
    mids = (g[:-1] + g[1:]) / 2
    x = np.concatenate([rng.uniform(0, 460, 4000), rng.uniform(0, 2 ** -4, 2000), mids, g,
                        np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    r = F.e4m3_round(x)
    for xi, ri in zip(x.tolist(), r.tolist()):
        a = min(xi, 448.0)
        d = np.abs(g - a)
        best = np.flatnonzero(d == d.min())
        if len(best) == 1:
            assert ri == g[best[0]], (xi, ri)
        else:                                  # a tie: the even code wins
            even = [i for i in best if i % 2 == 0]
            assert len(even) == 1 and ri == g[even[0]], (xi, ri)
    # signs, saturation, idempotence
    assert np.array_equal(F.e4m3_round(-x), -r)
    assert F.e4m3_round(np.array([1e6, -500.0, 464.0]))[0] == 448 and F.e4m3_round(np.array([-500.0]))[0] == -448
    assert np.array_equal(F.e4m3_round(g), g)
    assert F.e4m3_round(np.array([1.0625, 1.1875, 3 * 2 ** -11]))[:].tolist() == [1.0, 1.25, 2 ** -9]


def test_rounding_error_bound():
    rng = np.random.default_rng(22)
    x = rng.uniform(2 ** -6, 448, 20000)
    r = F.e4m3_round(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2 ** -4 * (1 + 1e-12))   # half a mantissa step


def test_weight_rows_on_the_grid_are_lossless():
    rng = np.random.default_rng(23)
    g = F.e4m3_grid()
    rows = []
    for k in (0, -3, 5, -12):
        v = rng.choice(np.concatenate([g, -g]), size=40)
        v[7] = 448.0 * rng.choice([-1, 1])
        rows.append(v * 2.0 ** k)
    w = np.array(rows, dtype=np.float32)
    vals, scale = F.quantize_rows(w)
    assert scale.tolist() == [2.0 ** k for k in (0, -3, 5, -12)]
    assert np.array_equal(F.dequantize_rows(vals, scale), w.astype(np.float64))


def test_power_of_two_scales():
    # the smallest 2^e with 2^e >= fl32(amax / 448)
    amax = np.array([448.0, 449.0, 447.0, 224.0, 0.5, 1e-30, 0.0, 3.0e5], dtype=np.float32)
    s = F.pow2_scale(amax)
    assert s.tolist()[:7] == [1.0, 2.0, 1.0, 0.5, 2.0 ** -9, 2.0 ** -108, 0.0]
    assert s[7] == 1024.0                            # 3e5 / 448 = 669.6 -> 2^10
    for a, sc in zip(amax[:6].tolist() + [3.0e5], s[:6].tolist() + [1024.0]):
        t = float(np.float32(np.float32(a) / np.float32(448)))
        assert sc >= t and sc / 2 < t


def test_weight_rule_per_row_and_zero_rows():
    w = np.array([[448.0, 1.0, -3.0], [0.5, -0.3, 0.1], [0.0, 0.0, 0.0]], dtype=np.float32)
    vals, scale = F.quantize_rows(w)
    assert scale[0] == 1.0 and scale[2] == 0.0 and not vals[2].any()
    assert vals[0].tolist() == [448.0, 1.0, -3.0]
    # row 1: s = 2^-9 (>= 0.5/448 = 2^-9.8); 0.5 -> 256, -0.3 / s = -153.6 -> -160, 0.1 / s = 51.2 -> 52
    assert scale[1] == 2.0 ** -9
    assert vals[1].tolist() == [256.0, -160.0, 52.0]


def test_activation_rule():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((5, 64))
    q = F.quantize_act_rows(x)
    # relative error of every element at most half a mantissa step (plus the
    # float32 rounding of the row), idempotent, sign-symmetric, power-of-two-equivariant
    big = np.abs(x) >= np.max(np.abs(x), axis=1, keepdims=True) * 2 ** -6
    assert np.all(np.abs(q - x)[big] <= np.abs(x)[big] * (2 ** -4 + 1e-6))
    np.testing.assert_array_equal(F.quantize_act_rows(q), q)
    np.testing.assert_array_equal(F.quantize_act_rows(-x), -q)
    np.testing.assert_array_equal(F.quantize_act_rows(x * 8.0), q * 8.0)


def test_activation_rule_is_applied_at_every_norm_output():
    shape = synth.small_shape(n_layers=3)
    w = synth.make_weights(shape, 25)
    seen = []

    def spy(v):
        seen.append(np.array(v, copy=True))
        return v                      # identity: the pass equals the plain one

    ids = [3, 9, 27, 1]
    got = O.Oracle(shape, w, quantize_norm_outputs=spy).forward(ids)
    np.testing.assert_array_equal(got, O.Oracle(shape, w).forward(ids))
    assert len(seen) == 2 * shape.n_layers + 1
    # the first is layer 0's input norm of the embedding rows, the last the final norm of the last row
    x = w["embed"][ids].astype(np.float64)
    np.testing.assert_allclose(seen[0], O.rms_norm(x, w["layers"][0]["attn_norm"], shape.rms_eps), rtol=1e-14)
    assert seen[-1].shape == (shape.hidden,)
    # with the fp8 rule the logits move, and stay within a few percent of the spread
    q = O.Oracle(shape, w, quantize_norm_outputs=F.quantize_act_rows).forward(ids)
    assert 0 < np.max(np.abs(q - got)) < 0.2 * np.std(got)
