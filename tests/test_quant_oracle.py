"""Pins of the int8 weight format in the oracle (oracle/quant.py): per-row
symmetric codes, round to nearest with ties to even, the forward pass run on
the dequantized values ("Milestones", M7, the quantization decision; the
format reading is in the module's header).

The checks are closed forms (rows that are integers times a power of two
quantize losslessly), brute force over all 255 codes, the half-integer ties,
the error bound, and a model whose every row is exactly representable, which
must give the unquantized logits bit for bit.
"""
import numpy as np
import pytest

import synth
from oracle import oracle as O
from oracle import quant as Q


def _exact_rows(rng, rows, cols, exps):
    """Rows of integers in [-127, 127] times 2^-e (e per row), each holding +-127."""
    k = rng.integers(-127, 128, size=(rows, cols))
    k[:, 0] = 127 * rng.choice([-1, 1], size=rows)
    return k, (k.astype(np.float64) * np.exp2(-np.asarray(exps, dtype=np.float64))[:, None]).astype(np.float32)


def test_rows_of_scaled_integers_are_lossless():
    rng = np.random.default_rng(11)
    exps = np.array([0, 3, 7, 12, 20])
    k, w = _exact_rows(rng, 5, 64, exps)
    codes, scale = Q.quantize_rows(w)
    assert codes.dtype == np.int8 and scale.dtype == np.float32
    assert np.array_equal(codes, k)
    assert np.array_equal(scale, np.exp2(-exps).astype(np.float32))
    assert np.array_equal(Q.dequantize_rows(codes, scale), w.astype(np.float64))


def test_scale_is_per_output_row():
    # one row's large value must not coarsen another row's codes
    w = np.array([[127.0, 1.0, -3.0], [0.5, -0.3, 0.1]], dtype=np.float32)
    codes, scale = Q.quantize_rows(w)
    assert scale.tolist() == [1.0, np.float32(0.5) / np.float32(127)]
    assert codes[0].tolist() == [127, 1, -3]
    assert codes[1].tolist() == [127, -76, 25]       # -0.3 * 254 = -76.2, 0.1 * 254 = 25.4


def test_ties_go_to_even_and_signs_are_symmetric():
    w = np.array([[127, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5]], dtype=np.float32)
    codes, scale = Q.quantize_rows(w)
    assert scale[0] == 1.0
    assert codes[0].tolist() == [127, 2, 4, -2, -4, 0, 0, 2, 126]
    c2, s2 = Q.quantize_rows(-w)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scale)


def test_zero_rows_and_empty_rows():
    w = np.zeros((3, 8), dtype=np.float32)
    w[1, 5] = -0.75
    codes, scale = Q.quantize_rows(w)
    assert scale[0] == 0 and scale[2] == 0 and not codes[0].any() and not codes[2].any()
    assert codes[1].tolist() == [0, 0, 0, 0, 0, -127, 0, 0]
    assert scale[1] == np.float32(0.75) / np.float32(127)
    c0, s0 = Q.quantize_rows(np.zeros((2, 0), np.float32))
    assert c0.shape == (2, 0) and s0.tolist() == [0.0, 0.0]
    with pytest.raises(ValueError):
        Q.quantize_rows(np.array([[0.1]], dtype=np.float64))    # not a float32 value


def test_brute_force_nearest_code():
    # every code is the nearest of the 255 candidates c * s (ties: even c),
    # away from values whose quotient sits within float32 rounding of a tie
    rng = np.random.default_rng(12)
    w = synth.round_to_bf16((rng.standard_normal((16, 96)) * 0.02).astype(np.float32))
    codes, scale = Q.quantize_rows(w)
    cand = np.arange(-127, 128, dtype=np.float64)
    checked = 0
    for n in range(w.shape[0]):
        s = float(scale[n])
        for kk in range(w.shape[1]):
            x = float(w[n, kk])
            frac = abs(x / s - np.floor(x / s) - 0.5)
            if frac < 1e-5:
                continue
            err = np.abs(x - cand * s)
            assert codes[n, kk] == int(cand[np.argmin(err)]), (n, kk)
            checked += 1
    assert checked > 0.99 * w.size


def test_error_bound_and_extremes():
    rng = np.random.default_rng(13)
    w = synth.round_to_bf16((rng.standard_normal((64, 1024)) * 0.02).astype(np.float32))
    codes, scale = Q.quantize_rows(w)
    deq = Q.dequantize_rows(codes, scale)
    s = scale.astype(np.float64)[:, None]
    # the float32 quotient may sit up to 127 * 2^-24 from the exact one
    assert np.all(np.abs(w - deq) <= s * (0.5 + 1e-5))
    assert np.all(np.max(np.abs(codes.astype(np.int32)), axis=1) == 127)
    nz = codes != 0
    assert np.all(np.sign(codes[nz]) == np.sign(w[nz]))
    # the amax element reconstructs to within float32 rounding of the scale
    i = np.argmax(np.abs(w), axis=1)
    assert np.allclose(deq[np.arange(64), i], w[np.arange(64), i], rtol=1e-6, atol=0)


def _exact_model(shape, seed):
    """A weight set whose every matrix row is integers times a power of two."""
    rng = np.random.default_rng(seed)
    w = synth.make_weights(shape, seed)

    def exact(a):
        e = rng.integers(12, 16, size=a.shape[0])
        return _exact_rows(rng, a.shape[0], a.shape[1], e)[1]
    w["embed"] = exact(w["embed"])
    for lw in w["layers"]:
        for k in Q.LAYER_MATRICES:
            lw[k] = exact(lw[k])
    return w


def test_forward_on_exact_weights_is_unchanged():
    shape = synth.small_shape()
    w = _exact_model(shape, 21)
    dq = Q.dequantized_weights(w)
    toks = synth.tokens(5, shape.vocab, 9)
    a = O.Oracle(shape, w).forward(toks, all_rows=True)
    b = O.Oracle(shape, dq).forward(toks, all_rows=True)
    assert np.array_equal(a, b)


def test_every_matrix_is_quantized_and_norms_are_not():
    shape = synth.small_shape()
    w = synth.make_weights(shape, 22)
    dq = Q.dequantized_weights(w)
    q = Q.quantize_weights(w)
    assert not np.array_equal(dq["embed"], w["embed"])
    assert np.array_equal(dq["final_norm"], w["final_norm"])
    for lw, dl, ql in zip(w["layers"], dq["layers"], q["layers"]):
        for k in Q.LAYER_MATRICES:
            assert dl[k].shape == lw[k].shape and ql[k][1].shape == (lw[k].shape[0],)
            assert not np.array_equal(dl[k], lw[k]), k
            assert np.all(np.abs(dl[k] - lw[k]) <= ql[k][1][:, None] * (0.5 + 1e-5)), k
        for k in synth.NORM_KEYS:
            assert np.array_equal(dl[k], lw[k])
    # the quantized model still predicts close to the unquantized one
    toks = synth.tokens(6, shape.vocab, 12)
    a = O.Oracle(shape, w).forward(toks)
    b = O.Oracle(shape, dq).forward(toks)
    assert 0 < np.max(np.abs(a - b)) < 0.05 * np.max(np.abs(a))
