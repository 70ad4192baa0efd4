"""8-bit floating-point (e4m3) weights and activations (test infrastructure;
same rules of use as oracle.py).

"Milestones", M7, asks for a measured decision on low-bit weights (quality,
memory and speed against the baseline); "ferrite", What it does, lists
8-bit formats among the ones it reads.  The pages fix no format.  This
module is the oracle of the library's fp8 option, whose reading is:

* Format: 8-bit floats with 1 sign bit, 4 exponent bits (bias 7) and 3
  mantissa bits, no infinities: exponent field e in 1..15 encodes
  (1 + m/8) * 2^(e - 7) except e = 15, m = 7, which is NaN; e = 0 encodes the
  subnormals (m/8) * 2^-6.  The largest finite magnitude is 448, the smallest
  positive 2^-9.  (This is the layout the gfx950 matrix cores take as their
  fp8 operand.)
* Rounding: a real value goes to the nearest representable value, a tie to
  the one with an even mantissa field; magnitudes beyond 448 saturate to 448;
  a result of zero is stored as code 0 (the positive zero) whatever the sign.
* Scales are powers of two, one per row: for a row with largest magnitude
  a > 0, ``t = a / 448`` (correctly rounded float32) and ``s = 2^e`` with e the
  smallest integer such that ``2^e >= t``; a zero row has scale 0 and codes 0.
  Then ``code = e4m3(x / s)`` (the division is exact), and ``code * s`` is
  exact in float32 and in bfloat16, so a code times its scale is the value
  the products use, and a matrix unit that takes a power-of-two scale per
  row (the gfx950 fp8 products take an 8-bit exponent per 32 operands) applies
  it without rounding.  A float format loses nothing to the power-of-two
  choice: only the window of representable magnitudes moves, by less than 2x.
* Weights: every matrix of the pass (wq, wk, wv, wo, w_gate, w_up, w_down
  and the tied embedding / head) is stored as codes with one scale per output
  row (row n of the ``[out, in]`` matrix).  Norm weights stay in the model's
  dtype.
* Activations: the outputs of the RMSNorms, which feed the Q/K/V projection,
  the gate/up projection and the tied head, are quantized per row by the same
  rule (the float32 row values) and the projection takes ``q * s``; so each
  product ``sum_k q_k c_k`` is a sum of products of two e4m3 values, which the
  fp8 matrix instructions compute exactly.  The inputs of the output and down
  projections (the attention output and the SwiGLU output) are not quantized:
  those products are weight-only.

The fp8 forward pass is the oracle's, on ``dequantized_weights`` and with
``quantize_act_rows`` applied to the norm outputs
(``Oracle(shape, dequantized_weights(w), quantize_norm_outputs=quantize_act_rows)``).
Every function is pinned by tests/test_fp8_oracle.py.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

FP8_MAX = 448.0
LAYER_MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def e4m3_decode(code: int) -> float:
    """The value of one 8-bit code (NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_grid() -> np.ndarray:
    """The 127 non-negative finite values in increasing order (0, 2^-9, ..., 448)."""
    vals = [e4m3_decode(c) for c in range(0x7F)]        # codes 0x00..0x7e: 0 and the positives
    return np.array(vals, dtype=np.float64)


_GRID = e4m3_grid()


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 value of each element (ties to an even mantissa field,
    saturating at +-448), returned as float64.  NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), FP8_MAX)
    # index of the largest grid value <= a
    i = np.searchsorted(_GRID, a, side="right") - 1
    i = np.clip(i, 0, len(_GRID) - 1)
    lo = _GRID[i]
    hi = _GRID[np.minimum(i + 1, len(_GRID) - 1)]
    d_lo = a - lo
    d_hi = hi - a
    # codes of the grid are their indices; an even code has an even mantissa field
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (i % 2 == 1) & (hi != lo))
    r = np.where(take_hi, hi, lo)
    out = np.where(x < 0, -r, r)
    return np.where(np.isnan(x), np.nan, out)


def e4m3_code(v: np.ndarray) -> np.ndarray:
    """The uint8 codes of values already on the e4m3 grid (inverse of e4m3_decode)."""
    v = np.asarray(v, dtype=np.float64)
    idx = np.searchsorted(_GRID, np.abs(v))
    if not np.all(_GRID[np.minimum(idx, len(_GRID) - 1)] == np.abs(v)):
        raise ValueError("value not on the e4m3 grid")
    return (idx | np.where(np.signbit(v) & (v != 0), 0x80, 0)).astype(np.uint8)


def pow2_scale(amax: np.ndarray) -> np.ndarray:
    """Per-row scales 2^e, e the smallest integer with 2^e >= fl32(amax / 448);
    0 where amax is 0 (float32)."""
    amax = np.asarray(amax, dtype=np.float32)
    t = (amax / np.float32(FP8_MAX)).astype(np.float32)           # correctly rounded float32
    m, e = np.frexp(t.astype(np.float64))                          # t = m * 2^e, m in [0.5, 1)
    e = np.where(m == 0.5, e - 1, e)                               # t itself a power of two
    s = np.ldexp(np.float64(1.0), e).astype(np.float32)
    return np.where(amax > 0, s, np.float32(0)).astype(np.float32)


def quantize_rows(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row e4m3 codes (as their float64 values) and power-of-two float32
    scales of a ``[rows, cols]`` float32-representable matrix."""
    w = np.asarray(w)
    if w.ndim != 2:
        raise ValueError("quantize_rows takes a matrix")
    x = w.astype(np.float32)
    if not np.array_equal(x.astype(w.dtype), w):
        raise ValueError("values are not float32-representable")
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    scale = pow2_scale(amax)
    vals = np.zeros(x.shape, dtype=np.float64)
    nz = scale > 0
    if np.any(nz):
        vals[nz] = e4m3_round(x[nz].astype(np.float64) / scale[nz, None])   # exact quotient
    return vals, scale


def dequantize_rows(vals: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """code * scale, exact in float64."""
    return np.asarray(vals, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[:, None]


def quantize_act_rows(x: np.ndarray) -> np.ndarray:
    """The activation rule applied to each row of x (last axis): the row's
    e4m3 codes times its power-of-two scale, on the row's float32 values."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1, x.shape[-1]).astype(np.float32)          # the rows as float32 values
    vals, scale = quantize_rows(flat)
    return dequantize_rows(vals, scale).reshape(x.shape)


def dequantized_weights(weights: dict) -> dict:
    """A weight dict whose matrices are replaced by their e4m3 code * scale
    values (float64); norm weights pass through."""
    layers = []
    for lw in weights["layers"]:
        d = dict(lw)
        for k in LAYER_MATRICES:
            d[k] = dequantize_rows(*quantize_rows(lw[k]))
        layers.append(d)
    return {"embed": dequantize_rows(*quantize_rows(weights["embed"])), "final_norm": weights["final_norm"],
            "layers": layers}


def quantize_weights(weights: dict) -> Dict[str, object]:
    """(values, scales) of every quantized matrix, as for the int8 format."""
    return {"embed": quantize_rows(weights["embed"]),
            "layers": [{k: quantize_rows(lw[k]) for k in LAYER_MATRICES} for lw in weights["layers"]]}
