"""Low-bit decode weights: the int8 weight format (test infrastructure; same
rules of use as oracle.py).

The pages leave the format open.  "Milestones", M7, asks whether low-bit
weights earn their complexity once a measured baseline exists, with the
quality, memory and speed differences recorded; "ferrite", What it does,
lists 8-bit block formats among the ones it reads.  The reading taken here:

* every matrix the forward pass multiplies by (wq, wk, wv, wo, w_gate, w_up,
  w_down and the tied embedding / head) is stored as signed 8-bit codes with
  one scale per output row (row n of the ``[out, in]`` matrix);
* symmetric and round-to-nearest: ``s_n = max_k |W[n, k]| / 127`` and
  ``q[n, k] = round(W[n, k] / s_n)``, ties to even, codes in [-127, 127];
  a row of zeros has scale 0 and codes 0;
* both decisions are taken in float32 (the weights are float32 or bfloat16
  values, so their float32 form is exact): the scale is the correctly rounded
  float32 quotient, and the code the nearest integer to the correctly rounded
  float32 quotient ``W / s_n``;
* the model computes with ``q[n, k] * s_n``, formed exactly (float64 here);
  norm weights stay in the model's dtype.  The embedding lookup and the head
  read the same codes, so the head stays tied.

The quantized forward pass is the oracle's forward pass run on
``dequantized_weights``; nothing else changes.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

QMAX = 127
# the matrices of one layer that are quantized, by the names the weight dict uses
LAYER_MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def quantize_rows(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric int8 codes and float32 scales of a ``[rows, cols]`` matrix."""
    w = np.asarray(w)
    if w.ndim != 2:
        raise ValueError("quantize_rows takes a matrix")
    x = w.astype(np.float32)
    if not np.array_equal(x.astype(w.dtype), w):
        raise ValueError("values are not float32-representable")
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    scale = (amax / np.float32(QMAX)).astype(np.float32)          # correctly rounded float32
    codes = np.zeros(x.shape, dtype=np.int8)
    nz = scale > 0
    if np.any(nz):
        r = (x[nz] / scale[nz, None]).astype(np.float32)          # correctly rounded float32
        codes[nz] = np.clip(np.rint(r), -QMAX, QMAX).astype(np.int8)
    return codes, scale


def dequantize_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """The values the model computes with: code * scale, exact in float64."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[:, None]


def quantize_weights(weights: dict) -> Dict[str, object]:
    """Codes and scales of every quantized matrix of a weight dict (as made by
    ``synth.make_weights``): ``{"embed": (codes, scale), "layers": [{name: (codes, scale)}]}``."""
    return {
        "embed": quantize_rows(weights["embed"]),
        "layers": [{k: quantize_rows(lw[k]) for k in LAYER_MATRICES} for lw in weights["layers"]],
    }


def dequantized_weights(weights: dict) -> dict:
    """A weight dict whose matrices are replaced by their dequantized values
    (float64); norm weights are passed through unchanged."""
    q = quantize_weights(weights)
    layers = []
    for lw, ql in zip(weights["layers"], q["layers"]):
        d = dict(lw)
        for k in LAYER_MATRICES:
            d[k] = dequantize_rows(*ql[k])
        layers.append(d)
    return {"embed": dequantize_rows(*q["embed"]), "final_norm": weights["final_norm"], "layers": layers}

