"""Prefill attention: fixed softmax shift from the q/k-norm score bound, and
its fallback to the running max.

The library bounds every base-2 score of a layer by
log2(e) sqrt(d) max|g_q| max|g_k| (times 1.01 for the bf16 rounding of q' and
k') and, where that bound is at most 63, shifts the softmax by it instead of a
running max (tests/test_score_bound.py checks the bound on the CPU).  Two
layers of the 0.6B widths, two prompts of 1,100 tokens (the MFMA attention
with a ragged last tile), against the float32 oracle at the bf16 bound.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from tests.gpu_common import TOL, check_argmax, check_logits, dev_tokens, need_gpu, weights

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _shape():
    return dataclasses.replace(synth.QWEN3_0P6B, n_layers=2)


def _bound(w, d):
    return max(LOG2E * np.sqrt(d) * np.max(np.abs(L["q_norm"])) * np.max(np.abs(L["k_norm"])) * 1.01
               for L in w["layers"])


def _scaled(w, f):
    out = dict(w)
    # bf16 models take bf16-representable values: round the scaled gains
    out["layers"] = [dict(L, q_norm=synth.round_to_bf16((L["q_norm"] * f).astype(np.float32)),
                          k_norm=synth.round_to_bf16((L["k_norm"] * f).astype(np.float32)))
                     for L in w["layers"]]
    return out


def _prefill(shape, w, toks, monkeypatch=None, fixed=None):
    from dense_gqa_transformer_amd.model import Model
    if monkeypatch is not None and fixed is not None:
        monkeypatch.setenv("FS_PREFILL_FIXED_SHIFT", fixed)
    model = Model(shape, w, max_seqs=2, max_ctx=1100)
    if monkeypatch is not None:
        monkeypatch.delenv("FS_PREFILL_FIXED_SHIFT", raising=False)
    try:
        return model.prefill(dev_tokens(toks), [0, 1]).cpu().numpy()
    finally:
        model.close()


def _errors(shape, w, toks, lg):
    orc = O.Oracle(shape, w, dtype=np.float32)
    out = []
    for b in range(toks.shape[0]):
        ref = orc.forward(toks[b])
        assert np.all(np.isfinite(lg[b]))
        out.append((float(np.max(np.abs(lg[b].astype(np.float64) - ref))), ref))
    return out


def _vs_oracle(shape, w, toks, lg, what):
    for b, (err, ref) in enumerate(_errors(shape, w, toks, lg)):
        check_logits(lg[b], ref, TOL["bf16"], f"{what} row {b}")
        check_argmax(int(np.argmax(lg[b])), ref, f"{what} row {b} argmax")
        print(f"{what} row {b} max-abs logit error {err:.3e}", flush=True)


def test_fixed_shift_near_its_limit(monkeypatch):
    # q/k norm gains scaled so the largest layer bound is 60 (probabilities as
    # small as 2^-120, still normal numbers).  Gains 1.5 times larger sharpen
    # the softmax, and every path's bf16 rounding of q' and k' then moves the
    # logits by more than at the default gains, so the fixed shift is held to
    # the running max's own error on the same weights, not to the bound set for
    # the default ones: the shift is exact in arithmetic, so both errors are
    # samples of the same rounding error (the fixed shift may not exceed twice
    # the running max's), while a wrong shift (overflow, flushed probabilities,
    # a term dropped) is off by orders of magnitude.
    shape = _shape()
    w0 = weights(shape)
    f = float(np.sqrt(60.0 / _bound(w0, shape.head_dim)))
    w = _scaled(w0, f)
    assert 55.0 < _bound(w, shape.head_dim) <= 63.0
    toks = synth.tokens(1101, shape.vocab, (2, 1100))
    fixed = _errors(shape, w, toks, _prefill(shape, w, toks))
    running = _errors(shape, w, toks, _prefill(shape, w, toks, monkeypatch, "0"))
    for b in range(2):
        ef, er = fixed[b][0], running[b][0]
        print(f"bound 60 row {b}: fixed shift {ef:.3e}, running max {er:.3e}", flush=True)
        assert ef <= 2.0 * er + 2e-3, f"row {b}: fixed-shift error {ef:.3e} vs running max {er:.3e}"


def test_running_max_switch(monkeypatch):
    # FS_PREFILL_FIXED_SHIFT=0 keeps the running-max softmax on the default weights
    shape = _shape()
    w = weights(shape)
    toks = synth.tokens(1102, shape.vocab, (2, 1100))
    lg = _prefill(shape, w, toks, monkeypatch, "0")
    _vs_oracle(shape, w, toks, lg, "running max")


def test_bound_over_63_falls_back_to_the_running_max(monkeypatch):
    # gains x2.2 put every layer's bound above 63: the library must take the
    # running-max kernel by itself, so its logits equal those of a model
    # created with the fixed shift switched off, bit for bit
    shape = _shape()
    w = _scaled(weights(shape), 2.2)
    assert _bound(w, shape.head_dim) > 63.0
    toks = synth.tokens(1103, shape.vocab, (2, 1100))
    auto = _prefill(shape, w, toks)
    off = _prefill(shape, w, toks, monkeypatch, "0")
    assert np.all(np.isfinite(auto))
    assert np.array_equal(auto, off)
