"""Shared helpers for the GPU parity tests (imported by test modules only)."""
import functools

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O

# max-abs logit tolerance per model dtype
TOL = {"f32": 1e-4, "bf16": 2e-2}
# argmax must match wherever the oracle's top-2 gap exceeds this
GAP = 1e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from dense_gqa_transformer_amd import native
    native.load()          # raises if the HIP library is missing


@functools.lru_cache(maxsize=2)
def weights(shape):
    return synth.make_weights(shape, 0)


@functools.lru_cache(maxsize=1)
def oracle_for(shape):
    return O.Oracle(shape, weights(shape))


def fresh_oracle(shape):
    return O.Oracle(shape, weights(shape))


def make_model(shape, max_seqs, max_ctx):
    from dense_gqa_transformer_amd.model import Model
    return Model(shape, weights(shape), max_seqs=max_seqs, max_ctx=max_ctx)


def dev_tokens(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


def check_logits(gpu, ref, tol, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, what
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU logits"
    err = float(np.max(np.abs(gpu - ref)))
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"
    return err


def check_argmax(gpu_id, ref_logits, what=""):
    ref_id = O.greedy_argmax_fast(ref_logits)
    if O.top2_gap(ref_logits) > GAP:
        assert int(gpu_id) == ref_id, f"{what}: argmax {int(gpu_id)} != oracle {ref_id}"
    else:
        # near-tie: any ID within GAP of the oracle's max is acceptable
        assert ref_logits[int(gpu_id)] >= np.max(ref_logits) - GAP, what
