"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no arithmetic of the forward pass.  It only defines model
shapes, draws random-init weights and token IDs from fixed seeds, and encodes
float32 values as bfloat16 bit patterns.  Both the CPU oracle (``oracle/``)
and the GPU library's callers (tests, ``bench.py``) take their inputs from here
and nowhere else.

Recipe (applies to every workload):
  * one ``numpy.random.Generator(PCG64(seed))`` per weight set, seed 0;
  * matrices ~ N(0, 0.02^2), norm weights ~ 1 + N(0, 0.1^2), drawn as float32
    in a fixed order: embed, then per layer attn_norm, wq, wk, wv, q_norm,
    k_norm, wo, mlp_norm, w_gate, w_up, w_down, then final_norm;
  * bf16 models round every drawn value to bfloat16 (round to nearest, ties to
    even) and keep the rounded value; its float32 widening is exact;
  * token IDs uniform on [0, vocab) from a per-workload seed.

Model shapes: the Qwen3-0.6B shape printed in "Coming back to Failed Star",
section "Second sitting: connect the story to the code" (V=151936, H=1024,
L=28, 16 query heads, 8 KV heads, d=128, I=3072); the first model named in
"Failed Star (fs)", section "How it's built" (GQA, RoPE, SwiGLU, RMSNorm).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

F32 = "f32"
BF16 = "bf16"

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
              "mlp_norm", "w_gate", "w_up", "w_down")
NORM_KEYS = ("attn_norm", "q_norm", "k_norm", "mlp_norm")


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    dtype: str = BF16
    rope_dim: int = 0          # rotated dims per head (0: all of head_dim)
    attn_gate: bool = False    # q projection carries a per-head output gate
    weight_format: str = "dtype"   # "dtype", "i8_row" (int8 codes + a scale per row) or "f8_row" (e4m3)

    @property
    def q_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def rot_dim(self) -> int:
        return self.rope_dim or self.head_dim

    @property
    def q_proj_width(self) -> int:
        """Rows of wq: per head the query, then (gated) its gate, interleaved by head."""
        return self.q_width * (2 if self.attn_gate else 1)

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    def layer_shapes(self) -> Dict[str, tuple]:
        h, q, kv, i, d = self.hidden, self.q_width, self.kv_width, self.ffn, self.head_dim
        return {
            "attn_norm": (h,), "wq": (self.q_proj_width, h), "wk": (kv, h), "wv": (kv, h),
            "q_norm": (d,), "k_norm": (d,), "wo": (h, q), "mlp_norm": (h,),
            "w_gate": (i, h), "w_up": (i, h), "w_down": (h, i),
        }


# Tiny fp32 model: 2 layers, hidden 256, 4 query / 2 KV heads, head_dim 64.
TINY = ModelShape(n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                  ffn=768, vocab=4096, dtype=F32)
# Qwen3-0.6B shape, bf16 weights.
QWEN3_0P6B = ModelShape(n_layers=28, hidden=1024, n_heads=16, n_kv_heads=8,
                        head_dim=128, ffn=3072, vocab=151936, dtype=BF16)
# The gated attention variant ("ferrite", What it does): 8 query / 2 KV heads
# of width 256, rotate-half RoPE on 64 of the 256 dims, a sigmoid gate on each
# head's output carried by the q projection (per-head interleaved [q | gate]).
GATED_TINY = ModelShape(n_layers=2, hidden=512, n_heads=8, n_kv_heads=2, head_dim=256,
                        ffn=1024, vocab=4096, dtype=F32, rope_dim=64, attn_gate=True)
GATED_BF16 = ModelShape(n_layers=2, hidden=512, n_heads=8, n_kv_heads=2, head_dim=256,
                        ffn=1024, vocab=4096, dtype=BF16, rope_dim=64, attn_gate=True)
# The same attention at the 0.6B shape's other widths (for measurement).
GATED_0P6B = ModelShape(n_layers=28, hidden=1024, n_heads=8, n_kv_heads=2, head_dim=256,
                        ffn=3072, vocab=151936, dtype=BF16, rope_dim=64, attn_gate=True)


# Int8 weights (one scale per output row) on the tiny fp32 model and the 0.6B shape.
TINY_I8 = dataclasses.replace(TINY, weight_format="i8_row")
QWEN3_0P6B_I8 = dataclasses.replace(QWEN3_0P6B, weight_format="i8_row")
# fp8 (e4m3) weights with power-of-two row scales, norm outputs quantized too.
TINY_F8 = dataclasses.replace(TINY, weight_format="f8_row")
QWEN3_0P6B_F8 = dataclasses.replace(QWEN3_0P6B, weight_format="f8_row")


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even; returns the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    lsb += np.uint32(0x7FFF)
    lsb += u                       # wraps only for NaN patterns, fixed below
    out = (lsb >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bfloat16 (RNE)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


def make_weights(shape: ModelShape, seed: int = 0, std: float = 0.02,
                 norm_std: float = 0.1) -> dict:
    """Random-init weights as float32 numpy arrays, ``[out, in]`` row-major.

    For bf16 models each array already holds bf16-rounded values, so
    ``f32_to_bf16_bits`` of it is lossless.  Returns
    ``{"embed", "final_norm", "layers": [dict per layer]}``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))

    def draw(shp, norm):
        a = rng.standard_normal(size=shp, dtype=np.float32)
        if norm:
            a *= np.float32(norm_std)
            a += np.float32(1.0)
        else:
            a *= np.float32(std)
        if shape.dtype == BF16:
            a = round_to_bf16(a)
        return a

    embed = draw((shape.vocab, shape.hidden), False)
    layers: List[dict] = []
    shp = shape.layer_shapes()
    for _ in range(shape.n_layers):
        layers.append({k: draw(shp[k], k in NORM_KEYS) for k in LAYER_KEYS})
    final_norm = draw((shape.hidden,), True)
    return {"embed": embed, "final_norm": final_norm, "layers": layers}


def tokens(seed: int, vocab: int, size) -> np.ndarray:
    """Uniform-random token IDs on [0, vocab), int32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, vocab, size=size).astype(np.int32)


def uniforms(seed: int, size) -> np.ndarray:
    """Uniform draws on [0, 1) as float32 (the random numbers a sampler consumes)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.random(size=size, dtype=np.float64)
    return np.minimum(u, np.nextafter(np.float32(1), np.float32(0))).astype(np.float32)


def logit_rows(seed: int, rows: int, vocab: int, std: float = 0.64) -> np.ndarray:
    """Synthetic fp32 logit rows ~ N(0, std^2), the spread the 0.6B-shape
    random-init model produces."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((rows, vocab), dtype=np.float32) * np.float32(std)).astype(np.float32)


def activation_rows(seed: int, rows: int, cols: int) -> np.ndarray:
    """Synthetic fp32 rows shaped like normalised activations: N(0, 1) times a
    per-row magnitude spread over 2^-4 .. 2^4, with one column in 64 scaled up
    8x (the outlier channels a norm gain produces)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    mag = np.exp2(rng.uniform(-4.0, 4.0, size=(rows, 1))).astype(np.float32)
    out_cols = rng.permutation(cols)[: max(1, cols // 64)]
    x[:, out_cols] *= np.float32(8.0)
    return (x * mag).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    prompts: tuple          # tuple of int32 arrays, one per sequence
    decode_steps: int       # greedy KV-cached steps after the prompt

    @property
    def batch(self) -> int:
        return len(self.prompts)

    @property
    def max_ctx(self) -> int:
        return max(len(p) for p in self.prompts) + self.decode_steps


def workload(name: str) -> Workload:
    """The five seeded workloads.

    tiny_fp32            : tiny fp32 model, one 16-token prompt, 16 decode steps
    scorer_0p6b          : 0.6B bf16, one 6-token prompt, last-token logits only
    decode_0p6b_bs1      : 0.6B bf16, 512-token prompt, 256 decode steps
    prefill_0p6b_4x4096  : 0.6B bf16, four 4096-token prompts, last-token logits
    decode_0p6b_bs64     : 0.6B bf16, 64 prompts of ragged length in
                           [256, 4096], 128 decode steps each
    gated_tiny_fp32      : gated-attention variant (fp32), one 16-token prompt,
                           16 decode steps
    gated_bf16           : gated-attention variant (bf16), two 160-token
                           prompts, 16 decode steps
    """
    if name == "tiny_fp32":
        t = tokens(101, TINY.vocab, (1, 16))
        return Workload(name, TINY, (t[0],), 16)
    if name == "scorer_0p6b":
        t = tokens(102, QWEN3_0P6B.vocab, (1, 6))
        return Workload(name, QWEN3_0P6B, (t[0],), 0)
    if name == "decode_0p6b_bs1":
        t = tokens(103, QWEN3_0P6B.vocab, (1, 512))
        return Workload(name, QWEN3_0P6B, (t[0],), 256)
    if name == "prefill_0p6b_4x4096":
        t = tokens(104, QWEN3_0P6B.vocab, (4, 4096))
        return Workload(name, QWEN3_0P6B, tuple(t[i] for i in range(4)), 0)
    if name == "decode_0p6b_bs64":
        lens = np.random.Generator(np.random.PCG64(105)).integers(256, 4097, 64)
        rng = np.random.Generator(np.random.PCG64(106))
        prompts = tuple(rng.integers(0, QWEN3_0P6B.vocab, size=int(n)).astype(np.int32)
                        for n in lens)
        return Workload(name, QWEN3_0P6B, prompts, 128)
    if name == "gated_tiny_fp32":
        t = tokens(107, GATED_TINY.vocab, (1, 16))
        return Workload(name, GATED_TINY, (t[0],), 16)
    if name == "gated_bf16":
        t = tokens(108, GATED_BF16.vocab, (2, 160))
        return Workload(name, GATED_BF16, (t[0], t[1]), 16)
    raise KeyError(name)


WORKLOADS = ("tiny_fp32", "scorer_0p6b", "decode_0p6b_bs1",
             "prefill_0p6b_4x4096", "decode_0p6b_bs64", "gated_tiny_fp32", "gated_bf16")


def small_shape(**kw) -> ModelShape:
    """A very small shape for brute-force checks (fp32)."""
    base = dict(n_layers=2, hidden=32, n_heads=4, n_kv_heads=2, head_dim=8,
                ffn=48, vocab=64, dtype=F32)
    base.update(kw)
    return ModelShape(**base)


_WEIGHT_CACHE: Dict[tuple, dict] = {}


def cached_weights(shape: ModelShape, seed: int = 0) -> dict:
    key = (shape, seed)
    if key not in _WEIGHT_CACHE:
        _WEIGHT_CACHE[key] = make_weights(shape, seed)
    return _WEIGHT_CACHE[key]
