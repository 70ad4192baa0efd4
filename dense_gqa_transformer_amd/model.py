"""Python face of the C ABI: a model handle plus the greedy argmax call.

PyTorch supplies device memory and the HIP stream; the forward pass itself
runs inside libfs.so.  Nothing here computes any part of the pass.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import native
from .native import FsConfig, FsLayerWeights, FsWeights, check, int_array

LAYER_KEYS = native.LAYER_FIELDS


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[ctypes.c_void_p]:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _to_device(a, torch_dtype, device) -> torch.Tensor:
    if isinstance(a, np.ndarray):
        a = torch.from_numpy(np.ascontiguousarray(a))
    return a.to(device=device, dtype=torch_dtype).contiguous()


class Model:
    """A model on one GPU: packed weights, KV cache of max_seqs x max_ctx.

    ``shape`` carries n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn,
    vocab, rms_eps, rope_theta and dtype ("f32" or "bf16"); ``weights`` is
    ``{"embed", "final_norm", "layers": [{attn_norm, wq, ...}]}`` of numpy
    arrays or tensors, ``[out, in]`` row-major.  The values are copied into
    library-owned memory; for bf16 models they must be bf16-representable.
    ``shape.weight_format == "i8_row"`` has the library store the matrices as
    int8 codes with one scale per output row (quantized at creation);
    ``"f8_row"`` as e4m3 codes with a power-of-two scale per row, the norm
    outputs that feed Q/K/V, gate/up and the head quantized likewise.
    """

    def __init__(self, shape, weights: dict, max_seqs: int, max_ctx: int,
                 device: str = "cuda", stream: Optional[torch.cuda.Stream] = None):
        lib = native.load()
        self.shape = shape
        self.device = torch.device(device)
        self.dtype = native.FS_BF16 if shape.dtype == "bf16" else native.FS_F32
        self.torch_dtype = torch.bfloat16 if self.dtype == native.FS_BF16 else torch.float32
        self.vocab = shape.vocab
        self.cfg = FsConfig(shape.n_layers, shape.hidden, shape.n_heads, shape.n_kv_heads,
                            shape.head_dim, shape.ffn, shape.vocab, float(shape.rms_eps),
                            float(shape.rope_theta), self.dtype, int(max_seqs), int(max_ctx),
                            int(getattr(shape, "rope_dim", 0)), int(bool(getattr(shape, "attn_gate", False))),
                            {"i8_row": native.FS_WEIGHTS_I8_ROW, "f8_row": native.FS_WEIGHTS_F8_ROW}.get(
                                getattr(shape, "weight_format", "dtype"), native.FS_WEIGHTS_DTYPE))
        with torch.cuda.device(self.device):
            keep = []

            def up(a):
                t = _to_device(a, self.torch_dtype, self.device)
                keep.append(t)
                return ctypes.c_void_p(t.data_ptr())

            layers = (FsLayerWeights * max(1, shape.n_layers))()
            for i, lw in enumerate(weights["layers"]):
                for k in LAYER_KEYS:
                    setattr(layers[i], k, up(lw[k]))
            w = FsWeights(up(weights["embed"]), up(weights["final_norm"]), layers)
            handle = ctypes.c_void_p()
            st = lib.fs_model_create(ctypes.byref(self.cfg), ctypes.byref(w), _stream_ptr(stream),
                                     ctypes.byref(handle))
            check(st)
            self._h = handle
            del keep
        self._lib = lib

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.fs_model_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ calls
    def prefill(self, tokens: torch.Tensor, slots: Sequence[int],
                logits: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """tokens: int32 [B, S] on the device; returns last-token logits [B, V] fp32."""
        assert tokens.dtype == torch.int32 and tokens.is_contiguous() and tokens.dim() == 2
        B, S = tokens.shape
        if logits is None:
            logits = torch.empty((B, self.vocab), dtype=torch.float32, device=self.device)
        check(self._lib.fs_prefill(self._h, _ptr(tokens), B, S, int_array(slots), _ptr(logits),
                                   _stream_ptr(stream)))
        return logits

    def decode_step(self, tokens: torch.Tensor, positions: Sequence[int], slots: Sequence[int],
                    logits: Optional[torch.Tensor] = None, next_ids: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> None:
        """tokens int32 [B] on the device; fills logits [B, V] and/or next_ids [B]."""
        B = len(slots)
        check(self._lib.fs_decode_step(self._h, _ptr(tokens), int_array(positions), int_array(slots), B,
                                       _ptr(logits), _ptr(next_ids), _stream_ptr(stream)))

    def slot_length(self, slot: int) -> int:
        return int(self._lib.fs_slot_length(self._h, slot))

    def timing(self, enable: bool) -> None:
        """Starts (clearing old records) or stops per-launch event timing."""
        check(self._lib.fs_timing(self._h, 1 if enable else 0))

    def timing_read(self, label: str):
        """(total milliseconds, launches) recorded for one step label."""
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        check(self._lib.fs_timing_read(self._h, label.encode(), ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def kernel_bench(self, label: str, reps: int = 20, slot: int = 0, position: int = 0,
                     stream: Optional[torch.cuda.Stream] = None) -> float:
        """Microseconds per launch of one decode kernel class replayed over all layers."""
        us = ctypes.c_double()
        check(self._lib.fs_kernel_bench(self._h, label.encode(), slot, position, reps, ctypes.byref(us),
                                        _stream_ptr(stream)))
        return us.value

    def decode_trace(self, n: int = 1024):
        """Clock stamps (100 MHz) of the last persistent decode step (FS_DECODE_TRACE=1)."""
        buf = (ctypes.c_int64 * n)()
        check(self._lib.fs_decode_trace(self._h, buf, n))
        return np.array(buf[:], dtype=np.int64)

    def sample(self, logits: torch.Tensor, temperature: float, top_k: int = 0, top_p: float = 1.0,
               u: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """One token per row of fp32 logits [B, V]: temperature -> top-k -> top-p ->
        renormalise -> draw with the caller's uniforms u [B] (fp32 in [0, 1))."""
        assert logits.dtype == torch.float32 and logits.is_contiguous() and logits.dim() == 2
        B, V = logits.shape
        if out is None:
            out = torch.empty((B,), dtype=torch.int32, device=logits.device)
        if u is not None:
            assert u.dtype == torch.float32 and u.is_contiguous() and u.numel() >= B
        sp = native.FsSampling(float(temperature), int(top_k), float(top_p))
        check(self._lib.fs_sample(self._h, _ptr(logits), B, V, ctypes.byref(sp),
                                  _ptr(u) if u is not None else None, _ptr(out), _stream_ptr(stream)))
        return out

    def generate(self, prompt, max_new_tokens: int, eos_ids=(), include_stop_id: bool = False,
                 sampling=None, uniforms: Optional[torch.Tensor] = None, slot: int = 0,
                 stream: Optional[torch.cuda.Stream] = None):
        """Generation for one sequence (fs_generate).  prompt: int32 token IDs
        (host array or device tensor); sampling = (temperature, top_k, top_p) or
        None for greedy, with uniforms fp32 [max_new_tokens] on the device.
        Returns (ids, stop_reason)."""
        if isinstance(prompt, torch.Tensor):
            pt = prompt.to(device=self.device, dtype=torch.int32).contiguous().view(-1)
        else:
            pt = torch.from_numpy(np.ascontiguousarray(np.asarray(prompt, dtype=np.int32))).to(self.device)
        eos = int_array(eos_ids) if len(eos_ids) else None
        sp = native.FsSampling(*[float(sampling[0]), int(sampling[1]), float(sampling[2])]) if sampling else None
        g = native.FsGeneration(int(max_new_tokens), eos, len(eos_ids), int(bool(include_stop_id)),
                                ctypes.pointer(sp) if sp is not None else None,
                                uniforms.data_ptr() if uniforms is not None else None)
        out = (ctypes.c_int32 * max(1, int(max_new_tokens)))()
        n = ctypes.c_int32()
        why = ctypes.c_int32()
        check(self._lib.fs_generate(self._h, _ptr(pt), int(pt.numel()), int(slot), ctypes.byref(g), out,
                                    ctypes.byref(n), ctypes.byref(why), _stream_ptr(stream)))
        return [int(out[i]) for i in range(n.value)], int(why.value)

    def kv_read(self, layer: int, slot: int, kv_head: int, pos0: int, n: int,
                stream: Optional[torch.cuda.Stream] = None):
        k = torch.empty((n, self.shape.head_dim), dtype=self.torch_dtype, device=self.device)
        v = torch.empty_like(k)
        check(self._lib.fs_kv_read(self._h, layer, slot, kv_head, pos0, n, _ptr(k), _ptr(v),
                                   _stream_ptr(stream)))
        return k, v


def quantize_rows_i8(src: torch.Tensor, stream: Optional[torch.cuda.Stream] = None):
    """Per-row int8 codes and fp32 scales of a device matrix [rows, cols] (fp32
    or bf16), by the library's quantizer (fs_quantize_rows_i8)."""
    lib = native.load()
    assert src.dim() == 2 and src.is_contiguous() and src.dtype in (torch.float32, torch.bfloat16)
    rows, cols = src.shape
    codes = torch.empty((rows, cols), dtype=torch.int8, device=src.device)
    scales = torch.empty((rows,), dtype=torch.float32, device=src.device)
    dt = native.FS_BF16 if src.dtype == torch.bfloat16 else native.FS_F32
    check(lib.fs_quantize_rows_i8(_ptr(src), dt, rows, cols, _ptr(codes), _ptr(scales), _stream_ptr(stream)))
    return codes, scales


def quantize_rows_f8(src: torch.Tensor, stream: Optional[torch.cuda.Stream] = None):
    """Per-row e4m3 codes and power-of-two fp32 scales of a device matrix
    [rows, cols] (fp32 or bf16), by the library's quantizer (fs_quantize_rows_f8)."""
    lib = native.load()
    assert src.dim() == 2 and src.is_contiguous() and src.dtype in (torch.float32, torch.bfloat16)
    rows, cols = src.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    scales = torch.empty((rows,), dtype=torch.float32, device=src.device)
    dt = native.FS_BF16 if src.dtype == torch.bfloat16 else native.FS_F32
    check(lib.fs_quantize_rows_f8(_ptr(src), dt, rows, cols, _ptr(codes), _ptr(scales), _stream_ptr(stream)))
    return codes, scales


def gemm_f8(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor,
            out: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """fs_gemm_f8: out[m, n] = a_scales[m] * w_scales[n] * sum_k a[m, k] * w[n, k]
    over e4m3 code matrices a [M, K], w [N, K] (uint8), fp32 out [M, N]."""
    lib = native.load()
    assert a_codes.dtype == torch.uint8 and w_codes.dtype == torch.uint8
    assert a_codes.dim() == 2 and w_codes.dim() == 2 and a_codes.shape[1] == w_codes.shape[1]
    assert a_codes.is_contiguous() and w_codes.is_contiguous()
    M, K = a_codes.shape
    N = w_codes.shape[0]
    assert a_scales.dtype == torch.float32 and a_scales.shape == (M,) and a_scales.is_contiguous()
    assert w_scales.dtype == torch.float32 and w_scales.shape == (N,) and w_scales.is_contiguous()
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    assert out.dtype == torch.float32 and out.shape == (M, N) and out.is_contiguous()
    check(lib.fs_gemm_f8(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, K, _ptr(out),
                         _stream_ptr(stream)))
    return out


def argmax(logits: torch.Tensor, out: Optional[torch.Tensor] = None,
           stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Greedy IDs of each row of fp32 logits [B, V] (lowest ID on ties, -1 if none finite)."""
    lib = native.load()
    assert logits.dtype == torch.float32 and logits.is_contiguous() and logits.dim() == 2
    B, V = logits.shape
    if out is None:
        out = torch.empty((B,), dtype=torch.int32, device=logits.device)
    check(lib.fs_argmax(_ptr(logits), B, V, _ptr(out), _stream_ptr(stream)))
    return out


def sample_noalloc(logits: torch.Tensor, temperature: float, top_k: int = 0, top_p: float = 1.0,
                   u: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """fs_sample_noalloc: Model.sample without a model, on the library's static
    scratch (rows up to FS_SAMPLE_NOALLOC_MAX_ROWS; the library allocates nothing)."""
    lib = native.load()
    assert logits.dtype == torch.float32 and logits.is_contiguous() and logits.dim() == 2
    B, V = logits.shape
    if out is None:
        out = torch.empty((B,), dtype=torch.int32, device=logits.device)
    if u is not None:
        assert u.dtype == torch.float32 and u.is_contiguous() and u.numel() >= B
    sp = native.FsSampling(float(temperature), int(top_k), float(top_p))
    check(lib.fs_sample_noalloc(_ptr(logits), B, V, ctypes.byref(sp), _ptr(u) if u is not None else None,
                                _ptr(out), _stream_ptr(stream)))
    return out
