"""ctypes binding of libfs.so (the C ABI in include/fs.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind these calls.  Importing this module fails loudly when the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfs.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "fs.h")

FS_OK = 0
FS_ERR_INVALID_ARG = -1
FS_ERR_OOM = -2
FS_ERR_HIP = -3
FS_ERR_CAPACITY = -4
FS_ERR_UNSUPPORTED = -5
STATUS_NAMES = {0: "FS_OK", -1: "FS_ERR_INVALID_ARG", -2: "FS_ERR_OOM", -3: "FS_ERR_HIP",
                -4: "FS_ERR_CAPACITY", -5: "FS_ERR_UNSUPPORTED"}
FS_F32 = 0
FS_BF16 = 1
FS_WEIGHTS_DTYPE = 0
FS_WEIGHTS_I8_ROW = 1
FS_WEIGHTS_F8_ROW = 2

LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
                "mlp_norm", "w_gate", "w_up", "w_down")


class FsConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("attn_gate", ctypes.c_int32),
                ("weight_format", ctypes.c_int32)]


class FsLayerWeights(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in LAYER_FIELDS]


class FsWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(FsLayerWeights))]


class FsSampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float)]


class FsGeneration(ctypes.Structure):
    _fields_ = [("max_new_tokens", ctypes.c_int32), ("eos_ids", ctypes.POINTER(ctypes.c_int32)),
                ("n_eos", ctypes.c_int32), ("include_stop_id", ctypes.c_int32),
                ("sampling", ctypes.POINTER(FsSampling)), ("uniforms", ctypes.c_void_p)]


FS_STOP_NONE, FS_STOP_EOS, FS_STOP_BUDGET, FS_STOP_CONTEXT = 0, 1, 2, 3


class FsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None


def load() -> ctypes.CDLL:
    """Loads libfs.so from the package directory (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m dense_gqa_transformer_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.fs_model_create.argtypes = [ctypes.POINTER(FsConfig), ctypes.POINTER(FsWeights), P, ctypes.POINTER(P)]
    lib.fs_model_create.restype = ctypes.c_int
    lib.fs_model_destroy.argtypes = [P]
    lib.fs_model_destroy.restype = None
    lib.fs_prefill.argtypes = [P, P, i32, i32, ctypes.POINTER(i32), P, P]
    lib.fs_prefill.restype = ctypes.c_int
    lib.fs_decode_step.argtypes = [P, P, ctypes.POINTER(i32), ctypes.POINTER(i32), i32, P, P, P]
    lib.fs_decode_step.restype = ctypes.c_int
    lib.fs_argmax.argtypes = [P, i32, i32, P, P]
    lib.fs_argmax.restype = ctypes.c_int
    lib.fs_quantize_rows_i8.argtypes = [P, i32, i32, i32, P, P, P]
    lib.fs_quantize_rows_i8.restype = ctypes.c_int
    lib.fs_quantize_rows_f8.argtypes = [P, i32, i32, i32, P, P, P]
    lib.fs_quantize_rows_f8.restype = ctypes.c_int
    lib.fs_gemm_f8.argtypes = [P, P, P, P, i32, i32, i32, P, P]
    lib.fs_gemm_f8.restype = ctypes.c_int
    lib.fs_sample.argtypes = [P, P, i32, i32, ctypes.POINTER(FsSampling), P, P, P]
    lib.fs_sample.restype = ctypes.c_int
    lib.fs_sample_noalloc.argtypes = [P, i32, i32, ctypes.POINTER(FsSampling), P, P, P]
    lib.fs_sample_noalloc.restype = ctypes.c_int
    lib.fs_generate.argtypes = [P, P, i32, i32, ctypes.POINTER(FsGeneration), ctypes.POINTER(i32),
                                ctypes.POINTER(i32), ctypes.POINTER(i32), P]
    lib.fs_generate.restype = ctypes.c_int
    lib.fs_slot_length.argtypes = [P, i32]
    lib.fs_slot_length.restype = i32
    lib.fs_kv_read.argtypes = [P, i32, i32, i32, i32, i32, P, P, P]
    lib.fs_kv_read.restype = ctypes.c_int
    lib.fs_timing.argtypes = [P, i32]
    lib.fs_timing.restype = ctypes.c_int
    lib.fs_timing_read.argtypes = [P, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_int64)]
    lib.fs_timing_read.restype = ctypes.c_int
    lib.fs_kernel_bench.argtypes = [P, ctypes.c_char_p, i32, i32, i32, ctypes.POINTER(ctypes.c_double), P]
    lib.fs_kernel_bench.restype = ctypes.c_int
    lib.fs_decode_trace.argtypes = [P, ctypes.POINTER(ctypes.c_int64), i32]
    lib.fs_decode_trace.restype = ctypes.c_int
    lib.fs_last_error.argtypes = []
    lib.fs_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().fs_last_error().decode()


def check(status: int) -> None:
    if status != FS_OK:
        raise FsError(status, last_error())


def header_functions(path: str = HEADER):
    """Names of the functions include/fs.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(fs_\w+)\s*\(", text, re.M)))


def int_array(values):
    vals = [int(v) for v in values]
    return (ctypes.c_int32 * len(vals))(*vals)
