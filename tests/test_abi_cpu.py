"""Host-side checks of the C ABI library: it loads, exports every declared
function, and rejects bad arguments before touching a device."""
import ctypes

import pytest

from dense_gqa_transformer_amd import native


def test_library_exports_every_declared_symbol():
    lib = native.load()
    names = native.header_functions()
    assert set(names) == {"fs_model_create", "fs_model_destroy", "fs_prefill", "fs_decode_step",
                          "fs_argmax", "fs_slot_length", "fs_kv_read", "fs_last_error",
                          "fs_timing", "fs_timing_read", "fs_kernel_bench", "fs_sample", "fs_generate",
                          "fs_quantize_rows_i8", "fs_sample_noalloc", "fs_decode_trace", "fs_quantize_rows_f8",
                          "fs_gemm_f8"}
    for n in names:
        assert hasattr(lib, n), n


def test_argument_errors_without_device():
    lib = native.load()
    assert lib.fs_argmax(None, 1, 10, None, None) == native.FS_ERR_INVALID_ARG
    assert "NULL" in native.last_error()
    fake = ctypes.c_void_p(0x1000)
    assert lib.fs_argmax(fake, 0, 10, fake, None) == native.FS_ERR_INVALID_ARG
    assert lib.fs_argmax(fake, 2, -1, fake, None) == native.FS_ERR_INVALID_ARG
    assert lib.fs_slot_length(None, 0) == -1
    assert lib.fs_prefill(None, None, 1, 1, None, None, None) == native.FS_ERR_INVALID_ARG
    assert lib.fs_decode_step(None, None, None, None, 1, None, None, None) == native.FS_ERR_INVALID_ARG
    assert lib.fs_kv_read(None, 0, 0, 0, 0, 1, None, None, None) == native.FS_ERR_INVALID_ARG
    assert lib.fs_timing(None, 1) == native.FS_ERR_INVALID_ARG
    sp = native.FsSampling(1.0, 0, 1.0)
    assert lib.fs_sample(None, fake, 1, 10, ctypes.byref(sp), fake, fake, None) == native.FS_ERR_INVALID_ARG
    ns = lib.fs_sample_noalloc
    assert ns(None, 1, 10, ctypes.byref(sp), fake, fake, None) == native.FS_ERR_INVALID_ARG
    assert ns(fake, 0, 10, ctypes.byref(sp), fake, fake, None) == native.FS_ERR_INVALID_ARG
    assert ns(fake, 65, 10, ctypes.byref(sp), fake, fake, None) == native.FS_ERR_CAPACITY
    assert "static" in native.last_error()
    assert ns(fake, 2, 10, ctypes.byref(native.FsSampling(1.0, 0, 1.5)), fake, fake, None) == native.FS_ERR_INVALID_ARG
    assert ns(fake, 2, 10, ctypes.byref(sp), None, fake, None) == native.FS_ERR_INVALID_ARG
    g = native.FsGeneration(4, None, 0, 0, None, None)
    n, why = ctypes.c_int32(), ctypes.c_int32()
    out = (ctypes.c_int32 * 4)()
    assert lib.fs_generate(None, fake, 3, 0, ctypes.byref(g), out, ctypes.byref(n), ctypes.byref(why),
                           None) == native.FS_ERR_INVALID_ARG
    q = lib.fs_quantize_rows_i8
    assert q(None, native.FS_BF16, 4, 64, fake, fake, None) == native.FS_ERR_INVALID_ARG
    assert q(fake, 9, 4, 64, fake, fake, None) == native.FS_ERR_UNSUPPORTED
    assert q(fake, native.FS_BF16, 0, 64, fake, fake, None) == native.FS_ERR_INVALID_ARG
    assert q(fake, native.FS_BF16, 4, 60, fake, fake, None) == native.FS_ERR_INVALID_ARG
    assert q(ctypes.c_void_p(0x1008), native.FS_BF16, 4, 64, fake, fake, None) == native.FS_ERR_INVALID_ARG
    gf = lib.fs_gemm_f8
    assert gf(None, fake, fake, fake, 4, 8, 64, fake, None) == native.FS_ERR_INVALID_ARG
    assert gf(fake, fake, fake, fake, 0, 8, 64, fake, None) == native.FS_ERR_INVALID_ARG
    assert gf(fake, fake, fake, fake, 4, 8, 96, fake, None) == native.FS_ERR_INVALID_ARG      # K % 64
    assert gf(fake, fake, fake, fake, 4, 12, 64, fake, None) == native.FS_ERR_INVALID_ARG     # N % 8
    assert gf(ctypes.c_void_p(0x1008), fake, fake, fake, 4, 8, 64, fake, None) == native.FS_ERR_INVALID_ARG


def _cfg(**kw):
    base = dict(n_layers=1, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn=768, vocab=4096,
                rms_eps=1e-6, rope_theta=1e6, dtype=native.FS_F32, max_seqs=1, max_ctx=32,
                rope_dim=0, attn_gate=0, weight_format=0)
    base.update(kw)
    return native.FsConfig(*[base[f] for f, _ in native.FsConfig._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), native.FS_ERR_UNSUPPORTED),
    (dict(head_dim=96), native.FS_ERR_UNSUPPORTED),
    (dict(n_heads=6, n_kv_heads=4), native.FS_ERR_INVALID_ARG),
    (dict(n_heads=12, n_kv_heads=4), native.FS_ERR_UNSUPPORTED),
    (dict(hidden=200), native.FS_ERR_UNSUPPORTED),
    (dict(hidden=8192), native.FS_ERR_UNSUPPORTED),
    (dict(max_ctx=0), native.FS_ERR_INVALID_ARG),
    (dict(vocab=0), native.FS_ERR_INVALID_ARG),
    (dict(weight_format=3), native.FS_ERR_UNSUPPORTED),
])
def test_create_rejects_bad_config(kw, status):
    lib = native.load()
    cfg = _cfg(**kw)
    w = native.FsWeights(None, None, None)
    out = ctypes.c_void_p()
    assert lib.fs_model_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(out)) == status
    assert out.value is None
    assert native.last_error() != ""


def test_create_rejects_null_weights():
    lib = native.load()
    cfg = _cfg()
    w = native.FsWeights(None, None, None)
    out = ctypes.c_void_p()
    assert lib.fs_model_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(out)) == native.FS_ERR_INVALID_ARG
    assert lib.fs_model_create(ctypes.byref(cfg), None, None, ctypes.byref(out)) == native.FS_ERR_INVALID_ARG
