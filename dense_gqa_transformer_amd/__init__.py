"""Dense GQA decoder forward pass (Qwen3-0.6B kind) on MI355X / gfx950.

The work runs in libfs.so (hand-written HIP kernels behind the C ABI in
include/fs.h); this package is its ctypes binding.
"""
from . import native  # noqa: F401

__all__ = ["native", "Model", "argmax"]


def __getattr__(name):
    if name in ("Model", "argmax"):
        from . import model
        return getattr(model, name)
    raise AttributeError(name)
