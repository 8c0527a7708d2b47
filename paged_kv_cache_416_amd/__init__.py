"""pkv: paged KV cache and decode attention for AMD MI355X (gfx950).

The compute path is libpkv.so (hand-written HIP kernels and a native host block-pool
allocator behind the C ABI of include/pkv.h). This package is a thin binding over it:
it marshals torch tensors (device memory, the current stream) and host arrays into the
C calls. It has no CPU fallback: if libpkv.so cannot be loaded or built, every call raises.
"""
from ._lib import PkvError, load  # noqa: F401
from .pool import OutOfBlocks, Pool  # noqa: F401

__all__ = ["PkvError", "OutOfBlocks", "Pool", "load", "kernels", "cache"]


def __getattr__(name):
    # torch-dependent modules load on first use
    if name in ("kernels", "cache"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
