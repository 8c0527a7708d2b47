"""ctypes declarations of libpkv.so (the C ABI in include/pkv.h). Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_ENOMEM, PKV_ENOSEQ, PKV_EHIP, PKV_EUNSUPPORTED, PKV_EEXIST = 0, -1, -2, -3, -4, -5, -6
PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
PKV_FLAG_SCALAR_GQA = 1
PKV_FLAG_CACHED_KV = 2
PKV_PARTITION_BALANCED = -1

STATUS_NAMES = {0: "PKV_OK", -1: "PKV_EINVAL", -2: "PKV_ENOMEM", -3: "PKV_ENOSEQ", -4: "PKV_EHIP",
                -5: "PKV_EUNSUPPORTED", -6: "PKV_EEXIST"}

_p = ctypes.c_void_p
_i32, _i64, _u32, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)

# name -> (restype, argtypes); every symbol include/pkv.h declares
SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_pool_create": (ctypes.c_int, [_i32, _i32, _pi32, ctypes.POINTER(_p)]),
    "pkv_pool_destroy": (None, [_p]),
    "pkv_pool_num_blocks": (_i32, [_p]),
    "pkv_pool_block_size": (_i32, [_p]),
    "pkv_pool_num_free": (_i32, [_p]),
    "pkv_block_ref_count": (_i32, [_p, _i32]),
    "pkv_seq_add": (ctypes.c_int, [_p, _i64]),
    "pkv_seq_free": (ctypes.c_int, [_p, _i64]),
    "pkv_seq_fork": (ctypes.c_int, [_p, _i64, _i64]),
    "pkv_seq_len": (_i64, [_p, _i64]),
    "pkv_seq_num_blocks": (_i32, [_p, _i64]),
    "pkv_seq_blocks": (_i32, [_p, _i64, _pi32, _i32]),
    "pkv_seq_append": (ctypes.c_int, [_p, _pi64, _pi32, _i32, _pi64, _pi32, _i32, _pi32]),
    "pkv_build_block_tables": (ctypes.c_int, [_p, _pi64, _i32, _i32, _i32, _pi32, _pi32]),
    "pkv_shared_prefix_lens": (ctypes.c_int, [_p, _pi64, _i32, _pi32]),
    "pkv_seq_migrate": (ctypes.c_int, [_p, _p, _pi64, _i32, _pi32, _i32, _pi32]),
    "pkv_prompt_digests": (ctypes.c_int, [_pi32, _i64, _i32, ctypes.POINTER(ctypes.c_uint8), _i64]),
    "pkv_seq_add_prompt": (ctypes.c_int, [_p, _i64, _pi32, _i32, _pi64, _pi32]),
    "pkv_pool_num_cached": (_i32, [_p]),
    "pkv_sim_paged": (ctypes.c_int, [_i32, _i32, _i32, _i32, _pi32, _pi32, _pi32, _i32, _i64, _pi64, _pi64, _pi64]),
    "pkv_sim_contiguous": (ctypes.c_int, [_i64, _i32, _pi32, _pi32, _pi32, _pi32, _i32, _i64, _pi64, _pi64, _pi64]),
    "pkv_reshape_and_cache": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _i64, _p, _i32, _i32, _i32, _i32, _i32,
                                             _p]),
    "pkv_copy_blocks": (ctypes.c_int, [ctypes.POINTER(_p), ctypes.POINTER(_p), _i32, _i64, _i64, _pi32, _i32, _p]),
    "pkv_swap_blocks": (ctypes.c_int, [ctypes.POINTER(_p), ctypes.POINTER(_p), _i32, _i64, _i64, _i64, _pi32, _i32,
                                       _p]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attention_decode": (ctypes.c_int, [_p, _p, _p, _p, _i64, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32,
                                                  _i32, _f32, _i32, _p, _sz, _i32, _u32, _p, _p]),
    "pkv_paged_attention_decode_step": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i64, _p, _i32, _p, _i32, _i32,
                                                       _i32, _i32, _i32, _i32, _f32, _i32, _p, _sz, _i32, _u32, _p,
                                                       _p]),
    "pkv_paged_attention_decode_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _i64, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                                          _i32, _i32, _f32, _i32, _i32, _u32, _p, _p]),
    "pkv_contiguous_attention_decode": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32,
                                                       _f32, _i32, _p, _sz, _i32, _u32, _p]),
    "pkv_read_probe": (ctypes.c_int, [_p, _sz, _p, _p]),
    "pkv_paged_attention_prefill": (ctypes.c_int, [_p, _p, _p, _p, _i64, _p, _i32, _p, _p, _i32, _i32, _i32, _i32,
                                                   _i32, _i32, _i32, _i32, _f32, _i32, _u32, _p]),
}

_lib = None


class PkvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def load(path: str | None = None):
    """Load libpkv.so; build it first if it is not there. Raises if neither works."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        from .build import build
        build()
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(rc):
    if rc != PKV_OK:
        raise PkvError(rc, load().pkv_last_error().decode(errors="replace"))
    return rc
