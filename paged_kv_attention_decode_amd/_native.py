"""ctypes loader for libpkv.so (the C ABI declared in include/pkv.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

# Every symbol include/pkv.h declares, with its ctypes signature.
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "pkv_kv_append": (_i, [_vp, _vp, _i, _vp, _i, _vp, _i, _vp, _vp, _i, _i, _i, _i, _vp]),
    "pkv_kv_append_fp8": (_i, [_vp, _vp, _i, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "pkv_kv_append_int8": (_i, [_vp, _vp, _i, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "pkv_kv_append_int4": (_i, [_vp, _vp, _i, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "pkv_decode_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "pkv_paged_attn_decode": (_i, [_vp, _i, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i, _i,
                                   _f, _i, _vp, _i, _vp, _sz, _vp]),
    "pkv_paged_attn_decode_fp8": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i,
                                       _i, _i, _f, _i, _vp, _i, _vp, _sz, _vp]),
    "pkv_paged_attn_decode_int8": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i,
                                        _i, _i, _f, _i, _vp, _i, _vp, _sz, _vp]),
    "pkv_paged_attn_decode_int4": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i,
                                        _i, _i, _f, _i, _vp, _i, _vp, _sz, _vp]),
    "pkv_decode_step": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i,
                             _i, _f, _i, _vp, _i, _vp, _sz, _vp]),
    "pkv_decode_step_quant": (_i, [_vp, _i, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i,
                                   _i, _i, _f, _i, _vp, _i, _vp, _sz, _vp]),
    "pkv_decode_step_noalloc": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i,
                                     _i, _i, _f, _i, _vp, _i, _vp]),
    "pkv_kv_append_chunk": (_i, [_vp, _vp, _i, _vp, _i, _vp, _i, _vp, _i, _vp, _vp, _i, _i, _i, _i, _vp]),
    "pkv_paged_prefill": (_i, [_vp, _i, _vp, _i, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _f,
                               _vp, _i, _vp]),
    "pkv_paged_prefill_fp8": (_i, [_vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i,
                                   _f, _vp, _i, _vp]),
    "pkv_alloc_pages": (_i, [_vp, _i, _vp, _i, _i, _vp, _vp, _i, _vp]),
    "pkv_release_pages": (_i, [_vp, _vp, _i, _vp, _i, _i, _i, _vp, _vp, _i, _vp]),
    "pkv_debug_gather": (_i, [_vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "pkv_debug_read_probe": (_i, [_vp, _sz, _vp, _vp]),
    "pkv_strerror": (ctypes.c_char_p, [_i]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (_i, []),
}

_lib = None


class NativeLibraryMissing(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libpkv.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NativeLibraryMissing(
                f"{LIB_PATH} is missing: build it with "
                "`python -m paged_kv_attention_decode_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
