"""ctypes declarations of libgdn.so's C ABI (include/gdn.h).

Raw entry points take plain integers for device pointers; the torch-facing
wrappers in ops.py marshal tensors into these calls.  Loading fails loudly if
the library has not been built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK = 0
GDN_ERR_NULL = 1
GDN_ERR_INVALID = 2
GDN_ERR_UNSUPPORTED = 3
GDN_ERR_ALIGN = 4
GDN_ERR_ALIAS = 5
GDN_ERR_WORKSPACE = 6
GDN_ERR_HIP = 7
STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_INVALID", 3: "GDN_ERR_UNSUPPORTED",
                4: "GDN_ERR_ALIGN", 5: "GDN_ERR_ALIAS", 6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_HIP"}

GDN_F32 = 0
GDN_BF16 = 1

# Size of the library-owned scratch array used by gdn_chunk_fwd_noalloc.
GDN_NOALLOC_SCRATCH_BYTES = 128 << 20

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in header order
PROTOTYPES = {
    "gdn_conv1d_fwd": (_i32, [_p, _i32, _p, _i32, _p, _i32, _i64, _p, _i32, _p, _p, _p]),
    "gdn_chunk_fwd": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _f32, _i32, _f32,
                             _i32, _i32, _i32, _i32, _i32, _p, _i32, _i64, _p, _p, _p, _i32,
                             _p, _p, _f32, _p, _sz, _p]),
    "gdn_chunk_fwd_noalloc": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _f32, _i32, _f32,
                                     _i32, _i32, _i32, _i32, _i32, _p, _i32, _i64, _p, _p, _p, _i32,
                                     _p, _p, _f32, _p]),
    "gdn_chunk_fwd_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32,
                                            ctypes.POINTER(_sz)]),
    "gdn_recurrent_step": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _f32, _i32, _f32,
                                  _i32, _i32, _i32, _i32, _i32, _p, _i32, _p, _p, _i32, _p, _p,
                                  _f32, _p]),
    "gdn_chunk_fwd_gated": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _i64, _i32, _p, _p,
                                   _f32, _i32, _f32, _i32, _i32, _i32, _i32, _i32, _p, _i32, _i64,
                                   _p, _p, _p, _i32, _p, _p, _f32, _p, _sz, _p]),
    "gdn_recurrent_step_gated": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _i64, _i32, _p,
                                        _p, _f32, _i32, _f32, _i32, _i32, _i32, _i32, _i32, _p, _i32,
                                        _p, _p, _i32, _p, _p, _f32, _p]),
    "gdn_recurrent_verify": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _f32, _i32, _f32,
                                    _i32, _i32, _i32, _i32, _i32, _i32, _p, _i32, _p, _p, _i32, _p,
                                    _i32, _p, _p, _f32, _p]),
    "gdn_conv1d_verify": (_i32, [_p, _i32, _p, _i32, _i32, _i32, _p, _i32, _p, _p, _p, _i32, _p]),
    "gdn_state_rows_copy": (_i32, [_p, _i64, _p, _p, _i64, _p, _i64, _i32, _p]),
    "gdn_conv1d_mixed": (_i32, [_p, _i32, _p, _i32, _p, _i32, _i64, _p, _i32, _p, _p, _p, _p]),
    "gdn_chunk_mixed": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _f32, _i32, _f32,
                               _i32, _i32, _i32, _i32, _i32, _p, _i32, _i64, _p, _i32, _p, _p,
                               _p, _i32, _p, _p, _f32, _p, _sz, _p]),
    "gdn_chunk_bwd": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _f32, _i32, _f32,
                             _i32, _i32, _i32, _i32, _p, _i32, _i64, _p, _p, _p,
                             _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "gdn_chunk_bwd_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i64, ctypes.POINTER(_sz)]),
    "gdn_conv1d_bwd": (_i32, [_p, _i32, _p, _i32, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "gdn_conv1d_bwd_workspace_size": (_i32, [_i32, _i32, _i64, ctypes.POINTER(_sz)]),
    "gdn_mixer_decode_step": (_i32, [_p, _i32, _p, _p, _p, _p, _f32, _i32, _f32, _i32, _i32, _i32, _i32, _i32,
                                     _p, _i32, _p, _p, _i32, _p, _p, _f32, _p]),
    "gdn_gated_rmsnorm": (_i32, [_p, _i32, _p, _i32, _p, _f32, _i64, _i32, _p, _i32, _p]),
    "gdn_status_string": (ctypes.c_char_p, [_i32]),
    "gdn_last_hip_error": (_i32, []),
    "gdn_version": (ctypes.c_char_p, []),
}

_lib = None


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{fn} failed: {self.status_name}{(' ' + detail) if detail else ''}")


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libgdn.so (once) and declare its prototypes."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m gated_deltanet_mixer_causal_amd.build` "
                           "(the HIP library is required; there is no fallback path)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != GDN_OK:
        detail = ""
        if status == GDN_ERR_HIP:
            detail = f"(hipError {load().gdn_last_hip_error()})"
        raise GdnError(fn, status, detail)
