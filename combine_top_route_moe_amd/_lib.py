"""ctypes loader for ``libmoe.so``, the C-ABI library of HIP kernels.

The library is built in-tree by ``_build.build()``; loading fails loudly when
it is missing, so nothing ever falls back to a CPU path.
"""

from __future__ import annotations

import ctypes
import os

from ._build import LIB

_c_int, _c_i64, _c_size, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes), mirroring include/moe.h
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_c_int]),
    "moe_device_check": (_c_int, [_c_int]),
    "moe_route": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "moe_permute_capacity": (_c_i64, [_c_int, _c_int, _c_int, _c_int]),
    "moe_permute_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "moe_permute": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                             _c_int, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp, _vp]),
    "moe_permute_noalloc_scratch_bytes": (_c_size, []),
    "moe_permute_noalloc": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_int, _c_int, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp]),
    "moe_grouped_ffn_workspace_bytes": (_c_size, [_c_i64, _c_int, _c_int, _c_int]),
    "moe_grouped_ffn": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                 _c_i64, _c_int, _vp, _c_size, _vp, _vp]),
    "moe_pack_ffn_weights": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "moe_grouped_ffn_fp8": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _c_i64, _c_int, _vp, _c_size, _vp, _vp]),
    "moe_pack_ffn_weights_fp8": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                          _c_int, _vp]),
    "moe_quant_rows_fp8": (_c_int, [_vp, _c_i64, _c_int, _vp, _vp, _vp, _c_i64, _vp]),
    "moe_grouped_ffn_w8a8_workspace_bytes": (_c_size, [_c_i64, _c_int, _c_int, _c_int]),
    "moe_grouped_ffn_w8a8": (_c_int, [_vp, _vp, _c_i64, _vp, _c_int, _vp, _vp, _c_int, _c_int,
                                      _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_int, _vp,
                                      _c_size, _vp, _vp]),
    "moe_fake_quant_rows": (_c_int, [_vp, _vp, _c_i64, _c_int, _vp, _c_int, _c_int, _vp, _vp,
                                     _vp, _vp]),
    "moe_scale_from_amax": (_c_int, [_vp, _vp, _c_int, _vp]),
    "moe_combine": (_c_int, [_vp, _c_i64, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                             _vp]),
    "moe_combine_check": (_c_int, [_vp, _c_i64, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                                   _vp]),
    "moe_copy_bytes": (_c_int, [_vp, _vp, _c_size, _vp]),
    "moe_read_bytes": (_c_int, [_vp, _c_size, _vp, _vp]),
}

_lib = None


def load(path: str = LIB) -> ctypes.CDLL:
    """Load the library once and attach the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library not found at {path}; build it first with "
            "`python -m combine_top_route_moe_amd._build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MoEError(RuntimeError):
    """A negative status returned by the C ABI."""

    def __init__(self, fn: str, status: int):
        text = load().moe_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise MoEError(fn, status)
