"""ctypes loader for libepx.so (the HIP kernels behind include/epx.h).

There is no fallback: if the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libepx.so")

EP_OK = 0
EP_EINVAL = -1
EP_ELAUNCH = -2
EP_ENOTSUP = -3
EP_ESCRATCH = -4
EP_NOALLOC_SCRATCH_BYTES = 4 << 20
EP_ZERO_PAD_ROWS = 1
EP_LAYOUT_LOOKBACK = 2
EP_LAYOUT_DIRECT = 4
EP_LAYOUT_BARRIER = 8
EP_LAYOUT_COUNT = 16
EP_FLAG_DROPPED = 1
EP_FLAG_BAD_ID = 2
EP_FLAG_INTERNAL = 4
EP_FLAG_MAP_OVERFLOW = 8
EP_MAX_GROUPS = 2048

# Every symbol include/epx.h declares.
SYMBOLS = ("ep_query", "ep_dispatch_layout", "ep_dispatch", "ep_dispatch_nvfp4", "ep_dispatch_fp8",
           "ep_combine", "ep_dispatch_bwd", "ep_combine_bwd", "ep_combine_bwd_probs",
           "ep_indices_to_multihot", "ep_multihot_to_indices", "ep_dispatch_layout_noalloc",
           "ep_combine_nvfp4", "ep_dispatch_with_layout", "ep_dispatch_nvfp4_with_layout",
           "ep_dispatch_fp8_with_layout", "ep_strerror", "ep_abi_version")


class EpCfg(ctypes.Structure):
    """Mirror of ep_cfg_t."""

    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_segments", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("align", ctypes.c_int32),
                ("seg_capacity", ctypes.c_int32), ("shared_expert", ctypes.c_int32),
                ("src_segment", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("recv_rows", ctypes.c_int64), ("flags", ctypes.c_uint32),
                ("reserved1", ctypes.c_uint32)]


class EpLayout(ctypes.Structure):
    """Mirror of ep_layout_t (device pointers)."""

    _fields_ = [(name, ctypes.c_void_p) for name in
                ("counts", "seg_base", "row_offsets", "scales_offsets", "token_row", "expert_ids",
                 "src_info", "flags")]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m combine_ep_dispatch_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        cfg_p, lay_p = ctypes.POINTER(EpCfg), ctypes.POINTER(EpLayout)
        L.ep_query.argtypes = [cfg_p, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_int32)]
        L.ep_dispatch_layout.argtypes = [cfg_p, P, P, I64, lay_p, P]
        L.ep_dispatch.argtypes = [cfg_p, lay_p, P, P, P]
        L.ep_dispatch_nvfp4.argtypes = [cfg_p, lay_p, P, P, P, P, P]
        L.ep_combine.argtypes = [cfg_p, lay_p, P, P, P, P]
        L.ep_dispatch_bwd.argtypes = [cfg_p, lay_p, P, P, P]
        L.ep_combine_bwd.argtypes = [cfg_p, lay_p, P, P, P, P]
        L.ep_combine_bwd_probs.argtypes = [cfg_p, lay_p, P, P, P, P]
        L.ep_dispatch_fp8.argtypes = [cfg_p, lay_p, P, P, P, P]
        L.ep_indices_to_multihot.argtypes = [cfg_p, P, P, P, P, P]
        L.ep_multihot_to_indices.argtypes = [cfg_p, P, P, P, P, P, P]
        L.ep_dispatch_layout_noalloc.argtypes = [cfg_p, P, lay_p, P]
        L.ep_combine_nvfp4.argtypes = [cfg_p, lay_p, P, P, P, P, P, P]
        L.ep_dispatch_with_layout.argtypes = [cfg_p, P, P, I64, lay_p, P, P, P]
        L.ep_dispatch_nvfp4_with_layout.argtypes = [cfg_p, P, P, I64, lay_p, P, P, P, P, P]
        L.ep_dispatch_fp8_with_layout.argtypes = [cfg_p, P, P, I64, lay_p, P, P, P, P]
        for name in SYMBOLS[:16]:
            getattr(L, name).restype = I
        L.ep_strerror.argtypes = [I]
        L.ep_strerror.restype = ctypes.c_char_p
        L.ep_abi_version.argtypes = []
        L.ep_abi_version.restype = I
        _lib = L
    return _lib
