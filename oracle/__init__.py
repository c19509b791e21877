"""CPU oracle for MoE expert-parallel dispatch and combine.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``smoke()`` in
``__graft_entry__.py`` and by the ``cpu_baseline`` leg of ``bench.py``;
never by the product package.  The arithmetic lives in ``oracle.c`` (plain,
single-threaded C built with gcc, no FMA contraction); this module only
builds it and marshals numpy arrays through ctypes.

Every function returns freshly allocated numpy arrays.  Buffers that the
oracle leaves untouched (rows past a segment's used rows) are pre-filled
with sentinels so that a test can tell "not written" apart from a value.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the loader at a deliberately mutated build of oracle.c
# (to show that the pins catch planted mistakes); never set in normal runs.
_LIB_OVERRIDE = os.environ.get("EPX_ORACLE_LIB_OVERRIDE")

SENTINEL_I32 = np.int32(-0x5A5A5A5B)   # never a valid row, id or token
SENTINEL_U16 = np.uint16(0x7FA5)        # a NaN payload nothing computes
SENTINEL_U8 = np.uint8(0xA5)

FLAG_DROPPED = 1
FLAG_BAD_ID = 2


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
               "-Wall", "-Wextra", "-shared", "-fPIC", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("S", ctypes.c_int32), ("K", ctypes.c_int32), ("A", ctypes.c_int32),
                ("C", ctypes.c_int32), ("shared", ctypes.c_int32),
                ("src_seg", ctypes.c_int32), ("recv_rows", ctypes.c_int64)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.orc_layout.restype = ctypes.c_int
        lib.orc_layout.argtypes = [P] * 10
        for name in ("orc_dispatch", "orc_dispatch_bwd"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [P] * 4
        for name in ("orc_combine", "orc_combine_bwd"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [P] * 5
        lib.orc_combine_bwd_probs.restype = None
        lib.orc_combine_bwd_probs.argtypes = [P] * 5
        lib.orc_combine_nvfp4.restype = None
        lib.orc_combine_nvfp4.argtypes = [P] * 7
        lib.orc_indices_to_multihot.restype = None
        lib.orc_indices_to_multihot.argtypes = [P] * 5
        lib.orc_multihot_to_indices.restype = ctypes.c_int32
        lib.orc_multihot_to_indices.argtypes = [P] * 5
        lib.orc_fp8_row.restype = None
        lib.orc_fp8_row.argtypes = [ctypes.c_int32, P, P, P]
        lib.orc_dispatch_fp8.restype = None
        lib.orc_dispatch_fp8.argtypes = [P] * 5
        lib.orc_e4m3_encode_signed.restype = ctypes.c_uint8
        lib.orc_e4m3_encode_signed.argtypes = [ctypes.c_float]
        lib.orc_dispatch_nvfp4.restype = None
        lib.orc_dispatch_nvfp4.argtypes = [P] * 6
        lib.orc_nvfp4_row.restype = None
        lib.orc_nvfp4_row.argtypes = [ctypes.c_int32, P, P, P, P]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_decode.restype = ctypes.c_float
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_e2m1_encode.restype = ctypes.c_uint8
        lib.orc_e2m1_encode.argtypes = [ctypes.c_float]
        lib.orc_e2m1_decode.restype = ctypes.c_float
        lib.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        lib.orc_bf16_rne.restype = ctypes.c_uint16
        lib.orc_bf16_rne.argtypes = [ctypes.c_float]
        lib.orc_bf16_to_f32.restype = ctypes.c_float
        lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        _lib = lib
    return _lib


@dataclass
class Cfg:
    """Problem description (mirrors the fields the pages' problem statement names)."""

    T: int
    H: int
    E: int
    S: int
    K: int
    A: int = 1
    C: int = 0
    shared: int = 0
    src_seg: int = 0
    recv_rows: int = 0

    @property
    def Kp(self) -> int:
        return self.K + self.shared

    @property
    def G(self) -> int:
        return self.E // self.S + self.shared

    def _c(self) -> _Cfg:
        return _Cfg(self.T, self.H, self.E, self.S, self.K, self.A, self.C, self.shared,
                    self.src_seg, self.recv_rows)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def layout(cfg: Cfg, topk_ids: np.ndarray) -> dict:
    lib = _load()
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32).reshape(cfg.T, cfg.K)
    NG, G1 = cfg.S * cfg.G, cfg.S * (cfg.G + 1)
    out = {
        "counts": np.full(NG, SENTINEL_I32, np.int32),
        "row_offsets": np.full(G1, SENTINEL_I32, np.int32),
        "scales_offsets": np.full(G1, SENTINEL_I32, np.int32),
        "seg_base": np.full(cfg.S + 1, SENTINEL_I32, np.int32),
        "token_row": np.full(cfg.T * cfg.Kp, SENTINEL_I32, np.int32),
        "expert_ids": np.full(cfg.recv_rows, SENTINEL_I32, np.int32),
        "src_info": np.full(2 * cfg.recv_rows, SENTINEL_I32, np.int32),
        "flags": np.full(1, SENTINEL_I32, np.int32),
    }
    c = cfg._c()
    rc = lib.orc_layout(ctypes.byref(c), _ptr(ids), *(_ptr(out[k]) for k in (
        "counts", "row_offsets", "scales_offsets", "seg_base", "token_row", "expert_ids",
        "src_info", "flags")))
    if rc != 0:
        raise ValueError("oracle layout: a row falls outside recv_rows")
    out["token_row"] = out["token_row"].reshape(cfg.T, cfg.Kp)
    out["src_info"] = out["src_info"].reshape(cfg.recv_rows, 2)
    out["row_offsets"] = out["row_offsets"].reshape(cfg.S, cfg.G + 1)
    out["scales_offsets"] = out["scales_offsets"].reshape(cfg.S, cfg.G + 1)
    out["counts"] = out["counts"].reshape(cfg.S, cfg.G)
    return out


def dispatch(cfg: Cfg, token_row: np.ndarray, x: np.ndarray) -> np.ndarray:
    lib = _load()
    recv = np.full((cfg.recv_rows, cfg.H), SENTINEL_U16, np.uint16)
    tr = np.ascontiguousarray(token_row, np.int32)
    xx = np.ascontiguousarray(x, np.uint16)
    lib.orc_dispatch(ctypes.byref(cfg._c()), _ptr(tr), _ptr(xx), _ptr(recv))
    return recv


def dispatch_nvfp4(cfg: Cfg, token_row: np.ndarray, x: np.ndarray):
    lib = _load()
    codes = np.full((cfg.recv_rows, cfg.H // 2), SENTINEL_U8, np.uint8)
    scales = np.full((cfg.recv_rows, cfg.H // 16), SENTINEL_U8, np.uint8)
    rowscale = np.full(cfg.recv_rows, SENTINEL_U16, np.uint16)
    tr = np.ascontiguousarray(token_row, np.int32)
    xx = np.ascontiguousarray(x, np.uint16)
    lib.orc_dispatch_nvfp4(ctypes.byref(cfg._c()), _ptr(tr), _ptr(xx), _ptr(codes),
                           _ptr(scales), _ptr(rowscale))
    return codes, scales, rowscale


SENTINEL_F32_BITS = np.uint32(0x7FA5A5A5)  # a NaN payload nothing computes
FLAG_MAP_OVERFLOW = 8


def indices_to_multihot(cfg: Cfg, topk_ids: np.ndarray, probs: Optional[np.ndarray]):
    """(routing_map uint8 [T, E], dense_probs float32 [T, E] or None)."""
    lib = _load()
    ids = np.ascontiguousarray(topk_ids, np.int32).reshape(cfg.T, cfg.K)
    rm = np.full((cfg.T, cfg.E), SENTINEL_U8, np.uint8)
    dp = None if probs is None else np.full((cfg.T, cfg.E), np.nan, np.float32)
    pp = None if probs is None else np.ascontiguousarray(probs, np.float32)
    lib.orc_indices_to_multihot(ctypes.byref(cfg._c()), _ptr(ids), _ptr(pp), _ptr(rm), _ptr(dp))
    return rm, dp


def multihot_to_indices(cfg: Cfg, routing_map: np.ndarray, dense_probs: Optional[np.ndarray]):
    """(topk_ids int32 [T, K], probs float32 [T, K], flags)."""
    lib = _load()
    rm = np.ascontiguousarray(routing_map, np.uint8).reshape(cfg.T, cfg.E)
    dp = None if dense_probs is None else np.ascontiguousarray(dense_probs, np.float32)
    ids = np.full((cfg.T, cfg.K), SENTINEL_I32, np.int32)
    pr = np.full((cfg.T, cfg.K), np.nan, np.float32)
    f = lib.orc_multihot_to_indices(ctypes.byref(cfg._c()), _ptr(rm), _ptr(dp), _ptr(ids), _ptr(pr))
    return ids, pr, int(f)


def fp8_row(x_row: np.ndarray):
    """FP8 dispatch of one token (bf16 bits [H]) -> (codes u8 [H], scales f32 [H/128])."""
    lib = _load()
    xx = np.ascontiguousarray(x_row, np.uint16)
    H = xx.shape[0]
    codes = np.zeros(H, np.uint8)
    scales = np.zeros(H // 128, np.float32)
    lib.orc_fp8_row(H, _ptr(xx), _ptr(codes), _ptr(scales))
    return codes, scales


def dispatch_fp8(cfg: Cfg, token_row: np.ndarray, x: np.ndarray):
    lib = _load()
    codes = np.full((cfg.recv_rows, cfg.H), SENTINEL_U8, np.uint8)
    scales = np.full((cfg.recv_rows, cfg.H // 128), SENTINEL_F32_BITS, np.uint32).view(np.float32)
    tr = np.ascontiguousarray(token_row, np.int32)
    xx = np.ascontiguousarray(x, np.uint16)
    lib.orc_dispatch_fp8(ctypes.byref(cfg._c()), _ptr(tr), _ptr(xx), _ptr(codes), _ptr(scales))
    return codes, scales


def nvfp4_row(x_row: np.ndarray):
    """Quantize one token (bf16 bits [H]) -> (codes [H/2], scales [H/16], rowscale bits)."""
    lib = _load()
    xx = np.ascontiguousarray(x_row, np.uint16)
    H = xx.shape[0]
    codes = np.zeros(H // 2, np.uint8)
    scales = np.zeros(H // 16, np.uint8)
    rs = np.zeros(1, np.uint16)
    lib.orc_nvfp4_row(H, _ptr(xx), _ptr(codes), _ptr(scales), _ptr(rs))
    return codes, scales, int(rs[0])


def combine(cfg: Cfg, token_row: np.ndarray, out: np.ndarray, probs: Optional[np.ndarray]):
    lib = _load()
    y = np.full((cfg.T, cfg.H), SENTINEL_U16, np.uint16)
    tr = np.ascontiguousarray(token_row, np.int32)
    oo = np.ascontiguousarray(out, np.uint16)
    pp = None if probs is None else np.ascontiguousarray(probs, np.float32)
    lib.orc_combine(ctypes.byref(cfg._c()), _ptr(tr), _ptr(oo), _ptr(pp), _ptr(y))
    return y


def combine_nvfp4(cfg: Cfg, token_row: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                  rowscale: np.ndarray, probs: Optional[np.ndarray]) -> np.ndarray:
    """Combine over NVFP4 expert-output rows (codes [R, H/2], E4M3 scales
    [R, H/16], bf16 rowscale bits [R]) -> y bf16 bits [T, H]."""
    lib = _load()
    y = np.full((cfg.T, cfg.H), SENTINEL_U16, np.uint16)
    tr = np.ascontiguousarray(token_row, np.int32)
    cc = np.ascontiguousarray(codes, np.uint8)
    ss = np.ascontiguousarray(scales, np.uint8)
    rs = np.ascontiguousarray(rowscale, np.uint16)
    pp = None if probs is None else np.ascontiguousarray(probs, np.float32)
    lib.orc_combine_nvfp4(ctypes.byref(cfg._c()), _ptr(tr), _ptr(cc), _ptr(ss), _ptr(rs), _ptr(pp), _ptr(y))
    return y


def dispatch_bwd(cfg: Cfg, token_row: np.ndarray, grad_recv: np.ndarray) -> np.ndarray:
    lib = _load()
    gx = np.full((cfg.T, cfg.H), SENTINEL_U16, np.uint16)
    tr = np.ascontiguousarray(token_row, np.int32)
    gr = np.ascontiguousarray(grad_recv, np.uint16)
    lib.orc_dispatch_bwd(ctypes.byref(cfg._c()), _ptr(tr), _ptr(gr), _ptr(gx))
    return gx


def combine_bwd(cfg: Cfg, token_row: np.ndarray, grad_y: np.ndarray,
                probs: Optional[np.ndarray]) -> np.ndarray:
    lib = _load()
    go = np.full((cfg.recv_rows, cfg.H), SENTINEL_U16, np.uint16)
    tr = np.ascontiguousarray(token_row, np.int32)
    gy = np.ascontiguousarray(grad_y, np.uint16)
    pp = None if probs is None else np.ascontiguousarray(probs, np.float32)
    lib.orc_combine_bwd(ctypes.byref(cfg._c()), _ptr(tr), _ptr(gy), _ptr(pp), _ptr(go))
    return go


def combine_bwd_probs(cfg: Cfg, token_row: np.ndarray, grad_y: np.ndarray,
                      out: np.ndarray) -> np.ndarray:
    """d loss / d probs [T, K] in float64 (the definition)."""
    lib = _load()
    gp = np.full((cfg.T, cfg.K), np.nan, np.float64)
    tr = np.ascontiguousarray(token_row, np.int32)
    gy = np.ascontiguousarray(grad_y, np.uint16)
    oo = np.ascontiguousarray(out, np.uint16)
    lib.orc_combine_bwd_probs(ctypes.byref(cfg._c()), _ptr(tr), _ptr(gy), _ptr(oo), _ptr(gp))
    return gp


def e4m3_encode(s: float) -> int:
    return int(_load().orc_e4m3_encode(float(s)))


def e4m3_decode(c: int) -> float:
    return float(_load().orc_e4m3_decode(int(c)))


def e2m1_encode(v: float) -> int:
    return int(_load().orc_e2m1_encode(float(v)))


def e2m1_decode(c: int) -> float:
    return float(_load().orc_e2m1_decode(int(c)))


def bf16_rne(f: float) -> int:
    return int(_load().orc_bf16_rne(float(f)))


def bf16_to_f32(h: int) -> float:
    return float(_load().orc_bf16_to_f32(int(h)))


def min_recv_rows(cfg: Cfg) -> int:
    """Rows a caller must allocate without reading counts (worst case over ids)."""
    if cfg.C > 0:
        return cfg.S * cfg.C
    routed = cfg.T * cfg.Kp
    return routed + min(routed, cfg.E + cfg.shared) * (cfg.A - 1)
