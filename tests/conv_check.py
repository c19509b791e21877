"""Build and load tests/libconvcheck.so (the exhaustive conversion checks of
tests/conv_check.hip).  Test infrastructure: built by __graft_entry__.build()
next to the product library, loaded only by tests/test_gpu_conversions.py."""

from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "conv_check.hip")
LIB = os.path.join(HERE, "libconvcheck.so")


def build() -> str:
    import sys

    sys.path.insert(0, ROOT)
    from combine_ep_dispatch_amd import build as b

    tmp = LIB + ".tmp"
    subprocess.run([b.hipcc(), *b.compile_flags(), "-shared", "-o", tmp, SRC], check=True)
    os.replace(tmp, LIB)
    return LIB


def load():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    P, I, U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
    L.conv_check_encode.argtypes = [I, U64, U64, P, P, P, P]
    L.conv_check_e2m1_decode.argtypes = [P, P, P]
    L.conv_check_e2m1_decode_scaled.argtypes = [P, P, P, P]
    L.conv_eval_sw.argtypes = [P, I, P, P, P, P]
    for f in (L.conv_check_encode, L.conv_check_e2m1_decode, L.conv_check_e2m1_decode_scaled, L.conv_eval_sw):
        f.restype = I
    return L
