"""Pins of the oracle's number formats against their published definitions.

E2M1 (OCP Microscaling element format): 1 sign, 2 exponent bits (bias 1), 1
mantissa bit; exponent field 0 is subnormal.  E4M3 (OCP 8-bit floating
point, "fn" variant): bias 7, largest finite 448, no infinities.  bfloat16:
upper half of an IEEE binary32, round to nearest-even.  The NVFP4 payload of
the MAX DistributedEPDispatchBlockScaledNVDynGlobalScales page is built from
these three formats.
"""

import numpy as np
import pytest
import torch


def e2m1_from_fields(code: int) -> float:
    """Value of an E2M1 code straight from its bit fields."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def test_e2m1_decode_matches_bit_fields(orc):
    for c in range(16):
        assert orc.e2m1_decode(c) == e2m1_from_fields(c), c


def test_e2m1_encode_roundtrips_every_code(orc):
    for c in range(16):
        v = e2m1_from_fields(c)
        if c == 8:  # -0.0 keeps its sign bit
            assert orc.e2m1_encode(-0.0) == 8
            continue
        assert orc.e2m1_encode(v) == c, (c, v)


def test_e2m1_ties_go_to_even_code(orc):
    mags = sorted({abs(e2m1_from_fields(c)) for c in range(8)})
    for lo, hi in zip(mags[:-1], mags[1:]):
        mid = (lo + hi) / 2
        c_lo = [c for c in range(8) if e2m1_from_fields(c) == lo][0]
        c_hi = [c for c in range(8) if e2m1_from_fields(c) == hi][0]
        want = c_lo if c_lo % 2 == 0 else c_hi
        assert orc.e2m1_encode(mid) == want, (lo, hi)
        assert orc.e2m1_encode(-mid) == want | 8
        # one float ulp either side of the tie leaves the tie rule alone
        assert orc.e2m1_encode(np.nextafter(np.float32(mid), np.float32(0))) == c_lo
        assert orc.e2m1_encode(np.nextafter(np.float32(mid), np.float32(10))) == c_hi


def test_e2m1_encode_is_nearest_and_saturates(orc):
    rng = np.random.default_rng(5)
    vals = np.concatenate([rng.uniform(-7, 7, 4000), rng.uniform(-0.3, 0.3, 500)]).astype(np.float32)
    mags = np.array([abs(e2m1_from_fields(c)) for c in range(8)])
    for v in vals:
        c = orc.e2m1_encode(float(v))
        got = abs(e2m1_from_fields(c))
        best = np.min(np.abs(mags - min(abs(float(v)), 6.0)))
        assert abs(got - min(abs(float(v)), 6.0)) == pytest.approx(best, abs=0), v
        assert (c >> 3) == int(np.signbit(v))
    for v in (6.0, 6.5, 7.0, 1e30):
        assert orc.e2m1_encode(v) == 7 and orc.e2m1_encode(-v) == 15


def test_e4m3_decode_matches_torch(orc):
    allb = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        want = allb[c]
        got = orc.e4m3_decode(c)
        if np.isnan(want):
            assert np.isnan(got), c
        else:
            assert got == want, (c, got, want)


def _torch_e4m3(vals: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_on_values_and_midpoints(orc):
    finite = np.array([orc.e4m3_decode(c) for c in range(0x7F)], dtype=np.float64)
    mids = (finite[:-1] + finite[1:]) / 2
    pts = np.concatenate([finite, mids]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(1e9))])
    rng = np.random.default_rng(11)
    pts = np.concatenate([pts, rng.uniform(0, 448, 20000).astype(np.float32),
                          np.exp2(rng.uniform(-12, 8.8, 20000)).astype(np.float32)])
    pts = pts[(pts >= 0) & (pts < 464)]
    want = _torch_e4m3(pts)
    got = np.array([orc.e4m3_encode(float(p)) for p in pts], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(pts[i]), int(got[i]), int(want[i])) for i in bad[:5]]


def test_e4m3_encode_saturates_to_finite(orc):
    for s in (448.0, 448.5, 463.99, 464.0, 480.0, 1e6, float("inf")):
        assert orc.e4m3_encode(s) == 0x7E


def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, 2000, dtype=np.uint32) << 16) | np.uint32(0x8000)
    vals = np.concatenate([bits, ties, np.array([0, 0x80000000, 0x7F7FFFFF, 0x7F7F8000, 1, 0x00008000],
                                                np.uint32)]).view(np.float32)
    vals = vals[np.isfinite(vals)]
    want = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_rne(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)
    for h in (0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x3B12):
        assert orc.bf16_rne(orc.bf16_to_f32(h)) == h
