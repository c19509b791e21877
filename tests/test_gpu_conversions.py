"""The gfx950 hardware conversions the kernels rely on, checked exhaustively
against the software definitions the kernels carry (epx_device.h), and
those definitions against the CPU oracle at every rounding boundary.

  * E2M1 encode, v_cvt_scalef32_pk_fp4_f32 with scale 1 (NVFP4 dispatch):
    equal to e2m1_encode on all 2^32 float patterns except NaN, which the
    kernels never convert (a block whose factor overflowed takes the
    software encoder).
  * E4M3 encode, v_cvt_pk_fp8_f32 (FP8 dispatch): equal to e4m3_signed on
    every float with |v| <= 464; the kernels pass it only |v| <= 448 up to
    one rounding.
  * bf16 rounding, v_cvt_pk_bf16_f32 (every bf16 output): equal to the bit
    formula on all 2^32 patterns, NaN included.
  * E2M1 decode, v_cvt_scalef32_pk_f32_fp4 with scale 1 (NVFP4 combine):
    equal to the bit-field decode for every byte in every byte position
    (with another scale it is not an exact multiply, so the kernel does not
    use one).
  * E4M3 decode, v_cvt_f32_fp8 (NVFP4 combine's block scales): equal to the
    software decode and to the oracle's on every finite code, NaN for the
    two NaN codes 0x7F and 0xFF as in the oracle.

The software encoders and the oracle (oracle/oracle.c: brute-force nearest
value, ties to the even code) are both monotone step functions of the
input, so agreeing at every decision boundary and one ulp either side of
it, on both signs, makes them agree everywhere; the boundary inputs are
generated here from the formats' definitions.  Together with the
exhaustive hardware checks this ties every code the kernels write to the
oracle's definition.
"""

import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def C():
    import conv_check

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()
    return conv_check.load()


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)


def tallies(run):
    counts = torch.zeros(8, dtype=torch.int64, device=DEV)
    first = torch.zeros(32, dtype=torch.int32, device=DEV)
    nfirst = torch.zeros(4, dtype=torch.int32, device=DEV)
    run(ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(first.data_ptr()), ctypes.c_void_p(nfirst.data_ptr()))
    torch.cuda.synchronize()
    c = counts.cpu().numpy().reshape(4, 2)
    f = first.cpu().numpy().view(np.uint32).reshape(4, 8)
    n = nfirst.cpu().numpy()
    return c, [f[i, :min(int(n[i]), 8)].tolist() for i in range(4)]


def encode_all(C, kind):
    def run(counts, first, nfirst):
        step = 1 << 30
        for b in range(0, 1 << 32, step):
            print(f"[gpu] conversion check kind {kind}: patterns {b:#x}..{b + step - 1:#x}", flush=True)
            assert C.conv_check_encode(kind, b, step, counts, first, nfirst, stream()) == 0
    return tallies(run)


FINITE = (1 << 32) - (1 << 24)  # exponent field 255 holds the 2 infinities and 2^24 - 2 NaNs


def test_e2m1_encode_exhaustive(C):
    c, first = encode_all(C, 0)
    assert c[0, 0] == FINITE and c[1, 0] == 2 and c[2, 0] == (1 << 24) - 2
    assert c[0, 1] == 0, [hex(u) for u in first[0]]  # every finite input
    assert c[1, 1] == 0, [hex(u) for u in first[1]]  # +-inf saturate to +-6 on both sides
    print(f"E2M1 encode: NaN inputs that differ from the software encoder: {c[2, 1]} of {c[2, 0]}")


def test_e4m3_encode_exhaustive(C):
    c, first = encode_all(C, 1)
    assert c[0, 0] + c[1, 0] == FINITE
    assert c[0, 1] == 0, [hex(u) for u in first[0]]  # every finite input with |v| <= 464
    print(f"E4M3 encode: finite inputs past 464 that differ (the hardware gives NaN): {c[1, 1]} of {c[1, 0]}")


def test_bf16_rounding_exhaustive(C):
    c, first = encode_all(C, 2)
    assert c[0, 0] == FINITE and c[1, 0] == 2 and c[2, 0] == (1 << 24) - 2
    assert c[:3, 1].tolist() == [0, 0, 0], first


def test_e2m1_decode_every_byte(C):
    out = torch.zeros(2048, dtype=torch.int32, device=DEV)
    ref = torch.zeros(2048, dtype=torch.int32, device=DEV)
    assert C.conv_check_e2m1_decode(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ref.data_ptr()), stream()) == 0
    torch.cuda.synchronize()
    o, r = out.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32)
    assert np.array_equal(o, r), np.nonzero(o != r)[0][:8]
    # and the bit-field decode is the format's table
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    want = np.empty(2048, np.float32)
    for byte in range(256):
        for sel in range(4):
            for half, nib in ((0, byte & 15), (1, byte >> 4)):
                want[(byte * 4 + sel) * 2 + half] = -mags[nib & 7] if nib & 8 else mags[nib & 7]
    assert np.array_equal(r, want.view(np.uint32))  # -0 for code 8 included


def test_e4m3_decode_every_byte(C, orc):
    out = torch.zeros(256, dtype=torch.int32, device=DEV)
    ref = torch.zeros(256, dtype=torch.int32, device=DEV)
    assert C.conv_check_e4m3_decode(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ref.data_ptr()), stream()) == 0
    torch.cuda.synchronize()
    o, r = out.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32)
    lib = orc._load()
    dec = lib.orc_e4m3_decode
    dec.restype, dec.argtypes = ctypes.c_float, [ctypes.c_uint8]
    nan_codes = (0x7F, 0xFF)
    for c in range(256):
        want = np.float32(dec(c))
        hw = o[c:c + 1].view(np.float32)[0]
        if c in nan_codes:
            assert np.isnan(hw) and np.isnan(want), (c, hw, want)
        else:
            assert o[c] == r[c] == want.view(np.uint32), (hex(c), hex(o[c]), hex(r[c]), want)


def test_e2m1_decode_with_block_scale(C):
    """The decode with the scale operand set to a block scale (every finite
    E4M3 code times every finite bf16 rowscale) against the software
    product e2m1 * bs, recorded by class.  Measured on MI355X, most products
    differ (246 137 428 of 263 115 576 in the normal range): the operand is
    not applied as an exact fp32 multiply, so the NVFP4 combine converts
    with scale 1 (exact, test above) and multiplies by the block scale in
    software.  Only the number of inputs is asserted."""
    def run(counts, first, nfirst):
        assert C.conv_check_e2m1_decode_scaled(counts, first, nfirst, stream()) == 0
    c, first = tallies(run)
    for cls, what in enumerate(("normal", "subnormal product", "subnormal block scale")):
        print(f"E2M1 decode x block scale, {what}: {c[cls, 1]} of {c[cls, 0]} differ; first {[hex(u) for u in first[cls]]}")
    assert c[0, 0] + c[1, 0] + c[2, 0] == 16 * 254 * (65536 - 256)  # 256 bf16 patterns are inf or NaN


def boundary_inputs():
    """Every rounding boundary of E2M1, E4M3 and bf16 and one float ulp
    either side, both signs, plus zeros, subnormals and saturation edges."""
    e4m3 = sorted({0.0} | {m * 2.0 ** -9 for m in range(8)} |
                  {(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8) if not (e == 15 and m == 7)})
    mids = [(a + b) / 2 for a, b in zip(e4m3, e4m3[1:])]
    e2m1 = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    e2m1_mids = [(a + b) / 2 for a, b in zip(e2m1, e2m1[1:])]
    pts = set(e4m3) | set(mids) | set(e2m1) | set(e2m1_mids) | {464.0, 480.0, 500.0, 1e30, 6.5, 7.0,
                                                               2.0 ** -10, 2.0 ** -12, 1e-40, 1e-45}
    base = np.array(sorted(pts), np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    down = np.nextafter(base, np.float32(-np.inf))
    vals = np.concatenate([base, up, down])
    vals = np.concatenate([vals, -vals])
    # bf16 ties: low 16 bits exactly 0x8000, and one ulp either side, over
    # every exponent, plus random patterns
    rng = np.random.default_rng(0)
    hi = rng.integers(0, 0x7F80, 4000).astype(np.uint32)
    ties = np.concatenate([(hi << 16) | 0x8000, (hi << 16) | 0x7FFF, (hi << 16) | 0x8001,
                           rng.integers(0, 0x7F800000, 4000).astype(np.uint32)])
    ties = np.concatenate([ties, ties | 0x80000000]).view(np.float32)
    return np.concatenate([vals, ties]).astype(np.float32)


def test_software_encoders_match_the_oracle_at_every_boundary(C, orc):
    x = boundary_inputs()
    n = x.size
    xin = torch.from_numpy(x).to(DEV)
    e2 = torch.zeros(n, dtype=torch.uint8, device=DEV)
    e4 = torch.zeros(n, dtype=torch.uint8, device=DEV)
    bf = torch.zeros(n, dtype=torch.int16, device=DEV)
    assert C.conv_eval_sw(ctypes.c_void_p(xin.data_ptr()), n, ctypes.c_void_p(e2.data_ptr()),
                          ctypes.c_void_p(e4.data_ptr()), ctypes.c_void_p(bf.data_ptr()), stream()) == 0
    torch.cuda.synchronize()
    e2, e4, bf = e2.cpu().numpy(), e4.cpu().numpy(), bf.cpu().numpy().view(np.uint16)
    lib = orc._load()
    bad = []
    for i, v in enumerate(x.tolist()):
        if abs(v) <= 1e30:
            if e2[i] != orc.e2m1_encode(v):
                bad.append(("e2m1", v, int(e2[i]), orc.e2m1_encode(v)))
            if e4[i] != lib.orc_e4m3_encode_signed(ctypes.c_float(v)):
                bad.append(("e4m3", v, int(e4[i]), int(lib.orc_e4m3_encode_signed(ctypes.c_float(v)))))
        if bf[i] != orc.bf16_rne(v):
            bad.append(("bf16", v, int(bf[i]), orc.bf16_rne(v)))
    assert not bad, bad[:10]
