"""Pins of the oracle's NVFP4 dispatch quantization with a per-token dynamic
global scale (MAX DistributedEPDispatchBlockScaledNVDynGlobalScales page,
execute: global scale 2688 / rowmax, block scales in output_scales, BF16
inverse global scale in output_rowwise_scales).

The pages print no quantized values, so the pins are:
  * a hand-worked token (tests/golden/nvfp4_worked_example.json);
  * the dequantization error bound, proved from the quantization steps:
    |x - e2m1(code) * e4m3(scale) * rowscale| <= (3/16) bmax + 2^-18 rowmax
    for every block (3/16 = half the widest relative E2M1 gap (1/6) plus the
    rounding slack of the E4M3 scale and the bf16 rowscale);
  * structural facts: the block holding rowmax gets scale 448 (0x7E) and its
    largest element the code 6; rowscale * 2688 = rowmax to bf16 precision;
    every copy of a token carries the same bytes; an all-zero token gives
    all-zero bytes.
"""

import json
import os

import numpy as np
import pytest

from combine_ep_dispatch_amd import workload as wl


def f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def e4m3_table(orc):
    return np.array([orc.e4m3_decode(c) for c in range(256)], np.float64)


def dequant(orc, codes, scales, rowscale_bits, H):
    lo = codes & 0xF
    hi = codes >> 4
    el = np.empty(H, np.int64)
    el[0::2] = lo
    el[1::2] = hi
    sc = e4m3_table(orc)[scales]
    return E2M1[el] * np.repeat(sc, 16) * float(f32(np.uint16(rowscale_bits)))


def test_worked_example(orc, golden_dir):
    with open(os.path.join(golden_dir, "nvfp4_worked_example.json")) as f:
        doc = json.load(f)
    x = wl.bf16_bits(np.array(doc["x"], np.float32))
    assert np.array_equal(f32(x), np.array(doc["x"], np.float32))  # exact in bf16
    codes, scales, rs = orc.nvfp4_row(x)
    assert codes.tobytes().hex().upper() == doc["codes_hex"]
    assert scales.tobytes().hex().upper() == doc["scales_hex"]
    assert rs == int(doc["rowscale_bits"], 16)


def rows_for_bound(rng, H):
    rows = [rng.standard_normal(H).astype(np.float32)]
    r = rng.standard_normal(H).astype(np.float32)
    r[rng.integers(0, H)] *= 50
    rows.append(r)
    # tiny blocks next to a huge one: E4M3-subnormal and zero block scales
    r = (rng.standard_normal(H) * 1e-4).astype(np.float32)
    r[0] = 300.0
    rows.append(r)
    r = (rng.standard_normal(H) * 10.0 ** rng.uniform(-6, 1, H)).astype(np.float32)
    rows.append(r)
    r = np.zeros(H, np.float32)
    r[rng.integers(0, H)] = -3.25
    rows.append(r)
    rows.append(rng.uniform(-6, 6, H).astype(np.float32))
    return rows


@pytest.mark.parametrize("seed", range(12))
def test_dequantization_error_bound(orc, seed):
    rng = np.random.default_rng(seed)
    H = 16 * int(rng.integers(1, 40))
    for r in rows_for_bound(rng, H):
        x = wl.bf16_bits(r)
        xf = f32(x).astype(np.float64)
        codes, scales, rs = orc.nvfp4_row(x)
        xh = dequant(orc, codes, scales, rs, H)
        rowmax = np.max(np.abs(xf))
        bmax = np.repeat(np.abs(xf).reshape(-1, 16).max(1), 16)
        assert np.all(np.abs(xf - xh) <= 3 / 16 * bmax + 2.0 ** -18 * rowmax), seed


def test_structure_of_the_global_scale(orc):
    rng = np.random.default_rng(7)
    for _ in range(50):
        H = 16 * int(rng.integers(1, 64))
        r = (rng.standard_normal(H) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        x = wl.bf16_bits(r)
        xf = f32(x)
        codes, scales, rs = orc.nvfp4_row(x)
        i = int(np.argmax(np.abs(xf)))
        rowmax = float(np.abs(xf[i]))
        assert scales[i // 16] == 0x7E
        c = (codes[i // 2] >> (4 * (i % 2))) & 0xF
        assert c & 7 == 7 and (c >> 3) == int(xf[i] < 0)
        assert abs(float(f32(np.uint16(rs))) * 2688.0 / rowmax - 1) <= 2.0 ** -8


def test_zero_token(orc):
    codes, scales, rs = orc.nvfp4_row(np.zeros(64, np.uint16))
    assert not codes.any() and not scales.any() and rs == 0
    # negative zeros are zeros too
    codes, scales, rs = orc.nvfp4_row(np.full(32, 0x8000, np.uint16))
    assert not codes.any() and not scales.any() and rs == 0


def test_every_copy_is_the_token_quantized_once(orc):
    w = wl.CONFIGS["nvfp4"]
    T, H = 48, 256
    d = wl.make_workload(wl.Workload("nv_small", T=T, H=H, E=16, S=4, K=3, align=8,
                                     shared_expert=1, src_segment=2,
                                     outlier_frac=0.05, outlier_scale=w.outlier_scale))
    cfg = orc.Cfg(T=T, H=H, E=16, S=4, K=3, A=8, shared=1, src_seg=2)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, d["topk_ids"])
    codes, scales, rowscale = orc.dispatch_nvfp4(cfg, L["token_row"], d["x"])
    for t in range(T):
        qc, qs, rs = orc.nvfp4_row(d["x"][t])
        for k in range(cfg.Kp):
            row = L["token_row"][t, k]
            assert row >= 0
            assert np.array_equal(codes[row], qc) and np.array_equal(scales[row], qs)
            assert rowscale[row] == rs
    used = np.zeros(cfg.recv_rows, bool)
    used[L["token_row"].ravel()] = True
    assert np.all(codes[~used] == orc.SENTINEL_U8)
    assert np.all(rowscale[~used] == orc.SENTINEL_U16)
