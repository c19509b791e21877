"""Pins of the oracle's combine over NVFP4 expert-output rows (MAX
DistributedEPDispatchBlockScaledNVDynGlobalScales page, execute: the NVFP4
row format with output_scales and output_rowwise_scales; NeMo AutoModel
token_dispatcher page, TokenDispatcherConfig.moe_router_dtype: fp32
weighted combine).

Reading: xhat = e2m1(code) * (e4m3(scale) * float(rowscale)), each an fp32
multiply; y = bf16(sum_k w_k * xhat_k) in fp32, ascending k (as combine).

Pins, none of which reuses the oracle's arithmetic:
  * a hand-worked token (tests/golden/nvfp4_combine_worked_example.json),
    re-derived here with exact rational arithmetic;
  * single-slot rows: every xhat is exact in fp32, so y is the bf16
    rounding of the product computed in float64 from independent decoders
    (a table of the eight E2M1 magnitudes and torch's float8_e4m3fn);
  * rows whose values are exactly bf16 (power-of-two scales): the result
    equals orc_combine over those values written as bf16 rows, bit for bit;
  * weighted sums against the float64 sum within the fp32 and bf16 rounding
    bound;
  * the round trip x -> NVFP4 dispatch -> NVFP4 combine (weights summing to
    1) stays within the NVFP4 block error bound of x;
  * masked and dropped slots contribute nothing.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from combine_ep_dispatch_amd import workload as wl

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def e4m3_values(codes):
    """float64 values of E4M3 codes, decoded by torch's float8_e4m3fn."""
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def to_bf16_bits(v64):
    """Round float64 values that are exact in float32 to bf16 (RNE), via torch."""
    t = torch.from_numpy(np.asarray(v64, np.float64).astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def xhat64(codes, scales, rowscale_bits, H):
    """float64 dequantization of NVFP4 rows [n, H/2], [n, H/16], [n]."""
    el = np.empty((codes.shape[0], H), np.int64)
    el[:, 0::2] = codes & 0xF
    el[:, 1::2] = codes >> 4
    sc = np.repeat(e4m3_values(scales), 16, axis=1)
    return E2M1[el] * sc * f32(rowscale_bits).astype(np.float64)[:, None]


def rne_bf16_exact(q: Fraction) -> int:
    """bf16 bits of an exact rational (normal range), round to nearest-even."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    m = a / Fraction(2) ** e * 128
    lo = math.floor(m)
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    if lo == 256:
        lo, e = 128, e + 1
    return sign | ((e + 127) << 7) | (lo - 128)


def one_token_cfg(orc, H, K, shared=0):
    return orc.Cfg(T=1, H=H, E=K, S=1, K=K, A=1, shared=shared, recv_rows=K + shared)


def test_worked_example(orc, golden_dir):
    with open(os.path.join(golden_dir, "nvfp4_combine_worked_example.json")) as f:
        doc = json.load(f)
    codes = np.stack([np.frombuffer(bytes.fromhex(h), np.uint8) for h in doc["codes_hex"]])
    scales = np.stack([np.frombuffer(bytes.fromhex(h), np.uint8) for h in doc["scales_hex"]])
    rs = np.array([int(b, 16) for b in doc["rowscale_bits"]], np.uint16)
    probs = np.array([doc["probs"]], np.float32)
    want = np.array([int(h, 16) for h in doc["y_hex"].split()], np.uint16)
    # the fixture's values, re-derived exactly: E2M1 magnitudes, E4M3 from
    # its bit fields, rowscale from its bf16 bits
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]

    def e4m3(c):
        e, m = (c >> 3) & 15, c & 7
        v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        return -v if c & 0x80 else v

    def bf16v(b):
        e, m = (b >> 7) & 0xFF, b & 0x7F
        v = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
        return -v if b & 0x8000 else v

    exact = []
    for h in range(32):
        acc = Fraction(0)
        for r, w in enumerate(doc["probs"]):
            byte = int(codes[r, h // 2])
            c = byte & 0xF if h % 2 == 0 else byte >> 4
            v = mags[c & 7] * (-1 if c & 8 else 1)
            acc += Fraction(w) * v * e4m3(int(scales[r, h // 16])) * bf16v(int(rs[r]))
        exact.append(rne_bf16_exact(acc))
    assert np.array_equal(np.array(exact, np.uint16), want)
    cfg = one_token_cfg(orc, 32, 2)
    tr = np.array([[0, 1]], np.int32)
    got = orc.combine_nvfp4(cfg, tr, codes, scales, rs, probs)
    assert np.array_equal(got.reshape(-1), want)


@pytest.mark.parametrize("seed", range(4))
def test_single_slot_is_the_rounded_exact_product(orc, seed):
    rng = np.random.default_rng(seed)
    H, n = 256, 64
    codes = rng.integers(0, 256, (n, H // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (n, H // 16), dtype=np.uint8)  # finite, non-negative E4M3
    scales[:, 0] |= 0x80 * (seed % 2)  # negative scales are decoded too
    # rowscales whose products stay in the fp32 normal range
    rs = wl.bf16_bits(np.exp2(rng.uniform(-60, 60, n)).astype(np.float32) * rng.choice([1, -1], n))
    want = to_bf16_bits(0.0 + xhat64(codes, scales, rs, H))  # combine starts from +0: -0 becomes +0
    for r in range(0, n, 16):
        cfg = orc.Cfg(T=16, H=H, E=1, S=1, K=1, A=1, recv_rows=n)
        tr = np.arange(r, r + 16, dtype=np.int32).reshape(16, 1)
        got = orc.combine_nvfp4(cfg, tr, codes, scales, rs, None)
        assert np.array_equal(got, want[r:r + 16]), r


def test_power_of_two_rows_match_bf16_combine(orc):
    """xhat = e2m1 * 2^k is exact in bf16: the NVFP4 combine must equal the
    bf16 combine over those rows, bit for bit (same weights, same order)."""
    rng = np.random.default_rng(5)
    T, H, E, K = 40, 64, 6, 3
    R = orc.min_recv_rows(orc.Cfg(T=T, H=H, E=E, S=2, K=K, A=2, shared=1, src_seg=1))
    codes = rng.integers(0, 256, (R, H // 2), dtype=np.uint8)
    scales = (rng.integers(1, 15, (R, H // 16)) << 3).astype(np.uint8)  # mantissa 0: powers of two
    rs = wl.bf16_bits(np.exp2(rng.integers(-8, 8, R)).astype(np.float32))
    rows = to_bf16_bits(xhat64(codes, scales, rs, H))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids[rng.random((T, K)) < 0.2] = -1
    logits = rng.standard_normal((T, K))
    probs = (np.exp(logits) / np.exp(logits).sum(1, keepdims=True)).astype(np.float32)
    for shared in (0, 1):
        cfg = orc.Cfg(T=T, H=H, E=E, S=2, K=K, A=2, shared=shared, src_seg=1, recv_rows=R)
        tr = orc.layout(cfg, ids)["token_row"]
        for p in (probs, None):
            a = orc.combine_nvfp4(cfg, tr, codes, scales, rs, p)
            b = orc.combine(cfg, tr, rows, p)
            assert np.array_equal(a, b), (shared, p is None)


def test_weighted_sum_within_rounding_bound(orc):
    rng = np.random.default_rng(9)
    T, H, E, K = 64, 128, 16, 8
    x = wl.bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    logits = rng.standard_normal((T, K)) * 2
    probs = (np.exp(logits) / np.exp(logits).sum(1, keepdims=True)).astype(np.float32)
    cfg = orc.Cfg(T=T, H=H, E=E, S=4, K=K, A=4, recv_rows=0)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    tr = orc.layout(cfg, ids)["token_row"]
    # expert outputs: independent random NVFP4 rows, one per receive row
    R = cfg.recv_rows
    codes = rng.integers(0, 256, (R, H // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x50, (R, H // 16), dtype=np.uint8)
    rs = wl.bf16_bits(np.exp2(rng.uniform(-4, 4, R)).astype(np.float32))
    got = f32(orc.combine_nvfp4(cfg, tr, codes, scales, rs, probs)).astype(np.float64)
    xh = xhat64(codes, scales, rs, H)
    ref = np.zeros((T, H))
    mag = np.zeros((T, H))
    for k in range(K):
        term = probs[:, k:k + 1].astype(np.float64) * xh[tr[:, k]]
        ref += term
        mag += np.abs(term)
    half_ulp = np.where(ref == 0, 0, np.exp2(np.floor(np.log2(np.abs(ref) + 1e-300)) - 8))
    assert np.all(np.abs(got - ref) <= half_ulp * 1.0001 + 2.0 ** -20 * mag)
    del x


def test_round_trip_within_block_bound(orc):
    """combine_nvfp4(dispatch_nvfp4(x)) with identity experts and weights
    summing to 1 returns x to within the NVFP4 block error bound
    (3/16 bmax + 2^-18 rowmax, proved for the quantizer) plus the fp32
    weight sum and bf16 rounding."""
    w = wl.CONFIGS["nvfp4"].at_tokens(256)
    d = wl.make_workload(w)
    cfg = orc.Cfg(T=w.T, H=w.H, E=w.E, S=w.S, K=w.K, A=w.align, recv_rows=0)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    tr = orc.layout(cfg, d["topk_ids"])["token_row"]
    codes, scales, rs = orc.dispatch_nvfp4(cfg, tr, d["x"])
    y = f32(orc.combine_nvfp4(cfg, tr, codes, scales, rs, d["probs"])).astype(np.float64)
    x = f32(d["x"]).astype(np.float64)
    H = w.H
    ax = np.abs(x).reshape(w.T, H // 16, 16)
    bmax = np.repeat(ax.max(axis=2), 16, axis=1)
    rowmax = ax.reshape(w.T, H).max(axis=1, keepdims=True)
    bound = 3.0 / 16 * bmax + 2.0 ** -18 * rowmax
    xh = np.abs(x) + bound
    slack = xh * (2.0 ** -8 + 2.0 ** -20)  # bf16 half ulp and the fp32 weight sum
    assert np.all(np.abs(y - x) <= bound + slack)


def test_masked_and_dropped_slots_add_nothing(orc):
    H = 32
    cfg = one_token_cfg(orc, H, 3)
    cfg.T = 2
    codes = np.full((3, H // 2), 0x22, np.uint8)
    scales = np.full((3, H // 16), 0x38, np.uint8)
    rs = np.full(3, 0x3F80, np.uint16)  # every element 1.0
    probs = np.array([[0.5, 0.25, 0.125], [0.5, 0.25, 0.125]], np.float32)
    tr = np.array([[0, -1, 2], [-1, -1, -1]], np.int32)
    y = orc.combine_nvfp4(cfg, tr, codes, scales, rs, probs)
    assert np.all(y[0] == np.uint16(0x3F20))  # 0.625
    assert np.all(y[1] == 0)                  # no kept slot: +0
