"""Pins of the oracle's FP8 (E4M3) dispatch quantization (NeMo AutoModel
fused_a2a page: init_hybrid_ep_buffer can use FP8 for the dispatch payload;
HybridEPDispatch.forward returns a scaling factor beside the hidden states).

Reading: per token and 128-element block, code = E4M3(x * 448/amax) (RNE,
saturating, sign kept), scale = amax/448.  Pins:
  * a hand-worked block (tests/golden/fp8_worked_example.json);
  * the codes equal torch's float8_e4m3fn cast of x * (448/amax) (a library
    routine), with -0 mapped to the sign-kept zero;
  * dequantization error |x - e4m3(code) * scale| <= 2^-4 |x| (three mantissa
    bits) + 2^-10 * scale (half the subnormal step) + rounding of the scale;
  * the block maximum decodes to +-448, and every copy carries equal bytes.
"""

import json
import os

import numpy as np
import torch

from combine_ep_dispatch_amd import workload as wl


def f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def e4m3_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def test_worked_example(orc, golden_dir):
    with open(os.path.join(golden_dir, "fp8_worked_example.json")) as f:
        doc = json.load(f)
    x = np.zeros(doc["H"], np.float32)
    x[: len(doc["x"])] = doc["x"]
    xb = wl.bf16_bits(x)
    assert np.array_equal(f32(xb), x)  # every value exact in bf16
    codes, scales = orc.fp8_row(xb)
    assert codes[:10].tobytes().hex().upper() == doc["codes_hex_first10"]
    assert not codes[10:].any()
    assert scales.view(np.uint32)[0] == int(doc["scale_bits"], 16)


def rows(rng, H):
    out = [rng.standard_normal(H).astype(np.float32)]
    r = rng.standard_normal(H).astype(np.float32)
    r[rng.integers(0, H)] *= 50
    out.append(r)
    out.append((rng.standard_normal(H) * 10.0 ** rng.uniform(-6, 3, H)).astype(np.float32))
    r = np.zeros(H, np.float32)
    r[5] = -1e-3
    out.append(r)
    out.append(np.zeros(H, np.float32))
    return out


def test_codes_match_torch_cast_and_error_bound(orc):
    rng = np.random.default_rng(2)
    dec = e4m3_values()
    for H in (128, 256, 1024):
        for r in rows(rng, H):
            xb = wl.bf16_bits(r)
            xf = f32(xb)
            codes, scales = orc.fp8_row(xb)
            for b in range(H // 128):
                blk = xf[128 * b: 128 * (b + 1)]
                cb = codes[128 * b: 128 * (b + 1)]
                amax = np.float32(np.abs(blk).max())
                if amax == 0:
                    assert not cb.any() and scales[b] == 0
                    continue
                inv = np.float32(448.0) / amax
                v = (blk * inv).astype(np.float32)
                want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
                # torch drops the sign of values that round to zero: keep it, as the reading says
                want = np.where((want & 0x7F) == 0, np.where(np.signbit(v), 0x80, 0x00), want).astype(np.uint8)
                assert np.array_equal(cb, want), (H, b)
                assert scales[b] == np.float32(amax / np.float32(448.0))
                xh = dec[cb] * np.float64(scales[b])
                bound = (2.0 ** -4 + 2.0 ** -20) * np.abs(blk) + 2.0 ** -10 * scales[b] * (1 + 2.0 ** -20)
                assert np.all(np.abs(blk - xh) <= bound), (H, b)
                i = int(np.argmax(np.abs(blk)))
                assert abs(dec[cb[i]]) == 448.0


def test_every_copy_is_the_token_quantized_once(orc):
    T, H = 40, 256
    d = wl.make_workload(wl.Workload("fp8_small", T=T, H=H, E=16, S=4, K=3, align=8, shared_expert=1,
                                     src_segment=1, outlier_frac=0.05, outlier_scale=50.0))
    cfg = orc.Cfg(T=T, H=H, E=16, S=4, K=3, A=8, shared=1, src_seg=1)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, d["topk_ids"])
    codes, scales = orc.dispatch_fp8(cfg, L["token_row"], d["x"])
    for t in range(T):
        qc, qs = orc.fp8_row(d["x"][t])
        for k in range(cfg.Kp):
            row = L["token_row"][t, k]
            assert np.array_equal(codes[row], qc) and np.array_equal(scales[row], qs)
    used = np.zeros(cfg.recv_rows, bool)
    used[L["token_row"].ravel()] = True
    assert np.all(codes[~used] == orc.SENTINEL_U8)
    assert np.all(scales[~used].view(np.uint32) == orc.SENTINEL_F32_BITS)
