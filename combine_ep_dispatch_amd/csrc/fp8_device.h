// FP8 (E4M3) block quantization shared by the FP8 dispatch kernels and the
// small layout kernel's fused FP8 dispatch (NeMo AutoModel fused_a2a page,
// init_hybrid_ep_buffer: FP8 dispatch payload with its scaling factor):
// per 128-element block, code = E4M3(x * (448 / amax)), scale = amax / 448.
// Every kernel that quantizes a token calls these, so the bits agree
// whichever kernel ran.
#pragma once

#include "epx_device.h"

namespace epx {

__device__ __forceinline__ uint32_t absmax16(const uint4& p, const uint4& q) {
    const uint32_t w[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    return m;
}

// Four E4M3 codes (elements 2i, 2i+1 of words w0, w1) packed little-endian.
__device__ __forceinline__ uint32_t codes4(uint32_t w0, uint32_t w1, float inv) {
    return e4m3_signed(bf16_lo(w0) * inv) | (e4m3_signed(bf16_hi(w0) * inv) << 8) |
           (e4m3_signed(bf16_lo(w1) * inv) << 16) | (e4m3_signed(bf16_hi(w1) * inv) << 24);
}

// The same by the hardware conversion: operand a goes to the lower byte of
// the selected half-word, b to the upper one.
__device__ __forceinline__ uint32_t codes4_hw(uint32_t w0, uint32_t w1, float inv) {
    int r = 0;
    r = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w0) * inv, bf16_hi(w0) * inv, r, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w1) * inv, bf16_hi(w1) * inv, r, true);
    return (uint32_t)r;
}

// Iteration `it` of a row: 8 blocks of 128 elements, block it*8 + lane/8
// in lanes 8j..8j+7, 16 elements per lane (one 2 KiB wave load).
// load_iteration fetches this lane's 16 elements (zeros past the last
// block); quantize_loaded gives its 16 codes and its block's scale (the
// same in all 8 lanes).
__device__ __forceinline__ void load_iteration(const uint4* xr, int32_t it, int lane, int32_t nblk, uint4& p,
                                               uint4& q) {
    const int32_t b = it * 8 + lane / 8;  // this lane's block
    p = make_uint4(0, 0, 0, 0);
    q = make_uint4(0, 0, 0, 0);
    if (b < nblk) {
        p = xr[128 * it + 2 * lane];
        q = xr[128 * it + 2 * lane + 1];
    }
}

__device__ __forceinline__ void quantize_loaded(uint4 p, uint4 q, uint4& code, float& scale) {
    uint32_t m = absmax16(p, q);
    m = max(m, (uint32_t)__shfl_xor((int)m, 4, kWave));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2, kWave));
    m = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
    const float amax = __uint_as_float(m << 16);
    if (amax == 0.0f) {
        code = make_uint4(0, 0, 0, 0);
        scale = 0.0f;
        return;
    }
    const float inv = 448.0f / amax;
    if (inv > 0.0f && inv <= __FLT_MAX__) {  // 0 when amax is inf
        code.x = codes4_hw(p.x, p.y, inv);
        code.y = codes4_hw(p.z, p.w, inv);
        code.z = codes4_hw(q.x, q.y, inv);
        code.w = codes4_hw(q.z, q.w, inv);
    } else {
        code.x = codes4(p.x, p.y, inv);
        code.y = codes4(p.z, p.w, inv);
        code.z = codes4(q.x, q.y, inv);
        code.w = codes4(q.z, q.w, inv);
    }
    scale = amax / 448.0f;
}

__device__ __forceinline__ void quantize_iteration(const uint4* xr, int32_t it, int lane, int32_t nblk, uint4& code,
                                                   float& scale) {
    uint4 p, q;
    load_iteration(xr, it, lane, nblk, p, q);
    quantize_loaded(p, q, code, scale);
}

}  // namespace epx
