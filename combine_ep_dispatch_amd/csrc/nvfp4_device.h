// NVFP4 block quantization shared by the NVFP4 dispatch kernels and the
// small layout kernel's fused NVFP4 dispatch (MAX
// DistributedEPDispatchBlockScaledNVDynGlobalScales page, execute: per-token
// global scale, E4M3 block scales, E2M1 codes).  Every kernel that quantizes
// a token calls these, so the bits agree whichever kernel ran.
#pragma once

#include "epx_device.h"

namespace epx {

__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t acc, uint32_t w) {
    const uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
    return max(acc, max(lo, hi));
}

// Two E2M1 codes per byte, element 2j in the low nibble.
__device__ __forceinline__ uint32_t codes_of_word(uint32_t w, float inv) {
    const uint32_t c0 = e2m1_encode(bf16_lo(w) * inv);
    const uint32_t c1 = e2m1_encode(bf16_hi(w) * inv);
    return c0 | (c1 << 4);
}

// Eight codes (words w0..w3) by the hardware conversion: operand a fills the
// low nibble of the selected byte, operand b the high one.
__device__ __forceinline__ uint32_t codes_of_words_hw(const uint4& w, float inv) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo(w.x) * inv, bf16_hi(w.x) * inv, 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo(w.y) * inv, bf16_hi(w.y) * inv, 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo(w.z) * inv, bf16_hi(w.z) * inv, 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo(w.w) * inv, bf16_hi(w.w) * inv, 1.0f, 3);
    return r;
}

__device__ __forceinline__ uint32_t codes_of_words_sw(const uint4& w, float inv) {
    return codes_of_word(w.x, inv) | (codes_of_word(w.y, inv) << 8) | (codes_of_word(w.z, inv) << 16) |
           (codes_of_word(w.w, inv) << 24);
}

// |x| max of a 16-element block (two 16-byte words) as bf16 bits: integer
// order = magnitude order for finite x.
__device__ __forceinline__ uint32_t block_amax(const uint4& q0, const uint4& q1) {
    uint32_t m = 0;
    m = absmax_bf16x2(m, q0.x);
    m = absmax_bf16x2(m, q0.y);
    m = absmax_bf16x2(m, q0.z);
    m = absmax_bf16x2(m, q0.w);
    m = absmax_bf16x2(m, q1.x);
    m = absmax_bf16x2(m, q1.y);
    m = absmax_bf16x2(m, q1.z);
    m = absmax_bf16x2(m, q1.w);
    return m;
}

// One block against the token's global scale g = 2688 / rowmax (rowmax > 0):
// E4M3 block scale and the 16 E2M1 codes.
__device__ __forceinline__ void quantize_block(const uint4& q0, const uint4& q1, uint32_t bmax, float g,
                                               uint2& code, uint32_t& sc) {
    const float d = __uint_as_float(bmax << 16) / 6.0f;
    const float s = d * g;
    const uint32_t c = e4m3_encode(s);
    const float sq = e4m3_decode(c);
    sc = c;
    if (sq == 0.0f) {
        code = make_uint2(0, 0);
        return;
    }
    const float inv = g / sq;
    if (inv <= __FLT_MAX__) {
        code.x = codes_of_words_hw(q0, inv);
        code.y = codes_of_words_hw(q1, inv);
    } else {
        code.x = codes_of_words_sw(q0, inv);
        code.y = codes_of_words_sw(q1, inv);
    }
}

}  // namespace epx
