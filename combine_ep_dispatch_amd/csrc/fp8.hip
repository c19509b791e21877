// FP8 (E4M3) dispatch (NeMo AutoModel fused_a2a page: init_hybrid_ep_buffer
// can use FP8 for the dispatch payload, and HybridEPDispatch.forward returns
// a scaling factor beside the dispatched hidden states).  Per token and
// 128-element block, with amax = max|x|:
//   code  = E4M3(x * (448 / amax))   RNE, saturating to 448, sign of the product kept
//   scale = amax / 448               fp32, so that code * scale reproduces x
// An all-zero block gives zero codes and scale 0.  Each token is quantized
// once and its bytes written to every kept (token, slot) row.
//
// One wave64 per token (four for batches under kSmallBatchTokens, taking
// alternate iterations).  Lanes form 8 groups of 8; group j owns block
// 8*it + j of iteration it and each lane 16 of its elements, so one wave
// load covers 2 KiB of the row and one wave store 1 KiB of codes, both
// contiguous.  The block amax is three xor-shuffles inside the 8-lane group.
// IEEE division and no contraction keep the result bit-identical to the
// plain definition.  The encode is gfx950's v_cvt_pk_fp8_f32 (OCP E4M3,
// RNE), two elements per instruction: for |v| <= 464 it equals the RNE,
// saturating, sign-kept encode (checked over all 2^32 float patterns), and
// here |v| <= 448 up to one rounding.  Past 464 it gives the NaN code, so a
// block whose factor 448 / amax overflowed (amax below 448/FLT_MAX) takes
// the software encoder instead.
#include "epx_device.h"

namespace epx {
namespace {

constexpr int kFp8Threads = 256;
constexpr int kFp8Waves = kFp8Threads / kWave;
constexpr int kFp8MaxIters = 16;  // H <= 1024 * 16
#ifndef EPX_FP8_SMALL_BATCH
#define EPX_FP8_SMALL_BATCH 4096
#endif
constexpr int kSmallBatchTokens = EPX_FP8_SMALL_BATCH;  // below this, 4 waves per token

__device__ __forceinline__ uint32_t e4m3_signed(float v) {
    return e4m3_encode(__builtin_fabsf(v)) | ((__float_as_uint(v) >> 24) & 0x80u);
}

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

// W waves per token (1, or 4 for small batches): wave `part` takes the
// iterations part, part + W, ...  A 128-element block lives in 8 lanes of
// one wave, so the waves of a token never exchange anything.
template <int NIT, int W>
__global__ __launch_bounds__(kFp8Threads) void k_fp8(Fp8Args a) {
    const int wv = threadIdx.x / kWave;
    const int32_t t = uniform((int32_t)(blockIdx.x * (kFp8Waves / W) + wv / W));
    if (t >= a.T) return;
    const int part = wv % W;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t nblk = a.H / 128;
    const uint4* xr = reinterpret_cast<const uint4*>(a.x + (int64_t)t * a.H);

    uint4 code[NIT];
    float scale[NIT];
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
        const int32_t it = part + j * W;        // this wave's iteration
        const int32_t b = it * 8 + lane / 8;  // this lane's block
        uint4 p = make_uint4(0, 0, 0, 0), q = make_uint4(0, 0, 0, 0);
        if (b < nblk) {
            p = xr[128 * it + 2 * lane];
            q = xr[128 * it + 2 * lane + 1];
        }
        uint32_t m = absmax16(p, q);
        m = max(m, (uint32_t)__shfl_xor((int)m, 4, kWave));
        m = max(m, (uint32_t)__shfl_xor((int)m, 2, kWave));
        m = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
        const float amax = __uint_as_float(m << 16);
        if (amax == 0.0f) {
            code[j] = make_uint4(0, 0, 0, 0);
            scale[j] = 0.0f;
        } else {
            const float inv = 448.0f / amax;
            if (inv > 0.0f && inv <= __FLT_MAX__) {  // 0 when amax is inf
                code[j].x = codes4_hw(p.x, p.y, inv);
                code[j].y = codes4_hw(p.z, p.w, inv);
                code[j].z = codes4_hw(q.x, q.y, inv);
                code[j].w = codes4_hw(q.z, q.w, inv);
            } else {
                code[j].x = codes4(p.x, p.y, inv);
                code[j].y = codes4(p.z, p.w, inv);
                code[j].z = codes4(q.x, q.y, inv);
                code[j].w = codes4(q.z, q.w, inv);
            }
            scale[j] = amax / 448.0f;
        }
    }

    const int32_t* tr = a.token_row + (int64_t)t * a.Kp;
    for (int32_t k = 0; k < a.Kp; ++k) {
        const int32_t row = tr[k];
        if (row < 0 || row >= a.R) continue;
        uint4* crow = reinterpret_cast<uint4*>(a.codes + (int64_t)row * a.H);
        float* srow = a.scales + (int64_t)row * nblk;
#pragma unroll
        for (int j = 0; j < NIT; ++j) {
            const int32_t it = part + j * W;
            const int32_t b = it * 8 + lane / 8;
            if (b < nblk) {
                crow[64 * it + lane] = code[j];
                if ((lane & 7) == 0) srow[b] = scale[j];
            }
        }
    }
}

template <int NIT, int W>
hipError_t launch_nit(const Fp8Args& a, hipStream_t stream) {
    constexpr int kTokensPerBlock = kFp8Waves / W;
    const unsigned blocks = (unsigned)((a.T + kTokensPerBlock - 1) / kTokensPerBlock);
    hipLaunchKernelGGL((k_fp8<NIT, W>), dim3(blocks), dim3(kFp8Threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int fp8_max_hidden() { return 1024 * kFp8MaxIters; }

hipError_t launch_fp8(const Fp8Args& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int nit = (a.H + 1023) / 1024;
    if (a.T < kSmallBatchTokens) {  // 4 waves per token
        switch ((nit + 3) / 4) {
            case 1: return launch_nit<1, 4>(a, stream);
            case 2: return launch_nit<2, 4>(a, stream);
            case 3: return launch_nit<3, 4>(a, stream);
            default: return launch_nit<4, 4>(a, stream);
        }
    }
    switch (nit) {
        case 1: return launch_nit<1, 1>(a, stream);
        case 2: return launch_nit<2, 1>(a, stream);
        case 3: case 4: return launch_nit<4, 1>(a, stream);
        case 5: case 6: return launch_nit<6, 1>(a, stream);
        case 7: return launch_nit<7, 1>(a, stream);
        case 8: return launch_nit<8, 1>(a, stream);
        case 9: case 10: case 11: case 12: return launch_nit<12, 1>(a, stream);
        default: return launch_nit<kFp8MaxIters, 1>(a, stream);
    }
}

}  // namespace epx
