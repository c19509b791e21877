// FP8 (E4M3) dispatch (NeMo AutoModel fused_a2a page: init_hybrid_ep_buffer
// can use FP8 for the dispatch payload, and HybridEPDispatch.forward returns
// a scaling factor beside the dispatched hidden states).  Per token and
// 128-element block, with amax = max|x|:
//   code  = E4M3(x * (448 / amax))   RNE, saturating to 448, sign of the product kept
//   scale = amax / 448               fp32, so that code * scale reproduces x
// An all-zero block gives zero codes and scale 0.  Each token is quantized
// once and its bytes written to every kept (token, slot) row.
//
// One workgroup of 8 waves per token: the waves quantize the row into LDS
// once (wave w takes iterations w, w + 8, ...), then wave w stores the
// codes and scales to the rows of slots w, w + 8, ...  Short store runs per
// wave rather than one wave storing all K' copies: at DeepSeek-V3 size the
// kernel went from 51.0 to 48.0 us, and from 5.8 to 4.8 us at T = 128.
// Outputs larger than the 256 MiB MALL take nontemporal code stores; smaller
// ones are stored plainly and stay in it.  Measured on MI355X, launches
// back to back / after a cache flush: DeepSeek-V3 size (231 MiB out) 47.8 /
// 49.2 us with plain stores against 48.0 / 63.3 us nontemporal; the skewed
// workload (258 MiB) 51.9 / 66.9 nontemporal against 66.1 / 55.6 plain,
// the plain stores' cold figure leaving the write-back of the MALL's dirty
// lines to whatever runs next.  One wave per token: 51.1 / 48.2 and
// 66.8 / 54.7 us; at T = 128 4.8 / 7.7 against 5.8 / 9.3 us.  Rows of
// fewer than 4 iterations (H < 3584) keep one wave per token.  4 and 2
// waves per token were slower than 8 warm and no better cold.  Batches
// past that kernel's grid (2^23 tokens) take one wave per token (four under
// kSmallBatchTokens, taking alternate iterations).  In an iteration, lanes
// form 8 groups of 8; group j owns block 8*it + j and each lane 16 of its
// elements, so one wave load covers 2 KiB of the row and one wave store
// 1 KiB of codes, both contiguous.  The block amax is three xor-shuffles
// inside the 8-lane group.
// IEEE division and no contraction keep the result bit-identical to the
// plain definition.  The encode is gfx950's v_cvt_pk_fp8_f32 (OCP E4M3,
// RNE), two elements per instruction: for |v| <= 464 it equals e4m3_signed,
// the RNE, saturating, sign-kept encode (tests/test_gpu_conversions.py runs
// both over all 2^32 float patterns), and here |v| <= 448 up to one
// rounding.  Past 464 it gives the NaN code, so a
// block whose factor 448 / amax overflowed (amax below 448/FLT_MAX) takes
// the software encoder instead.
#include "fp8_device.h"

namespace epx {
namespace {

constexpr int kFp8Threads = 256;
constexpr int kFp8Waves = kFp8Threads / kWave;
constexpr int kFp8MaxIters = 16;  // H <= 1024 * 16
#ifndef EPX_FP8_SMALL_BATCH
#define EPX_FP8_SMALL_BATCH 4096
#endif
constexpr int kSmallBatchTokens = EPX_FP8_SMALL_BATCH;  // below this, 4 waves per token

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
    // The token's K' rows, lane k holding slot k, loaded before the row is
    // quantized so that the store loop issues no load (a load there is
    // waited on together with the previous slot's stores).
    const int32_t my_row = lane < a.Kp ? a.token_row[(int64_t)t * a.Kp + lane] : -1;

    // every iteration's loads go out before the first is quantized (one
    // round trip per token, not one per iteration)
    uint4 p[NIT], q[NIT];
#pragma unroll
    for (int j = 0; j < NIT; ++j) load_iteration(xr, part + j * W, lane, nblk, p[j], q[j]);
    __builtin_amdgcn_sched_barrier(0);
    uint4 code[NIT];
    float scale[NIT];
#pragma unroll
    for (int j = 0; j < NIT; ++j) quantize_loaded(p[j], q[j], code[j], scale[j]);

    for (int32_t k = 0; k < a.Kp; ++k) {
        const int32_t row = __builtin_amdgcn_readlane(my_row, k);
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

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
#ifndef EPX_FP8_WPT
#define EPX_FP8_WPT 8  // waves per token (one workgroup per token)
#endif
// Outputs larger than this (the MALL) take nontemporal code stores: they
// could not stay in it anyway, and written straight through they no longer
// evict the inputs from it.  Smaller ones stay in it for their consumer.
#ifndef EPX_FP8_STREAM_MB
#define EPX_FP8_STREAM_MB 256
#endif
constexpr int64_t kFp8StreamBytes = int64_t(EPX_FP8_STREAM_MB) << 20;
#ifndef EPX_FP8_WG_MIN_ITERS
#define EPX_FP8_WG_MIN_ITERS 4
#endif

// One workgroup of WPT waves per token: the waves quantize the row's
// iterations into LDS once, then wave w stores the codes and scales of the
// token's slots w, w + WPT, ... (one short run of stores per slot row).
// LDS (dynamic): nit * 1 KiB of codes, then nit * 8 scales.
template <int WPT, bool NT>
__global__ __launch_bounds__(WPT * kWave) void k_fp8_wg(Fp8Args a) {
    extern __shared__ uint4 s_dyn[];
    const int32_t t = blockIdx.x;
    const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int32_t nblk = a.H / 128, nit = (nblk + 7) / 8;
    uint4* s_code = s_dyn;
    float* s_scale = reinterpret_cast<float*>(s_dyn + nit * kWave);
    const int32_t* tr = a.token_row + (int64_t)t * a.Kp;
    const int32_t row0 = wv < a.Kp ? tr[wv] : -1;  // fetched before the barrier
    const uint4* xr = reinterpret_cast<const uint4*>(a.x + (int64_t)t * a.H);
    for (int32_t it = wv; it < nit; it += WPT) {
        uint4 code;
        float scale;
        quantize_iteration(xr, it, lane, nblk, code, scale);
        s_code[it * kWave + lane] = code;
        if ((lane & 7) == 0) s_scale[it * 8 + lane / 8] = scale;
    }
    __syncthreads();
    for (int32_t k = wv; k < a.Kp; k += WPT) {
        const int32_t row = uniform(k == wv ? row0 : tr[k]);
        if (row < 0 || row >= a.R) continue;
        uint4* crow = reinterpret_cast<uint4*>(a.codes + (int64_t)row * a.H);
        float* srow = a.scales + (int64_t)row * nblk;
        for (int32_t it = 0; it < nit; ++it) {
            const int32_t b = it * 8 + lane / 8;
            if (b < nblk) {
                const uint4 c = s_code[it * kWave + lane];
                if (NT)
                    __builtin_nontemporal_store(v4u{c.x, c.y, c.z, c.w}, reinterpret_cast<v4u*>(crow + 64 * it + lane));
                else
                    crow[64 * it + lane] = c;
            }
        }
        for (int32_t b = lane; b < nblk; b += kWave) srow[b] = s_scale[b];
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
    constexpr int WPT = EPX_FP8_WPT;
    const int32_t nit = (a.H / 128 + 7) / 8;
    // One workgroup per token where a row has at least 4 iterations of 8
    // blocks (H >= 3584).  With 2 (H = 2048, capacity workload) 6 of its 8
    // waves idle while the row is quantized, and the kernel took 32.9 against
    // 26.6 us with one wave per token.
    if (nit >= EPX_FP8_WG_MIN_ITERS && (int64_t)a.T * WPT * kWave <= 0xFFFFFFFFll) {
        const size_t lds = (size_t)nit * kWave * sizeof(uint4) + (size_t)nit * 8 * sizeof(float);
        const int64_t out_bytes = (int64_t)a.T * a.Kp * (a.H + a.H / 128 * 4);
        if (out_bytes > kFp8StreamBytes)
            hipLaunchKernelGGL((k_fp8_wg<WPT, true>), dim3((unsigned)a.T), dim3(WPT * kWave), lds, stream, a);
        else
            hipLaunchKernelGGL((k_fp8_wg<WPT, false>), dim3((unsigned)a.T), dim3(WPT * kWave), lds, stream, a);
        return hipGetLastError();
    }
    // Narrow rows, and batches past that grid (2^23 tokens): one wave per
    // token (nit = (H + 1023) / 1024 as well: 1024 elements per iteration).
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
