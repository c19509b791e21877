// NVFP4 dispatch with a per-token dynamic global scale (MAX
// DistributedEPDispatchBlockScaledNVDynGlobalScales page, execute): every
// token is quantized against its own global scale g = 2688 / rowmax, block
// scales go to `scales`, the BF16 inverse of g to `rowscale`, and the packed
// E2M1 codes to `codes`, once per kept (token, slot) row.
//
// 2688 = 448 * 6: the largest finite E4M3 block scale times the largest
// E2M1 magnitude, so the block that holds rowmax gets scale 448.
//
// Rows of H % 64 == 0 with at least 256 blocks (every named workload but
// the narrow capacity one) take one workgroup of 8 waves per token
// (k_nvfp4_wg): the row is quantized into LDS once and each wave stores
// whole slot rows with 16-byte code and 4-byte scale stores.  Other rows
// take one wave64 per token (four for batches under kSmallBatchTokens,
// k_nvfp4): lane l holds 16-element blocks l, l+64, ... of the row in
// registers (two 16-byte loads per block), so a block's amax is
// lane-local and the row max is one wave reduction (plus an LDS exchange
// when a token has several waves); its bytes then go to each of the
// token's K' rows, 8 code bytes per block per lane (512 contiguous bytes
// per wave store) and one scale byte per block.  The token is quantized
// once (VALU only: there is no contraction here for MFMA).
// The code stores are nontemporal, as the bf16 dispatch's: with plain ones
// the 117 MB of codes at DeepSeek-V3 size waited dirty in the MALL and the
// next kernels wrote them back.  Measured on MI355X with one wave per
// token (graphs of the whole step, interleaved builds): DeepSeek-V3 step
// 413.4 -> 410.2 us, skewed 465.0 -> 452.0, NVFP4 workload 454.9 ->
// 451.9, capacity 204.8 -> 202.9 us, while that kernel alone got slower
// (29.6 -> 32.8 us back to back, 34.0 -> 36.7 us after a cache flush); the
// workgroup form with nontemporal codes then took the DeepSeek-V3 step to
// 407.6 us and the kernel back to 29.8 us.  A consumer that read the codes
// right away would find them in the MALL with plain stores.  Nontemporal
// scale stores as well cost more than they gave (step 412.5).
//
// Arithmetic is IEEE binary32 with round-to-nearest-even everywhere; the
// library is built with correctly rounded division and without FMA
// contraction, so the results are bit-identical to the plain definition.
// The E2M1 encode is gfx950's v_cvt_scalef32_pk_fp4_f32 with scale 1, two
// elements per instruction: on every finite and infinite input it equals
// e2m1_encode, the RNE, ties-to-even, saturating, sign-kept encode
// (tests/test_gpu_conversions.py runs both over all 2^32 float patterns,
// and e2m1_encode against the oracle at every rounding boundary).  It
// differs only on NaN, so a block whose
// per-element factor g / e4m3(s) overflowed (a row max below 2688/FLT_MAX,
// where 0 * inf can occur) takes the threshold encoder instead:
//   s = (bmax / 6) * g            -> E4M3, RNE, saturating to 448
//   v = x * (g / e4m3(s))         -> E2M1, RNE (ties to even), saturating
//                                   at 6, sign bit of v kept
//   rowscale = bf16(1 / g)
// Formats: OCP OFP8 E4M3 ("fn": bias 7, max finite 448), OCP MX E2M1.
#include "nvfp4_device.h"

namespace epx {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantWaves = kQuantThreads / kWave;
constexpr int kMaxBlocksPerLane = 16;  // H <= 16 * 64 * 16 = 16384
#ifndef EPX_NVFP4_NT_CODES
#define EPX_NVFP4_NT_CODES 1
#endif
#ifndef EPX_NVFP4_NT_SCALES
#define EPX_NVFP4_NT_SCALES 0
#endif
#ifndef EPX_NVFP4_SMALL_BATCH
#define EPX_NVFP4_SMALL_BATCH 4096
#endif
constexpr int kSmallBatchTokens = EPX_NVFP4_SMALL_BATCH;  // below this, 4 waves per token

// W waves per token (1, or 4 for small batches, where a token's quantize
// latency would otherwise leave the chip idle): wave `part` of the token
// holds blocks part*64 + lane + i*64*W, and with W > 1 the row max meets in
// LDS.  A workgroup is 4 waves, so with W = 4 it is one token and the early
// exit below is the same for the whole workgroup.
template <int NBL, int W>
__global__ __launch_bounds__(kQuantThreads) void k_nvfp4(Nvfp4Args a) {
    const int wv = threadIdx.x / kWave;
    const int32_t t = uniform((int32_t)(blockIdx.x * (kQuantWaves / W) + wv / W));
    if (t >= a.T) return;
    const int part = wv % W;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t nblk = a.H / 16;
    const uint4* xr = reinterpret_cast<const uint4*>(a.x + (int64_t)t * a.H);
    const int32_t b0 = part * kWave + lane;  // this lane's first block
    // The token's K' rows, lane k holding slot k, loaded with the row so
    // that the store loop below issues no load: a load there is waited on
    // together with the previous slot's stores (one round trip per slot).
    const int32_t my_row = lane < a.Kp ? a.token_row[(int64_t)t * a.Kp + lane] : -1;

    uint4 q[NBL][2];
    uint32_t bmax[NBL];
    uint32_t lmax = 0;
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
        const int32_t b = b0 + i * kWave * W;
        if (b < nblk) {
            q[i][0] = xr[2 * b];
            q[i][1] = xr[2 * b + 1];
        } else {
            q[i][0] = make_uint4(0, 0, 0, 0);
            q[i][1] = make_uint4(0, 0, 0, 0);
        }
        bmax[i] = block_amax(q[i][0], q[i][1]);
        lmax = max(lmax, bmax[i]);
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) lmax = max(lmax, (uint32_t)__shfl_xor((int)lmax, o, kWave));
    if (W > 1) {
        __shared__ uint32_t s_rmax[kQuantWaves];
        if (lane == 0) s_rmax[wv] = lmax;
        __syncthreads();
#pragma unroll
        for (int p2 = 0; p2 < W; ++p2) lmax = max(lmax, s_rmax[(wv / W) * W + p2]);
    }
    const float rowmax = __uint_as_float(lmax << 16);

    uint2 code[NBL];
    uint32_t sc[NBL];
    uint32_t rs = 0u;
    if (rowmax == 0.0f) {
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            code[i] = make_uint2(0, 0);
            sc[i] = 0u;
        }
    } else {
        const float g = 2688.0f / rowmax;
#pragma unroll
        for (int i = 0; i < NBL; ++i) quantize_block(q[i][0], q[i][1], bmax[i], g, code[i], sc[i]);
        rs = f32_to_bf16(1.0f / g);
    }

    const int64_t cstride = a.H / 2, sstride = nblk;
    for (int32_t k = 0; k < a.Kp; ++k) {
        const int32_t row = __builtin_amdgcn_readlane(my_row, k);
        if (row < 0 || row >= a.R) continue;
        uint8_t* crow = a.codes + (int64_t)row * cstride;
        uint8_t* srow = a.scales + (int64_t)row * sstride;
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            const int32_t b = b0 + i * kWave * W;
            if (b < nblk) {
#if EPX_NVFP4_NT_CODES
                typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));
                __builtin_nontemporal_store(v2u_t{code[i].x, code[i].y}, reinterpret_cast<v2u_t*>(crow + 8 * (int64_t)b));
#else
                *reinterpret_cast<uint2*>(crow + 8 * (int64_t)b) = code[i];
#endif
#if EPX_NVFP4_NT_SCALES
                __builtin_nontemporal_store((uint8_t)sc[i], srow + b);
#else
                srow[b] = (uint8_t)sc[i];
#endif
            }
        }
        if (part == 0 && lane == 0) a.rowscale[row] = (uint16_t)rs;
    }
}

#ifndef EPX_NVFP4_WG
#define EPX_NVFP4_WG 1
#endif
#ifndef EPX_NVFP4_WG_NT
#define EPX_NVFP4_WG_NT 1
#endif
constexpr int kWgWaves = 8;
constexpr int kWgMaxBlocks = 16 * kWave;  // H <= 16384: 1024 blocks

// One workgroup of 8 waves per token (rows with H % 64 == 0 and at least
// 256 blocks): lane l of wave w holds blocks w*64 + l + i*512; the row max
// meets in LDS, the codes and scales are quantized into LDS once, then wave
// w stores the codes, scales and rowscale of slots w, w + 8, ... with
// 16-byte code stores (nontemporal, as in k_nvfp4) and 4-byte scale
// stores.
template <int NB>
__global__ __launch_bounds__(kWgWaves * kWave) void k_nvfp4_wg(Nvfp4Args a) {
    // Declared as 16- and 4-byte words so that the stores below can read
    // them back as such (ds_read_b128 needs a 16-byte aligned address).
    __shared__ uint4 s_code4[kWgMaxBlocks / 2];
    __shared__ uint32_t s_sc4[kWgMaxBlocks / 4];
    __shared__ uint32_t s_rmax[kWgWaves];
    uint2* s_code = reinterpret_cast<uint2*>(s_code4);
    uint8_t* s_sc = reinterpret_cast<uint8_t*>(s_sc4);
    const int32_t t = blockIdx.x;
    const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int32_t nblk = a.H / 16;
    const int32_t* tr = a.token_row + (int64_t)t * a.Kp;
    const int32_t row0 = wv < a.Kp ? tr[wv] : -1;  // fetched before the barriers
    const uint4* xr = reinterpret_cast<const uint4*>(a.x + (int64_t)t * a.H);

    uint4 q[NB][2];
    uint32_t bmax[NB];
    uint32_t lmax = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int32_t b = wv * kWave + lane + i * kWgWaves * kWave;
        if (b < nblk) {
            q[i][0] = xr[2 * b];
            q[i][1] = xr[2 * b + 1];
        } else {
            q[i][0] = make_uint4(0, 0, 0, 0);
            q[i][1] = make_uint4(0, 0, 0, 0);
        }
        bmax[i] = block_amax(q[i][0], q[i][1]);
        lmax = max(lmax, bmax[i]);
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) lmax = max(lmax, (uint32_t)__shfl_xor((int)lmax, o, kWave));
    if (lane == 0) s_rmax[wv] = lmax;
    __syncthreads();
#pragma unroll
    for (int w2 = 0; w2 < kWgWaves; ++w2) lmax = max(lmax, s_rmax[w2]);
    const float rowmax = __uint_as_float(lmax << 16);
    const float g = rowmax == 0.0f ? 0.0f : 2688.0f / rowmax;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int32_t b = wv * kWave + lane + i * kWgWaves * kWave;
        if (b < nblk) {
            uint2 code = make_uint2(0, 0);
            uint32_t sc = 0u;
            if (rowmax != 0.0f) quantize_block(q[i][0], q[i][1], bmax[i], g, code, sc);
            s_code[b] = code;
            s_sc[b] = (uint8_t)sc;
        }
    }
    const uint16_t rs = rowmax == 0.0f ? (uint16_t)0 : (uint16_t)f32_to_bf16(1.0f / g);
    __syncthreads();

    const int32_t cvec = nblk / 2, swords = nblk / 4;  // 16-byte code vectors, 4-byte scale words
    for (int32_t k = wv; k < a.Kp; k += kWgWaves) {
        const int32_t row = uniform(k == wv ? row0 : tr[k]);
        if (row < 0 || row >= a.R) continue;
        uint4* crow = reinterpret_cast<uint4*>(a.codes + (int64_t)row * (a.H / 2));
        uint32_t* srow = reinterpret_cast<uint32_t*>(a.scales + (int64_t)row * nblk);
#if EPX_NVFP4_WG_NT
        typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
        for (int32_t v = lane; v < cvec; v += kWave) {
            const uint4 c = s_code4[v];
            __builtin_nontemporal_store(v4u_t{c.x, c.y, c.z, c.w}, reinterpret_cast<v4u_t*>(crow + v));
        }
#else
        for (int32_t v = lane; v < cvec; v += kWave) crow[v] = s_code4[v];
#endif
        for (int32_t v = lane; v < swords; v += kWave) srow[v] = s_sc4[v];
        if (lane == 0) a.rowscale[row] = rs;
    }
}

template <int NBL, int W>
hipError_t launch_nbl(const Nvfp4Args& a, hipStream_t stream) {
    constexpr int kTokensPerBlock = kQuantWaves / W;
    const unsigned blocks = (unsigned)((a.T + kTokensPerBlock - 1) / kTokensPerBlock);
    hipLaunchKernelGGL((k_nvfp4<NBL, W>), dim3(blocks), dim3(kQuantThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int nvfp4_max_hidden() { return 16 * kWave * kMaxBlocksPerLane; }

hipError_t launch_nvfp4(const Nvfp4Args& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int32_t nblk = a.H / 16;
    // Rows of H % 64 == 0 with at least 256 blocks and 4-byte aligned
    // scales, batches within its grid (2^23 tokens): one workgroup of 8
    // waves per token.  At DeepSeek-V3 dims T = 128 went from 5.7 to 4.3 us
    // and T = 1024 from 10.8 to 9.4 us against one wave per token.  With
    // plain code stores one wave per token stayed faster at T = 4096 (29.6
    // against 30.8 us); with nontemporal code stores in both the workgroup
    // form wins there too: 29.8 against 32.4 us, the whole step 407.6
    // against 411.3 us (NVFP4 workload 448.1 against 449.9 us, skewed equal,
    // T = 2048 15.1 against 16.7 us).
    if (EPX_NVFP4_WG && a.H % 64 == 0 && nblk >= 4 * kWave && (reinterpret_cast<uintptr_t>(a.scales) & 3) == 0 &&
        (int64_t)a.T * kWgWaves * kWave <= 0xFFFFFFFFll) {
        const int nb = (nblk + kWgWaves * kWave - 1) / (kWgWaves * kWave);  // blocks per lane
        if (nb == 1)
            hipLaunchKernelGGL(k_nvfp4_wg<1>, dim3((unsigned)a.T), dim3(kWgWaves * kWave), 0, stream, a);
        else
            hipLaunchKernelGGL(k_nvfp4_wg<2>, dim3((unsigned)a.T), dim3(kWgWaves * kWave), 0, stream, a);
        return hipGetLastError();
    }
    if (a.T < kSmallBatchTokens) {  // 4 waves per token
        const int nbl = (a.H / 16 + 4 * kWave - 1) / (4 * kWave);
        switch (nbl) {
            case 1: return launch_nbl<1, 4>(a, stream);
            case 2: return launch_nbl<2, 4>(a, stream);
            case 3: return launch_nbl<3, 4>(a, stream);
            default: return launch_nbl<4, 4>(a, stream);
        }
    }
    const int nbl = (a.H / 16 + kWave - 1) / kWave;
    switch (nbl) {
        case 1: return launch_nbl<1, 1>(a, stream);
        case 2: return launch_nbl<2, 1>(a, stream);
        case 3: return launch_nbl<3, 1>(a, stream);
        case 4: return launch_nbl<4, 1>(a, stream);
        case 5: case 6: return launch_nbl<6, 1>(a, stream);
        case 7: return launch_nbl<7, 1>(a, stream);
        case 8: return launch_nbl<8, 1>(a, stream);
        case 9: case 10: case 11: case 12: return launch_nbl<12, 1>(a, stream);
        default: return launch_nbl<kMaxBlocksPerLane, 1>(a, stream);
    }
}

}  // namespace epx
