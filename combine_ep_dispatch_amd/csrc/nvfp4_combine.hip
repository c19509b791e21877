// Combine over NVFP4 expert-output rows: the rows arrive in the format the
// MAX DistributedEPDispatchBlockScaledNVDynGlobalScales page's execute
// produces (E2M1 codes, E4M3 block scales in output_scales, the bf16 inverse
// global scale in output_rowwise_scales), and combine dequantizes them as it
// reads them:
//   xhat = e2m1(code) * (e4m3(scale) * float(rowscale))
//   y[t] = bf16( sum_k w_k * xhat(row(t,k)) )   fp32, ascending k, from +0
// with one rounding per multiply and add (no FMA), w_k as in the bf16
// combine (NeMo AutoModel token_dispatcher page,
// TokenDispatcherConfig.moe_router_dtype: fp32 weighting).
//
// One wave per (token, piece of 64 blocks = 1024 elements).  Lane l owns
// block b = 64*piece + l: per slot row it loads the block's 8 code bytes
// and its scale byte (wave loads of 512 and 64 contiguous bytes) through
// buffer descriptors whose base is the row (wave-uniform), and the row's
// rowscale; the loads of up to 8 slots are issued before any is used.  A
// masked or dropped slot gets an empty descriptor (its loads return 0) and
// weight 0, so it adds +0 to every sum, which leaves the sum unchanged: a
// sum that starts at +0 never becomes -0 in round-to-nearest.  That keeps
// the slot loop free of per-slot branches.  The E2M1 values come from
// gfx950's v_cvt_scalef32_pk_f32_fp4 with scale 1.0 (two exact values per
// instruction), the E4M3 scale from v_cvt_f32_fp8 (exact; NaN for the
// codes 0x7F and 0xFF); tests/test_gpu_conversions.py checks both against
// the software decodes on every byte.  The block scale and the element
// product are ordinary fp32 multiplies in the order above.  A row is 4034
// bytes instead of 14336 for bf16 at H = 7168, so the kernel reads 3.6x
// fewer bytes than ep_combine; it is bound by the VALU: three fp32
// operations per element and slot (packed fp32 math stays off).
#include "epx_device.h"

namespace epx {
namespace {

constexpr int kCqThreads = 128;  // two waves per workgroup, as the bf16 gathers
constexpr int kCqWaves = kCqThreads / kWave;
constexpr int kCqBatch = 8;      // slots whose loads are in flight together

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3: 32-bit data, raw addressing

// The 16 E2M1 values of one block: 8 code bytes, element 2j in the low
// nibble of byte j.
__device__ __forceinline__ void e2m1_block(v2u c, float (&v)[16]) {
    f32x2_t p;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 0);
    v[0] = p.x, v[1] = p.y;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 1);
    v[2] = p.x, v[3] = p.y;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 2);
    v[4] = p.x, v[5] = p.y;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 3);
    v[6] = p.x, v[7] = p.y;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 0);
    v[8] = p.x, v[9] = p.y;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 1);
    v[10] = p.x, v[11] = p.y;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 2);
    v[12] = p.x, v[13] = p.y;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 3);
    v[14] = p.x, v[15] = p.y;
}

template <bool WEIGHTED>
__global__ __launch_bounds__(kCqThreads) void k_combine_nvfp4(CombineNvfp4Args a, int32_t pieces) {
    const int32_t wave = uniform((int32_t)(blockIdx.x * kCqWaves + threadIdx.x / kWave));
    const int32_t t = wave / pieces;
    if (t >= a.T) return;
    const int32_t piece = wave - t * pieces;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t nblk = a.H / 16;
    const int32_t b = piece * kWave + lane;  // lanes past the last block read past their descriptors: 0

    // Slot row and weight of slot `lane` (both loads issued before either is
    // tested); rows outside [0, R) read as -1 and get weight 0.
    const int32_t r_raw = a.token_row[(int64_t)t * a.Kp + min(lane, a.Kp - 1)];
    float w_lane = 1.0f;
    if (WEIGHTED) w_lane = a.probs[(int64_t)t * a.K + min(lane, a.K - 1)];
    // Left to itself the scheduler tests the row before it sends the weight
    // load: two round trips before the payload loads can start.
    __builtin_amdgcn_sched_barrier(0);
    const int32_t my_row = (lane < a.Kp && r_raw >= 0 && r_raw < a.R) ? r_raw : -1;
    const float my_w = my_row < 0 ? 0.0f : (lane < a.K ? w_lane : 1.0f);

    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    const int32_t cstride = a.H / 2;
    for (int32_t k0 = 0; k0 < a.Kp; k0 += kCqBatch) {
        v2u cw[kCqBatch];
        uint32_t sc[kCqBatch], rs[kCqBatch];
#pragma unroll
        for (int kk = 0; kk < kCqBatch; ++kk) {
            const int32_t row = k0 + kk < a.Kp ? __builtin_amdgcn_readlane(my_row, k0 + kk) : -1;
            const bool valid = row >= 0;
            const int64_t r = valid ? row : 0;
            const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(a.codes + r * cstride), (short)0, valid ? cstride : 0, kBufferFlags);
            const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(a.scales + r * nblk), (short)0, valid ? nblk : 0, kBufferFlags);
            // the row's rowscale through an empty descriptor as well: a
            // conditional load here would be waited on at once, with the
            // loads of the earlier slots, one round trip per slot
            const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(a.rowscale + r), (short)0, valid ? 2 : 0, kBufferFlags);
            cw[kk] = __builtin_amdgcn_raw_buffer_load_b64(rc, 8 * b, 0, 0);
            sc[kk] = __builtin_amdgcn_raw_buffer_load_b8(rsc, b, 0, 0);
            rs[kk] = __builtin_amdgcn_raw_buffer_load_b16(rrs, 0, 0, 0);
        }
#pragma unroll
        for (int kk = 0; kk < kCqBatch; ++kk) {
            if (k0 + kk >= a.Kp) break;
            const float w = WEIGHTED ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), k0 + kk)) : 1.0f;
            // block scale * float(rowscale)
            const float bs = __builtin_amdgcn_cvt_f32_fp8((int)sc[kk], 0) * bf16_lo(rs[kk]);
            float v[16];
            e2m1_block(cw[kk], v);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float xh = v[i] * bs;
                if (WEIGHTED) {
                    const float p = w * xh;
                    acc[i] = acc[i] + p;
                } else {
                    acc[i] = acc[i] + xh;
                }
            }
        }
    }
    if (b >= nblk) return;
    v4u* dst = reinterpret_cast<v4u*>(a.y + (int64_t)t * a.H + 16 * (int64_t)b);
    v4u o0, o1;
    o0.x = pack_bf16x2(acc[0], acc[1]);
    o0.y = pack_bf16x2(acc[2], acc[3]);
    o0.z = pack_bf16x2(acc[4], acc[5]);
    o0.w = pack_bf16x2(acc[6], acc[7]);
    o1.x = pack_bf16x2(acc[8], acc[9]);
    o1.y = pack_bf16x2(acc[10], acc[11]);
    o1.z = pack_bf16x2(acc[12], acc[13]);
    o1.w = pack_bf16x2(acc[14], acc[15]);
    __builtin_nontemporal_store(o0, dst);
    __builtin_nontemporal_store(o1, dst + 1);
}

}  // namespace

int combine_nvfp4_pieces(int32_t H) { return (H / 16 + kWave - 1) / kWave; }

hipError_t launch_combine_nvfp4(const CombineNvfp4Args& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int32_t pieces = combine_nvfp4_pieces(a.H);
    const dim3 blocks((unsigned)(((int64_t)a.T * pieces + kCqWaves - 1) / kCqWaves));
    if (a.probs != nullptr)
        hipLaunchKernelGGL(k_combine_nvfp4<true>, blocks, dim3(kCqThreads), 0, stream, a, pieces);
    else
        hipLaunchKernelGGL(k_combine_nvfp4<false>, blocks, dim3(kCqThreads), 0, stream, a, pieces);
    return hipGetLastError();
}

}  // namespace epx
