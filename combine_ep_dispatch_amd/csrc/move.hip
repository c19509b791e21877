// Payload movement for MoE expert-parallel dispatch and combine on gfx950.
//
//  k_scatter<false>  dispatch: recv[token_row[t,k]] = x[t] (bit copy)
//                    (NeMo AutoModel fused_a2a page, HybridEPDispatch.forward
//                    with fuse_permute)
//  k_scatter<true>   combine backward: grad_out[token_row[t,k]] =
//                    bf16(w_k * grad_y[t]) (HybridEPCombine.backward:
//                    redispatch through the saved layout)
//  k_gather<W>       combine / dispatch backward: y[t] = bf16(sum_k w_k *
//                    src[token_row[t,k]]), fp32, ascending k
//                    (HybridEPCombine.forward, HybridEPDispatch.backward;
//                    NeMo AutoModel token_dispatcher page,
//                    TokenDispatcherConfig.moe_router_dtype: fp32 weighting)
//
// All three are HBM-bound row movers.  One wave64 owns one (token, piece of
// the hidden dimension): a piece is 64 lanes x VPL 16-byte vectors, so every
// load and store instruction of the wave covers 1 KiB of one row,
// contiguous.  The token index is wave-uniform, so token_row and probs come
// in through scalar loads.  A token's x row is read once and written K'
// times; combine issues the loads of up to 8 slots before reducing them in
// slot order.
#include "epx_device.h"

namespace epx {
namespace {

constexpr int kMoveThreads = 256;
constexpr int kMoveWaves = kMoveThreads / kWave;
constexpr int kVpl = 2;       // 16-byte vectors per lane per piece
constexpr int kSlotBatch = 8;  // slots whose loads are in flight together in k_gather

__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float w) {
    uint4 o;
    o.x = pack_bf16x2(w * bf16_lo(v.x), w * bf16_hi(v.x));
    o.y = pack_bf16x2(w * bf16_lo(v.y), w * bf16_hi(v.y));
    o.z = pack_bf16x2(w * bf16_lo(v.z), w * bf16_hi(v.z));
    o.w = pack_bf16x2(w * bf16_lo(v.w), w * bf16_hi(v.w));
    return o;
}

template <bool SCALED>
__global__ __launch_bounds__(kMoveThreads) void k_scatter(MoveArgs a, int32_t Hv, int32_t pieces) {
    const int32_t wave = uniform((int32_t)(blockIdx.x * kMoveWaves + threadIdx.x / kWave));
    const int32_t t = wave / pieces;
    if (t >= a.T) return;
    const int32_t piece = wave - t * pieces;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t v0 = piece * (kWave * kVpl) + lane;

    const uint4* src = static_cast<const uint4*>(a.src) + (int64_t)t * Hv;
    uint4 buf[kVpl];
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
        const int32_t v = v0 + i * kWave;
        buf[i] = v < Hv ? src[v] : make_uint4(0, 0, 0, 0);
    }
    const int32_t* tr = a.token_row + (int64_t)t * a.Kp;
    for (int32_t k = 0; k < a.Kp; ++k) {
        const int32_t row = tr[k];
        if (row < 0 || row >= a.R) continue;
        uint4* dst = static_cast<uint4*>(a.dst) + (int64_t)row * Hv;
        if (SCALED) {
            const float w = (a.probs != nullptr && k < a.K) ? a.probs[(int64_t)t * a.K + k] : 1.0f;
#pragma unroll
            for (int i = 0; i < kVpl; ++i) {
                const int32_t v = v0 + i * kWave;
                if (v < Hv) dst[v] = scale_bf16x8(buf[i], w);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kVpl; ++i) {
                const int32_t v = v0 + i * kWave;
                if (v < Hv) dst[v] = buf[i];
            }
        }
    }
}

__device__ __forceinline__ void accumulate(float (&acc)[8], uint4 v, float w, bool weighted) {
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = bf16_lo(q[j]), hi = bf16_hi(q[j]);
        if (weighted) {
            const float plo = w * lo, phi = w * hi;
            acc[2 * j] = acc[2 * j] + plo;
            acc[2 * j + 1] = acc[2 * j + 1] + phi;
        } else {
            acc[2 * j] = acc[2 * j] + lo;
            acc[2 * j + 1] = acc[2 * j + 1] + hi;
        }
    }
}

template <bool WEIGHTED>
__global__ __launch_bounds__(kMoveThreads) void k_gather(MoveArgs a, int32_t Hv, int32_t pieces) {
    const int32_t wave = uniform((int32_t)(blockIdx.x * kMoveWaves + threadIdx.x / kWave));
    const int32_t t = wave / pieces;
    if (t >= a.T) return;
    const int32_t piece = wave - t * pieces;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t v0 = piece * (kWave * kVpl) + lane;
    const int32_t* tr = a.token_row + (int64_t)t * a.Kp;
    const uint4* src = static_cast<const uint4*>(a.src);

    float acc[kVpl][8];
#pragma unroll
    for (int i = 0; i < kVpl; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    for (int32_t k0 = 0; k0 < a.Kp; k0 += kSlotBatch) {
        int32_t rows[kSlotBatch];
        float wts[kSlotBatch];
        uint4 buf[kSlotBatch][kVpl];
#pragma unroll
        for (int kk = 0; kk < kSlotBatch; ++kk) {
            const int32_t k = k0 + kk;
            const int32_t r = k < a.Kp ? tr[k] : -1;
            rows[kk] = r < a.R ? r : -1;
            wts[kk] = (WEIGHTED && k < a.K) ? a.probs[(int64_t)t * a.K + (k < a.K ? k : 0)] : 1.0f;
        }
#pragma unroll
        for (int kk = 0; kk < kSlotBatch; ++kk) {
            const uint4* r = src + (int64_t)(rows[kk] < 0 ? 0 : rows[kk]) * Hv;
#pragma unroll
            for (int i = 0; i < kVpl; ++i) {
                const int32_t v = v0 + i * kWave;
                buf[kk][i] = (rows[kk] >= 0 && v < Hv) ? r[v] : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int kk = 0; kk < kSlotBatch; ++kk) {
            if (rows[kk] < 0) continue;  // masked or dropped: contributes nothing
#pragma unroll
            for (int i = 0; i < kVpl; ++i) accumulate(acc[i], buf[kk][i], wts[kk], WEIGHTED);
        }
    }
    uint4* dst = static_cast<uint4*>(a.dst) + (int64_t)t * Hv;
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
        const int32_t v = v0 + i * kWave;
        if (v < Hv) {
            uint4 o;
            o.x = pack_bf16x2(acc[i][0], acc[i][1]);
            o.y = pack_bf16x2(acc[i][2], acc[i][3]);
            o.z = pack_bf16x2(acc[i][4], acc[i][5]);
            o.w = pack_bf16x2(acc[i][6], acc[i][7]);
            dst[v] = o;
        }
    }
}

struct Grid {
    int32_t Hv, pieces;
    dim3 blocks;
};

Grid move_grid(const MoveArgs& a) {
    Grid g;
    g.Hv = a.H / 8;
    g.pieces = (g.Hv + kWave * kVpl - 1) / (kWave * kVpl);
    const int64_t waves = (int64_t)a.T * g.pieces;
    g.blocks = dim3((unsigned)((waves + kMoveWaves - 1) / kMoveWaves));
    return g;
}

// Zero the byte range [b0, b1) of `base` with 16-byte stores where aligned.
__device__ void zero_bytes(uint8_t* base, int64_t b0, int64_t b1) {
    const int64_t a0 = (b0 + 15) & ~int64_t(15), a1 = b1 & ~int64_t(15);
    if (a0 >= a1) {
        for (int64_t i = b0 + threadIdx.x; i < b1; i += blockDim.x) base[i] = 0;
        return;
    }
    for (int64_t i = b0 + threadIdx.x; i < a0; i += blockDim.x) base[i] = 0;
    for (int64_t i = a1 + threadIdx.x; i < b1; i += blockDim.x) base[i] = 0;
    uint4* v = reinterpret_cast<uint4*>(base + a0);
    const int64_t nv = (a1 - a0) / 16;
    for (int64_t i = threadIdx.x; i < nv; i += blockDim.x) v[i] = make_uint4(0, 0, 0, 0);
}

__global__ __launch_bounds__(256) void k_zero_pad_rows(uint8_t* base, int64_t row_bytes, ep_layout_t L,
                                                       int32_t G, int32_t A, int32_t C, int64_t R) {
    const int32_t g = blockIdx.x;
    const int32_t s = g / G, gl = g - s * G;
    const int32_t cnt = L.counts[g];
    const int32_t al = ((cnt + A - 1) / A) * A;
    const int32_t off = L.row_offsets[s * (G + 1) + gl];
    int64_t first = (int64_t)off + cnt, last = (int64_t)off + al;
    if (C > 0) {
        if (first > C) first = C;
        if (last > C) last = C;
    }
    if (first >= last) return;
    int64_t r0 = (int64_t)L.seg_base[s] + first, r1 = (int64_t)L.seg_base[s] + last;
    if (r0 < 0) r0 = 0;
    if (r1 > R) r1 = R;  // never past the buffer, whatever the layout holds
    if (r0 >= r1) return;
    zero_bytes(base, r0 * row_bytes, r1 * row_bytes);
}

}  // namespace

hipError_t launch_scatter(const MoveArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const Grid g = move_grid(a);
    hipLaunchKernelGGL(k_scatter<false>, g.blocks, dim3(kMoveThreads), 0, stream, a, g.Hv, g.pieces);
    return hipGetLastError();
}

hipError_t launch_gather_reduce(const MoveArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const Grid g = move_grid(a);
    if (a.probs != nullptr)
        hipLaunchKernelGGL(k_gather<true>, g.blocks, dim3(kMoveThreads), 0, stream, a, g.Hv, g.pieces);
    else
        hipLaunchKernelGGL(k_gather<false>, g.blocks, dim3(kMoveThreads), 0, stream, a, g.Hv, g.pieces);
    return hipGetLastError();
}

hipError_t launch_scatter_scaled(const MoveArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const Grid g = move_grid(a);
    hipLaunchKernelGGL(k_scatter<true>, g.blocks, dim3(kMoveThreads), 0, stream, a, g.Hv, g.pieces);
    return hipGetLastError();
}

hipError_t launch_zero_pad_rows(void* base, int64_t row_bytes, const ep_layout_t& L, int32_t S, int32_t G,
                                int32_t A, int32_t C, int64_t R, hipStream_t stream) {
    const int32_t NG = S * G;
    if (NG == 0 || row_bytes == 0 || A == 1 || R == 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_pad_rows, dim3((unsigned)NG), dim3(256), 0, stream,
                       static_cast<uint8_t*>(base), row_bytes, L, G, A, C, R);
    return hipGetLastError();
}

}  // namespace epx
