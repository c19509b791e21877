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
// All three are HBM-bound row movers.  A piece is 64 lanes x VPL 16-byte
// vectors of one row, so each wave load or store instruction moves 1 KiB,
// contiguous.  When the pieces tile the row exactly the lane guards vanish.
//  - The scatters run one wave per (token, piece, slot), with 2 KiB pieces:
//    the wave loads its row index, weight and payload piece together (one
//    round trip), then issues its nontemporal stores.  The K' slot waves
//    of a (token, piece) are consecutive waves on one XCD (see
//    ScatterGrid), so a token's x row is fetched from HBM once and re-read
//    by the other slots from L2, and no wave is idle whatever K' is (with
//    K' = 9, slot blocks of 8 waves left 7 of every 16 idle, and the
//    combine-backward scatter of a cold input took 133 instead of 107 us).
//    Workgroups of 8 waves: 4 shortened the DeepSeek-V3 step (409 against
//    413 us) but slowed the weighted scatter of a cold input (116 against
//    101 us), and with it the skewed workload's step (479 against 462 us).
//    Short waves with streaming stores keep many more
//    writes in flight than one wave storing all K' copies: at DeepSeek-V3
//    size the dispatch scatter went from 106 to ~92 us and the
//    combine-backward one from 102 to ~90.  The (token, piece, slot) of a
//    wave comes from the workgroup index with masks, shifts and multiplies
//    by precomputed reciprocals: the per-wave scalar work bounds these
//    short waves, and a division there cost more than the store.
//  - The gathers run one wave per (token, piece): the token's K' receive
//    rows (and weights) arrive with one vector load, lane k holding slot k,
//    are broadcast with v_readlane so every row address is wave-uniform, and
//    the loads of up to 8 slots are issued before they are reduced in slot
//    order.  The output row is written with nontemporal stores: with plain
//    stores its lines stayed dirty in L2 and the MALL, and the next kernel
//    paid for their write-back while reading its own cold input.  At
//    DeepSeek-V3 size the whole six-kernel step went from ~455 to ~417 us,
//    and combine alone from 91 to 88 us.  Stores through a buffer
//    descriptor with device scope (sc1) ran the gathers 2% faster back to
//    back (86.2 against 87.9 us) and made the step slower (451 against
//    413 us): their lines wait in the MALL and the next kernel writes them
//    back.  The same holds for the scatters (step 434 us).
//  - Both movers sit at the ceiling of their memory pattern on MI355X: a
//    probe that issues the gathers' loads and stores at DeepSeek-V3 size
//    (the same rows, 8 nontemporal 1 KiB reads and one nontemporal 1 KiB
//    write per wave) with no arithmetic took 87.2 us, combine 88.0 us; the
//    same probe without the writes took 69 us (6.8 TB/s of reads).
#include "epx_device.h"

#ifndef EPX_SCATTER_VPL
#define EPX_SCATTER_VPL 2
#endif
#ifndef EPX_SCATTER_WAVES
#define EPX_SCATTER_WAVES 8  // waves per scatter workgroup (one (token, piece, slot) each)
#endif
#ifndef EPX_GATHER_VPL
#define EPX_GATHER_VPL 1
#endif
#ifndef EPX_NT_LOADS
#define EPX_NT_LOADS 1
#endif
#ifndef EPX_SCATTER_NT_LOADS
#define EPX_SCATTER_NT_LOADS 0
#endif
#ifndef EPX_NT_STORES
#define EPX_NT_STORES 1  // gathers: nontemporal output stores
#endif
#ifndef EPX_SCATTER_NT_STORES
#define EPX_SCATTER_NT_STORES 1
#endif
// Cache-policy bits for the output stores (1 = sc0, 2 = nt, 16 = sc1), -1
// for the plain global forms above.
#ifndef EPX_GATHER_STORE_AUX
#define EPX_GATHER_STORE_AUX -1
#endif
#ifndef EPX_GATHER_LOAD_AUX
#define EPX_GATHER_LOAD_AUX -1
#endif
#ifndef EPX_SCATTER_STORE_AUX
#define EPX_SCATTER_STORE_AUX -1
#endif

namespace epx {
namespace {

constexpr int kMoveThreads = 256;
constexpr int kMoveWaves = kMoveThreads / kWave;
#ifndef EPX_GATHER_THREADS
#define EPX_GATHER_THREADS 128  // 2 waves: 1.5-2% faster than 1, 4 or 8 at DeepSeek-V3 size
#endif
constexpr int kGatherThreads = EPX_GATHER_THREADS;
constexpr int kGatherWaves = kGatherThreads / kWave;
constexpr int kSlotBatch = 8;  // slots whose loads are in flight together in k_gather

// One launch holds at most 2^32 - 1 work-items per grid dimension (the
// dispatch packet's grid size is a 32-bit count of work-items), so the
// movers split larger batches into token chunks.
constexpr int64_t kMaxLaunchItems = 0xFFFFFFFFll;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4u load_stream(const v4u* p) {
#if EPX_NT_LOADS
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

__device__ __forceinline__ v4u load_scatter_src(const v4u* p) {
#if EPX_SCATTER_NT_LOADS
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data, raw addressing
constexpr int kCachePolicyNt = 2;         // buffer load/store cache-policy bit: nontemporal

// 16-byte store to vector v of a wave-uniform row base through a buffer
// descriptor carrying the cache-policy bits AUX.
template <int AUX>
__device__ __forceinline__ void store_policy(v4u* row, int32_t v, int32_t row_bytes, v4u val) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, (short)0, row_bytes, kBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b128(val, rs, v * 16, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ v4u load_policy(const v4u* row, int32_t v, int32_t row_bytes) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<v4u*>(row), (short)0, row_bytes, kBufferWord3);
    return __builtin_amdgcn_raw_buffer_load_b128(rs, v * 16, 0, AUX);
}

__device__ __forceinline__ void store_scatter_dst(v4u* p, v4u v) {
#if EPX_SCATTER_NT_STORES
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

__device__ __forceinline__ void store_stream(v4u* p, v4u v) {
#if EPX_NT_STORES
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

__device__ __forceinline__ v4u scale_bf16x8(v4u v, float w) {
    v4u o;
    o.x = pack_bf16x2(w * bf16_lo(v.x), w * bf16_hi(v.x));
    o.y = pack_bf16x2(w * bf16_lo(v.y), w * bf16_hi(v.y));
    o.z = pack_bf16x2(w * bf16_lo(v.z), w * bf16_hi(v.z));
    o.w = pack_bf16x2(w * bf16_lo(v.w), w * bf16_hi(v.w));
    return o;
}

// Slot rows of token t in lane k (k < Kp), -1 elsewhere; rows outside [0, R)
// read as -1 so that no later address can leave the buffers.
__device__ __forceinline__ int32_t slot_row_of_lane(const MoveArgs& a, int32_t t, int lane) {
    int32_t r = -1;
    if (lane < a.Kp) {
        r = a.token_row[(int64_t)t * a.Kp + lane];
        if (r >= a.R) r = -1;
    }
    return r;
}

// Slot row and weight of token t in lane k together (row as above; weight
// probs[t,k] for k < K, 1 for the shared slot, lanes past it and without
// probs).  Both loads are issued before either value is tested: each reads
// at a lane index clamped into the token's slots (K >= 1) instead of under
// a lane branch, whose result test would otherwise wait for the row before
// the weight load is sent (a second round trip to memory before the payload
// loads can start).
__device__ __forceinline__ void slot_row_and_weight_of_lane(const MoveArgs& a, int32_t t, int lane, int32_t& row,
                                                            float& w) {
    const int32_t r = a.token_row[(int64_t)t * a.Kp + min(lane, a.Kp - 1)];
    float p = 1.0f;
    if (a.probs != nullptr) p = a.probs[(int64_t)t * a.K + min(lane, a.K - 1)];
    row = (lane < a.Kp && r < a.R) ? r : -1;
    w = lane < a.K ? p : 1.0f;
}

// Geometry of the scatter grid.  Workgroups are handed to the 8 XCDs
// round-robin by index, and the K' slot waves of one (token, piece) should
// share an XCD's L2 so that the piece is fetched once.  Workgroup b = 8q + x
// runs on XCD x; with W = EPX_SCATTER_WAVES waves per workgroup, that XCD's
// waves j = W q + w (w = wave in the workgroup) take the (token, piece,
// slot) triples of (token, piece) numbers x, x + 8, x + 16, ... in order:
// local pair l = j / K', slot k = j - l K', pair rest = 8 l + x.  Every
// wave has a slot, whatever K' is, and the K' waves of a pair are
// consecutive on one XCD (with K' = W = 8, one workgroup per pair).  Then t = rest / pieces and p = rest - t * pieces.
// The divisions are multiplies by host-computed reciprocals, exact below
// 2^31 where the 64-bit product cannot overflow; the launcher keeps both
// numerators below 2^26.  t0 is added to t for launches split in token
// chunks [t0, t1).  Indices past the last (token, piece) exit.
struct ScatterGrid {
    int32_t Hv, pieces, t0, t1;  // this launch covers tokens [t0, t1)
    uint64_t div_mul, kp_mul;
    uint32_t div_shift, kp_shift;
};

template <bool SCALED, bool FULL>
__global__ __launch_bounds__(EPX_SCATTER_WAVES * kWave) void k_scatter(MoveArgs a, ScatterGrid g) {
    constexpr int VPL = EPX_SCATTER_VPL;
    const uint32_t j = (blockIdx.x >> 3) * EPX_SCATTER_WAVES + uniform((uint32_t)(threadIdx.x / kWave));
    const uint32_t l = (uint32_t)(((uint64_t)j * g.kp_mul) >> g.kp_shift);
    const int32_t k = (int32_t)(j - l * (uint32_t)a.Kp);
    const uint32_t rest = (l << 3) | (blockIdx.x & 7u);
    const uint32_t tr = (uint32_t)(((uint64_t)rest * g.div_mul) >> g.div_shift);
    const int32_t p = (int32_t)(rest - tr * (uint32_t)g.pieces);
    const int32_t t = g.t0 + (int32_t)tr;
    if (t >= g.t1) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t Hv = g.Hv;

    // Row, weight and payload depend only on (t, k, p): all loads go out
    // before any is waited on.
    const int32_t row_raw = a.token_row[(int64_t)t * a.Kp + k];
    float w = 1.0f;
    if (SCALED && a.probs != nullptr && k < a.K) w = a.probs[(int64_t)t * a.K + k];
    const v4u* src = reinterpret_cast<const v4u*>(a.src) + (int64_t)t * Hv;
    v4u buf[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int32_t v = (p * VPL + i) * kWave + lane;
        buf[i] = (FULL || v < Hv) ? load_scatter_src(src + v) : v4u{0, 0, 0, 0};
    }
    // The compiler would otherwise sink the payload loads (and the
    // destination's kernel arguments) below the row test and pay two round
    // trips per wave.
#pragma unroll
    for (int i = 0; i < VPL; ++i) asm volatile("" ::"v"(buf[i].x), "v"(buf[i].y), "v"(buf[i].z), "v"(buf[i].w));
    void* const dst_base = a.dst;
    const int64_t R = a.R;
    asm volatile("" ::"s"(dst_base), "s"(R));
    const int32_t row = uniform(row_raw);
    if (row < 0 || row >= R) return;  // masked, dropped, or outside the buffer
    v4u* dst = reinterpret_cast<v4u*>(dst_base) + (int64_t)row * Hv;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int32_t v = (p * VPL + i) * kWave + lane;
        if (FULL || v < Hv) {
            const v4u val = SCALED ? scale_bf16x8(buf[i], w) : buf[i];
            if constexpr (EPX_SCATTER_STORE_AUX >= 0)
                store_policy<EPX_SCATTER_STORE_AUX>(dst, v, Hv * 16, val);
            else
                store_scatter_dst(dst + v, val);
        }
    }
}

__device__ __forceinline__ void accumulate(float (&acc)[8], v4u v, float w, bool weighted) {
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

// Tokens [t0, t1) of the batch, one wave per (token, piece).
template <bool WEIGHTED, bool FULL>
__global__ __launch_bounds__(kGatherThreads) void k_gather(MoveArgs a, int32_t Hv, int32_t pieces, int32_t t0,
                                                           int32_t t1) {
    constexpr int VPL = EPX_GATHER_VPL;
    const int32_t wave = uniform((int32_t)(blockIdx.x * kGatherWaves + threadIdx.x / kWave));
    const int32_t tr = wave / pieces;
    const int32_t t = t0 + tr;
    if (t >= t1) return;
    const int32_t piece = wave - tr * pieces;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t v0 = piece * (kWave * VPL) + lane;
    const v4u* src = reinterpret_cast<const v4u*>(a.src);

    int32_t my_row;
    float my_w = 1.0f;
    if (WEIGHTED)
        slot_row_and_weight_of_lane(a, t, lane, my_row, my_w);
    else
        my_row = slot_row_of_lane(a, t, lane);

    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    for (int32_t k0 = 0; k0 < a.Kp; k0 += kSlotBatch) {
        int32_t rows[kSlotBatch];
        v4u buf[kSlotBatch][VPL];
#pragma unroll
        for (int kk = 0; kk < kSlotBatch; ++kk) {
            const int32_t k = k0 + kk;
            rows[kk] = k < a.Kp ? __builtin_amdgcn_readlane(my_row, k) : -1;
            const v4u* r = src + (int64_t)(rows[kk] < 0 ? 0 : rows[kk]) * Hv;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int32_t v = v0 + i * kWave;
                if constexpr (EPX_GATHER_LOAD_AUX >= 0)
                    buf[kk][i] = (rows[kk] >= 0 && (FULL || v < Hv)) ? load_policy<EPX_GATHER_LOAD_AUX>(r, v, Hv * 16)
                                                                      : v4u{0, 0, 0, 0};
                else
                    buf[kk][i] = (rows[kk] >= 0 && (FULL || v < Hv)) ? load_stream(r + v) : v4u{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int kk = 0; kk < kSlotBatch; ++kk) {
            if (rows[kk] < 0) continue;  // masked or dropped: contributes nothing
            const float w =
                WEIGHTED ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), k0 + kk)) : 1.0f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) accumulate(acc[i], buf[kk][i], w, WEIGHTED);
        }
    }
    v4u* dst = reinterpret_cast<v4u*>(a.dst) + (int64_t)t * Hv;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int32_t v = v0 + i * kWave;
        if (FULL || v < Hv) {
            v4u o;
            o.x = pack_bf16x2(acc[i][0], acc[i][1]);
            o.y = pack_bf16x2(acc[i][2], acc[i][3]);
            o.z = pack_bf16x2(acc[i][4], acc[i][5]);
            o.w = pack_bf16x2(acc[i][6], acc[i][7]);
            if constexpr (EPX_GATHER_STORE_AUX >= 0)
                store_policy<EPX_GATHER_STORE_AUX>(dst, v, Hv * 16, o);
            else
                store_stream(dst + v, o);
        }
    }
}

// Router-probability gradient: grad_probs[t,k] = <grad_y[t], expert_out[row(t,k)]>
// (the derivative of combine's weighted sum with respect to its weights;
// NeMo AutoModel fused_a2a page, HybridEPDispatch.backward returns a
// probability gradient beside the hidden-state gradient).  One workgroup per
// token; thread i takes 16-byte vectors i, i+256, ... of the row and keeps
// one fp32 partial per slot (multiply, then add: no contraction), for up to
// 8 slots per pass.  The partials are reduced by a fixed butterfly inside
// each wave and then across the 4 waves in wave order, so the result is
// deterministic.  Masked, invalid and dropped slots get 0.
__global__ __launch_bounds__(kMoveThreads) void k_probs_grad(MoveArgs a, int32_t Hv, float* grad_probs) {
    __shared__ float s_part[kMoveWaves][kSlotBatch];
    const int32_t t = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int32_t my_row = slot_row_of_lane(a, t, lane);
    const v4u* gy = reinterpret_cast<const v4u*>(a.src) + (int64_t)t * Hv;
    const v4u* out = reinterpret_cast<const v4u*>(a.dst);
    for (int32_t k0 = 0; k0 < a.K; k0 += kSlotBatch) {
        int32_t rows[kSlotBatch];
        float acc[kSlotBatch];
#pragma unroll
        for (int kk = 0; kk < kSlotBatch; ++kk) {
            rows[kk] = k0 + kk < a.K ? __builtin_amdgcn_readlane(my_row, k0 + kk) : -1;
            acc[kk] = 0.0f;
        }
        for (int32_t v = threadIdx.x; v < Hv; v += kMoveThreads) {
            const v4u g = gy[v];
            const uint32_t gq[4] = {g.x, g.y, g.z, g.w};
            // Every slot's load goes out before any is used: under a
            // per-slot branch the compiler waited on each load in turn.  A
            // masked or dropped slot loads through an empty descriptor (no
            // memory access, zeros) and is skipped below.
            v4u ov[kSlotBatch];
#pragma unroll
            for (int kk = 0; kk < kSlotBatch; ++kk) {
                const bool valid = rows[kk] >= 0;
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<v4u*>(out + (int64_t)(valid ? rows[kk] : 0) * Hv), (short)0, valid ? Hv * 16 : 0,
                    kBufferWord3);
                ov[kk] = __builtin_amdgcn_raw_buffer_load_b128(rs, v * 16, 0, kCachePolicyNt);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < kSlotBatch; ++kk) {
                if (rows[kk] < 0) continue;
                const v4u o = ov[kk];
                const uint32_t oq[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p0 = bf16_lo(gq[j]) * bf16_lo(oq[j]);
                    acc[kk] = acc[kk] + p0;
                    const float p1 = bf16_hi(gq[j]) * bf16_hi(oq[j]);
                    acc[kk] = acc[kk] + p1;
                }
            }
        }
#pragma unroll
        for (int kk = 0; kk < kSlotBatch; ++kk) {
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) acc[kk] = acc[kk] + __shfl_xor(acc[kk], o, kWave);
        }
        if (lane == 0) {
#pragma unroll
            for (int kk = 0; kk < kSlotBatch; ++kk) s_part[w][kk] = acc[kk];
        }
        __syncthreads();
        if (threadIdx.x < kSlotBatch && k0 + (int)threadIdx.x < a.K) {
            const int kk = threadIdx.x;
            float sum = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < kMoveWaves; ++w2) sum = sum + s_part[w2][kk];
            grad_probs[(int64_t)t * a.K + k0 + kk] = sum;  // rows < 0 summed zeros: exactly 0
        }
        __syncthreads();
    }
}

struct Grid {
    int32_t Hv, pieces;
    bool full;
};

Grid move_grid(const MoveArgs& a, int vpl) {
    Grid g;
    g.Hv = a.H / 8;
    const int per_piece = kWave * vpl;
    g.pieces = (g.Hv + per_piece - 1) / per_piece;
    g.full = g.Hv % per_piece == 0;
    return g;
}

// q / d = (q * m) >> (32 + l) with l = ceil(log2 d) and
// m = floor(2^(32+l) / d) + 1 (Granlund and Montgomery, division by
// invariant integers): exact for every q < 2^32, and m < 2^33, so the 64-bit
// product q * m is exact for q < 2^31.
void reciprocal(uint32_t d, uint64_t& m, uint32_t& shift) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    shift = 32 + l;
    m = (uint64_t)(((unsigned __int128)1 << (32 + l)) / d) + 1;
}

template <bool SCALED>
hipError_t scatter(const MoveArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    ScatterGrid g;
    g.Hv = a.H / 8;
    const int per_piece = kWave * EPX_SCATTER_VPL;
    g.pieces = (g.Hv + per_piece - 1) / per_piece;
    const bool full = g.Hv % per_piece == 0;
    reciprocal((uint32_t)g.pieces, g.div_mul, g.div_shift);
    reciprocal((uint32_t)a.Kp, g.kp_mul, g.kp_shift);
    // A launch covers the (token, piece) pairs rounded up to a multiple of
    // 8, times K' waves, in workgroups of EPX_SCATTER_WAVES waves per XCD.
    const int64_t max_blocks = kMaxLaunchItems / (EPX_SCATTER_WAVES * kWave);
    const int64_t chunk = ((max_blocks - 8) / a.Kp * EPX_SCATTER_WAVES - 8) / g.pieces;
    if (chunk < 1) return hipErrorInvalidValue;
    for (int64_t t0 = 0; t0 < a.T; t0 += chunk) {
        const int64_t tokens = a.T - t0 < chunk ? a.T - t0 : chunk;
        const int64_t pairs_per_xcd = ((tokens * g.pieces + 7) & ~int64_t(7)) >> 3;
        const int64_t blocks_per_xcd = (pairs_per_xcd * a.Kp + EPX_SCATTER_WAVES - 1) / EPX_SCATTER_WAVES;
        const int64_t n = blocks_per_xcd * 8;
        g.t0 = (int32_t)t0;
        g.t1 = (int32_t)(t0 + tokens);
        if (full)
            hipLaunchKernelGGL((k_scatter<SCALED, true>), dim3((unsigned)n), dim3(EPX_SCATTER_WAVES * kWave), 0,
                               stream, a, g);
        else
            hipLaunchKernelGGL((k_scatter<SCALED, false>), dim3((unsigned)n), dim3(EPX_SCATTER_WAVES * kWave), 0,
                               stream, a, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <bool WEIGHTED>
hipError_t gather(const MoveArgs& a, hipStream_t stream) {
    const Grid g = move_grid(a, EPX_GATHER_VPL);
    const int64_t chunk = kMaxLaunchItems / kGatherThreads * kGatherWaves / g.pieces;
    if (chunk < 1) return hipErrorInvalidValue;
    for (int64_t t0 = 0; t0 < a.T; t0 += chunk) {
        const int64_t tokens = a.T - t0 < chunk ? a.T - t0 : chunk;
        const dim3 blocks((unsigned)((tokens * g.pieces + kGatherWaves - 1) / kGatherWaves));
        const int32_t c0 = (int32_t)t0, c1 = (int32_t)(t0 + tokens);
        if (g.full)
            hipLaunchKernelGGL((k_gather<WEIGHTED, true>), blocks, dim3(kGatherThreads), 0, stream, a, g.Hv, g.pieces,
                               c0, c1);
        else
            hipLaunchKernelGGL((k_gather<WEIGHTED, false>), blocks, dim3(kGatherThreads), 0, stream, a, g.Hv,
                               g.pieces, c0, c1);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
    int64_t r0 = (int64_t)L.seg_base[s] + first, r1 = (int64_t)L.seg_base[s] + last;
    if (r0 < 0) r0 = 0;
    if (r1 > R) r1 = R;  // never past the buffer, whatever the layout holds
    if (r0 >= r1) return;
    zero_bytes(base, r0 * row_bytes, r1 * row_bytes);
}

}  // namespace

hipError_t launch_scatter(const MoveArgs& a, hipStream_t stream) { return scatter<false>(a, stream); }

hipError_t launch_scatter_scaled(const MoveArgs& a, hipStream_t stream) { return scatter<true>(a, stream); }

hipError_t launch_gather_reduce(const MoveArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    return a.probs != nullptr ? gather<true>(a, stream) : gather<false>(a, stream);
}

hipError_t launch_probs_grad(const MoveArgs& a, float* grad_probs, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    hipLaunchKernelGGL(k_probs_grad, dim3((unsigned)a.T), dim3(kMoveThreads), 0, stream, a, a.H / 8, grad_probs);
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
