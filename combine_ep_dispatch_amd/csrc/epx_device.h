// Device-side helpers and kernel launchers shared by the epx HIP sources.
// gfx950 (CDNA4) only: wave64, 64 KiB of LDS per workgroup used at most.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epx.h"

namespace epx {

constexpr int kWave = 64;
constexpr int kMaxSlots = EP_MAX_SLOTS;  // K + shared_expert: one slot per lane

// ---------------------------------------------------------------------------
// Layout pass geometry.
// ---------------------------------------------------------------------------
constexpr int kLayoutThreads = 256;                      // 4 waves
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kWorkspaceHeader = 256;                    // reserved header before the descriptors
// Direct path: the histogram launch stores each tile's per-group counts as a
// row of a [tile][group] table.  Up to this many tiles every rank workgroup
// sums each group's whole column (its prefix over earlier tiles and the
// group total).  Past it the table is cut into chunks of this many rows: a
// launch between the two turns each chunk's counts into prefixes within the
// chunk and writes the chunk's sums to a [chunk][group] table, and every
// rank workgroup sums that table's column and adds its own row: a fixed
// number of loads per workgroup, so the layout's cost stays linear in the
// slots (a whole column per workgroup would grow with the square of the
// tile count).
constexpr int kDirectMaxTiles = 256;
inline int64_t direct_chunks(int64_t tiles) {
    return tiles <= kDirectMaxTiles ? 0 : (tiles + kDirectMaxTiles - 1) / kDirectMaxTiles;
}

// Direct-path column sums: lanes that share one group's column (a power of
// two, lanes * NG <= 256 where NG allows), each summing every lanes-th tile
// with kDirectBatch loads in flight.
constexpr int kDirectBatch = 64;
__host__ __device__ inline int direct_lanes_per_group(int NG) {
    return NG > 128 ? 1 : (NG > 64 ? 2 : (NG > 32 ? 4 : (NG > 16 ? 8 : (NG > 8 ? 16 : (NG > 4 ? 32 : 64)))));
}

// Routed slots per thread in one layout tile (1, 2, 4 or 8).  Smaller tiles
// mean more workgroups, each ranking fewer slots; the cost is more rows in
// each column of the direct count table, and past kDirectBatch per lane a
// column sum takes another round trip to memory.  Measured on MI355X: going
// from 4 or 8 slots per thread down to 2 pays for that extra round trip
// (fewer serial match-any rounds per wave), going from 2 to 1 does not.  So:
// 1 when that fits one batch of loads, else the smallest of 2, 4, 8 that
// keeps one chunk (at most kDirectMaxTiles tiles), else 8.
inline int layout_slots_per_thread(int64_t routed_slots, int NG) {
    auto tiles_at = [&](int spt) {
        return (routed_slots + (int64_t)kLayoutThreads * spt - 1) / ((int64_t)kLayoutThreads * spt);
    };
    if (tiles_at(1) <= (int64_t)kDirectBatch * direct_lanes_per_group(NG) && tiles_at(1) <= kDirectMaxTiles) return 1;
    for (int spt = 2; spt < 8; spt *= 2)
        if (tiles_at(spt) <= kDirectMaxTiles) return spt;
    return 8;
}
inline int64_t layout_tiles(int64_t routed_slots, int NG) {
    const int64_t tile = (int64_t)kLayoutThreads * layout_slots_per_thread(routed_slots, NG);
    const int64_t nt = (routed_slots + tile - 1) / tile;
    return nt < 1 ? 1 : nt;
}

// Up to this many routed slots (two slots per thread of one tile) the
// layout is one launch in which every workgroup ranks all slots in LDS to
// learn the group totals.  Measured on MI355X (DeepSeek-V3 shape), against
// the count path below: 5.0 against 5.8 us at 8 slots, 5.2 against 6.1 at
// 128, 6.0 against 6.2 at 512, 7.4 against 6.2 at 1024 (the serial
// match-any rounds of the whole tile then cost more than the count).
#ifndef EPX_SMALL_MAX_SLOTS
#define EPX_SMALL_MAX_SLOTS 512
#endif
constexpr int64_t kSmallMaxSlots = EPX_SMALL_MAX_SLOTS;

// Up to this many routed slots the layout is one launch in which every
// workgroup counts every slot into per-group LDS counters (split at its own
// tile: the counts before it are its in-group prefix), then ranks its tile
// of 256 slots.  Nothing is read that another workgroup wrote.  Measured on
// MI355X (DeepSeek-V3 shape, uniform and Zipf-1.2 routing), against the two
// kernels: 6.5 against 9.4 us at 1280-2048 slots, 7.0 against 9.4 at 4096,
// 8.2 against 9.5 at 8192, 10.3 against 9.5 at 16384 (every workgroup's
// count of all slots then costs more than the second launch), 16.3 against
// 11.5 at 32768.
constexpr int64_t kCountMaxSlots = 8192;
// Forced with EP_LAYOUT_COUNT the path takes at most this many routed slots:
// every one of its (slots / 256) workgroups counts every slot, so its cost
// grows with the square of the batch (262 144 slots: 1024 workgroups of
// 262 144 LDS additions each).
constexpr int64_t kCountForcedMaxSlots = int64_t(1) << 18;
// Forced with EP_LAYOUT_BARRIER the single pass takes at most this many
// routed slots: every workgroup reads every tile's counts, so its cost grows
// with the square of the tile count (MI355X, 256 groups: 147 us at 2^20
// routed slots, 29 ms at 2^24, against 46 us and 0.22 ms for the default).
constexpr int64_t kBarrierForcedMaxSlots = int64_t(1) << 20;

// Layout kernel paths.
constexpr int kLayoutSinglePass = 0;  // k_layout_sp: ticketed tiles, decoupled look-back
constexpr int kLayoutDirect = 1;      // k_layout_hist + k_layout_rank over a [tile][group] count table
constexpr int kLayoutSmall = 2;       // k_layout_rank alone: one tile, every workgroup ranks it
constexpr int kLayoutCount = 3;       // k_layout_rank alone: every workgroup counts every slot

// Single-pass layout tiles: 256 x {1, 2, 4, 8} slots, the smallest tile
// that gives at most kSpTargetTiles tiles (16, 32 and 64 measured within 1
// us of each other at 8k-32k routed slots).  A workgroup remembers at most
// kSpMaxTilesPerBlock tiles it took, so the single pass needs
// tiles <= 32 x the workgroups that can run at once; a layout call never
// gives it more than kSpMaxTiles tiles (8192 = 32 x one workgroup per CU).
#ifndef EPX_SP_TILES
#define EPX_SP_TILES 32
#endif
constexpr int kSpTargetTiles = EPX_SP_TILES;
constexpr int kSpMaxTilesPerBlock = 32;
constexpr int64_t kSpMaxTiles = 8192;

// Routed slots (T*K) a layout call takes.  Up to here the chunk-sum column
// a direct-path rank workgroup reads stays short (at most 32 chunks), and
// the single pass, when a caller forces it, runs at most kSpMaxTiles tiles
// of 256 x 8 slots, which the workgroups that are sure to be resident (one
// per CU) can hold.
constexpr int64_t kLayoutMaxSlots = int64_t(1) << 24;
static_assert(kLayoutMaxSlots <= kSpMaxTiles * 256 * 8, "the single pass must take every layout");
inline int sp_slots_per_thread(int64_t routed_slots) {
    for (int spt = 1; spt < 8; spt *= 2)
        if (routed_slots <= (int64_t)kLayoutThreads * spt * kSpTargetTiles) return spt;
    return 8;
}
inline int64_t sp_tiles(int64_t routed_slots) {
    const int64_t tile = (int64_t)kLayoutThreads * sp_slots_per_thread(routed_slots);
    const int64_t nt = (routed_slots + tile - 1) / tile;
    return nt < 1 ? 1 : nt;
}
// Single-pass workgroups: every tile has one; at least min(groups, 64) so
// that the groups' metadata runs are spread out.
inline int64_t sp_blocks(int64_t tiles, int NG) {
    const int64_t g = NG < 64 ? NG : 64;
    return tiles > g ? tiles : g;
}

// Look-back descriptor value word: 2 status bits over a 30-bit count.
constexpr uint32_t kDescAgg = 1u << 30;   // tile aggregate only
constexpr uint32_t kDescInc = 2u << 30;   // inclusive prefix through this tile
constexpr uint32_t kDescValue = (1u << 30) - 1;

// ---------------------------------------------------------------------------
// Number helpers (bit-exact definitions, no fused multiply-add anywhere: the
// library is built with -ffp-contract=off).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest-even; NaN keeps sign and payload top
// bits and is made quiet (bit 6 of the bf16 set).  This is gfx950's
// v_cvt_pk_bf16_f32, two values per instruction: on all 2^32 float
// patterns it equals bf16_rne_bits below, denormals and NaN included
// (tests/test_gpu_conversions.py).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// E4M3 ("fn" variant of OCP OFP8: bias 7, largest finite 448, exponent
// field 0 subnormal with step 2^-9).
// Non-negative finite s -> E4M3 code, RNE, saturating to 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
    if (!(s > 0.0f)) return 0u;
    if (s >= 448.0f) return 0x7Eu;
    if (s < 0.015625f) {                 // below 2^-6: subnormal step 2^-9
        return (uint32_t)__builtin_rintf(s * 512.0f);  // exact scaling, RNE; 8 -> 0x08 = 2^-6
    }
    uint32_t u = __float_as_uint(s);
    u += 0x7FFFFu + ((u >> 20) & 1u);    // round the mantissa to 3 bits, ties to even
    const uint32_t c = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);  // rebias 127 -> 7
    return c > 0x7Eu ? 0x7Eu : c;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    const uint32_t e = c >> 3, m = c & 7u;
    if (e == 0u) return (float)m * 0.001953125f;  // m * 2^-9, exact
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Signed E4M3 encode: RNE, saturating to +-448, sign bit of v kept (-0 and
// tiny negatives give 0x80).  Finite v only.
__device__ __forceinline__ uint32_t e4m3_signed(float v) {
    return e4m3_encode(__builtin_fabsf(v)) | ((__float_as_uint(v) >> 24) & 0x80u);
}

// E4M3 code with its sign bit -> value (finite codes).
__device__ __forceinline__ float e4m3_decode_signed(uint32_t c) {
    return __uint_as_float(__float_as_uint(e4m3_decode(c & 0x7Fu)) | ((c & 0x80u) << 24));
}

// v -> E2M1 code (OCP MX: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).  The
// thresholds are the midpoints between magnitudes; at a midpoint the even
// code wins (the comparison is strict toward the odd neighbour); past 5
// it saturates at 6; the sign bit of v is kept.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    const float a = __builtin_fabsf(v);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
                 (a > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// E2M1 code -> value, from its bit fields: exponent e = bits 2..1 (bias 1),
// mantissa m = bit 0; e = 0 is subnormal (m * 0.5).
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const uint32_t mag = e == 0u ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
    return __uint_as_float(mag | ((c & 8u) << 28));
}

// float -> bf16 bits by the bit formula: round to nearest-even on the
// dropped 16 bits; NaN keeps sign and payload top bits and is made quiet.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Count of set bits of `m` in lanes below this one (the in-wave rank).
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive sum over lanes 0..lane of the wave, by DPP row shifts (1, 2, 4,
// 8 within each row of 16 lanes) and row broadcasts (lane 15 into the next
// row, lane 31 into rows 2 and 3): six cross-lane adds with no LDS round
// trip.  Every lane of the wave must be active.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// Workgroup barrier for LDS traffic only: the fences order LDS accesses
// (a wait on the LDS counter) but not global memory, so global loads and
// stores in flight stay in flight across it (__syncthreads also waits for
// every outstanding global access of the wave, stores included).  Only for
// code in which no thread reads global memory that another thread of its
// workgroup wrote.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Lanes of the wave holding the same key as this lane.  Every lane of the
// wave must be active; keys are < 2^nbits.
__device__ __forceinline__ uint64_t match_any(uint32_t key, int nbits) {
    uint64_t m = ~0ull;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t on = __builtin_amdgcn_ballot_w64(bit);
        m &= bit ? on : ~on;
    }
    return m;
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
    return __builtin_amdgcn_readfirstlane(v);
}

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files).  All return a hipError_t of the
// launch; shapes are validated by the caller (api.hip).
// ---------------------------------------------------------------------------
struct LayoutArgs {
    const int32_t* topk_ids;
    uint32_t* desc;      // direct path: [tiles][NG] tile counts
    uint32_t* chunk_sums;  // direct path past kDirectMaxTiles tiles: [chunks][NG] column sums of the chunks
    void* sp_header;     // single pass: workspace header (generation, ticket, ...)
    uint64_t* sp_desc;   // single pass: [tiles][NG] look-back descriptors
    ep_layout_t out;
    int32_t T, K, Kp, E, S, G, NG, E_loc, A, C, shared, src_seg;
    int64_t recv_rows;
    int32_t tiles;             // tiles of the path that runs
    int32_t chunks;            // direct path: direct_chunks(tiles) (0: no chunk sums)
    int32_t mode;              // kLayoutSinglePass, kLayoutDirect, kLayoutSmall or kLayoutCount
    int32_t lookback;          // single pass: tile prefixes by decoupled look-back (else from all aggregates)
    int32_t rank_blocks;       // workgroups of the rank pass / single pass: max(tiles, min(NG, 256))
    int32_t slots_per_thread;  // 1, 2, 4 or 8 (layout_slots_per_thread)
    // Small path only: a dispatch fused in (x nullptr: layout only), the
    // bf16 one into recv, the NVFP4 one into codes, scales and rowscale, or
    // the FP8 one into f8_codes and f8_scales.
    const uint16_t* x;   // [T, H]
    uint16_t* recv;      // [R, H] (nullptr: no bf16 dispatch)
    uint8_t* codes;      // [R, H/2] (nullptr: no NVFP4 dispatch)
    uint8_t* scales;     // [R, H/16]
    uint16_t* rowscale;  // [R]
    uint8_t* f8_codes;   // [R, H] (nullptr: no FP8 dispatch)
    float* f8_scales;    // [R, H/128]
    int32_t H;
    int32_t fused_rpu;   // rows per unit of the fused dispatch (>= 1)
};
hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream);

struct MoveArgs {
    const void* src;
    void* dst;
    const int32_t* token_row;
    const float* probs;  // nullptr: weight 1
    int32_t T, K, Kp, H;
    int64_t R;           // receive rows; a token_row entry outside [0, R) is skipped
};
hipError_t launch_scatter(const MoveArgs& a, hipStream_t stream);         // dispatch: bit copy
hipError_t launch_scatter_scaled(const MoveArgs& a, hipStream_t stream);  // combine-bwd: w_k * row
hipError_t launch_gather_reduce(const MoveArgs& a, hipStream_t stream);   // combine / dispatch-bwd
// grad_probs [T,K] = <grad_y[t] (a.src), expert_out[row(t,k)] (a.dst, read only)>
hipError_t launch_probs_grad(const MoveArgs& a, float* grad_probs, hipStream_t stream);

struct Nvfp4Args {
    const uint16_t* x;
    uint8_t* codes;
    uint8_t* scales;
    uint16_t* rowscale;
    const int32_t* token_row;
    int32_t T, Kp, H;
    int64_t R;           // receive rows; a token_row entry outside [0, R) is skipped
};
hipError_t launch_nvfp4(const Nvfp4Args& a, hipStream_t stream);
int nvfp4_max_hidden();

struct Fp8Args {
    const uint16_t* x;
    uint8_t* codes;    // [R, H] E4M3
    float* scales;     // [R, H/128]
    const int32_t* token_row;
    int32_t T, Kp, H;
    int64_t R;
};
hipError_t launch_fp8(const Fp8Args& a, hipStream_t stream);
int fp8_max_hidden();

struct CombineNvfp4Args {
    const uint8_t* codes;      // [R, H/2]
    const uint8_t* scales;     // [R, H/16]
    const uint16_t* rowscale;  // [R] bf16 bits
    const int32_t* token_row;  // [T, K']
    const float* probs;        // [T, K] or nullptr: weight 1
    uint16_t* y;               // [T, H] bf16 bits
    int32_t T, K, Kp, H;
    int64_t R;                 // receive rows; a token_row entry outside [0, R) is skipped
};
hipError_t launch_combine_nvfp4(const CombineNvfp4Args& a, hipStream_t stream);
int combine_nvfp4_pieces(int32_t H);

struct RouteArgs {
    int32_t* ids;         // [T, K]
    float* probs;         // [T, K] or nullptr
    uint8_t* map;         // [T, E]
    float* dense_probs;   // [T, E] or nullptr
    int32_t* flags;       // OR-ed with EP_FLAG_MAP_OVERFLOW, or nullptr
    int32_t T, K, E;
};
hipError_t launch_indices_to_multihot(const RouteArgs& a, hipStream_t stream);
hipError_t launch_multihot_to_indices(const RouteArgs& a, hipStream_t stream);

// Zero the payload bytes of every pad row ([count, align_up(count)) of each
// group, below capacity).  row_bytes = bytes of one row of `base`.
hipError_t launch_zero_pad_rows(void* base, int64_t row_bytes, const ep_layout_t& L, int32_t S,
                                int32_t G, int32_t A, int32_t C, int64_t R, hipStream_t stream);

}  // namespace epx
