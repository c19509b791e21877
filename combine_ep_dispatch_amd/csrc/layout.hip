// Dispatch layout for one GPU's share of MoE expert-parallel dispatch:
// per-group counts, aligned row offsets, stable in-group ranks, token_row,
// expert_ids and src_info, plus the capacity-overflow flag.
//
// Semantics (page title, API item):
//  - NeMo AutoModel token_dispatcher page: dispatch_postprocess counts the
//    tokens per expert; _align_up / moe_router_expert_pad_multiple pad each
//    expert's rows to a multiple; _assert_no_hybridep_overflow: truncation
//    at capacity raises a one-element device overflow flag.
//  - NeMo AutoModel fused_a2a page, HybridEPDispatch.forward: -1 marks an
//    unused top-k slot; rows are grouped by local expert.
//  - MAX DistributedEPDispatchBlockScaledNVDynGlobalScales page, execute:
//    row_offsets, expert_ids per received token, src_info, atomic counters
//    coordinating work across thread blocks.
//
// Four paths, all with the same results (the host picks one by size or by
// the EP_LAYOUT_* flag the caller sets):
//
// Small (up to 512 routed slots): k_layout_rank alone; every workgroup
// ranks the one tile to learn the group totals, workgroup 0 writes the
// per-slot results and the others spread the groups' metadata runs.  As
// every workgroup then knows every slot's row, a dispatch can be fused in
// (ep_dispatch_with_layout, ep_dispatch_nvfp4_with_layout,
// ep_dispatch_fp8_with_layout): workgroup b takes units b, b + gridDim.x,
// ..., a unit being a token and a run of its K' rows (as few rows per unit
// as let the units fit one round of workgroups); it loads the token's bf16
// row, or quantizes it to NVFP4 or FP8, once and stores it to each of the
// unit's rows.  At DeepSeek-V3 dims
// (one process, interleaved) that is 5.4 us against 4.3 + 3.0 us for the
// two calls at T = 16 and 7.4 against 5.0 + 3.5 us at T = 64; for NVFP4
// 6.6 against 4.3 + 3.9 us and 7.9 against 5.0 + 4.0 us.
//
// Count (default up to 8192 routed slots, forced with EP_LAYOUT_COUNT up to
// 2^18):
// k_layout_rank alone; every workgroup counts all routed slots into LDS
// counters per group (those before its tile apart: its in-group prefix),
// then ranks its own tile of 256 slots as the two-kernel path does.
//
// Two kernels (default past 8192 routed slots, any size with
// EP_LAYOUT_DIRECT; a third launch between them past 256 tiles):
//  1. k_layout_hist   per tile of 256 x {1,2,4,8} routed slots, a wave64
//                     match-any over the group key (one ballot per key bit);
//                     the lowest lane of each match set adds the set's
//                     popcount into an LDS counter, so a hot expert costs one
//                     LDS atomic per wave instead of one per slot.  Each tile
//                     stores its per-group counts as one row of a
//                     [tile][group] table; tile 0 also clears the flags word.
//  2. k_layout_rank   every workgroup reads, for each group, the group's
//                     column of tile counts (lanes over groups, so wave loads
//                     are contiguous; 64 loads in flight per lane, and several
//                     lanes per group when groups are few; four groups per
//                     16-byte load up to 128 groups) and sums it twice:
//                     over all tiles (the group total) and over the tiles
//                     before its own (its in-group prefix).  No workgroup
//                     waits on another, and there are no atomics on global
//                     memory but the flags.  It then scans the aligned group
//                     sizes into group start rows, ranks its tile's slots
//                     inside their groups (per-wave running counters in LDS,
//                     one 4-byte word per group so neighbouring groups share
//                     no bank word, touched only by the lowest lane of each
//                     match set), and writes token_row and src_info; the
//                     last workgroup writes counts, offsets and segment
//                     bases.  With one group per lane and one batch of
//                     column loads the loads go out before the in-tile
//                     ranks, which run while they are in flight (the
//                     layout kernels' barriers wait on LDS only, see
//                     lds_barrier).  The fused shared-expert rows,
//                     and expert_ids of whole groups (pad rows included) as
//                     coalesced runs, are spread over at least
//                     min(groups, 256) workgroups.
//     Past 256 tiles, k_layout_chunks runs between the two: per chunk of 256
//     table rows and group it turns the counts into prefixes within the
//     chunk and sums them, and each rank workgroup reads the chunk sums and
//     its own row instead of a whole column: fixed work per workgroup, so
//     the cost stays linear in the slots (MI355X, 256 groups: 46 us at 2^20
//     routed slots, 222 us at 2^24; with whole columns 4.8 ms there).
//
// Single pass (EP_LAYOUT_LOOKBACK or EP_LAYOUT_BARRIER): k_layout_sp, one
// kernel with ticketed tiles, described above it.  Measured on MI355X it is
// slower than the two kernels at every size (DeepSeek-V3 share: 14.8
// against 12.0 us per launch; the look-back flavour 19.9; at 2^24 routed
// slots the look-back takes 0.83 ms): a position needs the totals of all
// groups, so the single pass waits for the slowest tile's counts through
// memory-side loads across the XCDs, which costs more than the second
// launch.  The barrier flavour reads every tile's counts in every
// workgroup, so its cost grows with the square of the tile count (29 ms at
// 2^24 slots); it is refused past 2^20 routed slots.
#include "fp8_device.h"
#include "nvfp4_device.h"

namespace epx {
namespace {

#ifndef EPX_DIRECT_QUADS
#define EPX_DIRECT_QUADS 1
#endif

// A wait on another workgroup gives up (EP_FLAG_INTERNAL) once the
// workgroup has run this many ticks of the 100 MHz wall clock (about 0.34 s);
// every later wait of the workgroup then gives up at once, so a call whose
// waits cannot end still finishes in bounded time.
constexpr uint64_t kWaitTicks = 1ull << 25;
// Fused NVFP4 dispatch: 16-element blocks per row (H <= 16384) and per thread.
constexpr int kQuantMaxBlocks = 1024;
constexpr int kQuantBlocksPerThread = kQuantMaxBlocks / kLayoutThreads;
// Fused FP8 dispatch: iterations of 8 128-element blocks per row (H <= 16384)
// and per wave.
constexpr int kF8ItersPerWave = 16 / kLayoutWaves;

// Receive row of the fused shared-expert slot of token t: rank t of its
// group, or -1 past the segment's capacity or the buffer.
__device__ __forceinline__ int32_t shared_row_of(const int32_t* s_start, const int32_t* s_lim, int32_t g, int32_t t,
                                                 uint32_t R) {
    const uint32_t r = (uint32_t)s_start[g] + (uint32_t)t;
    return (r < (uint32_t)s_lim[g] && r < R) ? (int32_t)r : -1;
}

typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
constexpr int kRowRsrcWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data, raw addressing

// Buffer resource over `bytes` bytes at p: loads past the end return zeros
// and stores past it are dropped, with no memory access, so the row loads
// and stores below need no per-vector branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, kRowRsrcWord3);
}

// A row of 8-element vectors as 16-element blocks: thread `tid` gets blocks
// tid, tid + 256, ... (16-byte vectors 2b and 2b + 1) of the row the
// resource covers, zeros past it (rows up to 16384 elements).
__device__ __forceinline__ void load_token_blocks(__amdgpu_buffer_rsrc_t rs, int tid,
                                                  uint4 (&q)[kQuantBlocksPerThread][2]) {
#pragma unroll
    for (int i = 0; i < kQuantBlocksPerThread; ++i) {
        const int32_t b = tid + i * kLayoutThreads;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, (2 * b + h) * 16, 0, 0);
            q[i][h].x = v.x;
            q[i][h].y = v.y;
            q[i][h].z = v.z;
            q[i][h].w = v.w;
        }
    }
}

// The same blocks stored to the row the resource covers.
__device__ __forceinline__ void store_token_blocks(__amdgpu_buffer_rsrc_t rs, int tid,
                                                   const uint4 (&q)[kQuantBlocksPerThread][2]) {
#pragma unroll
    for (int i = 0; i < kQuantBlocksPerThread; ++i) {
        const int32_t b = tid + i * kLayoutThreads;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            __builtin_amdgcn_raw_buffer_store_b128(v4u_t{q[i][h].x, q[i][h].y, q[i][h].z, q[i][h].w}, rs,
                                                   (2 * b + h) * 16, 0, 0);
    }
}

__device__ __forceinline__ int32_t align_up(int32_t count, int32_t multiple) {
    if ((multiple & (multiple - 1)) == 0) return (count + multiple - 1) & -multiple;  // power of two
    return ((count + multiple - 1) / multiple) * multiple;
}

template <int SPT>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_hist(LayoutArgs a) {
    constexpr int kTileSlots = kLayoutThreads * SPT;
    __shared__ int32_t s_hist[EP_MAX_GROUPS];
    __shared__ int32_t s_gof[EP_MAX_GROUPS];  // group of each routed expert
    const int tid = threadIdx.x;
    const int64_t routed = (int64_t)a.T * a.K;
    const int nbits = 32 - __clz(a.NG);  // keys live in [0, NG]; NG = "no group"
    const int64_t base = (int64_t)blockIdx.x * kTileSlots;
    // All of the tile's ids are loaded first, so that their latency hides
    // behind the LDS set-up and they cost one round trip, not one per slot
    // per thread.
    int32_t eid[SPT];
#pragma unroll
    for (int it = 0; it < SPT; ++it) {
        const int64_t f = base + it * kLayoutThreads + tid;
        eid[it] = f < routed ? a.topk_ids[f] : -1;
    }
    for (int g = tid; g < a.NG; g += kLayoutThreads) s_hist[g] = 0;
    for (int e = tid; e < a.E; e += kLayoutThreads)
        s_gof[e] = (e / a.E_loc) * a.G + a.shared + (e % a.E_loc);
    lds_barrier();

#pragma unroll
    for (int it = 0; it < SPT; ++it) {
        const int32_t e = eid[it];
        uint32_t key = (uint32_t)a.NG;
        if ((uint32_t)e < (uint32_t)a.E) key = (uint32_t)s_gof[e];
        const uint64_t m = match_any(key, nbits);
        if (key != (uint32_t)a.NG && lanes_below(m) == 0)
            atomicAdd(&s_hist[key], (int32_t)__popcll(m));
    }
    lds_barrier();
    uint32_t* row = a.desc + (int64_t)blockIdx.x * a.NG;
    for (int g = tid; g < a.NG; g += kLayoutThreads) row[g] = (uint32_t)s_hist[g];
    if (blockIdx.x == 0 && tid == 0) a.out.flags[0] = 0;
}

// Direct-path column sums.  Lane r of the tpg lanes that share a column
// sums its entries j = r, r + tpg, ... below n (col[j * stride]): all of
// them into tot, those below `split` into pre.  Loads are unconditional, at
// clamped 32-bit offsets (n * stride < 2^25), and masked afterwards: no
// branch around a load and no 64-bit address temporaries, which let the
// compiler reuse pending loads' registers and wait on each load in turn.
// kDirectBatch loads per lane are in flight together: one round trip to
// memory for up to kDirectBatch * tpg entries.
__device__ __forceinline__ void column_sums(const uint32_t* col, uint32_t stride, int n, int split, int r, int tpg,
                                            int32_t& tot, int32_t& pre) {
    constexpr int kBatch = kDirectBatch;
    for (int j0 = r; j0 < n; j0 += kBatch * tpg) {
        uint32_t v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int j = j0 + i * tpg;
            v[i] = col[(uint32_t)min(j, n - 1) * stride];
        }
        // Every load of the batch is issued before the first is consumed:
        // left to itself the scheduler may interleave the sums with the
        // issue to save registers, which waits on the first loads with half
        // the batch not yet sent (a second round trip to memory).
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int j = j0 + i * tpg;
            const int32_t c = j < n ? (int32_t)v[i] : 0;
            tot += c;
            pre += j < split ? c : 0;
        }
    }
}

// The same over four adjacent columns at once, one 16-byte load per entry
// (col[j * stride] holds the four columns' entries j).
__device__ __forceinline__ void quad_sums(const uint4* col, uint32_t stride, int n, int split, int r, int tpq,
                                          int32_t (&tot)[4], int32_t (&pre)[4]) {
    constexpr int kBatch4 = kDirectBatch / 4;
    for (int j0 = r; j0 < n; j0 += kBatch4 * tpq) {
        uint4 v[kBatch4];
#pragma unroll
        for (int i = 0; i < kBatch4; ++i) {
            const int j = j0 + i * tpq;
            v[i] = col[(uint32_t)min(j, n - 1) * stride];
        }
        __builtin_amdgcn_sched_barrier(0);  // the whole batch in flight first
#pragma unroll
        for (int i = 0; i < kBatch4; ++i) {
            const int j = j0 + i * tpq;
            const bool in = j < n, before = j < split;
            const int32_t c[4] = {(int32_t)v[i].x, (int32_t)v[i].y, (int32_t)v[i].z, (int32_t)v[i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                tot[q] += in ? c[q] : 0;
                pre[q] += before ? c[q] : 0;
            }
        }
    }
}

// Direct path past kDirectMaxTiles tiles: for chunk c of kDirectMaxTiles
// rows of the tile-count table and group g, turns the chunk's counts into
// exclusive prefixes within the chunk (in place) and writes their total to
// chunk_sums[c][g].  One lane per group, kDirectBatch rows in flight; a
// wave's loads and stores cover 64 adjacent groups of one row.  Grid:
// (chunks, groups / kLayoutThreads).
__global__ __launch_bounds__(kLayoutThreads) void k_layout_chunks(LayoutArgs a) {
    const int NG = a.NG;
    const int g = (int)blockIdx.y * kLayoutThreads + (int)threadIdx.x;
    const int t0 = (int)blockIdx.x * kDirectMaxTiles;
    const int n = min(kDirectMaxTiles, a.tiles - t0);
    if (g >= NG) return;
    uint32_t* col = a.desc + (uint32_t)t0 * (uint32_t)NG + g;
    uint32_t run = 0;
    for (int j0 = 0; j0 < n; j0 += kDirectBatch) {
        uint32_t v[kDirectBatch];
#pragma unroll
        for (int i = 0; i < kDirectBatch; ++i) v[i] = col[(uint32_t)min(j0 + i, n - 1) * (uint32_t)NG];
        __builtin_amdgcn_sched_barrier(0);  // the whole batch in flight first
#pragma unroll
        for (int i = 0; i < kDirectBatch; ++i) {
            if (j0 + i < n) {
                col[(uint32_t)(j0 + i) * (uint32_t)NG] = run;
                run += v[i];
            }
        }
    }
    a.chunk_sums[(int64_t)blockIdx.x * NG + g] = run;
}

// CHUNKS (direct mode past kDirectMaxTiles tiles): the column sums come
// from the chunk sums plus the tile's own chunk; a separate instantiation,
// so that the common case keeps its own register allocation (it measured
// 0.4 us slower with a run-time branch here).  MAXG (256 or EP_MAX_GROUPS)
// sizes the LDS arrays: up to 256 groups a workgroup takes 9 KiB of LDS
// instead of 72 KiB, so that several fit on a CU when there are more
// workgroups than CUs.
template <int SPT, int MODE, bool CHUNKS = false, int MAXG = EP_MAX_GROUPS>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_rank(LayoutArgs a) {
    constexpr bool DIRECT = MODE == kLayoutDirect, SMALL = MODE == kLayoutSmall, COUNT = MODE == kLayoutCount;
    constexpr int kTileSlots = kLayoutThreads * SPT;
    constexpr int kSlotsPerWave = kWave * SPT;
    constexpr int J = MAXG / kLayoutThreads;  // groups per thread in the per-group loops
    static_assert(MAXG % 8 == 0 && MAXG <= EP_MAX_GROUPS, "group arrays");
    __shared__ __align__(16) int32_t s_cnt[MAXG];    // group totals
    __shared__ __align__(16) int32_t s_start[MAXG];  // first row of the group (clamped at capacity)
    __shared__ __align__(16) int32_t s_lim[MAXG];    // first row past the segment's capacity
    __shared__ int32_t s_pref[MAXG];   // slots of the group in earlier tiles
    __shared__ int32_t s_gof[MAXG];    // group of each routed expert
    __shared__ int32_t s_wcnt[kLayoutWaves][MAXG];  // per-wave counts / prefixes (a 4-byte word each)
    __shared__ int32_t s_wsum[kLayoutWaves];
    __shared__ int32_t s_flag;
    __shared__ int32_t s_rowof[SMALL ? kTileSlots : 1];  // small path with a dispatch fused: each slot's row
    __shared__ uint2 s_qcode[SMALL ? kQuantMaxBlocks : 1];  // fused NVFP4: one token's codes, 8 bytes per block
    __shared__ uint8_t s_qsc[SMALL ? kQuantMaxBlocks : 1];  // and its E4M3 block scales
    __shared__ uint32_t s_qmax[kLayoutWaves];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int NG = a.NG, G = a.G;
    // Workgroups past the last tile own no slots: they only fill their share
    // of the groups' metadata runs (below), which at small T is most of the
    // work (every group padded to a multiple of A).  In the single-pass mode
    // every workgroup ranks the one tile (to learn the group totals) and
    // workgroup 0 alone writes the per-slot results.
    const uint32_t tile = blockIdx.x;
    const uint32_t slot_tile = SMALL ? 0u : tile;
    const bool owns_tile = SMALL ? tile == 0 : tile < (uint32_t)a.tiles;
    // This tile's routed slots: wave w owns [w*64*SPT, (w+1)*64*SPT), in SPT
    // rounds of 64.  The ids are fetched first so their latency hides behind the
    // offset scan.
    const int64_t routed = (int64_t)a.T * a.K;
    const int64_t wslot0 = (int64_t)slot_tile * kTileSlots + (int64_t)w * kSlotsPerWave;
    int32_t eid[SPT];
#pragma unroll
    for (int it = 0; it < SPT; ++it) {
        const int64_t f = wslot0 + it * kWave + lane;
        eid[it] = f < routed ? a.topk_ids[f] : -1;
    }
    // Small path with a dispatch fused: a unit is one token and a run of up
    // to `rpu` (LayoutArgs::fused_rpu) of its K' rows; the token is loaded
    // (and for NVFP4 quantized) once per unit and stored to each of the
    // unit's rows.
    // (Loading each workgroup's first x row here, ahead of the ranks,
    // measured 0.1-0.3 us slower.)
    const bool fused = SMALL && a.x != nullptr;
    const int32_t fused_rpu = a.fused_rpu;
    const int32_t fused_chunks = fused ? (a.Kp + fused_rpu - 1) / fused_rpu : 1;  // units per token
    const int32_t fused_units = fused ? a.T * fused_chunks : 0;
    const int32_t shared_group = a.shared ? a.src_seg * G : -1;
    if (tid == 0) s_flag = 0;
    int32_t flag = 0;

    // In-tile ranks (per-wave running counters + match-any), then the
    // per-wave exclusive prefixes and the tile's aggregate per group.
    uint32_t key[SPT], rnk[SPT];
    int32_t agg[J];
    auto rank_slots = [&]() {
        // ---- in-tile ranks (per-wave running counters + match-any) ----
        const int nbits = 32 - __clz(NG);
#pragma unroll
        for (int it = 0; it < SPT; ++it) {
            const int32_t e = eid[it];
            const uint32_t k = (uint32_t)e < (uint32_t)a.E ? (uint32_t)s_gof[e] : (uint32_t)NG;
            if (e != -1 && (uint32_t)e >= (uint32_t)a.E) flag |= EP_FLAG_BAD_ID;  // -1 = masked slot
            const uint64_t m = match_any(k, nbits);
            const uint32_t r = lanes_below(m);
            // only the lowest lane of each key touches LDS; the others take
            // its value by a cross-lane read
            int32_t before = 0;
            if (k != (uint32_t)NG && r == 0) {
                before = s_wcnt[w][k];
                s_wcnt[w][k] = before + (int32_t)__popcll(m);
            }
            before = __shfl(before, (int)__builtin_ctzll(m), kWave);
            rnk[it] = k != (uint32_t)NG ? (uint32_t)before + r : 0u;
            key[it] = k;
        }
        lds_barrier();

        // ---- per-wave exclusive prefixes and the tile aggregate per group ----
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int g = tid + j * kLayoutThreads;
            agg[j] = 0;
            if (g < NG) {
                int32_t run = 0;
#pragma unroll
                for (int w2 = 0; w2 < kLayoutWaves; ++w2) {
                    const int32_t c = s_wcnt[w2][g];
                    s_wcnt[w2][g] = run;
                    run += c;
                }
                agg[j] = run;
            }
        }
    };

    if (COUNT) {
        // Group totals and this tile's in-group prefix by counting every
        // routed slot in LDS: slots before the tile into s_pref, the rest
        // into s_cnt.  No workgroup reads anything another one wrote.
        for (int g = tid; g < NG; g += kLayoutThreads) {
            s_cnt[g] = 0;
            s_pref[g] = 0;
        }
        for (int e = tid; e < a.E; e += kLayoutThreads)
            s_gof[e] = (e / a.E_loc) * G + a.shared + (e % a.E_loc);
        lds_barrier();
        const int64_t mine0 = (int64_t)tile * kTileSlots;
        auto count = [&](int32_t e, int64_t f) {
            if ((uint32_t)e < (uint32_t)a.E)
                atomicAdd(f < mine0 ? &s_pref[s_gof[e]] : &s_cnt[s_gof[e]], 1);
            else if (e != -1)
                flag |= EP_FLAG_BAD_ID;
        };
        // The ids from a 16-byte boundary on as int4 vectors, kCountBatch
        // per thread in flight; the few before it and after the last whole
        // vector one by one.
        const int64_t head = min<int64_t>((int64_t)((16u - ((uintptr_t)a.topk_ids & 15u)) & 15u) / 4, routed);
        const int64_t nvec = (routed - head) / 4;
        const int4* vids = reinterpret_cast<const int4*>(a.topk_ids + head);
        constexpr int kCountBatch = 16;
        for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)kLayoutThreads * kCountBatch) {
            int4 q[kCountBatch];
#pragma unroll
            for (int i = 0; i < kCountBatch; ++i) {
                const int64_t v = v0 + i * kLayoutThreads + tid;
                q[i] = vids[v < nvec ? v : 0];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kCountBatch; ++i) {
                const int64_t v = v0 + i * kLayoutThreads + tid;
                if (v < nvec) {
                    const int64_t f = head + 4 * v;
                    count(q[i].x, f);
                    count(q[i].y, f + 1);
                    count(q[i].z, f + 2);
                    count(q[i].w, f + 3);
                }
            }
        }
        for (int64_t f = tid; f < head; f += kLayoutThreads) count(a.topk_ids[f], f);
        for (int64_t f = head + 4 * nvec + tid; f < routed; f += kLayoutThreads) count(a.topk_ids[f], f);
        lds_barrier();
        for (int g = tid; g < NG; g += kLayoutThreads)
            s_cnt[g] = s_cnt[g] + s_pref[g] + (g == shared_group ? a.T : 0);
    }
    // Direct path with one group per lane and one batch of column loads
    // (129 to 256 groups and at most kDirectBatch tiles, as at the DeepSeek-V3
    // share): the loads go out first, and the in-tile ranks, which need none
    // of them, run while they are in flight (the workgroup barriers here
    // wait on LDS only).
    const bool early = DIRECT && !CHUNKS && MAXG == kLayoutThreads && NG > kLayoutThreads / 2 &&
                       a.tiles <= kDirectBatch;
    if (early) {
        for (int e = tid; e < a.E; e += kLayoutThreads)
            s_gof[e] = (e / a.E_loc) * G + a.shared + (e % a.E_loc);
#pragma unroll
        for (int w2 = 0; w2 < kLayoutWaves; ++w2)
            if (tid < NG) s_wcnt[w2][tid] = 0;
        lds_barrier();
        // The ids must be in before the column loads go out: a wait on them
        // with the column loads in flight would also wait on the first of
        // those (the vector-memory counter a wait names holds at most 63).
        int32_t ids = 0;
#pragma unroll
        for (int it = 0; it < SPT; ++it) ids |= eid[it];
        __asm__ volatile("" : : "v"(ids));
        const uint32_t* col = a.desc + min(tid, NG - 1);
        uint32_t v[kDirectBatch];
#pragma unroll
        for (int i = 0; i < kDirectBatch; ++i) v[i] = col[(uint32_t)min(i, a.tiles - 1) * (uint32_t)NG];
        __builtin_amdgcn_sched_barrier(0);
        rank_slots();
        int32_t tot = 0, pre = 0;
#pragma unroll
        for (int i = 0; i < kDirectBatch; ++i) {
            const int32_t c = i < a.tiles ? (int32_t)v[i] : 0;
            tot += c;
            pre += i < (int)tile ? c : 0;
        }
        if (tid < NG) {
            s_cnt[tid] = tot + (tid == shared_group ? a.T : 0);
            s_pref[tid] = pre;
        }
        lds_barrier();
    }
    // Direct path: the group totals and this tile's in-group prefix from the
    // [tile][group] table; past kDirectMaxTiles tiles from the chunk sums
    // (totals, and the prefix over earlier chunks) plus this tile's row,
    // which k_layout_chunks turned into prefixes within its chunk.
    // Workgroups past the last tile need only the totals.
    const int my_chunk = CHUNKS ? min((int)(tile / kDirectMaxTiles), a.chunks) : 0;
    const bool in_chunk = CHUNKS && tile < (uint32_t)a.tiles;
    if (DIRECT && EPX_DIRECT_QUADS && (NG & 3) == 0 && NG <= 128) {
        // Four groups per 16-byte load (rows are 16-byte aligned when
        // NG % 4 == 0).  tpq (a power of two, tpq * NG / 4 <= 256, at most a
        // wave) lanes share a quad of groups: lane r sums entries r, r + tpq,
        // ...; with 16 loads in flight per lane that is one round trip for
        // up to 16 * tpq entries (the same as the one-group-per-load form
        // below wherever that bounds the tile size; at least 256 otherwise),
        // with a quarter of its load instructions.  Measured on MI355X
        // against that form: skewed (128 groups) 14.4 -> 14.0 us, capacity
        // (64) 20.0 -> 19.4 us; with 256 groups (4 lanes per quad, so a wave
        // load spans 4 table rows) 10.5 -> 11.1 us, so only up to 128.
        const int Q = NG / 4;
        const int tpq = min(4 * direct_lanes_per_group(NG), kWave);  // a quad's lanes stay in one wave
        const int r = tid & (tpq - 1);
        const uint4* table = reinterpret_cast<const uint4*>(a.desc);
        const uint4* chunks = reinterpret_cast<const uint4*>(a.chunk_sums);
        for (int q = tid / tpq; q < Q; q += kLayoutThreads / tpq) {
            int32_t tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
            if (!CHUNKS) {
                quad_sums(table + q, (uint32_t)Q, a.tiles, (int)tile, r, tpq, tot, pre);
            } else {
                // the tile's own row of in-chunk prefixes, in flight with
                // the chunk-sum loads; one lane of the quad adds it
                const uint4 own = table[(uint32_t)min((int)tile, a.tiles - 1) * (uint32_t)Q + (uint32_t)q];
                quad_sums(chunks + q, (uint32_t)Q, a.chunks, my_chunk, r, tpq, tot, pre);
                if (r == 0 && in_chunk) {
                    pre[0] += (int32_t)own.x;
                    pre[1] += (int32_t)own.y;
                    pre[2] += (int32_t)own.z;
                    pre[3] += (int32_t)own.w;
                }
            }
            for (int o = 1; o < tpq; o <<= 1) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    tot[c] += __shfl_xor(tot[c], o, kWave);
                    pre[c] += __shfl_xor(pre[c], o, kWave);
                }
            }
            if (r == 0) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int g = 4 * q + c;
                    s_cnt[g] = tot[c] + (g == shared_group ? a.T : 0);
                    s_pref[g] = pre[c];
                }
            }
        }
    } else if (DIRECT && !early) {
        // tpg (a power of two, tpg * NG <= 256) lanes share a group; their
        // partial sums meet by xor-shuffles inside the lane group (all lanes
        // of a group are active or inactive together).
        const int tpg = direct_lanes_per_group(NG);
        const int r = tid & (tpg - 1);
        for (int g = tid / tpg; g < NG; g += kLayoutThreads / tpg) {
            int32_t tot = 0, pre = 0;
            if (!CHUNKS) {
                column_sums(a.desc + g, (uint32_t)NG, a.tiles, (int)tile, r, tpg, tot, pre);
            } else {
                const uint32_t own = a.desc[(uint32_t)min((int)tile, a.tiles - 1) * (uint32_t)NG + (uint32_t)g];
                column_sums(a.chunk_sums + g, (uint32_t)NG, a.chunks, my_chunk, r, tpg, tot, pre);
                if (r == 0 && in_chunk) pre += (int32_t)own;
            }
            for (int o = 1; o < tpg; o <<= 1) {
                tot += __shfl_xor(tot, o, kWave);
                pre += __shfl_xor(pre, o, kWave);
            }
            if (r == 0) {
                s_cnt[g] = tot + (g == shared_group ? a.T : 0);
                s_pref[g] = pre;
            }
        }
    }
    if (!early) {
        if (!COUNT)
            for (int e = tid; e < a.E; e += kLayoutThreads)
                s_gof[e] = (e / a.E_loc) * G + a.shared + (e % a.E_loc);
#pragma unroll
        for (int w2 = 0; w2 < kLayoutWaves; ++w2)
            for (int g = tid; g < NG; g += kLayoutThreads) s_wcnt[w2][g] = 0;
        lds_barrier();
    }

    // Single pass: the group totals come from ranking the one tile.
    if (SMALL) {
        rank_slots();
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int g = tid + j * kLayoutThreads;
            if (g < NG) {
                s_cnt[g] = agg[j] + (g == shared_group ? a.T : 0);
                s_pref[g] = 0;
            }
        }
        lds_barrier();
    }

    // ---- aligned exclusive prefix P over all groups (segment-major) ----
    // Thread i covers groups [8i, 8i + 8) (NG <= MAXG <= 2048 = 256 * 8;
    // threads past MAXG / 8 hold none).  Counts,
    // starts and limits move between LDS and registers as 16-byte vectors
    // and no step branches per group, so each pass waits on LDS once rather
    // than once per group (measured on MI355X: this phase took 1.9 us of the
    // DeepSeek-V3 rank launch with a branch and a load per group).
    const bool has8 = tid * 8 < MAXG;
    int32_t P[8], al[8];
    int32_t tsum = 0;
    {
        const int4* c4 = reinterpret_cast<const int4*>(s_cnt) + 2 * tid;
        int4 lo = make_int4(0, 0, 0, 0), hi = lo;
        if (has8) {
            lo = c4[0];
            hi = c4[1];
        }
        int32_t c[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const int32_t A = a.A;
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = tid * 8 + j < NG ? c[j] : 0;
        if ((A & (A - 1)) == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) al[j] = (c[j] + A - 1) & -A;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) al[j] = (c[j] + A - 1) / A * A;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) tsum += al[j];
    }
    const int32_t incl = wave_inclusive_sum(tsum);
    if (lane == kWave - 1) s_wsum[w] = incl;
    lds_barrier();
    int32_t wbase = 0, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < kLayoutWaves; ++w2) {
        if (w2 < w) wbase += s_wsum[w2];
        total += s_wsum[w2];
    }
    {
        int32_t run = wbase + incl - tsum;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            P[j] = run;
            run += al[j];
        }
    }
    int4* st4 = reinterpret_cast<int4*>(s_start) + 2 * tid;
    int4* li4 = reinterpret_cast<int4*>(s_lim) + 2 * tid;
    if (has8) {
        st4[0] = make_int4(P[0], P[1], P[2], P[3]);
        st4[1] = make_int4(P[4], P[5], P[6], P[7]);
        if (a.C == 0) {  // without a capacity a group starts at P and nothing is dropped
            li4[0] = make_int4(0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF);
            li4[1] = li4[0];
        }
    }
    lds_barrier();

    // Counts, offsets and segment bases: the last workgroup writes them.  It
    // owns no tile when there are more workgroups than tiles, and otherwise
    // the last, possibly ragged one; the tile-0 workgroup, which writes the
    // flags word and (on the small path) every slot's results, stays off
    // this chain of LDS reads (phase stamps at the DeepSeek-V3 share: the
    // writer workgroup ran 1 us longer than the median one, and the rank
    // launch ends with its slowest workgroup).
    if (tile == gridDim.x - 1) {
        for (int g = tid; g < NG; g += kLayoutThreads) a.out.counts[g] = s_cnt[g];
        const int n = a.S * (G + 1);
        for (int idx = tid; idx < n; idx += kLayoutThreads) {
            const int s = idx / (G + 1), gl = idx - s * (G + 1);
            const int gi = s * G + gl;
            int32_t off = (gi < NG ? s_start[gi] : total) - s_start[s * G];
            if (a.C > 0 && off > a.C) off = a.C;
            a.out.row_offsets[idx] = off;
            a.out.scales_offsets[idx] = off;
        }
        for (int s = tid; s <= a.S; s += kLayoutThreads)
            a.out.seg_base[s] = a.C > 0 ? s * a.C : (s < a.S ? s_start[s * G] : total);
    }
    if (a.C > 0) {
        // P -> absolute first row (clamped at capacity) and capacity limit.
        // The segment index advances with g instead of being divided out
        // each time; groups past NG read a clamped (unused) entry.
        int32_t seg[8], segp[8];
        {
            int s = (tid * 8) / G, gl = tid * 8 - s * G;
#pragma unroll
            for (int j = 0; j < 8; ++j, ++gl) {
                if (gl == G) {
                    ++s;
                    gl = 0;
                }
                seg[j] = min(s, a.S - 1);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) segp[j] = s_start[seg[j] * G];
        int32_t st[8], li[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            st[j] = seg[j] * a.C + min(P[j] - segp[j], a.C);
            li[j] = (seg[j] + 1) * a.C;
        }
        lds_barrier();
        if (has8) {
            st4[0] = make_int4(st[0], st[1], st[2], st[3]);
            st4[1] = make_int4(st[4], st[5], st[6], st[7]);
            li4[0] = make_int4(li[0], li[1], li[2], li[3]);
            li4[1] = make_int4(li[4], li[5], li[6], li[7]);
        }
    }

    if (!SMALL && !early) rank_slots();

    lds_barrier();

    // ---- write the routed slots of this tile ----
    const uint32_t R = (uint32_t)a.recv_rows;
#pragma unroll
    for (int it = 0; it < SPT; ++it) {
        const int64_t f = wslot0 + it * kWave + lane;
        if (!owns_tile || f >= routed) continue;
        const uint32_t t = (uint32_t)f / (uint32_t)a.K, k = (uint32_t)f - t * (uint32_t)a.K;
        int32_t* tr = &a.out.token_row[(int64_t)t * a.Kp + k];
        const uint32_t g = key[it];
        if (g == (uint32_t)NG) {
            *tr = -1;
            continue;
        }
        const uint32_t row = (uint32_t)s_start[g] + (uint32_t)s_pref[g] + (uint32_t)s_wcnt[w][g] + rnk[it];
        if (row >= (uint32_t)s_lim[g]) {
            *tr = -1;
            flag |= EP_FLAG_DROPPED;
            continue;
        }
        if (row >= R) {
            *tr = -1;
            flag |= EP_FLAG_INTERNAL;
            continue;
        }
        *tr = (int32_t)row;
        a.out.src_info[2 * (int64_t)row] = (int32_t)t;
        a.out.src_info[2 * (int64_t)row + 1] = (int32_t)k;
    }

    // ---- the fused shared expert: token t is rank t of group 0 of src_seg ----
    if (a.shared) {
        const int32_t per_tile = (a.T + a.rank_blocks - 1) / a.rank_blocks;
        const int32_t t0 = (int32_t)tile * per_tile;
        const int32_t t1 = min(a.T, t0 + per_tile);
        const uint32_t st0 = (uint32_t)s_start[shared_group], lim0 = (uint32_t)s_lim[shared_group];
        for (int32_t t = t0 + tid; t < t1; t += kLayoutThreads) {
            int32_t* tr = &a.out.token_row[(int64_t)t * a.Kp + a.K];
            const uint32_t row = st0 + (uint32_t)t;
            if (row >= lim0) {
                *tr = -1;
                flag |= EP_FLAG_DROPPED;
            } else if (row >= R) {
                *tr = -1;
                flag |= EP_FLAG_INTERNAL;
            } else {
                *tr = (int32_t)row;
                a.out.src_info[2 * (int64_t)row] = t;
                a.out.src_info[2 * (int64_t)row + 1] = a.K;
            }
        }
    }

    // ---- expert_ids of every used row, and pad-row src_info, of groups
    // g = blockIdx (mod rank_blocks).  A group's rows are contiguous and all hold the
    // group's expert (E for the fused shared expert), so they are written as
    // one coalesced run instead of one scattered word per slot; pad rows get
    // -1 in expert_ids and src_info.
    for (int g = (int)tile; g < NG; g += a.rank_blocks) {
        const int32_t c = s_cnt[g];
        const int32_t n = align_up(c, a.A);
        const int32_t gs = g / G, gl = g - gs * G;
        const int32_t expert = (a.shared && gl == 0) ? a.E : gs * a.E_loc + (gl - a.shared);
        for (int32_t r = tid; r < n; r += kLayoutThreads) {
            const uint32_t row = (uint32_t)s_start[g] + (uint32_t)r;
            if (row >= (uint32_t)s_lim[g]) break;
            if (row >= R) {
                flag |= EP_FLAG_INTERNAL;
                break;
            }
            const bool pad = r >= c;
            a.out.expert_ids[row] = pad ? -1 : expert;
            if (pad) {
                a.out.src_info[2 * (int64_t)row] = -1;
                a.out.src_info[2 * (int64_t)row + 1] = -1;
            }
        }
    }

    // ---- small path with a dispatch fused in: every workgroup ranked the
    // whole tile, so each knows every slot's row (the same rows and drops as
    // token_row) ----
    if (SMALL && a.x != nullptr) {
#pragma unroll
        for (int it = 0; it < SPT; ++it) {
            const int64_t f = wslot0 + it * kWave + lane;
            if (f >= routed) continue;
            const uint32_t g = key[it];
            int32_t row = -1;
            if (g != (uint32_t)NG) {
                const uint32_t r = (uint32_t)s_start[g] + (uint32_t)s_pref[g] + (uint32_t)s_wcnt[w][g] + rnk[it];
                if (r < (uint32_t)s_lim[g] && r < R) row = (int32_t)r;
            }
            s_rowof[f] = row;
        }
        lds_barrier();
        // Workgroup b takes units b, b + gridDim.x, ...: unit u is token
        // t = u / chunks and its slots k in [c rpu, (c + 1) rpu), c = u - t
        // chunks.  Slot k < K has row s_rowof[t K + k], the shared-expert slot
        // rank t of its group; -1 (masked, dropped) is skipped.  Every branch
        // on t and on a row is workgroup-uniform.
        const int32_t nv = a.H / 8;  // 16-byte vectors per row
        const int32_t nblk = a.H / 16;
        auto row_of = [&](int32_t t, int32_t k) -> int32_t {
            return uniform(k < a.K ? s_rowof[t * a.K + k] : shared_row_of(s_start, s_lim, shared_group, t, R));
        };
        for (int32_t u = (int32_t)blockIdx.x; u < fused_units; u += (int32_t)gridDim.x) {
            const int32_t t = u / fused_chunks;
            const int32_t k0 = (u - t * fused_chunks) * fused_rpu, k1 = min(a.Kp, k0 + fused_rpu);
            if (a.recv != nullptr) {
                // bf16: the token's bits, every load of the row out before
                // the first store
                if (a.H <= kQuantMaxBlocks * 16) {
                    uint4 q[kQuantBlocksPerThread][2];
                    load_token_blocks(row_rsrc(a.x + (int64_t)t * a.H, a.H * 2), tid, q);
                    for (int32_t k = k0; k < k1; ++k) {
                        const int32_t row = row_of(t, k);
                        if (row >= 0) store_token_blocks(row_rsrc(a.recv + (int64_t)row * a.H, a.H * 2), tid, q);
                    }
                } else {
                    const uint4* src = reinterpret_cast<const uint4*>(a.x + (int64_t)t * a.H);
                    for (int32_t k = k0; k < k1; ++k) {
                        const int32_t row = row_of(t, k);
                        if (row < 0) continue;
                        uint4* dst = reinterpret_cast<uint4*>(a.recv + (int64_t)row * a.H);
                        for (int32_t v = tid; v < nv; v += kLayoutThreads) dst[v] = src[v];
                    }
                }
                continue;
            }
            if (a.f8_codes != nullptr) {
                // FP8: wave w quantizes iterations w, w + 4, ... of the row
                // (8 blocks of 128 elements each, in the FP8 dispatch's lane
                // layout and block arithmetic) and stores its codes and block
                // scales to each of the unit's rows; the waves share nothing.
                const int32_t nb8 = a.H / 128, nit = (nb8 + 7) / 8;
                const __amdgpu_buffer_rsrc_t xs = row_rsrc(a.x + (int64_t)t * a.H, a.H * 2);
                uint4 p8[kF8ItersPerWave], q8[kF8ItersPerWave];
#pragma unroll
                for (int j = 0; j < kF8ItersPerWave; ++j) {
                    const int32_t it = w + j * kLayoutWaves;  // zeros past the row, like load_iteration
                    const v4u_t v0 = __builtin_amdgcn_raw_buffer_load_b128(xs, (128 * it + 2 * lane) * 16, 0, 0);
                    const v4u_t v1 = __builtin_amdgcn_raw_buffer_load_b128(xs, (128 * it + 2 * lane + 1) * 16, 0, 0);
                    p8[j] = make_uint4(v0.x, v0.y, v0.z, v0.w);
                    q8[j] = make_uint4(v1.x, v1.y, v1.z, v1.w);
                }
                uint4 c8[kF8ItersPerWave];
                float s8[kF8ItersPerWave];
#pragma unroll
                for (int j = 0; j < kF8ItersPerWave; ++j) {
                    c8[j] = make_uint4(0, 0, 0, 0);
                    s8[j] = 0.0f;
                    if (w + j * kLayoutWaves < nit) quantize_loaded(p8[j], q8[j], c8[j], s8[j]);
                }
                for (int32_t k = k0; k < k1; ++k) {
                    const int32_t row = row_of(t, k);
                    if (row < 0) continue;
                    const __amdgpu_buffer_rsrc_t cs = row_rsrc(a.f8_codes + (int64_t)row * a.H, a.H);
                    float* srow = a.f8_scales + (int64_t)row * nb8;
#pragma unroll
                    for (int j = 0; j < kF8ItersPerWave; ++j) {
                        const int32_t it = w + j * kLayoutWaves;
                        if (it >= nit) break;
                        __builtin_amdgcn_raw_buffer_store_b128(v4u_t{c8[j].x, c8[j].y, c8[j].z, c8[j].w}, cs,
                                                               (64 * it + lane) * 16, 0, 0);
                        const int32_t b = it * 8 + lane / 8;
                        if ((lane & 7) == 0 && b < nb8) srow[b] = s8[j];
                    }
                }
                continue;
            }
            // NVFP4: the token is quantized (the row max meets in LDS, codes
            // and block scales are staged in LDS) with the NVFP4 dispatch's
            // block arithmetic, then stored to each of the unit's rows.
            uint4 q[kQuantBlocksPerThread][2];
            load_token_blocks(row_rsrc(a.x + (int64_t)t * a.H, a.H * 2), tid, q);
            uint32_t bmax[kQuantBlocksPerThread];
            uint32_t lmax = 0;
#pragma unroll
            for (int j = 0; j < kQuantBlocksPerThread; ++j) {
                bmax[j] = block_amax(q[j][0], q[j][1]);
                lmax = max(lmax, bmax[j]);
            }
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) lmax = max(lmax, (uint32_t)__shfl_xor((int)lmax, o, kWave));
            if (lane == 0) s_qmax[w] = lmax;
            lds_barrier();
#pragma unroll
            for (int w2 = 0; w2 < kLayoutWaves; ++w2) lmax = max(lmax, (uint32_t)s_qmax[w2]);
            const float rowmax = __uint_as_float(lmax << 16);
            const float gs = rowmax == 0.0f ? 0.0f : 2688.0f / rowmax;
#pragma unroll
            for (int j = 0; j < kQuantBlocksPerThread; ++j) {
                const int32_t b = tid + j * kLayoutThreads;
                if (b < nblk) {
                    uint2 code = make_uint2(0, 0);
                    uint32_t sc = 0u;
                    if (rowmax != 0.0f) quantize_block(q[j][0], q[j][1], bmax[j], gs, code, sc);
                    s_qcode[b] = code;
                    s_qsc[b] = (uint8_t)sc;
                }
            }
            lds_barrier();
            const uint16_t rs = rowmax == 0.0f ? (uint16_t)0 : (uint16_t)f32_to_bf16(1.0f / gs);
            for (int32_t k = k0; k < k1; ++k) {
                const int32_t row = row_of(t, k);
                if (row < 0) continue;
                uint2* crow = reinterpret_cast<uint2*>(a.codes + (int64_t)row * (a.H / 2));
                uint8_t* srow = a.scales + (int64_t)row * nblk;
                for (int32_t b = tid; b < nblk; b += kLayoutThreads) {
                    crow[b] = s_qcode[b];
                    srow[b] = s_qsc[b];
                }
                if (tid == 0) a.rowscale[row] = rs;
            }
            lds_barrier();  // the staging is reused by the next unit
        }
    }

    if (SMALL || COUNT) {
        // No earlier launch cleared the flags word, so workgroup 0 stores it
        // whole.  Every bit is a function of the group totals, starts and
        // limits (and, for a bad id, of the ids every workgroup counted), so
        // it also covers rows other workgroups handled: a group drops slots
        // if start + count > limit, and reaches past the buffer if its used
        // rows (pad included) end beyond R.
        if (tile != 0) return;
        for (int g = tid; g < NG; g += kLayoutThreads) {
            const uint32_t st = (uint32_t)s_start[g], lim = (uint32_t)s_lim[g], c = (uint32_t)s_cnt[g];
            if (st + c > lim) flag |= EP_FLAG_DROPPED;
            const uint32_t end = min(st + (uint32_t)align_up((int32_t)c, a.A), lim);
            if (end > st && end > R) flag |= EP_FLAG_INTERNAL;
        }
        if (flag) atomicOr(&s_flag, flag);
        lds_barrier();
        if (tid == 0) a.out.flags[0] = s_flag;
        return;
    }
    if (flag) atomicOr(&s_flag, flag);
    lds_barrier();
    if (tid == 0 && s_flag) atomicOr(a.out.flags, s_flag);
}

// ---------------------------------------------------------------------------
// Single-pass layout: one launch at any size.
//
// Workgroups whose index is below the tile count are tile workers: each
// takes tile numbers from an atomic ticket until none are left, so a tile is
// only ever taken by a running workgroup, and a workgroup only waits on
// others once every tile has been handed out (and, in the look-back, only on
// tiles with smaller tickets, taken earlier).  Per tile: rank its slots
// inside their groups (match-any + per-wave counters) and publish the tile's
// per-group aggregate.  Every position needs the totals of all groups (a
// group's first row depends on the sizes of all groups before it), so each
// workgroup then reads the aggregates of the other tiles.  The tile's
// in-group prefix over earlier tiles comes either from
//  - LOOKBACK = true: a decoupled look-back inside the ticket loop
//    (windows of predecessor descriptors read in one round trip, folded
//    nearest-first until an inclusive prefix is met; the tile then publishes
//    its own inclusive prefix), the totals being that prefix plus the
//    aggregates of the later tiles; or
//  - LOOKBACK = false: the same read of every tile's aggregate that gives the
//    totals (the sum over the tiles before this one).
// Every wait re-polls all the still unpublished entries of its window in one
// round trip.  The workgroup then scans the aligned group sizes into group
// start rows and writes its tiles' token_row and src_info; src_info goes
// through LDS in group-major order, so each wave store covers consecutive
// receive rows.  expert_ids and pad-row metadata of whole groups are written
// as coalesced runs by all workgroups.
//
// Workspace: a header {generation | ticket, departures, flag bits}, then
// two arrays of 64-bit descriptors [tile][group] = generation:32 |
// status:2 | value:30: the look-back descriptors (aggregate, upgraded to the
// inclusive prefix) and the tiles' aggregates alone (written once).  The
// generation tells descriptors of this call from stale ones, so they are
// never cleared.  Every flag bit is known once the totals are (dropped
// slots and rows past the buffer follow from the group sizes), so each
// workgroup reports its bits with its departure right then, in one atomic
// add; the last one out writes the flags word, bumps the generation and
// resets the ticket and the departure word, which leaves the workspace
// ready for the next call.
struct SpHeader {
    uint64_t ctl;     // generation (high 32 bits) | next tile ticket (low 32 bits)
    uint64_t depart;  // 16-bit fields: workgroups that have left (bits 0-15), and
                      // of those, how many saw a dropped slot, a bad id, or gave
                      // up a wait (bits 16-31, 32-47, 48-63)
};
// One workgroup's departure: its count and flag bits in the fields of
// SpHeader::depart (grids stay below 2^16 workgroups).
__device__ __forceinline__ uint64_t sp_departure(int32_t f) {
    return 1ull | ((f & EP_FLAG_DROPPED) ? 1ull << 16 : 0ull) | ((f & EP_FLAG_BAD_ID) ? 1ull << 32 : 0ull) |
           ((f & EP_FLAG_INTERNAL) ? 1ull << 48 : 0ull);
}
__device__ __forceinline__ int32_t sp_flags_of(uint64_t d) {
    return ((d >> 16) & 0xFFFFu ? EP_FLAG_DROPPED : 0) | ((d >> 32) & 0xFFFFu ? EP_FLAG_BAD_ID : 0) |
           ((d >> 48) & 0xFFFFu ? EP_FLAG_INTERNAL : 0);
}

__device__ __forceinline__ uint64_t sp_load(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sp_store(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool sp_published(uint64_t d, uint32_t gen) {
    return (uint32_t)(d >> 32) == gen && ((uint32_t)d & ~kDescValue) != 0u;
}
__device__ __forceinline__ int32_t sp_value(uint64_t d) { return (int32_t)((uint32_t)d & kDescValue); }

// Sum over tiles u in [lo, hi) of the published value src[u * NG + g]
// (tiles at or after `split` also go to *after`), W loads in flight; the
// unpublished entries of a window are re-polled together until published or
// the workgroup's wait budget runs out (then EP_FLAG_INTERNAL).
template <int W>
__device__ __forceinline__ int32_t sp_sum(const uint64_t* src, int NG, int g, uint32_t lo, uint32_t hi,
                                          uint32_t split, int32_t* after, uint32_t gen, uint64_t t_begin,
                                          int32_t& flag) {
    const uint64_t zero = ((uint64_t)gen << 32) | kDescAgg;
    int32_t acc = 0, acc_after = 0;
    for (uint32_t u = lo; u < hi; u += W) {
        uint64_t d[W];
#pragma unroll
        for (int i = 0; i < W; ++i) d[i] = u + i < hi ? sp_load(&src[(int64_t)(u + i) * NG + g]) : zero;
        for (;;) {
            bool pending = false;
#pragma unroll
            for (int i = 0; i < W; ++i) pending |= !sp_published(d[i], gen);
            if (!pending) break;
            if (wall_clock64() - t_begin > kWaitTicks) {
                flag |= EP_FLAG_INTERNAL;
#pragma unroll
                for (int i = 0; i < W; ++i) d[i] = sp_published(d[i], gen) ? d[i] : zero;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            // the whole window again; published entries are kept
            for (int i = 0; i < W; ++i) {
                const uint64_t n = u + i < hi ? sp_load(&src[(int64_t)(u + i) * NG + g]) : zero;
                d[i] = sp_published(d[i], gen) ? d[i] : n;
            }
        }
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const int32_t v = sp_value(d[i]);
            acc += v;
            acc_after += u + i >= split ? v : 0;
        }
    }
    if (after != nullptr) *after = acc_after;
    return acc;
}

// Decoupled look-back for tile t > 0 and group g: the sum of the values of
// descriptors t-1, t-2, ... folded nearest-first up to and including the
// first inclusive one, W descriptors per round trip; when the nearest
// unfolded entry is not yet published, the unfolded entries of the window
// are re-polled together.
template <int W>
__device__ __forceinline__ int32_t sp_lookback(const uint64_t* desc, int NG, int g, uint32_t t, uint32_t gen,
                                               uint64_t t_begin, int32_t& flag) {
    int32_t acc = 0;
    bool done = false;
    for (int64_t p = (int64_t)t - 1; !done; p -= W) {
        uint64_t d[W];
#pragma unroll
        for (int i = 0; i < W; ++i) d[i] = p - i >= 0 ? sp_load(&desc[(p - i) * NG + g]) : 0ull;
        uint64_t folded = 0;  // bit i: entry i already added
        for (;;) {
            bool blocked = false;
#pragma unroll
            for (int i = 0; i < W; ++i) {
                if (done || blocked || ((folded >> i) & 1u)) continue;
                if (p - i < 0) {  // tile 0 is inclusive from the start: not reached
                    done = true;
                    continue;
                }
                if (!sp_published(d[i], gen)) {
                    blocked = true;
                    continue;
                }
                acc += sp_value(d[i]);
                folded |= 1ull << i;
                if ((uint32_t)d[i] & kDescInc) done = true;
            }
            if (done || !blocked) break;
            if (wall_clock64() - t_begin > kWaitTicks) {
                flag |= EP_FLAG_INTERNAL;
                done = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int i = 0; i < W; ++i)
                if (!((folded >> i) & 1u) && p - i >= 0) d[i] = sp_load(&desc[(p - i) * NG + g]);
        }
    }
    return acc;
}

template <int SPT, int MAXG, bool LOOKBACK>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_sp(LayoutArgs a) {
    constexpr int J = MAXG / kLayoutThreads;  // groups per thread, contiguous: tid*J + j
    constexpr int W = 32 / J;                 // descriptors per group per round trip
    constexpr int kTileSlots = kLayoutThreads * SPT;
    constexpr int kSlotsPerWave = kWave * SPT;
    __shared__ int32_t s_cnt[MAXG];    // group totals
    __shared__ int32_t s_start[MAXG];  // first row of the group (clamped at capacity)
    __shared__ int32_t s_lim[MAXG];    // first row past the segment's capacity
    __shared__ int32_t s_base[MAXG];   // tile: first row of the group's run minus its stage offset
    __shared__ int32_t s_wcnt[kLayoutWaves][MAXG];  // per-wave counters, then stage offsets
    __shared__ uint16_t s_gof[MAXG];   // group of each routed expert (E <= NG)
    __shared__ int2 s_stage[kTileSlots];  // (row, flat slot) in group-major order
    __shared__ int32_t s_wsum[kLayoutWaves];
    __shared__ int32_t s_flag, s_ntiles, s_nstage;
    __shared__ uint32_t s_ticket, s_gen;
    __shared__ int32_t s_tiles[kSpMaxTilesPerBlock];

    const uint64_t t_begin = wall_clock64();
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int NG = a.NG, G = a.G;
    SpHeader* hdr = reinterpret_cast<SpHeader*>(a.sp_header);
    const uint32_t NT = (uint32_t)a.tiles;
    uint64_t* desc = a.sp_desc;                     // [NT][NG] aggregate, then inclusive prefix
    uint64_t* aggs = a.sp_desc + (int64_t)NT * NG;  // [NT][NG] aggregate only (written once)
    const bool worker = blockIdx.x < NT;
    const int64_t routed = (int64_t)a.T * a.K;
    const int32_t shared_group = a.shared ? a.src_seg * G : -1;
    const int nbits = 32 - __clz(NG);  // keys live in [0, NG]; NG = "no group"

    // Ticket (workers) or generation (the rest) first; the ids of tile
    // blockIdx.x are fetched meanwhile, in case the ticket is that tile.
    if (tid == 0) {
        if (worker) {
            const uint64_t c = __hip_atomic_fetch_add(&hdr->ctl, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_gen = (uint32_t)(c >> 32);
            s_ticket = (uint32_t)c;
        } else {
            s_gen = (uint32_t)(sp_load(&hdr->ctl) >> 32);
            s_ticket = NT;
        }
        s_flag = 0;
        s_ntiles = 0;
    }
    int32_t eid[SPT];
    auto load_ids = [&](uint32_t t) {
        const int64_t f0 = (int64_t)t * kTileSlots + (int64_t)w * kSlotsPerWave + lane;
#pragma unroll
        for (int it = 0; it < SPT; ++it) {
            const int64_t f = f0 + it * kWave;
            eid[it] = f < routed ? a.topk_ids[f] : -1;
        }
    };
    if (worker) load_ids(blockIdx.x);
    for (int e = tid; e < a.E; e += kLayoutThreads)
        s_gof[e] = (uint16_t)((e / a.E_loc) * G + a.shared + (e % a.E_loc));
    __syncthreads();
    const uint32_t gen = s_gen;

    uint32_t key[SPT], rnk[SPT];
    int32_t agg[J], tgo[J];
    int32_t flag = 0;
    // Ranks of the tile's slots in their groups: wave w owns slots
    // [w*64*SPT, (w+1)*64*SPT) of the tile, in SPT rounds of 64, so the
    // stable order (ascending slot index) is wave, round, lane.  Leaves
    // s_wcnt[w][g] = this wave's stage offset for group g (the tile's
    // earlier groups, then earlier waves), agg = the tile's count per owned
    // group, tgo = the tile's stage offset of each owned group, and the
    // number of staged (valid) slots in s_nstage.
    auto rank_tile = [&]() {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int g = tid * J + j;
#pragma unroll
            for (int w2 = 0; w2 < kLayoutWaves; ++w2)
                if (g < NG) s_wcnt[w2][g] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < SPT; ++it) {
            const int32_t e = eid[it];
            const uint32_t k = (uint32_t)e < (uint32_t)a.E ? (uint32_t)s_gof[e] : (uint32_t)NG;
            if (e != -1 && (uint32_t)e >= (uint32_t)a.E) flag |= EP_FLAG_BAD_ID;  // -1 = masked slot
            const uint64_t m = match_any(k, nbits);
            const uint32_t r = lanes_below(m);
            // only the lowest lane of each key touches LDS; the others take
            // its value by a cross-lane read
            int32_t before = 0;
            if (k != (uint32_t)NG && r == 0) {
                before = s_wcnt[w][k];
                s_wcnt[w][k] = before + (int32_t)__popcll(m);
            }
            before = __shfl(before, (int)__builtin_ctzll(m), kWave);
            rnk[it] = (uint32_t)before + r;
            key[it] = k;
        }
        __syncthreads();
        int32_t tsum = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int g = tid * J + j;
            int32_t run = 0;
            if (g < NG) {
#pragma unroll
                for (int w2 = 0; w2 < kLayoutWaves; ++w2) {
                    const int32_t c = s_wcnt[w2][g];
                    s_wcnt[w2][g] = run;
                    run += c;
                }
            }
            agg[j] = run;
            tgo[j] = tsum;
            tsum += run;
        }
        // exclusive scan of the per-thread sums: stage offsets of the groups
        const int32_t incl = wave_inclusive_sum(tsum);
        if (lane == kWave - 1) s_wsum[w] = incl;
        __syncthreads();
        int32_t wb = 0, tot = 0;
#pragma unroll
        for (int w2 = 0; w2 < kLayoutWaves; ++w2) {
            wb += w2 < w ? s_wsum[w2] : 0;
            tot += s_wsum[w2];
        }
        const int32_t tbase = wb + incl - tsum;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int g = tid * J + j;
            tgo[j] += tbase;
            if (g < NG) {
#pragma unroll
                for (int w2 = 0; w2 < kLayoutWaves; ++w2) s_wcnt[w2][g] += tgo[j];
            }
        }
        if (tid == 0) s_nstage = tot;
        __syncthreads();
    };

    // ---- phase 1: tiles by ticket; publish aggregates (and, with the
    // look-back, resolve and publish inclusive prefixes) ----
    int32_t pref[J];
    uint32_t t = s_ticket;
    bool live = false;  // key/rnk/s_wcnt/agg/tgo hold the last tile taken
    while (t < NT) {
        if (t != blockIdx.x || live) load_ids(t);
        rank_tile();
        // The next ticket travels meanwhile (its value is stored only
        // afterwards, so nothing waits for it here); a workgroup with a full
        // tile list stops taking tickets.
        uint32_t next_ticket = NT;
        if (tid == 0) {
            s_tiles[s_ntiles] = (int32_t)t;
            s_ntiles += 1;
            if (s_ntiles < kSpMaxTilesPerBlock)
                next_ticket = (uint32_t)__hip_atomic_fetch_add(&hdr->ctl, 1ull, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int g = tid * J + j;
            pref[j] = 0;
            if (g < NG) {
                const uint64_t aggd = ((uint64_t)gen << 32) | kDescAgg | (uint32_t)agg[j];
                sp_store(&aggs[(int64_t)t * NG + g], aggd);
                if (LOOKBACK) sp_store(&desc[(int64_t)t * NG + g], t == 0 ? aggd ^ (kDescAgg | kDescInc) : aggd);
            }
        }
        if (LOOKBACK && t > 0) {
            for (int j = 0; j < J; ++j) {
                const int g = tid * J + j;
                if (g < NG) {
                    pref[j] = sp_lookback<W>(desc, NG, g, t, gen, t_begin, flag);
                    sp_store(&desc[(int64_t)t * NG + g],
                             ((uint64_t)gen << 32) | kDescInc | (uint32_t)(pref[j] + agg[j]));
                }
            }
        }
        if (tid == 0) s_ticket = next_ticket;
        live = true;
        __syncthreads();
        const uint32_t next = s_ticket;
        if (next < NT) __syncthreads();  // s_wcnt is reused by the next tile
        else break;
        t = next;
    }

    // ---- phase 2: group totals (every tile has been handed to a running
    // workgroup by now, so the waits end) ----
    for (int j = 0; j < J; ++j) {
        const int g = tid * J + j;
        if (g >= NG) continue;
        int32_t tot;
        if (LOOKBACK) {
            // The totals are the exclusive prefix of a tile past the last
            // one: the look-back from the last tile folds aggregates back to
            // the first inclusive prefix it meets, a few round trips however
            // many tiles there are (summing every later tile's aggregate
            // instead makes the pass quadratic in the tile count).
            tot = sp_lookback<W>(desc, NG, g, NT, gen, t_begin, flag);
        } else {
            int32_t from_t = 0;  // tiles >= t
            tot = sp_sum<W>(aggs, NG, g, 0, NT, live ? t : NT, &from_t, gen, t_begin, flag);
            if (live) pref[j] = tot - from_t;
        }
        s_cnt[g] = tot + (g == shared_group ? a.T : 0);
    }
    __syncthreads();

    // ---- aligned exclusive prefix over all groups (segment-major) ----
    int32_t al[J];
    int32_t asum = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int g = tid * J + j;
        al[j] = g < NG ? align_up(s_cnt[g], a.A) : 0;
        asum += al[j];
    }
    const int32_t aincl = wave_inclusive_sum(asum);
    if (lane == kWave - 1) s_wsum[w] = aincl;
    __syncthreads();
    int32_t awb = 0, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < kLayoutWaves; ++w2) {
        awb += w2 < w ? s_wsum[w2] : 0;
        total += s_wsum[w2];
    }
    {
        int32_t run = awb + aincl - asum;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int g = tid * J + j;
            if (g < NG) s_start[g] = run;
            run += al[j];
        }
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int g = tid; g < NG; g += kLayoutThreads) a.out.counts[g] = s_cnt[g];
        const int n = a.S * (G + 1);
        for (int idx = tid; idx < n; idx += kLayoutThreads) {
            const int s = idx / (G + 1), gl = idx - s * (G + 1);
            const int gi = s * G + gl;
            int32_t off = (gi < NG ? s_start[gi] : total) - s_start[s * G];
            if (a.C > 0 && off > a.C) off = a.C;
            a.out.row_offsets[idx] = off;
            a.out.scales_offsets[idx] = off;
        }
        for (int s = tid; s <= a.S; s += kLayoutThreads)
            a.out.seg_base[s] = a.C > 0 ? s * a.C : (s < a.S ? s_start[s * G] : total);
    }
    // absolute first row (clamped at capacity) and capacity limit per group;
    // workgroup 0 derives the dropped / past-the-buffer bits from them: a
    // group drops slots iff start + count passes its limit, and reaches
    // past the buffer iff its used rows (pad included) end beyond R
    const uint32_t R = (uint32_t)a.recv_rows;
    int32_t st[J], li[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int g = tid * J + j;
        st[j] = 0;
        li[j] = 0;
        if (g < NG) {
            const int s = g / G;
            const int32_t segp = s_start[s * G];
            int32_t off = s_start[g] - segp;
            if (a.C > 0) {
                if (off > a.C) off = a.C;
                st[j] = s * a.C + off;
                li[j] = (s + 1) * a.C;
            } else {
                st[j] = segp + off;
                li[j] = 0x7FFFFFFF;
            }
            if (blockIdx.x == 0) {
                const uint32_t c = (uint32_t)s_cnt[g], s0 = (uint32_t)st[j], l0 = (uint32_t)li[j];
                if (s0 + c > l0) flag |= EP_FLAG_DROPPED;
                const uint32_t end = min(s0 + (uint32_t)align_up((int32_t)c, a.A), l0);
                if (end > s0 && end > R) flag |= EP_FLAG_INTERNAL;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int g = tid * J + j;
        if (g < NG) {
            s_start[g] = st[j];
            s_lim[g] = li[j];
        }
    }

    // ---- flags and departure: one atomic add carries this workgroup's
    // count and flag bits.  Its result is only looked at at the very end (by
    // the last workgroup out), so nothing waits for it here; every ticket
    // this workgroup took was returned before, so the reset below comes
    // after every ticket of the call. ----
    if (flag) atomicOr(&s_flag, flag);
    __syncthreads();
    uint64_t departed = 0;
    const uint64_t mine = sp_departure(s_flag);
    if (tid == 0) departed = __hip_atomic_fetch_add(&hdr->depart, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- phase 3: token_row and src_info of this workgroup's tiles ----
    const int ntiles = worker ? s_ntiles : 0;
    for (int q = ntiles - 1; q >= 0; --q) {
        const uint32_t tt = (uint32_t)s_tiles[q];
        if (q != ntiles - 1) {  // an earlier tile of this workgroup: rank it again
            __syncthreads();
            load_ids(tt);
            rank_tile();
            for (int j = 0; j < J; ++j) {
                const int g = tid * J + j;
                pref[j] = 0;
                if (g < NG) {
                    if (LOOKBACK)  // its published inclusive prefix, less its aggregate
                        pref[j] = sp_value(sp_load(&desc[(int64_t)tt * NG + g])) - agg[j];
                    else           // every aggregate is published by now
                        pref[j] = sp_sum<W>(aggs, NG, g, 0, tt, tt, nullptr, gen, t_begin, flag);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int g = tid * J + j;
            if (g < NG) s_base[g] = st[j] + pref[j] - tgo[j];
        }
        __syncthreads();
        const int64_t f0 = (int64_t)tt * kTileSlots + (int64_t)w * kSlotsPerWave + lane;
#pragma unroll
        for (int it = 0; it < SPT; ++it) {
            const int64_t f = f0 + it * kWave;
            if (f >= routed) continue;
            const uint32_t tk = (uint32_t)f / (uint32_t)a.K, k = (uint32_t)f - tk * (uint32_t)a.K;
            int32_t* tr = &a.out.token_row[(int64_t)tk * a.Kp + k];
            const uint32_t g = key[it];
            if (g == (uint32_t)NG) {
                *tr = -1;
                continue;
            }
            const int32_t pos = s_wcnt[w][g] + (int32_t)rnk[it];
            const uint32_t row = (uint32_t)(s_base[g] + pos);
            const int32_t out = (row >= (uint32_t)s_lim[g] || row >= R) ? -1 : (int32_t)row;
            *tr = out;
            s_stage[pos] = make_int2(out, (int32_t)f);
        }
        __syncthreads();
        const int32_t n = s_nstage;
        for (int32_t i = tid; i < n; i += kLayoutThreads) {
            const int2 e = s_stage[i];
            if (e.x < 0) continue;
            const uint32_t tk = (uint32_t)e.y / (uint32_t)a.K;
            *reinterpret_cast<int2*>(&a.out.src_info[2 * (int64_t)e.x]) =
                make_int2((int32_t)tk, e.y - (int32_t)(tk * (uint32_t)a.K));
        }
    }

    // ---- the fused shared expert: token t is rank t of group 0 of src_seg ----
    __syncthreads();
    const int32_t nb = (int32_t)gridDim.x;
    if (a.shared) {
        const int32_t per = (a.T + nb - 1) / nb;
        const int32_t t0 = (int32_t)blockIdx.x * per;
        const int32_t t1 = min(a.T, t0 + per);
        const uint32_t st0 = (uint32_t)s_start[shared_group], lim0 = (uint32_t)s_lim[shared_group];
        for (int32_t tk = t0 + tid; tk < t1; tk += kLayoutThreads) {
            int32_t* tr = &a.out.token_row[(int64_t)tk * a.Kp + a.K];
            const uint32_t row = st0 + (uint32_t)tk;
            if (row >= lim0 || row >= R) {
                *tr = -1;
            } else {
                *tr = (int32_t)row;
                *reinterpret_cast<int2*>(&a.out.src_info[2 * (int64_t)row]) = make_int2(tk, a.K);
            }
        }
    }

    // ---- expert_ids of every used row and pad-row src_info, by group ----
    for (int g = (int)blockIdx.x; g < NG; g += nb) {
        const int32_t c = s_cnt[g];
        const int32_t n = align_up(c, a.A);
        const int32_t gs = g / G, gl = g - gs * G;
        const int32_t expert = (a.shared && gl == 0) ? a.E : gs * a.E_loc + (gl - a.shared);
        for (int32_t r = tid; r < n; r += kLayoutThreads) {
            const uint32_t row = (uint32_t)s_start[g] + (uint32_t)r;
            if (row >= (uint32_t)s_lim[g] || row >= R) break;
            const bool pad = r >= c;
            a.out.expert_ids[row] = pad ? -1 : expert;
            if (pad) *reinterpret_cast<int2*>(&a.out.src_info[2 * (int64_t)row]) = make_int2(-1, -1);
        }
    }

    // ---- the last workgroup out writes the flags word and resets the
    // header for the next call (no read of this call touches it later) ----
    if (tid == 0 && (departed & 0xFFFFu) == gridDim.x - 1u) {
        const uint64_t all = departed + mine;
        a.out.flags[0] = sp_flags_of(all);
        __hip_atomic_store(&hdr->depart, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sp_store(&hdr->ctl, (uint64_t)(gen + 1u) << 32);
    }
}

}  // namespace

// The rank kernel with LDS arrays for at most 256 groups where they suffice.
template <int SPT, int MODE, bool CHUNKS>
void launch_rank(const LayoutArgs& a, hipStream_t stream) {
    if (a.NG <= kLayoutThreads)
        hipLaunchKernelGGL((k_layout_rank<SPT, MODE, CHUNKS, kLayoutThreads>), dim3((unsigned)a.rank_blocks),
                           dim3(kLayoutThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((k_layout_rank<SPT, MODE, CHUNKS, EP_MAX_GROUPS>), dim3((unsigned)a.rank_blocks),
                           dim3(kLayoutThreads), 0, stream, a);
}

template <int SPT>
void launch_spt(const LayoutArgs& a, hipStream_t stream) {
    const dim3 block(kLayoutThreads);
    if (a.mode == kLayoutSmall) {
        launch_rank<SPT, kLayoutSmall, false>(a, stream);
    } else if (a.mode == kLayoutCount) {
        launch_rank<SPT, kLayoutCount, false>(a, stream);
    } else if (a.mode == kLayoutDirect) {
        hipLaunchKernelGGL((k_layout_hist<SPT>), dim3((unsigned)a.tiles), block, 0, stream, a);
        if (a.chunks > 0)
            hipLaunchKernelGGL(k_layout_chunks,
                               dim3((unsigned)a.chunks, (unsigned)((a.NG + kLayoutThreads - 1) / kLayoutThreads)), block,
                               0, stream, a);
        if (a.chunks > 0)
            launch_rank<SPT, kLayoutDirect, true>(a, stream);
        else
            launch_rank<SPT, kLayoutDirect, false>(a, stream);
    } else if (a.NG <= kLayoutThreads) {
        if (a.lookback)
            hipLaunchKernelGGL((k_layout_sp<SPT, kLayoutThreads, true>), dim3((unsigned)a.rank_blocks), block, 0,
                               stream, a);
        else
            hipLaunchKernelGGL((k_layout_sp<SPT, kLayoutThreads, false>), dim3((unsigned)a.rank_blocks), block, 0,
                               stream, a);
    } else {
        if (a.lookback)
            hipLaunchKernelGGL((k_layout_sp<SPT, EP_MAX_GROUPS, true>), dim3((unsigned)a.rank_blocks), block, 0,
                               stream, a);
        else
            hipLaunchKernelGGL((k_layout_sp<SPT, EP_MAX_GROUPS, false>), dim3((unsigned)a.rank_blocks), block, 0,
                               stream, a);
    }
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
    switch (a.slots_per_thread) {
        case 1: launch_spt<1>(a, stream); break;
        case 2: launch_spt<2>(a, stream); break;
        case 4: launch_spt<4>(a, stream); break;
        default: launch_spt<8>(a, stream); break;
    }
    return hipGetLastError();
}

}  // namespace epx
