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
// Two launches on the caller's stream (the direct path, up to
// kDirectMaxTiles tiles; every configuration up to ~500k routed slots):
//  1. k_layout_hist   per tile of 256 x {2,4,8} routed slots (chosen so that
//                     there are about 64 tiles), a wave64 match-any over
//                     the group key (one ballot per key bit); the lowest lane
//                     of each match set adds the set's popcount into an LDS
//                     counter, so a hot expert costs one LDS atomic per wave
//                     instead of one per slot.  Each tile stores its
//                     per-group counts as one row of a [tile][group]
//                     table; tile 0 also clears the flags word.
//  2. k_layout_rank   every workgroup reads, for each group, the group's
//                     column of tile counts (lanes over groups, so wave
//                     loads are contiguous; 64 loads in flight per lane, and
//                     several lanes per group when groups are few) and sums
//                     it twice: over all tiles (the group total) and over the
//                     tiles before its own (its in-group prefix).  No workgroup waits on another, and
//                     there are no atomics on global memory but the flags.
//                     It then scans the aligned group sizes into group start
//                     rows, ranks its tile's slots inside their groups
//                     (per-wave running counters in LDS + match-any), and
//                     writes counts (tile 0), offsets, token_row and
//                     src_info.  The fused shared-expert rows, and
//                     expert_ids of whole groups (pad rows included) as
//                     coalesced runs, are spread over at least
//                     min(groups, 256) workgroups: the ones past the last
//                     tile do only this.
// Above kDirectMaxTiles the per-workgroup row sums would grow with the tile
// count, so three launches are used instead (also on request, with
// EP_LAYOUT_LOOKBACK; the results are the same):
//  0. k_layout_clear  zero the counts (the shared group gets T) and flags.
//  1. k_layout_hist   publishes each tile's per-group aggregate as a
//                     look-back descriptor ([tile][group], 2 status bits
//                     over a 30-bit count; tile 0 publishes its inclusive
//                     prefix) and adds its nonzero counters into `counts`.
//  2. k_layout_rank   resolves its per-group prefix by decoupled look-back
//                     (16 predecessor descriptors per round trip, folded
//                     nearest-first until an inclusive prefix is met) and
//                     upgrades its own descriptors to inclusive prefixes.
//                     Every aggregate is published by the previous launch,
//                     so no workgroup ever waits on another one.
// Invalid ids are detected where the slots are ranked (k_layout_rank).
#include "epx_device.h"

namespace epx {
namespace {

constexpr int kMaxSpins = 1 << 22;  // look-back gives up (EP_FLAG_INTERNAL) after this
constexpr int kLookback = 16;       // predecessor descriptors read per round trip

__device__ __forceinline__ int32_t align_up(int32_t count, int32_t multiple) {
    if ((multiple & (multiple - 1)) == 0) return (count + multiple - 1) & -multiple;  // power of two
    return ((count + multiple - 1) / multiple) * multiple;
}

__device__ __forceinline__ uint32_t desc_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void desc_store(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void k_layout_clear(LayoutArgs a) {
    const int32_t shared_group = a.shared ? a.src_seg * a.G : -1;
    for (int g = threadIdx.x; g < a.NG; g += blockDim.x) a.out.counts[g] = (g == shared_group) ? a.T : 0;
    if (threadIdx.x == 0) a.out.flags[0] = 0;
}

template <int SPT, bool DIRECT>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_hist(LayoutArgs a) {
    constexpr int kTileSlots = kLayoutThreads * SPT;
    __shared__ int32_t s_hist[EP_MAX_GROUPS];
    __shared__ int32_t s_gof[EP_MAX_GROUPS];  // group of each routed expert
    const int tid = threadIdx.x;
    for (int g = tid; g < a.NG; g += kLayoutThreads) s_hist[g] = 0;
    for (int e = tid; e < a.E; e += kLayoutThreads)
        s_gof[e] = (e / a.E_loc) * a.G + a.shared + (e % a.E_loc);
    __syncthreads();

    const int64_t routed = (int64_t)a.T * a.K;
    const int nbits = 32 - __clz(a.NG);  // keys live in [0, NG]; NG = "no group"
    const int64_t base = (int64_t)blockIdx.x * kTileSlots;
#pragma unroll
    for (int it = 0; it < SPT; ++it) {
        const int64_t f = base + it * kLayoutThreads + tid;
        uint32_t key = (uint32_t)a.NG;
        if (f < routed) {
            const int32_t e = a.topk_ids[f];
            if ((uint32_t)e < (uint32_t)a.E) key = (uint32_t)s_gof[e];
        }
        const uint64_t m = match_any(key, nbits);
        if (key != (uint32_t)a.NG && lanes_below(m) == 0)
            atomicAdd(&s_hist[key], (int32_t)__popcll(m));
    }
    __syncthreads();
    if (DIRECT) {
        uint32_t* row = a.desc + (int64_t)blockIdx.x * a.NG;
        for (int g = tid; g < a.NG; g += kLayoutThreads) row[g] = (uint32_t)s_hist[g];
        if (blockIdx.x == 0 && tid == 0) a.out.flags[0] = 0;
    } else {
        const uint32_t status = blockIdx.x == 0 ? kDescInc : kDescAgg;  // tile 0: prefix 0 + aggregate
        uint32_t* desc = a.desc + (int64_t)blockIdx.x * a.NG;
        for (int g = tid; g < a.NG; g += kLayoutThreads) {
            const int32_t c = s_hist[g];
            desc_store(&desc[g], status | (uint32_t)c);
            if (c) atomicAdd(&a.out.counts[g], c);
        }
    }
}

template <int SPT, int MODE>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_rank(LayoutArgs a) {
    constexpr bool DIRECT = MODE == kLayoutDirect, SMALL = MODE == kLayoutSmall, LOOKBACK = MODE == kLayoutLookback;
    constexpr int kTileSlots = kLayoutThreads * SPT;
    constexpr int kSlotsPerWave = kWave * SPT;
    __shared__ int32_t s_cnt[EP_MAX_GROUPS];    // group totals
    __shared__ int32_t s_start[EP_MAX_GROUPS];  // first row of the group (clamped at capacity)
    __shared__ int32_t s_lim[EP_MAX_GROUPS];    // first row past the segment's capacity
    __shared__ int32_t s_pref[EP_MAX_GROUPS];   // slots of the group in earlier tiles
    __shared__ int32_t s_gof[EP_MAX_GROUPS];    // group of each routed expert
    __shared__ uint16_t s_wcnt[kLayoutWaves][EP_MAX_GROUPS];  // per-wave counts / prefixes
    __shared__ int32_t s_wsum[kLayoutWaves];
    __shared__ int32_t s_flag;

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
    const int32_t shared_group = a.shared ? a.src_seg * G : -1;
    if (tid == 0) s_flag = 0;
    if (DIRECT) {
        // Group totals and this tile's in-group prefix from the [tile][group]
        // table.  tpg (a power of two, tpg * NG <= 256) lanes share a group:
        // lane r of the group sums tiles r, r + tpg, ...; with 64 loads in
        // flight per lane this is one round trip for up to 64 * tpg tiles.
        // The partial sums meet by xor-shuffles inside the lane group (all
        // lanes of a group are active or inactive together).
        constexpr int kBatch = kDirectBatch;
        const int tpg = direct_lanes_per_group(NG);
        const int r = tid & (tpg - 1);
        for (int g = tid / tpg; g < NG; g += kLayoutThreads / tpg) {
            const uint32_t* col = a.desc + g;
            int32_t tot = 0, pre = 0;
            for (int j0 = r; j0 < a.tiles; j0 += kBatch * tpg) {
                // Unconditional loads at clamped 32-bit offsets (tiles * NG
                // < 2^20), masked afterwards: no branch around a load and no
                // 64-bit address temporaries, which let the compiler reuse
                // pending loads' registers and wait on each load in turn.
                uint32_t v[kBatch];
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const int j = j0 + i * tpg;
                    v[i] = col[(uint32_t)min(j, a.tiles - 1) * (uint32_t)NG];
                }
                // Every load of the batch is issued before the first is
                // consumed: left to itself the scheduler may interleave the
                // sums with the issue to save registers, which waits on the
                // first loads with half the batch not yet sent (a second
                // round trip to memory).
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const int j = j0 + i * tpg;
                    const int32_t n = j < a.tiles ? (int32_t)v[i] : 0;
                    tot += n;
                    pre += j < (int)tile ? n : 0;
                }
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
    } else if (LOOKBACK) {
        for (int g = tid; g < NG; g += kLayoutThreads) s_cnt[g] = a.out.counts[g];
    }
    for (int e = tid; e < a.E; e += kLayoutThreads)
        s_gof[e] = (e / a.E_loc) * G + a.shared + (e % a.E_loc);
#pragma unroll
    for (int w2 = 0; w2 < kLayoutWaves; ++w2)
        for (int g = tid; g < NG; g += kLayoutThreads) s_wcnt[w2][g] = 0;
    __syncthreads();

    // In-tile ranks (per-wave running counters + match-any), then the
    // per-wave exclusive prefixes and the tile's aggregate per group.
    uint32_t key[SPT], rnk[SPT];
    int32_t flag = 0;
    int32_t agg[EP_MAX_GROUPS / kLayoutThreads];
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
            rnk[it] = 0;
            if (k != (uint32_t)NG) {
                const uint32_t before = s_wcnt[w][k];
                rnk[it] = before + r;
                if (r == 0) s_wcnt[w][k] = (uint16_t)(before + (uint32_t)__popcll(m));
            }
            key[it] = k;
        }
        __syncthreads();

        // ---- per-wave exclusive prefixes and the tile aggregate per group ----
#pragma unroll
        for (int j = 0; j < EP_MAX_GROUPS / kLayoutThreads; ++j) {
            const int g = tid + j * kLayoutThreads;
            agg[j] = 0;
            if (g < NG) {
                int32_t run = 0;
#pragma unroll
                for (int w2 = 0; w2 < kLayoutWaves; ++w2) {
                    const int32_t c = s_wcnt[w2][g];
                    s_wcnt[w2][g] = (uint16_t)run;
                    run += c;
                }
                agg[j] = run;
            }
        }
    };

    // Single pass: the group totals come from ranking the one tile.
    if (SMALL) {
        rank_slots();
#pragma unroll
        for (int j = 0; j < EP_MAX_GROUPS / kLayoutThreads; ++j) {
            const int g = tid + j * kLayoutThreads;
            if (g < NG) {
                s_cnt[g] = agg[j] + (g == shared_group ? a.T : 0);
                s_pref[g] = 0;
            }
        }
        __syncthreads();
    }

    // ---- aligned exclusive prefix P over all groups (segment-major) ----
    // Thread i covers groups [8i, 8i + 8); NG <= 2048 = 256 * 8.
    int32_t al[8];
    int32_t tsum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int g = tid * 8 + j;
        al[j] = g < NG ? align_up(s_cnt[g], a.A) : 0;
        tsum += al[j];
    }
    int32_t incl = tsum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int32_t n = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += n;
    }
    if (lane == kWave - 1) s_wsum[w] = incl;
    __syncthreads();
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
            const int g = tid * 8 + j;
            if (g < NG) s_start[g] = run;
            run += al[j];
        }
    }
    __syncthreads();

    // Counts (direct and single-pass paths), offsets and segment bases: one
    // tile writes them.
    if (tile == 0) {
        if (!LOOKBACK)
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
    // P -> absolute first row (clamped at capacity) and capacity limit.  The
    // segment index advances with g instead of being divided out each time.
    int32_t st[8], li[8];
    int s = (tid * 8) / G, gl = tid * 8 - s * G;
#pragma unroll
    for (int j = 0; j < 8; ++j, ++gl) {
        const int g = tid * 8 + j;
        if (gl == G) {
            ++s;
            gl = 0;
        }
        st[j] = 0;
        li[j] = 0;
        if (g < NG) {
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
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int g = tid * 8 + j;
        if (g < NG) {
            s_start[g] = st[j];
            s_lim[g] = li[j];
        }
    }

    if (!SMALL) rank_slots();

    // ---- decoupled look-back over earlier tiles (look-back path only) ----
#pragma unroll
    for (int j = 0; j < EP_MAX_GROUPS / kLayoutThreads; ++j) {
        const int g = tid + j * kLayoutThreads;
        if (!LOOKBACK || g >= NG) continue;
        uint32_t pref = 0;
        if (owns_tile && tile > 0 && s_cnt[g] > 0 && g != shared_group) {
            // Read a window of kLookback predecessors at once (independent
            // loads, one round trip), then fold them nearest-first until an
            // inclusive prefix is found.  Tile 0's descriptor is inclusive
            // from the start, so the walk ends at or before it.  Every
            // descriptor was published by the histogram launch; the wait
            // below is only a guard and gives up after kMaxSpins polls.
            bool done = false;
            for (int64_t p = (int64_t)tile - 1; !done && p >= 0; p -= kLookback) {
                uint32_t d[kLookback];
#pragma unroll
                for (int i = 0; i < kLookback; ++i)
                    d[i] = (p - i >= 0) ? desc_load(&a.desc[(p - i) * NG + g]) : kDescInc;
#pragma unroll
                for (int i = 0; i < kLookback; ++i) {
                    if (done || p - i < 0) {
                        done = true;
                        continue;
                    }
                    const uint32_t* dp = &a.desc[(p - i) * NG + g];
                    uint32_t di = d[i];
                    int spins = 0;
                    while ((di & ~kDescValue) == 0u) {  // not published yet
                        if (++spins > kMaxSpins) {
                            flag |= EP_FLAG_INTERNAL;
                            di = kDescInc;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                        di = desc_load(dp);
                    }
                    pref += di & kDescValue;
                    if (di & kDescInc) done = true;
                }
            }
            desc_store(&a.desc[(int64_t)tile * NG + g], kDescInc | (pref + (uint32_t)agg[j]));
        }
        s_pref[g] = (int32_t)pref;
    }
    __syncthreads();

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

    if (SMALL) {
        // No earlier launch cleared the flags word, so workgroup 0 stores it
        // whole.  Every bit is a function of the group totals, starts and
        // limits, so it also covers rows other workgroups handled: a group
        // drops slots if start + count > limit, and reaches past the buffer
        // if its used rows (pad included) end beyond R.
        if (tile != 0) return;
        for (int g = tid; g < NG; g += kLayoutThreads) {
            const uint32_t st = (uint32_t)s_start[g], lim = (uint32_t)s_lim[g], c = (uint32_t)s_cnt[g];
            if (st + c > lim) flag |= EP_FLAG_DROPPED;
            const uint32_t end = min(st + (uint32_t)align_up((int32_t)c, a.A), lim);
            if (end > st && end > R) flag |= EP_FLAG_INTERNAL;
        }
        if (flag) atomicOr(&s_flag, flag);
        __syncthreads();
        if (tid == 0) a.out.flags[0] = s_flag;
        return;
    }
    if (flag) atomicOr(&s_flag, flag);
    __syncthreads();
    if (tid == 0 && s_flag) atomicOr(a.out.flags, s_flag);
}

}  // namespace

template <int SPT, bool DIRECT>
void launch_passes(const LayoutArgs& a, hipStream_t stream) {
    constexpr int kMode = DIRECT ? kLayoutDirect : kLayoutLookback;
    const dim3 block(kLayoutThreads);
    if (!DIRECT) hipLaunchKernelGGL(k_layout_clear, dim3(1), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((k_layout_hist<SPT, DIRECT>), dim3((unsigned)a.tiles), block, 0, stream, a);
    hipLaunchKernelGGL((k_layout_rank<SPT, kMode>), dim3((unsigned)a.rank_blocks), block, 0, stream, a);
}

template <int SPT>
void launch_spt(const LayoutArgs& a, hipStream_t stream) {
    if (a.mode == kLayoutSmall)
        hipLaunchKernelGGL((k_layout_rank<SPT, kLayoutSmall>), dim3((unsigned)a.rank_blocks), dim3(kLayoutThreads),
                           0, stream, a);
    else if (a.mode == kLayoutDirect)
        launch_passes<SPT, true>(a, stream);
    else
        launch_passes<SPT, false>(a, stream);
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
