/*
 * epx: MoE expert-parallel token dispatch and combine for one GPU's share of
 * the work, on AMD Instinct MI355X (gfx950).
 *
 * Destination ranks are modelled as segments of one receive buffer in HBM:
 * segment s holds the rows for experts [s*E/S, (s+1)*E/S).  Nothing here
 * moves data between GPUs.
 *
 * Conventions for every call below:
 *  - All buffers are caller-owned device memory (e.g. torch tensors).  The
 *    library never allocates, frees or synchronizes; every call enqueues its
 *    kernels on `stream` (a hipStream_t, NULL = the null stream) and returns.
 *  - Calls are stateless and reentrant.  Two calls that share an output
 *    buffer or a workspace must be ordered by the caller (same stream).
 *  - bf16 values travel as uint16_t bit patterns; float is IEEE binary32.
 *  - Payload pointers (x, recv, expert_out, y, grads, codes) must be 16-byte
 *    aligned; index buffers 4-byte aligned.
 *  - Return value: EP_OK, or a negative status (see ep_strerror).  Argument
 *    errors are found on the host before anything is enqueued.  Data errors
 *    (dropped slots, ids out of range) are reported on the device, in the
 *    layout's flags word, and never make a call fail.
 *
 * Sources for the semantics (page title, API item):
 *  [FA] NeMo AutoModel fused_a2a page: HybridEPDispatch.forward (tokens
 *       [tokens, hidden] -> [dispatched_tokens, hidden] grouped by local
 *       expert; topk_idx with -1 for unused slots; pad_multiple;
 *       num_permuted_tokens as a static, host-known output extent),
 *       HybridEPDispatch.backward (combine the gradients),
 *       HybridEPCombine.forward / backward (restore token order;
 *       redispatch the gradients).
 *  [TD] NeMo AutoModel token_dispatcher page: _align_up,
 *       TokenDispatcherConfig.moe_router_expert_pad_multiple,
 *       TokenDispatcherConfig.moe_router_dtype (fp32 weighted averaging),
 *       _assert_no_hybridep_overflow (device overflow flag, truncation at
 *       capacity), _HybridEPManager._calibrate_hybridep_capacity,
 *       _DeepepManager reversed_mapping_for_combine.
 *  [MX] MAX DistributedEPDispatchBlockScaledNVDynGlobalScales page, execute:
 *       NVFP4 with a per-token global scale 2688/rowmax, output_scales,
 *       output_rowwise_scales (BF16 inverse global scale), row_offsets,
 *       scales_offsets, expert_ids, src_info, atomic_counters,
 *       fused_shared_expert.
 */
#ifndef EPX_H
#define EPX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EPX_ABI_VERSION 1

/* Status codes. */
#define EP_OK 0
#define EP_EINVAL (-1)   /* an argument fails a host-side check                */
#define EP_ELAUNCH (-2)  /* the HIP runtime reported an error enqueueing work  */
#define EP_ENOTSUP (-3)  /* the current device is not gfx950                   */
#define EP_ESCRATCH (-4) /* ep_dispatch_layout_noalloc: the layout needs more
                            scratch than EP_NOALLOC_SCRATCH_BYTES             */
/* A HIP grid dimension holds at most 2^32 - 1 work-items.  ep_dispatch,
 * ep_combine, ep_dispatch_bwd and ep_combine_bwd split larger batches into
 * several launches.  The calls that launch one grid per batch return
 * EP_EINVAL past it: ep_dispatch_nvfp4, ep_dispatch_fp8 and the routing-map
 * conversions from T = 2^26 - 16 tokens (one wave per token), and
 * ep_combine_bwd_probs from T = 2^24 - 4 (one 256-thread workgroup per
 * token). */

/* Bits of ep_cfg_t.flags. */
#define EP_ZERO_PAD_ROWS 1u    /* also write zeros into the payload of pad rows */
/* ep_dispatch_layout path selection: at most one of the next four bits;
   every path gives the same results, they differ only in speed. */
#define EP_LAYOUT_LOOKBACK 2u  /* one kernel: ticketed tiles, each tile's prefix
                                  by decoupled look-back */
#define EP_LAYOUT_DIRECT 4u    /* two kernels: tile-count table, then ranks */
#define EP_LAYOUT_BARRIER 8u   /* one kernel: ticketed tiles, each tile's prefix
                                  from one read of every tile's counts; at
                                  most 2^20 routed slots (T*K), else
                                  EP_EINVAL: its cost grows with the square
                                  of the tile count */
#define EP_LAYOUT_COUNT 16u    /* one kernel: every workgroup counts every
                                  routed slot (no workspace traffic); at
                                  most 2^18 routed slots (T*K), else
                                  EP_EINVAL: its cost grows with the square
                                  of the batch */

/* Bits of the device flags word (ep_layout_t.flags[0]). */
#define EP_FLAG_DROPPED 1      /* a slot was dropped at segment capacity [TD]  */
#define EP_FLAG_BAD_ID 2       /* an expert id outside [-1, E) (slot masked)   */
#define EP_FLAG_INTERNAL 4     /* a layout row past recv_rows, or a single-pass
                                  wait gave up (neither happens in valid use) */
#define EP_FLAG_MAP_OVERFLOW 8 /* a routing-map row marked more than top_k experts */

/* Largest number of groups S * (E/S + shared_expert) a layout may have. */
#define EP_MAX_GROUPS 2048
/* Largest number of slots per token, K + shared_expert. */
#define EP_MAX_SLOTS 64

/*
 * Problem description.  Field names follow the pages' statement of the
 * problem ([MX] hidden_size, top_k, n_experts; [FA] num_local_experts,
 * pad_multiple, num_permuted_tokens).
 *
 * Groups: segment s has G = E/S + shared_expert groups.  With a fused
 * shared expert ([MX] fused_shared_expert) group 0 of every segment is the
 * shared group; only segment src_segment receives rows in it (every token
 * once, as top-k slot index `top_k`, expert id `num_experts`, weight 1 in
 * combine).  Routed expert e goes to segment e/(E/S), group shared+e%(E/S).
 */
typedef struct ep_cfg_t {
    int32_t num_tokens;    /* T >= 0 tokens of this GPU's share                   */
    int32_t hidden;        /* H >= 8, multiple of 8 (bf16 calls) or 16 (NVFP4)     */
    int32_t num_experts;   /* E >= 1 routed experts                               */
    int32_t num_segments;  /* S >= 1 destination segments, E % S == 0             */
    int32_t top_k;         /* K, 1 <= K <= E, K + shared_expert <= EP_MAX_SLOTS  */
    int32_t align;         /* A >= 1: each group's rows are padded to a multiple  */
    int32_t seg_capacity;  /* C >= 0: 0 = packed segments; > 0 = C rows per
                              segment, slots past it are dropped and flagged      */
    int32_t shared_expert; /* 0 or 1                                              */
    int32_t src_segment;   /* 0 <= src_segment < S (ignored without shared)       */
    int32_t reserved0;     /* must be 0                                           */
    int64_t recv_rows;     /* R: rows of every receive-side buffer (expert_ids,
                              src_info, recv, codes, ...); R >= ep_query's
                              min_recv_rows and R < 2^31.  A host integer, so no
                              call ever reads a count back from the device [FA]. */
    uint32_t flags;        /* EP_ZERO_PAD_ROWS, at most one EP_LAYOUT_* bit, or 0 */
    uint32_t reserved1;    /* must be 0                                           */
} ep_cfg_t;

/*
 * The dispatch "handle" ([FA] handle; [TD] overflow flag kept last): device
 * arrays written by ep_dispatch_layout and read by every later call.  K' =
 * K + shared_expert, G = groups per segment, R = recv_rows.
 *   counts         int32 [S*G]      valid slots per group ([TD] tokens per expert)
 *   seg_base       int32 [S+1]      first row of each segment (packed: running
 *                                   sum of used rows; capacity: s*C)
 *   row_offsets    int32 [S*(G+1)]  per segment, exclusive prefix of the
 *                                   aligned group sizes, clamped to C ([MX])
 *   scales_offsets int32 [S*(G+1)]  offsets into the block-scale rows; scales
 *                                   are row-major, so equal to row_offsets ([MX])
 *   token_row      int32 [T*K']     receive row of slot (t,k); -1 if the slot
 *                                   is masked, invalid or dropped ([TD] the
 *                                   reversed mapping used by combine)
 *   expert_ids     int32 [R]        expert of every used row, -1 on pad rows;
 *                                   shared rows carry E ([MX])
 *   src_info       int32 [R*2]      (token t, slot k) of every used row,
 *                                   (-1,-1) on pad rows ([MX])
 *   flags          int32 [1]        EP_FLAG_* bits for this dispatch ([TD])
 * Rows of a segment past its used rows are not written.  Within a group,
 * rows follow ascending slot index t*K'+k (stable, deterministic).
 */
typedef struct ep_layout_t {
    int32_t* counts;
    int32_t* seg_base;
    int32_t* row_offsets;
    int32_t* scales_offsets;
    int32_t* token_row;
    int32_t* expert_ids;
    int32_t* src_info;
    int32_t* flags;
} ep_layout_t;

/*
 * Sizes the caller must allocate for `cfg` (host only, no device work).
 *   min_recv_rows   packed: T*K' + min(T*K', E+shared)*(A-1) (every group
 *                   padded by at most A-1 rows, [TD] _align_up); capacity:
 *                   S*C.
 *   workspace_bytes scratch device memory for ep_dispatch_layout.
 *   groups_per_seg  G = E/S + shared_expert.
 * Any output pointer may be NULL.  Returns EP_OK or EP_EINVAL; recv_rows is
 * not checked here.
 */
int ep_query(const ep_cfg_t* cfg, int64_t* min_recv_rows, int64_t* workspace_bytes,
             int32_t* groups_per_seg);

/*
 * Build the receive layout from top-k expert ids ([FA] HybridEPDispatch
 * routing-metadata preprocessing; [TD] dispatch_postprocess counts;
 * [MX] row_offsets, expert_ids, src_info).
 *   topk_ids   int32 [T*K], row-major; -1 = unused slot ([FA] topk_idx)
 *   workspace  >= workspace_bytes from ep_query, 16-byte aligned, zero-filled
 *              before its first use; every call leaves it ready for the
 *              next one (reuse it: the single-pass kernels keep a generation
 *              count and a ticket in it).  Not shared by calls that may run
 *              at the same time.
 *   layout     the arrays above, all written here (src_info 8-byte aligned)
 * Steps: per tile of routed slots, a wavefront ballot/popcount histogram
 * and in-group ranks (stable, ascending slot index); each tile's prefix
 * over earlier tiles; the aligned group sizes scanned into group start rows;
 * token_row, expert_ids and src_info written.  Paths (same results):
 *  - up to 512 routed slots: one kernel in which every workgroup ranks
 *    all slots itself;
 *  - up to 8192 routed slots (by default; EP_LAYOUT_COUNT at any size): one
 *    kernel in which every workgroup counts all slots per group in LDS,
 *    then ranks its own tile;
 *  - otherwise (by default; EP_LAYOUT_DIRECT at any size): two kernels, a
 *    [tile][group] count table then the ranks, with a third launch between
 *    them past 256 tiles that sums the table in chunks of 256 tiles;
 *  - EP_LAYOUT_LOOKBACK / EP_LAYOUT_BARRIER: one kernel, tiles taken from
 *    an atomic ticket, each tile's prefix by decoupled look-back (or from
 *    one read of every tile's counts, whose cost grows with the square of
 *    the tile count); slower than the two kernels at every size measured.
 * At most 2^24 routed slots (T*K), else EP_EINVAL: up to there every path
 * costs about linearly in the slots (the single pass runs at most 8192
 * tiles).  The other calls take any T*K' < 2^30 with a valid token_row.
 * Data errors go to layout->flags; a single-pass wait that cannot end gives
 * up after about 0.3 s and sets EP_FLAG_INTERNAL.
 */
int ep_dispatch_layout(const ep_cfg_t* cfg, const int32_t* topk_ids, void* workspace,
                       int64_t workspace_bytes, const ep_layout_t* layout, void* stream);

/*
 * bf16 dispatch ([FA] HybridEPDispatch.forward with fuse_permute):
 *   recv[token_row[t,k], :] = x[t, :] bit for bit, for every kept slot.
 *   x     bf16 [T, H];  recv  bf16 [R, H].
 * Uses layout->token_row (and counts/row_offsets/seg_base when
 * EP_ZERO_PAD_ROWS is set).  Unused rows of recv are not written.
 */
int ep_dispatch(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* x,
                uint16_t* recv, void* stream);

/*
 * Layout and bf16 dispatch in one call ([FA] HybridEPDispatch.forward: the
 * permutation and the dispatch of one batch in a single call).  Same
 * arguments, outputs and errors as ep_dispatch_layout followed by
 * ep_dispatch on the same stream, and the same results bit for bit.  Up to
 * 512 routed slots (T*K; decode-sized batches) with no EP_LAYOUT_* path
 * flag, one kernel computes the layout and copies the payload rows: every
 * workgroup already ranks all slots there, so the copy needs no second
 * launch.  Larger batches, or a forced path, run the layout launches and
 * then the dispatch scatter.
 */
int ep_dispatch_with_layout(const ep_cfg_t* cfg, const int32_t* topk_ids, void* workspace,
                            int64_t workspace_bytes, const ep_layout_t* layout, const uint16_t* x,
                            uint16_t* recv, void* stream);

/*
 * NVFP4 dispatch with a per-token dynamic global scale ([MX] execute):
 * every token is quantized once and its bytes written to each kept row.
 *   x         bf16 [T, H] (H % 16 == 0)
 *   codes     uint8 [R, H/2]   E2M1 element codes, element 2j in the low
 *                              nibble of byte j, 2j+1 in the high nibble
 *   scales    uint8 [R, H/16]  E4M3 block scale of each 16-element block
 *   rowscale  bf16  [R]        bf16(1/g), the inverse global scale
 * Per token, in IEEE fp32 with round-to-nearest-even:
 *   rowmax = max|x|;  g = 2688 / rowmax;
 *   per block: s = (bmax / 6) * g -> E4M3 (RNE, saturating to 448);
 *              v = x * (g / e4m3(s)) -> E2M1 (RNE, ties to even, saturating
 *              at 6, sign bit of v kept); zero scale -> zero codes.
 *   An all-zero token gives zero codes, zero scales and rowscale +0.
 * Tokens must be finite; a token with 0 < rowmax < 2688/FLT_MAX (where g
 * overflows) is outside the contract.
 */
int ep_dispatch_nvfp4(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* x,
                      uint8_t* codes, uint8_t* scales, uint16_t* rowscale, void* stream);

/*
 * Layout and NVFP4 dispatch in one call ([MX] execute: the expert layout,
 * the per-token global scales and the NVFP4 payload of one batch in a
 * single call).  Same arguments, outputs and errors as ep_dispatch_layout
 * followed by ep_dispatch_nvfp4 on the same stream, and the same results
 * bit for bit.  Up to 512 routed slots (T*K) with no EP_LAYOUT_* path flag,
 * one kernel computes the layout and quantizes each token once into LDS,
 * then stores its codes, block scales and rowscale to each of its rows;
 * larger batches, or a forced path, run the layout launches and then the
 * NVFP4 dispatch.
 */
int ep_dispatch_nvfp4_with_layout(const ep_cfg_t* cfg, const int32_t* topk_ids, void* workspace,
                                  int64_t workspace_bytes, const ep_layout_t* layout, const uint16_t* x,
                                  uint8_t* codes, uint8_t* scales, uint16_t* rowscale, void* stream);

/*
 * FP8 dispatch ([FA] init_hybrid_ep_buffer: FP8 communication in the
 * dispatch phase; HybridEPDispatch.forward returns a scaling factor beside
 * the hidden states).  The pages give no format; this library reads it as
 * E4M3 codes with one fp32 factor per token and 128-element block:
 *   x       bf16 [T, H] (H % 128 == 0, H <= 16384)
 *   codes   uint8 [R, H]       E4M3 ("fn") codes
 *   scales  float [R, H/128]   dequantization factors
 * Per block, in IEEE fp32 with round-to-nearest-even: amax = max|x|;
 *   codes = E4M3(x * (448 / amax))  (saturating to 448, sign of the product kept)
 *   scale = amax / 448
 * An all-zero block gives zero codes and scale 0.  Every copy of a token
 * carries the same bytes.  Blocks with 0 < amax < 448/FLT_MAX are outside
 * the contract.
 */
int ep_dispatch_fp8(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* x,
                    uint8_t* codes, float* scales, void* stream);

/*
 * Layout and FP8 dispatch in one call ([FA] HybridEPDispatch.forward: the
 * permutation and the FP8 payload with its scaling factor from one call).
 * Same arguments, outputs and errors as ep_dispatch_layout followed by
 * ep_dispatch_fp8 on the same stream, and the same results bit for bit.  Up
 * to 512 routed slots (T*K) with no EP_LAYOUT_* path flag, one kernel
 * computes the layout and quantizes each token once per run of its rows,
 * storing codes and block scales to each; larger batches, or a forced path,
 * run the layout launches and then the FP8 dispatch.
 */
int ep_dispatch_fp8_with_layout(const ep_cfg_t* cfg, const int32_t* topk_ids, void* workspace,
                                int64_t workspace_bytes, const ep_layout_t* layout, const uint16_t* x,
                                uint8_t* codes, float* scales, void* stream);

/*
 * Combine ([FA] HybridEPCombine.forward; [TD] moe_router_dtype fp32):
 *   y[t, :] = bf16_rne( sum_{k=0..K'-1, token_row[t,k] >= 0}
 *                       w_k * float(expert_out[token_row[t,k], :]) )
 * accumulated in fp32 in ascending k, one rounding per multiply and per add
 * (no fused multiply-add), starting from +0.  w_k = probs[t,k] for routed
 * slots (1 when probs is NULL) and 1 for the shared slot.
 *   expert_out bf16 [R, H];  probs float [T, K] or NULL;  y bf16 [T, H].
 * Pad and dropped rows are never read.
 */
int ep_combine(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* expert_out,
               const float* probs, uint16_t* y, void* stream);

/*
 * Combine over NVFP4 expert-output rows ([MX] execute: the NVFP4 row format,
 * output_scales, output_rowwise_scales; [TD] moe_router_dtype fp32): the
 * expert outputs come back in the dispatch's NVFP4 format and are
 * dequantized as they are read:
 *   xhat = e2m1(code) * (e4m3(scale[h/16]) * float(rowscale[row]))
 *   y[t, h] = bf16_rne( sum_{k, token_row[t,k] >= 0} w_k * xhat(token_row[t,k], h) )
 * each product an fp32 multiply, accumulated in fp32 in ascending k from +0
 * with no fused multiply-add; w_k as in ep_combine.
 *   codes     uint8 [R, H/2]   element 2j in the low nibble of byte j (8-byte aligned)
 *   scales    uint8 [R, H/16]  E4M3 block scales, sign bit decoded; the NaN
 *                              codes 0x7F / 0xFF are outside the contract
 *   rowscale  bf16  [R]
 *   probs     float [T, K] or NULL;  y  bf16 [T, H]  (H % 16 == 0)
 * Pad and dropped rows are never read.  Returns EP_EINVAL past one grid:
 * T * ceil(H/1024) waves of 64 work-items must stay below 2^32.
 */
int ep_combine_nvfp4(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint8_t* codes, const uint8_t* scales,
                     const uint16_t* rowscale, const float* probs, uint16_t* y, void* stream);

/*
 * Dispatch backward ([FA] HybridEPDispatch.backward: combine the
 * gradients): grad_x[t] = bf16_rne( sum_k float(grad_recv[token_row[t,k]]) ),
 * fp32, ascending k, unweighted (dispatch is a copy); 0 if no slot is kept.
 *   grad_recv bf16 [R, H];  grad_x bf16 [T, H].
 */
int ep_dispatch_bwd(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* grad_recv,
                    uint16_t* grad_x, void* stream);

/*
 * Combine backward ([FA] HybridEPCombine.backward: redispatch through the
 * saved layout): grad_expert_out[token_row[t,k]] = bf16_rne(w_k * float(grad_y[t]))
 * for every kept slot, w_k as in ep_combine.
 *   grad_y bf16 [T, H];  probs float [T, K] or NULL;  grad_expert_out bf16 [R, H].
 */
int ep_combine_bwd(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* grad_y,
                   const float* probs, uint16_t* grad_expert_out, void* stream);

/*
 * Router-probability gradient ([FA] HybridEPDispatch.backward returns a
 * probability gradient beside the hidden-state gradient): with combine
 * y[t] = sum_k p[t,k] * out[row(t,k)],
 *   grad_probs[t,k] = <grad_y[t], expert_out[token_row[t,k]]>  (k < K)
 * as an fp32 dot product over H; 0 for masked, invalid and dropped slots.
 * The summation order is fixed (each of 256 threads sums its strided
 * share of the row in order, then a fixed tree), so results are
 * deterministic; they equal the exact dot product to within about
 * (8*ceil(H/2048) + 10) * 2^-24 * sum_h |grad_y[t,h] * out[row,h]|.
 *   grad_y bf16 [T, H];  expert_out bf16 [R, H];  grad_probs float [T, K].
 */
int ep_combine_bwd_probs(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* grad_y,
                         const uint16_t* expert_out, float* grad_probs, void* stream);

/*
 * Compact top-k -> dense routing form ([TD] _HybridEPManager._indices_to_multihot;
 * [FA] HybridEPDispatch.forward accepts a Boolean routing map [tokens,
 * experts] with dense probabilities).  Only the fields T, E, K (and their
 * validity) of cfg are used.
 *   topk_ids     int32 [T, K]; -1 and ids outside [0, E) mark nothing
 *   probs        float [T, K]; required iff dense_probs is not NULL
 *   routing_map  uint8 [T, E]: 1 where some slot names the expert, else 0
 *   dense_probs  float [T, E] or NULL: sum of the probabilities of the slots
 *                naming the expert, added in slot order; 0 elsewhere
 */
int ep_indices_to_multihot(const ep_cfg_t* cfg, const int32_t* topk_ids, const float* probs,
                           uint8_t* routing_map, float* dense_probs, void* stream);

/*
 * Dense routing form -> compact top-k (the reverse; [FA] routing_map takes
 * precedence over topk_idx, so a caller holding both converts the map).
 *   routing_map  uint8 [T, E]; any nonzero byte marks the expert
 *   dense_probs  float [T, E]; required iff probs is not NULL
 *   topk_ids     int32 [T, K]: the marked experts in ascending order, then -1
 *   probs        float [T, K] or NULL: their dense probabilities, then 0
 *   flags        int32 [1] or NULL: OR-ed with EP_FLAG_MAP_OVERFLOW when a
 *                row marks more than K experts (the lowest K are kept); the
 *                caller clears it
 */
int ep_multihot_to_indices(const ep_cfg_t* cfg, const uint8_t* routing_map, const float* dense_probs,
                           int32_t* topk_ids, float* probs, int32_t* flags, void* stream);

/*
 * ep_dispatch_layout without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * ep_dispatch_layout, except that the workspace is a buffer built into the
 * library: EP_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the first call
 * on that GPU until the process ends.  Returns EP_ESCRATCH, before anything
 * is enqueued, when ep_query's workspace_bytes for cfg exceeds it.  Every
 * call on one GPU shares that buffer: two calls that may run at the same
 * time on one GPU (different streams, no ordering between them) race and
 * give undefined layouts; calls on one stream are ordered and safe.  Never
 * allocates, frees or synchronizes.
 */
#define EP_NOALLOC_SCRATCH_BYTES (4 << 20)
int ep_dispatch_layout_noalloc(const ep_cfg_t* cfg, const int32_t* topk_ids, const ep_layout_t* layout,
                               void* stream);

/* Static description of a status code. */
const char* ep_strerror(int status);

/* EPX_ABI_VERSION of the built library. */
int ep_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EPX_H */
