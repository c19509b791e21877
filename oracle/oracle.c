/*
 * CPU oracle for MoE expert-parallel dispatch and combine (one GPU's share).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only tests/, the smoke check in __graft_entry__.py and the
 * cpu_baseline leg of bench.py use it.  It shares no code, header, table or
 * constant with the HIP library; the only thing both sides share is the
 * seeded input generator.
 *
 * Plain, slow, single-threaded and scalar on purpose: every function below
 * is the definition of the step it computes, written out in the order the
 * pages describe it, so that it can be read against them by eye.  Build
 * with  gcc -O2 -fno-fast-math -ffp-contract=off  (no FMA contraction, no
 * excess precision: every float operation is one IEEE binary32 operation
 * rounded to nearest-even).
 *
 * Sources (page title, API item):
 *  - NeMo AutoModel fused_a2a page, HybridEPDispatch.forward / backward and
 *    HybridEPCombine.forward / backward: dispatch permutes [tokens, hidden]
 *    into [dispatched_tokens, hidden] grouped by local expert, -1 marks an
 *    unused top-k slot; combine restores [tokens, hidden]; the backward of
 *    dispatch combines gradients, the backward of combine redispatches them.
 *  - NeMo AutoModel token_dispatcher page: _align_up (round a count up to a
 *    multiple), TokenDispatcherConfig.moe_router_expert_pad_multiple
 *    (per-expert padding), TokenDispatcherConfig.moe_router_dtype (fp32
 *    weighted averaging), _assert_no_hybridep_overflow (truncation at
 *    capacity sets a device overflow flag), _DeepepManager
 *    reversed_mapping_for_combine (the inverse permutation used by combine).
 *  - MAX DistributedEPDispatchBlockScaledNVDynGlobalScales page, execute:
 *    each token is quantized to NVFP4 against its own global scale
 *    2688 / rowmax, block scales go to output_scales, the BF16 inverse of
 *    the global scale to output_rowwise_scales; row_offsets,
 *    scales_offsets, expert_ids (one per received token) and src_info
 *    (origin and token index of each received token); fused_shared_expert.
 *  - Number formats: OCP 8-bit floating point (E4M3, "fn" variant: bias 7,
 *    no infinities, 0x7F/0xFF are NaN, largest finite 448); OCP
 *    Microscaling (E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6); bfloat16
 *    = upper 16 bits of IEEE binary32, rounded to nearest-even.
 *
 * Readings where the pages are silent (the design notes list each one too):
 *  - segment of expert e is e / (E/S); with a fused shared expert every
 *    segment gets an extra group 0, only segment src_seg receives rows in
 *    it (all T tokens, slot index K, expert id E, weight 1 in combine);
 *  - within a group, rows follow ascending flattened slot index t*K'+k;
 *  - capacity mode: positions >= C inside a segment are dropped;
 *  - pad rows carry expert id -1 and source (-1,-1), payload untouched;
 *  - NVFP4 op order: g = 2688/rowmax; per 16-block s = (bmax/6)*g encoded
 *    E4M3 (RNE, saturate to finite), v = x * (g / decode(scale)) encoded
 *    E2M1 (RNE, ties to even code, saturate at 6, sign = sign bit of v),
 *    low nibble = even element, rowscale = bf16(1/g).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t T, H, E, S, K;   /* tokens, hidden, routed experts, segments, top-k */
    int32_t A;               /* per-group row alignment (pad multiple), >= 1    */
    int32_t C;               /* rows per segment; 0 = packed (no capacity)      */
    int32_t shared;          /* 1 = fused shared expert                          */
    int32_t src_seg;         /* segment holding the shared group                 */
    int64_t recv_rows;       /* receive rows the caller allocated                */
} orc_cfg;

#define ORC_FLAG_DROPPED 1
#define ORC_FLAG_BAD_ID 2

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 -> float: the 16 bits become the upper half of a binary32. */
float orc_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* float -> bfloat16, round to nearest, ties to even, written as a choice
 * between the two bf16 neighbours of f (truncation and its successor). */
uint16_t orc_bf16_rne(float f)
{
    uint32_t u = bits_from_f32(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);   /* keep sign, quiet */
    uint16_t lo = (uint16_t)(u >> 16);                      /* toward zero       */
    uint32_t rem = u & 0xFFFFu;                             /* dropped bits      */
    if (rem > 0x8000u) return (uint16_t)(lo + 1);
    if (rem < 0x8000u) return lo;
    return (lo & 1u) ? (uint16_t)(lo + 1) : lo;             /* exact tie: even   */
}

/* E4M3 ("fn") code -> value.  Exponent field 0 is subnormal: m * 2^-9. */
float orc_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexpf((float)m, -9);
    else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -v : v;
}

/* Non-negative float -> E4M3 code: the nearest finite E4M3 value, ties to
 * the code with an even mantissa; values beyond the largest finite (448)
 * saturate to it.  Brute force over the 127 non-negative finite codes. */
uint8_t orc_e4m3_encode(float s)
{
    if (!(s > 0.0f)) return 0;                 /* 0 (and out-of-contract NaN) */
    if (s >= 448.0f) return 0x7E;              /* saturate to finite          */
    static float value[0x7F];
    static int have_values = 0;
    if (!have_values) {
        for (int c = 0; c <= 0x7E; ++c) value[c] = orc_e4m3_decode((uint8_t)c);
        have_values = 1;
    }
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs((double)value[c] - (double)s);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)best;
}

/* E2M1 code -> value (OCP MX element format). */
float orc_e2m1_decode(uint8_t c)
{
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float v = mag[c & 7];
    return (c & 8) ? -v : v;
}

/* float -> E2M1 code: nearest magnitude, ties to the even code, saturating
 * at 6; the sign bit is the sign bit of v (so -0 and tiny negatives keep
 * it).  Brute force over the 8 magnitudes. */
uint8_t orc_e2m1_encode(float v)
{
    double a = fabs((double)v);
    if (a >= 6.0) return (uint8_t)(7 | (signbit(v) ? 8 : 0));   /* saturate */
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double err = fabs((double)orc_e2m1_decode((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 8 : 0));
}

/* ------------------------------------------------------------------ */
/* Layout: counts, aligned offsets, stable placement, metadata          */
/* ------------------------------------------------------------------ */

static int32_t align_up(int32_t count, int32_t multiple)
{
    /* token_dispatcher page, _align_up: next multiple of `multiple`. */
    return ((count + multiple - 1) / multiple) * multiple;
}

int32_t orc_groups_per_segment(const orc_cfg* c) { return c->E / c->S + c->shared; }

/* Group of slot (t, k), or -1 if the slot is masked.  *eid receives the
 * expert id recorded for the row, *bad is set for ids outside [-1, E). */
static int32_t slot_group(const orc_cfg* c, const int32_t* ids, int32_t t, int32_t k,
                          int32_t* eid, int* bad)
{
    int32_t E_loc = c->E / c->S, G = E_loc + c->shared;
    if (k == c->K) {                      /* the fused shared-expert slot */
        *eid = c->E;
        return c->src_seg * G + 0;
    }
    int32_t e = ids[(int64_t)t * c->K + k];
    if (e == -1) return -1;               /* unused top-k slot             */
    if (e < 0 || e >= c->E) { *bad = 1; return -1; }
    *eid = e;
    return (e / E_loc) * G + c->shared + (e % E_loc);
}

/*
 * Outputs (caller-allocated):
 *   counts        [S*G]       valid slots per group
 *   row_offsets   [S*(G+1)]   aligned exclusive prefix per segment (clamped to C)
 *   scales_offsets[S*(G+1)]   same as row_offsets (row-major scales)
 *   seg_base      [S+1]       first row of each segment
 *   token_row     [T*K']      receive row of slot (t,k), -1 masked/dropped
 *   expert_ids    [recv_rows] expert of each used row, -1 on pad rows
 *   src_info      [recv_rows*2] (t, k) of each used row, (-1,-1) on pad rows
 *   flags         [1]         bit0 dropped at capacity, bit1 invalid id
 * Rows past a segment's used rows are left untouched.
 * Returns 0, or -1 if a row would fall outside recv_rows.
 */
int orc_layout(const orc_cfg* c, const int32_t* ids, int32_t* counts, int32_t* row_offsets,
               int32_t* scales_offsets, int32_t* seg_base, int32_t* token_row,
               int32_t* expert_ids, int32_t* src_info, int32_t* flags)
{
    const int32_t S = c->S, G = orc_groups_per_segment(c), Kp = c->K + c->shared;
    const int32_t NG = S * G;
    int bad = 0, dropped = 0;

    /* 1. counts per group (token_dispatcher page, dispatch_postprocess:
     *    "number of tokens per expert"). */
    for (int32_t g = 0; g < NG; ++g) counts[g] = 0;
    for (int32_t t = 0; t < c->T; ++t)
        for (int32_t k = 0; k < Kp; ++k) {
            int32_t eid, g = slot_group(c, ids, t, k, &eid, &bad);
            if (g >= 0) counts[g] += 1;
        }

    /* 2. aligned exclusive prefix inside each segment (_align_up, pad
     *    multiple); unclamped offsets kept in `off`. */
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)S * (G + 1));
    for (int32_t s = 0; s < S; ++s) {
        off[s * (G + 1)] = 0;
        for (int32_t g = 0; g < G; ++g)
            off[s * (G + 1) + g + 1] = off[s * (G + 1) + g] + align_up(counts[s * G + g], c->A);
    }
    for (int32_t s = 0; s < S; ++s)
        for (int32_t g = 0; g <= G; ++g) {
            int64_t o = off[s * (G + 1) + g];
            if (c->C > 0 && o > c->C) o = c->C;
            row_offsets[s * (G + 1) + g] = (int32_t)o;
            scales_offsets[s * (G + 1) + g] = (int32_t)o;
        }
    seg_base[0] = 0;
    for (int32_t s = 0; s < S; ++s)
        seg_base[s + 1] = c->C > 0 ? (s + 1) * c->C
                                   : seg_base[s] + (int32_t)off[s * (G + 1) + G];

    /* 3. stable placement: walk slots in flattened order, each group hands
     *    out consecutive ranks. */
    int32_t* cursor = (int32_t*)calloc((size_t)NG, sizeof(int32_t));
    int rc = 0;
    for (int32_t t = 0; t < c->T; ++t)
        for (int32_t k = 0; k < Kp; ++k) {
            int64_t f = (int64_t)t * Kp + k;
            int32_t eid = -1, g = slot_group(c, ids, t, k, &eid, &bad);
            token_row[f] = -1;
            if (g < 0) continue;
            int32_t s = g / G, gl = g % G;
            int64_t pos = off[s * (G + 1) + gl] + cursor[g]++;
            if (c->C > 0 && pos >= c->C) { dropped = 1; continue; }
            int64_t row = seg_base[s] + pos;
            if (row >= c->recv_rows) { rc = -1; continue; }
            token_row[f] = (int32_t)row;
            expert_ids[row] = eid;
            src_info[2 * row] = t;
            src_info[2 * row + 1] = k;
        }

    /* 4. pad rows of every group: metadata -1. */
    for (int32_t g = 0; g < NG; ++g) {
        int32_t s = g / G, gl = g % G;
        for (int32_t r = counts[g]; r < align_up(counts[g], c->A); ++r) {
            int64_t pos = off[s * (G + 1) + gl] + r;
            if (c->C > 0 && pos >= c->C) break;
            int64_t row = seg_base[s] + pos;
            if (row >= c->recv_rows) { rc = -1; break; }
            expert_ids[row] = -1;
            src_info[2 * row] = -1;
            src_info[2 * row + 1] = -1;
        }
    }
    flags[0] = (dropped ? ORC_FLAG_DROPPED : 0) | (bad ? ORC_FLAG_BAD_ID : 0);
    free(cursor);
    free(off);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Payload movement                                                    */
/* ------------------------------------------------------------------ */

/* bf16 dispatch: recv[token_row[t,k]] = x[t], bit for bit. */
void orc_dispatch(const orc_cfg* c, const int32_t* token_row, const uint16_t* x, uint16_t* recv)
{
    const int32_t Kp = c->K + c->shared;
    for (int32_t t = 0; t < c->T; ++t)
        for (int32_t k = 0; k < Kp; ++k) {
            int32_t row = token_row[(int64_t)t * Kp + k];
            if (row < 0) continue;
            memcpy(recv + (int64_t)row * c->H, x + (int64_t)t * c->H, sizeof(uint16_t) * c->H);
        }
}

/* Weight of slot k of token t: the routing probability, 1 for the shared
 * slot, 1 for every slot when probs is NULL. */
static float slot_weight(const orc_cfg* c, const float* probs, int32_t t, int32_t k)
{
    if (probs == NULL || k >= c->K) return 1.0f;
    return probs[(int64_t)t * c->K + k];
}

/* combine: y[t] = bf16( sum_k w_k * float(out[row(t,k)]) ), fp32, k ascending. */
void orc_combine(const orc_cfg* c, const int32_t* token_row, const uint16_t* out,
                 const float* probs, uint16_t* y)
{
    const int32_t Kp = c->K + c->shared;
    for (int32_t t = 0; t < c->T; ++t)
        for (int32_t h = 0; h < c->H; ++h) {
            float acc = 0.0f;
            for (int32_t k = 0; k < Kp; ++k) {
                int32_t row = token_row[(int64_t)t * Kp + k];
                if (row < 0) continue;
                float w = slot_weight(c, probs, t, k);
                float v = orc_bf16_to_f32(out[(int64_t)row * c->H + h]);
                float prod = w * v;
                acc = acc + prod;
            }
            y[(int64_t)t * c->H + h] = orc_bf16_rne(acc);
        }
}

/* dispatch backward: grad_x[t] = bf16( sum_k float(grad_recv[row(t,k)]) ). */
void orc_dispatch_bwd(const orc_cfg* c, const int32_t* token_row, const uint16_t* grad_recv,
                      uint16_t* grad_x)
{
    orc_combine(c, token_row, grad_recv, NULL, grad_x);
}

/* combine backward: grad_out[row(t,k)] = bf16( w_k * float(grad_y[t]) ). */
void orc_combine_bwd(const orc_cfg* c, const int32_t* token_row, const uint16_t* grad_y,
                     const float* probs, uint16_t* grad_out)
{
    const int32_t Kp = c->K + c->shared;
    for (int32_t t = 0; t < c->T; ++t)
        for (int32_t k = 0; k < Kp; ++k) {
            int32_t row = token_row[(int64_t)t * Kp + k];
            if (row < 0) continue;
            float w = slot_weight(c, probs, t, k);
            for (int32_t h = 0; h < c->H; ++h) {
                float prod = w * orc_bf16_to_f32(grad_y[(int64_t)t * c->H + h]);
                grad_out[(int64_t)row * c->H + h] = orc_bf16_rne(prod);
            }
        }
}

/* Router-probability gradient (NeMo AutoModel fused_a2a page,
 * HybridEPDispatch.backward returns a probability gradient next to the
 * hidden-state gradient): combine is y[t] = sum_k p[t,k] * out[row(t,k)],
 * so d loss / d p[t,k] = <grad_y[t], out[row(t,k)]>.  The dot product is
 * taken in double (the definition, not a rounding order); masked, invalid
 * and dropped slots get 0.  grad_probs is [T, K] (the shared slot carries
 * no probability). */
void orc_combine_bwd_probs(const orc_cfg* c, const int32_t* token_row, const uint16_t* grad_y,
                           const uint16_t* out, double* grad_probs)
{
    const int32_t Kp = c->K + c->shared;
    for (int32_t t = 0; t < c->T; ++t)
        for (int32_t k = 0; k < c->K; ++k) {
            int32_t row = token_row[(int64_t)t * Kp + k];
            double dot = 0.0;
            if (row >= 0)
                for (int32_t h = 0; h < c->H; ++h)
                    dot += (double)orc_bf16_to_f32(grad_y[(int64_t)t * c->H + h]) *
                           (double)orc_bf16_to_f32(out[(int64_t)row * c->H + h]);
            grad_probs[(int64_t)t * c->K + k] = dot;
        }
}

/* ------------------------------------------------------------------ */
/* Combine over NVFP4 expert outputs                                   */
/* ------------------------------------------------------------------ */

/* Combine whose expert outputs arrive as NVFP4 rows: codes [rows, H/2]
 * (element 2j in the low nibble of byte j), E4M3 block scales [rows, H/16]
 * and a bf16 rowscale per row, the layout the MAX
 * DistributedEPDispatchBlockScaledNVDynGlobalScales page's execute
 * produces (output_scales, output_rowwise_scales: the BF16 inverse of the
 * per-token global scale).  Element h of row r dequantizes as
 *     xhat = e2m1(code) * (e4m3(scale[h/16]) * float(rowscale))
 * (reading: the block's combined scale first, then the element, each an
 * IEEE fp32 multiply rounded to nearest-even; both products are exact
 * unless they fall below the fp32 normal range), and combine sums
 * w_k * xhat over the kept slots in ascending k in fp32, exactly as
 * orc_combine does with bf16 rows. */
void orc_combine_nvfp4(const orc_cfg* c, const int32_t* token_row, const uint8_t* codes,
                       const uint8_t* scales, const uint16_t* rowscale, const float* probs, uint16_t* y)
{
    const int32_t Kp = c->K + c->shared, H = c->H;
    for (int32_t t = 0; t < c->T; ++t)
        for (int32_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t k = 0; k < Kp; ++k) {
                int32_t row = token_row[(int64_t)t * Kp + k];
                if (row < 0) continue;
                float w = slot_weight(c, probs, t, k);
                uint8_t byte = codes[(int64_t)row * (H / 2) + h / 2];
                uint8_t code = (h % 2 == 0) ? (uint8_t)(byte & 0x0F) : (uint8_t)(byte >> 4);
                float block_scale = orc_e4m3_decode(scales[(int64_t)row * (H / 16) + h / 16]) *
                                    orc_bf16_to_f32(rowscale[row]);
                float xhat = orc_e2m1_decode(code) * block_scale;
                float prod = w * xhat;
                acc = acc + prod;
            }
            y[(int64_t)t * H + h] = orc_bf16_rne(acc);
        }
}

/* ------------------------------------------------------------------ */
/* Compact top-k <-> dense routing map                                  */
/* ------------------------------------------------------------------ */

/* NeMo AutoModel token_dispatcher page, _HybridEPManager._indices_to_multihot:
 * top-k indices (and their probabilities) become a multihot [T, E] map and
 * a dense [T, E] probability matrix.  Readings: -1 and ids outside [0, E)
 * set nothing; an expert named by two slots of one token is set once and
 * its probabilities add, in slot order (so a combine over the dense form
 * weights that expert's output by the same total). */
void orc_indices_to_multihot(const orc_cfg* c, const int32_t* ids, const float* probs,
                             uint8_t* routing_map, float* dense_probs)
{
    for (int32_t t = 0; t < c->T; ++t) {
        for (int32_t e = 0; e < c->E; ++e) {
            routing_map[(int64_t)t * c->E + e] = 0;
            if (dense_probs) dense_probs[(int64_t)t * c->E + e] = 0.0f;
        }
        for (int32_t k = 0; k < c->K; ++k) {
            int32_t e = ids[(int64_t)t * c->K + k];
            if (e < 0 || e >= c->E) continue;
            routing_map[(int64_t)t * c->E + e] = 1;
            if (dense_probs && probs)
                dense_probs[(int64_t)t * c->E + e] = dense_probs[(int64_t)t * c->E + e] + probs[(int64_t)t * c->K + k];
        }
    }
}

/* The reverse direction (NeMo AutoModel fused_a2a page,
 * HybridEPDispatch.forward takes either a dense routing map or compact
 * indices).  Readings: the experts a token's row marks (any nonzero byte)
 * fill its slots in ascending expert order, the rest get -1 and
 * probability 0; a row marking more than K experts keeps the lowest K and
 * raises flag bit 3 (value 8).  Returns the flag bits. */
int32_t orc_multihot_to_indices(const orc_cfg* c, const uint8_t* routing_map, const float* dense_probs,
                                int32_t* ids, float* probs)
{
    int32_t flags = 0;
    for (int32_t t = 0; t < c->T; ++t) {
        int32_t n = 0;
        for (int32_t e = 0; e < c->E; ++e) {
            if (!routing_map[(int64_t)t * c->E + e]) continue;
            if (n == c->K) {
                flags |= 8;
                break;
            }
            ids[(int64_t)t * c->K + n] = e;
            if (probs) probs[(int64_t)t * c->K + n] = dense_probs ? dense_probs[(int64_t)t * c->E + e] : 0.0f;
            ++n;
        }
        for (; n < c->K; ++n) {
            ids[(int64_t)t * c->K + n] = -1;
            if (probs) probs[(int64_t)t * c->K + n] = 0.0f;
        }
    }
    return flags;
}

/* ------------------------------------------------------------------ */
/* FP8 (E4M3) dispatch                                                 */
/* ------------------------------------------------------------------ */

/* NeMo AutoModel fused_a2a page: init_hybrid_ep_buffer can use FP8 for the
 * dispatch payload, and HybridEPDispatch.forward returns a scaling factor
 * next to the dispatched hidden states.  Reading (the pages give no
 * format): per token and 128-element block, amax = max|x|,
 *   code  = E4M3(x * (448 / amax))  (RNE, saturating, sign bit of the product kept)
 *   scale = amax / 448               (fp32, the dequantization factor)
 * so that code * scale reproduces x; an all-zero block gives zero codes and
 * scale 0. */
uint8_t orc_e4m3_encode_signed(float v)
{
    uint8_t c = orc_e4m3_encode(fabsf(v));
    return signbit(v) ? (uint8_t)(c | 0x80) : c;
}

void orc_fp8_row(int32_t H, const uint16_t* x, uint8_t* codes, float* scales)
{
    for (int32_t b = 0; b < H / 128; ++b) {
        const uint16_t* xb = x + 128 * b;
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            float a = fabsf(orc_bf16_to_f32(xb[i]));
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            memset(codes + 128 * b, 0, 128);
            scales[b] = 0.0f;
            continue;
        }
        float inv = 448.0f / amax;
        for (int i = 0; i < 128; ++i) {
            float v = orc_bf16_to_f32(xb[i]) * inv;
            codes[128 * b + i] = orc_e4m3_encode_signed(v);
        }
        scales[b] = amax / 448.0f;
    }
}

void orc_dispatch_fp8(const orc_cfg* c, const int32_t* token_row, const uint16_t* x, uint8_t* codes,
                      float* scales)
{
    const int32_t Kp = c->K + c->shared, H = c->H;
    uint8_t* qc = (uint8_t*)malloc((size_t)H);
    float* qs = (float*)malloc(sizeof(float) * (size_t)(H / 128));
    for (int32_t t = 0; t < c->T; ++t) {
        orc_fp8_row(H, x + (int64_t)t * H, qc, qs);
        for (int32_t k = 0; k < Kp; ++k) {
            int32_t row = token_row[(int64_t)t * Kp + k];
            if (row < 0) continue;
            memcpy(codes + (int64_t)row * H, qc, (size_t)H);
            memcpy(scales + (int64_t)row * (H / 128), qs, sizeof(float) * (size_t)(H / 128));
        }
    }
    free(qc);
    free(qs);
}

/* ------------------------------------------------------------------ */
/* NVFP4 quantization with a per-token dynamic global scale             */
/* ------------------------------------------------------------------ */

/* One token: codes [H/2] (two E2M1 per byte, low nibble first), scales
 * [H/16] (E4M3 block scales), rowscale = bf16 inverse global scale. */
void orc_nvfp4_row(int32_t H, const uint16_t* x, uint8_t* codes, uint8_t* scales,
                   uint16_t* rowscale)
{
    /* (i)-(ii) row maximum of |x| */
    float rowmax = 0.0f;
    for (int32_t h = 0; h < H; ++h) {
        float a = fabsf(orc_bf16_to_f32(x[h]));
        if (a > rowmax) rowmax = a;
    }
    if (rowmax == 0.0f) {                      /* (iii) all-zero token */
        memset(codes, 0, (size_t)H / 2);
        memset(scales, 0, (size_t)H / 16);
        *rowscale = orc_bf16_rne(0.0f);
        return;
    }
    float g = 2688.0f / rowmax;                /* global scale 2688 / rowmax */
    uint8_t code[16];
    for (int32_t b = 0; b < H / 16; ++b) {
        const uint16_t* xb = x + 16 * b;
        float bmax = 0.0f;                     /* (iv) block amax */
        for (int i = 0; i < 16; ++i) {
            float a = fabsf(orc_bf16_to_f32(xb[i]));
            if (a > bmax) bmax = a;
        }
        float d = bmax / 6.0f;
        float s = d * g;
        uint8_t sc = orc_e4m3_encode(s);
        float sq = orc_e4m3_decode(sc);
        scales[b] = sc;
        if (sq == 0.0f) {                      /* (v) zero scale: zero codes */
            memset(code, 0, sizeof code);
        } else {
            float inv = g / sq;
            for (int i = 0; i < 16; ++i) {
                float v = orc_bf16_to_f32(xb[i]) * inv;
                code[i] = orc_e2m1_encode(v);  /* (vi) */
            }
        }
        for (int j = 0; j < 8; ++j)            /* (vii) low nibble = even element */
            codes[8 * b + j] = (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
    }
    *rowscale = orc_bf16_rne(1.0f / g);        /* (ix) BF16 inverse of the global scale */
}

/* NVFP4 dispatch: quantize each token, copy its bytes to every row it goes to. */
void orc_dispatch_nvfp4(const orc_cfg* c, const int32_t* token_row, const uint16_t* x,
                        uint8_t* codes, uint8_t* scales, uint16_t* rowscale)
{
    const int32_t Kp = c->K + c->shared, H = c->H;
    uint8_t* qc = (uint8_t*)malloc((size_t)H / 2);
    uint8_t* qs = (uint8_t*)malloc((size_t)H / 16);
    for (int32_t t = 0; t < c->T; ++t) {
        uint16_t rs;
        orc_nvfp4_row(H, x + (int64_t)t * H, qc, qs, &rs);
        for (int32_t k = 0; k < Kp; ++k) {
            int32_t row = token_row[(int64_t)t * Kp + k];
            if (row < 0) continue;
            memcpy(codes + (int64_t)row * (H / 2), qc, (size_t)H / 2);
            memcpy(scales + (int64_t)row * (H / 16), qs, (size_t)H / 16);
            rowscale[row] = rs;
        }
    }
    free(qc);
    free(qs);
}
