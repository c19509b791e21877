/* Drives every oracle function over small seeded cases, edge cases
 * included, for a build under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitizers.py).  Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t T, H, E, S, K, A, C, shared, src_seg;
    int64_t recv_rows;
} orc_cfg;

int orc_layout(const orc_cfg*, const int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*,
               int32_t*, int32_t*);
void orc_dispatch(const orc_cfg*, const int32_t*, const uint16_t*, uint16_t*);
void orc_dispatch_nvfp4(const orc_cfg*, const int32_t*, const uint16_t*, uint8_t*, uint8_t*, uint16_t*);
void orc_dispatch_fp8(const orc_cfg*, const int32_t*, const uint16_t*, uint8_t*, float*);
void orc_combine(const orc_cfg*, const int32_t*, const uint16_t*, const float*, uint16_t*);
void orc_dispatch_bwd(const orc_cfg*, const int32_t*, const uint16_t*, uint16_t*);
void orc_combine_bwd(const orc_cfg*, const int32_t*, const uint16_t*, const float*, uint16_t*);
void orc_combine_bwd_probs(const orc_cfg*, const int32_t*, const uint16_t*, const uint16_t*, double*);
void orc_combine_nvfp4(const orc_cfg*, const int32_t*, const uint8_t*, const uint8_t*, const uint16_t*,
                       const float*, uint16_t*);
void orc_indices_to_multihot(const orc_cfg*, const int32_t*, const float*, uint8_t*, float*);
int32_t orc_multihot_to_indices(const orc_cfg*, const uint8_t*, const float*, int32_t*, float*);

static uint64_t rng_state = 88172645463325252ull;
static uint32_t rnd(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 11);
}

static int64_t min_rows(const orc_cfg* c)
{
    if (c->C > 0) return (int64_t)c->S * c->C;
    int64_t routed = (int64_t)c->T * (c->K + c->shared), groups = c->E + c->shared;
    return routed + (routed < groups ? routed : groups) * (c->A - 1);
}

static void run(orc_cfg c)
{
    c.recv_rows = min_rows(&c);
    const int32_t G = c.E / c.S + c.shared, Kp = c.K + c.shared;
    const int64_t R = c.recv_rows;
    int32_t* ids = malloc(sizeof(int32_t) * (size_t)(c.T * c.K + 1));
    for (int64_t i = 0; i < (int64_t)c.T * c.K; ++i) {
        uint32_t r = rnd() % 100;
        ids[i] = r < 8 ? -1 : (r < 10 ? (int32_t)(c.E + r) : (int32_t)(rnd() % (uint32_t)c.E));
    }
    uint16_t* x = malloc(sizeof(uint16_t) * (size_t)(c.T * c.H + 1));
    for (int64_t i = 0; i < (int64_t)c.T * c.H; ++i) x[i] = (uint16_t)(0x3C00 + (rnd() % 0x800)) ^ (uint16_t)((rnd() & 1) << 15);
    float* probs = malloc(sizeof(float) * (size_t)(c.T * c.K + 1));
    for (int64_t i = 0; i < (int64_t)c.T * c.K; ++i) probs[i] = (float)(rnd() % 1000) / 1000.0f;
    int32_t *counts = malloc(4 * (size_t)(c.S * G)), *ro = malloc(4 * (size_t)(c.S * (G + 1))),
            *so = malloc(4 * (size_t)(c.S * (G + 1))), *sb = malloc(4 * (size_t)(c.S + 1)),
            *tr = malloc(4 * (size_t)(c.T * Kp + 1)), *eid = malloc(4 * (size_t)(R + 1)),
            *src = malloc(8 * (size_t)(R + 1)), flags;
    if (orc_layout(&c, ids, counts, ro, so, sb, tr, eid, src, &flags) != 0) {
        printf("layout out of rows\n");
        exit(1);
    }
    uint16_t* recv = calloc((size_t)(R * c.H + 1), 2);
    orc_dispatch(&c, tr, x, recv);
    if (c.H % 16 == 0) {
        uint8_t *codes = calloc((size_t)(R * c.H / 2 + 1), 1), *sc = calloc((size_t)(R * c.H / 16 + 1), 1);
        uint16_t* rs = calloc((size_t)(R + 1), 2);
        orc_dispatch_nvfp4(&c, tr, x, codes, sc, rs);
        uint16_t* yq = malloc(sizeof(uint16_t) * (size_t)(c.T * c.H + 1));
        orc_combine_nvfp4(&c, tr, codes, sc, rs, probs, yq);
        orc_combine_nvfp4(&c, tr, codes, sc, rs, NULL, yq);
        free(yq);
        free(codes);
        free(sc);
        free(rs);
    }
    if (c.H % 128 == 0) {
        uint8_t* codes = calloc((size_t)(R * c.H + 1), 1);
        float* sc = calloc((size_t)(R * c.H / 128 + 1), 4);
        orc_dispatch_fp8(&c, tr, x, codes, sc);
        free(codes);
        free(sc);
    }
    uint16_t* y = calloc((size_t)(c.T * c.H + 1), 2);
    orc_combine(&c, tr, recv, probs, y);
    orc_combine(&c, tr, recv, NULL, y);
    orc_dispatch_bwd(&c, tr, recv, y);
    orc_combine_bwd(&c, tr, x, probs, recv);
    double* gp = calloc((size_t)(c.T * c.K + 1), 8);
    orc_combine_bwd_probs(&c, tr, x, recv, gp);
    uint8_t* map = calloc((size_t)(c.T * c.E + 1), 1);
    float* dense = calloc((size_t)(c.T * c.E + 1), 4);
    orc_indices_to_multihot(&c, ids, probs, map, dense);
    orc_multihot_to_indices(&c, map, dense, ids, probs);
    free(map);
    free(dense);
    free(gp);
    free(y);
    free(recv);
    free(counts);
    free(ro);
    free(so);
    free(sb);
    free(tr);
    free(eid);
    free(src);
    free(ids);
    free(x);
    free(probs);
}

int main(void)
{
    /* T, H, E, S, K, A, C, shared, src_seg */
    orc_cfg cases[] = {
        {0, 16, 4, 2, 2, 4, 0, 0, 0, 0},      {1, 16, 4, 2, 2, 4, 0, 1, 1, 0},
        {37, 128, 12, 3, 4, 4, 0, 1, 2, 0},   {64, 256, 8, 2, 2, 16, 0, 0, 0, 0},
        {50, 32, 16, 4, 3, 1, 20, 1, 0, 0},   {80, 48, 6, 6, 6, 3, 0, 0, 0, 0},
        {200, 256, 64, 4, 8, 128, 0, 1, 3, 0}, {100, 16, 8, 1, 8, 2, 7, 0, 0, 0},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) run(cases[i]);
    printf("oracle sanitizer run ok\n");
    return 0;
}
