/*
 * Driver for running the CPU oracle (oracle/oracle.c) under AddressSanitizer
 * and UndefinedBehaviorSanitizer: tests/test_oracle_sanitize_cpu.py compiles
 * it together with oracle.c and runs it on the CPU.  Inputs come from a fixed
 * linear congruential generator, shaped like the tiny test layers; the driver
 * checks only that every call succeeds and returns finite values, so a
 * sanitizer report (or a non-zero exit) is the failure being looked for.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_router_logits(const uint16_t *x, const float *wr, int64_t T, int64_t H, int64_t E,
                         float *logits);
int oracle_topk(const float *logits, int64_t T, int64_t E, int64_t k, int routing, int32_t *idx,
                double *w);
int oracle_permute(const int32_t *idx, int64_t T, int64_t k, int64_t E, int32_t *counts,
                   int32_t *offsets, int32_t *perm, int32_t *inv);
int oracle_decode_matrix(int fmt, int64_t H, int64_t I, int64_t E, const uint8_t *packed,
                         int64_t expert, int which, double *dst);
int oracle_expert_ffn(int fmt, int64_t H, int64_t I, int64_t E, const uint8_t *packed,
                      int64_t expert, const uint16_t *x, double *h, double *y);
int oracle_moe_forward(int fmt, int64_t H, int64_t I, int64_t E, int64_t k, int routing,
                       const uint8_t *packed, const uint16_t *x, const float *wr, int64_t T,
                       const int64_t *tokens, int64_t n, double *out, int32_t *idx, double *w,
                       float *logits);

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;

static uint32_t lcg(void) {
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg_state >> 33);
}

/* a float in [-1, 1) */
static float lcg_unit(void) { return (float)(lcg() & 0xFFFFFF) / 8388608.0f - 1.0f; }

/* bf16 bits of a value in [-2, 2) (truncated: any bf16 will do here) */
static uint16_t lcg_bf16(void) {
    float f = 2.0f * lcg_unit();
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* fp16 bits of a value in [-1, 1): sign, exponent 10..14, random mantissa */
static uint16_t lcg_fp16(void) {
    return (uint16_t)(((lcg() & 1u) << 15) | ((10u + lcg() % 5u) << 10) | (lcg() & 0x3FFu));
}

static int failures = 0;

static void check(int ok, const char *what) {
    if (!ok) {
        printf("FAIL %s\n", what);
        ++failures;
    }
}

static int all_finite(const double *v, int64_t n) {
    for (int64_t i = 0; i < n; i++)
        if (!isfinite(v[i])) return 0;
    return 1;
}

/* MXFP4 layer: random code bytes, E8M0 bytes in [120, 126] in the scale regions */
static uint8_t *make_mxfp4(int64_t H, int64_t I, int64_t E, size_t *bytes) {
    const int64_t gc = 2 * I * H / 2, gs = 2 * I * H / 32, dc = H * I / 2, ds = H * I / 32;
    const int64_t per = gc + gs + dc + ds;
    uint8_t *p = malloc((size_t)(per * E));
    for (int64_t e = 0; e < E; e++) {
        uint8_t *q = p + e * per;
        for (int64_t i = 0; i < per; i++) q[i] = (uint8_t)lcg();
        for (int64_t i = 0; i < gs; i++) q[gc + i] = (uint8_t)(120 + lcg() % 7);
        for (int64_t i = 0; i < ds; i++) q[gc + gs + dc + i] = (uint8_t)(120 + lcg() % 7);
    }
    *bytes = (size_t)(per * E);
    return p;
}

/* VQ layer (with or without the residual stage): fp16 books in [-1, 1),
 * random index bytes, fp16 gains in [-1, 1) */
static uint8_t *make_vq(int64_t H, int64_t I, int64_t E, int res, size_t *bytes) {
    const int64_t books = (8192 + (res ? 256 : 0)) * 8;
    int64_t per = 0;
    const int64_t mats[2][2] = {{2 * I, H}, {H, I}};
    for (int m = 0; m < 2; m++) {
        const int64_t nvec = mats[m][0] * mats[m][1] / 8;
        per += nvec * 3 / 2 + nvec / 8 + (res ? nvec : 0) + mats[m][0] * 2;
    }
    const size_t total = (size_t)(books * 2 + per * E);
    uint8_t *p = malloc(total);
    uint16_t *bk = (uint16_t *)p;
    for (int64_t i = 0; i < books; i++) bk[i] = lcg_fp16();
    uint8_t *ex = p + books * 2;
    for (int64_t e = 0; e < E; e++) {
        uint8_t *q = ex + e * per;
        for (int m = 0; m < 2; m++) {
            const int64_t nvec = mats[m][0] * mats[m][1] / 8;
            const int64_t idx_bytes = nvec * 3 / 2 + nvec / 8 + (res ? nvec : 0);
            for (int64_t i = 0; i < idx_bytes; i++) q[i] = (uint8_t)lcg();
            uint16_t *gain = (uint16_t *)(q + idx_bytes);
            for (int64_t i = 0; i < mats[m][0]; i++) gain[i] = lcg_fp16();
            q += idx_bytes + mats[m][0] * 2;
        }
    }
    *bytes = total;
    return p;
}

static void run_layer(const char *name, int fmt, int64_t H, int64_t I, int64_t E, int64_t k,
                      int64_t T, const uint8_t *packed) {
    uint16_t *x = malloc(sizeof(uint16_t) * (size_t)(T * H));
    float *wr = malloc(sizeof(float) * (size_t)(E * H));
    for (int64_t i = 0; i < T * H; i++) x[i] = lcg_bf16();
    for (int64_t i = 0; i < E * H; i++) wr[i] = 0.02f * lcg_unit();

    /* routing: logits, top-k (both weightings), grouping */
    float *logits = malloc(sizeof(float) * (size_t)(T * E));
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)(T * k));
    double *w = malloc(sizeof(double) * (size_t)(T * k));
    int32_t *counts = malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *perm = malloc(sizeof(int32_t) * (size_t)(T * k));
    int32_t *inv = malloc(sizeof(int32_t) * (size_t)(T * k));
    check(oracle_router_logits(x, wr, T, H, E, logits) == 0, name);
    for (int routing = 0; routing < 2; routing++) {
        check(oracle_topk(logits, T, E, k, routing, idx, w) == 0, name);
        check(all_finite(w, T * k), "finite routing weights");
    }
    check(oracle_permute(idx, T, k, E, counts, offsets, perm, inv) == 0, name);
    check(offsets[E] == T * k, "every route placed");

    /* one expert decoded whole, one route through its FFN */
    double *dense = malloc(sizeof(double) * (size_t)(2 * I * H));
    check(oracle_decode_matrix(fmt, H, I, E, packed, E - 1, 0, dense) == 0, name);
    check(oracle_decode_matrix(fmt, H, I, E, packed, E - 1, 1, dense) == 0, name);
    check(all_finite(dense, H * I), "finite decoded weights");
    double *h = malloc(sizeof(double) * (size_t)I);
    double *y = malloc(sizeof(double) * (size_t)H);
    check(oracle_expert_ffn(fmt, H, I, E, packed, E - 1, x, h, y) == 0, name);
    check(all_finite(y, H), "finite expert output");

    /* the whole layer, all tokens and a listed subset (last token first) */
    double *out = malloc(sizeof(double) * (size_t)(T * H));
    float *lg = malloc(sizeof(float) * (size_t)(T * E));
    check(oracle_moe_forward(fmt, H, I, E, k, 0, packed, x, wr, T, NULL, 0, out, idx, w, lg) == 0,
          name);
    check(all_finite(out, T * H), "finite layer output");
    const int64_t sub[2] = {T - 1, 0};
    check(oracle_moe_forward(fmt, H, I, E, k, 1, packed, x, wr, T, sub, 2, out, idx, w, lg) == 0,
          name);
    check(all_finite(out, 2 * H), "finite sampled output");
    printf("%s ok\n", name);
    free(x); free(wr); free(logits); free(idx); free(w); free(counts); free(offsets);
    free(perm); free(inv); free(dense); free(h); free(y); free(out); free(lg);
}

int main(void) {
    size_t bytes;
    uint8_t *mx = make_mxfp4(256, 128, 8, &bytes);
    run_layer("mxfp4", 1, 256, 128, 8, 2, 16, mx);
    free(mx);
    uint8_t *vq = make_vq(256, 256, 8, 1, &bytes);
    run_layer("vq13r8", 2, 256, 256, 8, 2, 16, vq);
    free(vq);
    uint8_t *vq13 = make_vq(256, 256, 8, 0, &bytes);
    run_layer("vq13", 3, 256, 256, 8, 2, 16, vq13);
    free(vq13);
    printf("%d failures\n", failures);
    return failures;
}
