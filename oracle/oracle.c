/*
 * oracle.c -- plain CPU reference of the routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no source, table
 * or helper with the GPU library; it is slow on purpose and written so that a
 * reader can check every step against the definitions below by eye.
 *
 * What it computes, for every token t (MiMo-V2.6-Flash-RL routed-expert
 * layer: each token uses 8 of 256 routed experts and the layer has no
 * shared expert -- TrevorJS GGUF card, "Architecture notes"; router kept in
 * F32 -- savrn mixed-quant card, first paragraph and "Quantization
 * targets"):
 *
 *   l[e]   = sum_h x[t,h] * Wr[e,h]                 (fp32, canonical order)
 *   idx    = the k experts with the largest l, ties to the lower index
 *   w[s]   = softmax over the k selected logits      (double), or, with
 *            sigmoid routing, sigma(l_s) / sum_j sigma(l_j) over them
 *   h_s[i] = silu(G_e[i,:] x) * (U_e[i,:] x)         (double)
 *   y_s[j] = D_e[j,:] h_s                            (double)
 *   out[t] = sum_{s<k} w[s] * y_s, in slot order     (double)
 *
 * Expert weights are decoded exactly (E2M1 times E8M0 for MXFP4 -- TrevorJS
 * card, "Architecture notes"; codebook vectors times an F16 row gain for VQ
 * -- Baekpica VQ card, "Recipe").  The expert arithmetic is done in double:
 * the pages require wide accumulation because expert intermediates exceed
 * fp16's 65504 (TrevorJS card, "Recipe", layer-47 note; benthecarman EXL3
 * card, "Bitrate", layer-47 note).
 *
 * Readings taken where the pages are silent (each is pinned by a test):
 *  - routing weights are a softmax over the k selected logits, no extra scale;
 *    the TrevorJS card ("Architecture notes") names sigmoid routing for MiMo,
 *    read as the same selection with weights sigma(l_s) normalised over the
 *    k selected experts, again with no extra scale;
 *  - the fp32 router logit is summed in the canonical order of
 *    oracle_router_logits so that routing can be compared bit for bit;
 *  - ties between equal logits go to the lower expert index;
 *  - gate/up is one matrix of 2I rows, rows [0, I) gate and [I, 2I) up;
 *  - the activation is plain SwiGLU, h = silu(g) * u, with no clamp or bias;
 *  - the byte layouts are this project's own (see the layout comments).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_FMT_MXFP4 1
#define OR_FMT_VQ13R8 2
#define OR_FMT_VQ13 3
#define OR_VQ_ENTRIES 8192
#define OR_VQ_RES_ENTRIES 256

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* element encodings                                                         */
/* ------------------------------------------------------------------------ */

/* E2M1 (the FP4 element of MXFP4): 1 sign bit, 2 exponent bits with bias 1,
 * 1 mantissa bit.  Exponent field 0 is subnormal: m/2.  Otherwise
 * 2^(e-1) * (1 + m/2).  (Two such values per byte -- savrn card, "Why this
 * model needs an asymmetric layout".) */
double oracle_e2m1(int code) {
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E8M0 block scale: 2^(e-127); the all-ones byte encodes NaN.  (One E8M0
 * exponent per 32 values -- TrevorJS card, "Architecture notes".) */
double oracle_e8m0(int e) {
    if (e == 255) return NAN;
    return ldexp(1.0, e - 127);
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits.  Used for the
 * VQ row gains and codebooks (F16 row gain -- Baekpica VQ card, "Recipe"). */
double oracle_fp16(uint16_t b) {
    int s = (b >> 15) & 1;
    int e = (b >> 10) & 31;
    int m = b & 1023;
    double mag;
    if (e == 0) mag = ldexp((double)m, -24);
    else if (e == 31) mag = (m == 0) ? INFINITY : NAN;
    else mag = ldexp(1024.0 + m, e - 25);
    return s ? -mag : mag;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
float oracle_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* packed layouts                                                            */
/* ------------------------------------------------------------------------ */

/* One MXFP4 matrix of N rows by K columns: tiles of 16 rows x 32 columns,
 * tile (n/16, k/32) at index (n/16)*(K/32) + k/32.  A tile has 256 code bytes
 * (tile row r in bytes 16r..16r+15, column c in byte c/2, even c in the low
 * nibble) and 16 scale bytes, one per tile row. */
double oracle_mxfp4_weight(const uint8_t *codes, const uint8_t *scales,
                           int64_t N, int64_t K, int64_t n, int64_t k) {
    (void)N;
    int64_t tile = (n / 16) * (K / 32) + k / 32;
    int64_t r = n % 16, c = k % 32;
    uint8_t byte = codes[tile * 256 + r * 16 + c / 2];
    int code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
    return oracle_e2m1(code) * oracle_e8m0(scales[tile * 16 + r]);
}

/* One VQ matrix of N rows by K columns (Baekpica VQ card, "Recipe": every 8
 * consecutive weights of a row are one 13-bit codebook index -- a 12-bit code
 * stream plus a 1-bit plane -- times an F16 row gain; the R13+8 stage adds an
 * 8-bit index into a 256-entry residual book).  Weight
 *   w[n][k] = gain[n] * (Cb[i13][k%8] + Rb[i8][k%8]).
 * Layout: tiles of 16 rows x 256 columns, tile (n/16, k/256) at index
 * (n/16)*(K/256) + k/256, 512 vectors each.  Vector (tile row r, vector column
 * j = (k%256)/8) sits at stream position ((j/8)*16 + r)*8 + j%8 of its tile.
 * code12 is a little-endian 12-bit stream, plane a little-endian bit stream
 * (the plane bit is bit 12 of the index), res one byte per vector.  A layer
 * of the 13-bit stage alone (res and rb both NULL) has w = gain * Cb[i13]. */
double oracle_vq_weight(const uint8_t *code12, const uint8_t *plane,
                        const uint8_t *res, const uint16_t *gain,
                        const uint16_t *cb, const uint16_t *rb,
                        int64_t N, int64_t K, int64_t n, int64_t k) {
    (void)N;
    int64_t tile = (n / 16) * (K / 256) + k / 256;
    int64_t r = n % 16, j = (k % 256) / 8, d = k % 8;
    int64_t pos = tile * 512 + ((j / 8) * 16 + r) * 8 + (j % 8);
    int64_t bit = pos * 12;
    uint32_t two = (uint32_t)code12[bit / 8] | ((uint32_t)code12[bit / 8 + 1] << 8);
    int i12 = (int)((two >> (bit % 8)) & 0xFFF);
    int p = (plane[pos / 8] >> (pos % 8)) & 1;
    int i13 = i12 | (p << 12);
    double c = oracle_fp16(cb[(int64_t)i13 * 8 + d]);
    if (res == NULL) return oracle_fp16(gain[n]) * c;
    int i8 = res[pos];
    double rr = oracle_fp16(rb[(int64_t)i8 * 8 + d]);
    return oracle_fp16(gain[n]) * (c + rr);
}

/* Byte offsets of the regions of one expert; the same sizes are documented
 * with the header of the packed formats. */
typedef struct {
    int fmt;
    int64_t H, I, E;
    const uint8_t *packed;
} layer_t;

static int64_t mx_expert_bytes(int64_t H, int64_t I) {
    return 2 * I * H / 2 + 2 * I * H / 32 + H * I / 2 + H * I / 32;
}

/* with_res: the matrix has the residual index region (VQ13R8) or not (VQ13) */
static int64_t vq_matrix_bytes(int64_t N, int64_t K, int with_res) {
    int64_t nvec = N * K / 8;
    return nvec * 3 / 2 + nvec / 8 + (with_res ? nvec : 0) + N * 2;
}

static int64_t vq_expert_bytes(int64_t H, int64_t I, int with_res) {
    return vq_matrix_bytes(2 * I, H, with_res) + vq_matrix_bytes(H, I, with_res);
}

/* Weight of expert e, matrix m (0 = gate/up [2I x H], 1 = down [H x I]). */
static double layer_weight(const layer_t *L, int64_t e, int m, int64_t n, int64_t k) {
    int64_t H = L->H, I = L->I;
    int64_t N = m == 0 ? 2 * I : H;
    int64_t K = m == 0 ? H : I;
    if (L->fmt == OR_FMT_MXFP4) {
        const uint8_t *base = L->packed + e * mx_expert_bytes(H, I);
        const uint8_t *gc = base;
        const uint8_t *gs = gc + 2 * I * H / 2;
        const uint8_t *dc = gs + 2 * I * H / 32;
        const uint8_t *ds = dc + H * I / 2;
        return m == 0 ? oracle_mxfp4_weight(gc, gs, N, K, n, k)
                      : oracle_mxfp4_weight(dc, ds, N, K, n, k);
    } else {
        /* VQ13R8: [Cb][Rb] then experts with a res region; VQ13: [Cb] then
         * experts without one */
        const int with_res = L->fmt == OR_FMT_VQ13R8;
        const uint16_t *cb = (const uint16_t *)L->packed;
        const uint16_t *rb = with_res ? cb + OR_VQ_ENTRIES * 8 : NULL;
        const int64_t books = (OR_VQ_ENTRIES + (with_res ? OR_VQ_RES_ENTRIES : 0)) * 8 * 2;
        const uint8_t *base = L->packed + books + e * vq_expert_bytes(H, I, with_res);
        if (m == 1) base += vq_matrix_bytes(2 * I, H, with_res);
        int64_t nvec = N * K / 8;
        const uint8_t *c12 = base;
        const uint8_t *pl = c12 + nvec * 3 / 2;
        const uint8_t *rs = with_res ? pl + nvec / 8 : NULL;
        const uint16_t *gn = (const uint16_t *)(pl + nvec / 8 + (with_res ? nvec : 0));
        return oracle_vq_weight(c12, pl, rs, gn, cb, rb, N, K, n, k);
    }
}

/* Decode one whole matrix into row-major doubles (test helper). */
int oracle_decode_matrix(int fmt, int64_t H, int64_t I, int64_t E, const uint8_t *packed,
                         int64_t expert, int which, double *dst) {
    layer_t L = {fmt, H, I, E, packed};
    if (expert < 0 || expert >= E || (which != 0 && which != 1)) return -1;
    int64_t N = which == 0 ? 2 * I : H;
    int64_t K = which == 0 ? H : I;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            dst[n * K + k] = layer_weight(&L, expert, which, n, k);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* routing                                                                   */
/* ------------------------------------------------------------------------ */

/* Canonical fp32 router logit (the pages only say the router stays F32; the
 * order is this project's reading, fixed so that routing is reproducible bit
 * for bit).  H must be a multiple of 256.  Partial sum c (c = 0..63) takes the
 * columns k with (k/4) mod 64 == c, in ascending k, each step a fused
 * multiply-add p = fmaf(x_k, W_k, p) starting from +0.  The 64 partials are
 * then added as a pairwise tree of adjacent blocks: for s = 1, 2, 4, ..., 32,
 * p[c] = p[c] + p[c+s] for every c that is a multiple of 2s; the logit is
 * p[0]. */
static float router_logit(const uint16_t *x, const float *w, int64_t H) {
    float p[64];
    for (int c = 0; c < 64; c++) p[c] = 0.0f;
    for (int64_t k = 0; k < H; k++) {
        int c = (int)((k / 4) % 64);
        p[c] = fmaf(oracle_bf16(x[k]), w[k], p[c]);
    }
    for (int s = 1; s < 64; s *= 2)
        for (int c = 0; c < 64; c += 2 * s) p[c] = p[c] + p[c + s];
    return p[0];
}

int oracle_router_logits(const uint16_t *x, const float *wr, int64_t T, int64_t H, int64_t E,
                         float *logits) {
    if (H % 256 != 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t te = 0; te < T * E; te++) {
        int64_t t = te / E, e = te % E;
        logits[te] = router_logit(x + t * H, wr + e * H, H);
    }
    return 0;
}

/* The same dot products in double, plain ascending order (diagnostic). */
int oracle_router_logits_f64(const uint16_t *x, const float *wr, int64_t T, int64_t H, int64_t E,
                             double *logits) {
#pragma omp parallel for schedule(static)
    for (int64_t te = 0; te < T * E; te++) {
        int64_t t = te / E, e = te % E;
        double acc = 0.0;
        for (int64_t k = 0; k < H; k++) acc += (double)oracle_bf16(x[t * H + k]) * (double)wr[e * H + k];
        logits[te] = acc;
    }
    return 0;
}

/* The logistic function in double, evaluated on the side where exp() cannot
 * overflow: 1/(1+e^-v) for v >= 0, e^v/(1+e^v) for v < 0. */
static double or_sigmoid(double v) {
    if (v >= 0.0) return 1.0 / (1.0 + exp(-v));
    const double z = exp(v);
    return z / (1.0 + z);
}

/* Top-k selection: repeatedly take the unselected expert with the largest
 * logit; a strict comparison keeps the lower index on equal logits (so -0 and
 * +0 tie).  Slots are ordered by (logit descending, index ascending).  Weights,
 * in double: routing 0, softmax over the k selected logits; routing 1 (sigmoid
 * routing -- TrevorJS card, "Architecture notes"), sigma(l_s) divided by the
 * sum of sigma over the k selected logits.  (The logistic form is used for
 * logits above -700; below that every sigma underflows in double and the
 * ratio is undefined here.)  (k = 8 selected experts per token -- TrevorJS
 * card, "Architecture notes"; the calibration counts of the ProCreations IQ3
 * card, "Calibration", confirm 8 routes for each token.) */
int oracle_topk(const float *logits, int64_t T, int64_t E, int64_t k, int routing, int32_t *idx,
                double *w) {
    if (routing != 0 && routing != 1) return -1;
    if (k < 1 || k > E) return -1;
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        char *taken = calloc((size_t)E, 1);
        if (!taken) return -2;
        for (int64_t s = 0; s < k; s++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            idx[t * k + s] = (int32_t)best;
        }
        free(taken);
        if (routing == 0) {
            double m = (double)l[idx[t * k]];
            double sum = 0.0;
            for (int64_t s = 0; s < k; s++) sum += exp((double)l[idx[t * k + s]] - m);
            for (int64_t s = 0; s < k; s++) w[t * k + s] = exp((double)l[idx[t * k + s]] - m) / sum;
        } else {
            double sum = 0.0;
            for (int64_t s = 0; s < k; s++) sum += or_sigmoid((double)l[idx[t * k + s]]);
            for (int64_t s = 0; s < k; s++)
                w[t * k + s] = or_sigmoid((double)l[idx[t * k + s]]) / sum;
        }
    }
    return 0;
}

/* Grouping of routes by expert: route r = t*k + s.  counts[e] = number of
 * routes to e; offsets = exclusive prefix sum (E+1 entries); perm lists the
 * routes sorted by (expert, token) -- a stable counting sort on the expert id;
 * inv[r] is the position of route r in perm. */
int oracle_permute(const int32_t *idx, int64_t T, int64_t k, int64_t E,
                   int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv) {
    int64_t R = T * k;
    for (int64_t e = 0; e < E; e++) counts[e] = 0;
    for (int64_t r = 0; r < R; r++) {
        if (idx[r] < 0 || idx[r] >= E) return -1;
        counts[idx[r]]++;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = malloc(sizeof(int32_t) * (size_t)E);
    if (!fill) return -2;
    for (int64_t e = 0; e < E; e++) fill[e] = offsets[e];
    for (int64_t r = 0; r < R; r++) {
        int32_t p = fill[idx[r]]++;
        perm[p] = (int32_t)r;
        inv[r] = p;
    }
    free(fill);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* expert feed-forward                                                       */
/* ------------------------------------------------------------------------ */

/* silu(g) = g * sigmoid(g), evaluated without overflow for either sign. */
static double silu(double g) {
    if (g >= 0.0) return g / (1.0 + exp(-g));
    double z = exp(g);
    return g * z / (1.0 + z);
}

/* y = D_e (silu(G_e x) * U_e x), all in double. */
static void expert_ffn(const layer_t *L, int64_t e, const double *x, double *h, double *y) {
    int64_t H = L->H, I = L->I;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; i++) {
        double g = 0.0, u = 0.0;
        for (int64_t k = 0; k < H; k++) {
            g += layer_weight(L, e, 0, i, k) * x[k];
            u += layer_weight(L, e, 0, I + i, k) * x[k];
        }
        h[i] = silu(g) * u;
    }
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < H; j++) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; i++) acc += layer_weight(L, e, 1, j, i) * h[i];
        y[j] = acc;
    }
}

/* Expert FFN of one explicit route (test helper): h [I] and y [H] in double. */
int oracle_expert_ffn(int fmt, int64_t H, int64_t I, int64_t E, const uint8_t *packed,
                      int64_t expert, const uint16_t *x, double *h, double *y) {
    layer_t L = {fmt, H, I, E, packed};
    if (expert < 0 || expert >= E) return -1;
    double *xd = malloc(sizeof(double) * (size_t)H);
    if (!xd) return -2;
    for (int64_t k = 0; k < H; k++) xd[k] = oracle_bf16(x[k]);
    expert_ffn(&L, expert, xd, h, y);
    free(xd);
    return 0;
}

/* The whole layer for the listed tokens (all tokens when tokens == NULL):
 * out [n][H] double, idx [n][k], w [n][k] double, logits [n][E] fp32.
 * routing: 0 softmax, 1 sigmoid (see oracle_topk). */
int oracle_moe_forward(int fmt, int64_t H, int64_t I, int64_t E, int64_t k, int routing,
                       const uint8_t *packed, const uint16_t *x, const float *wr, int64_t T,
                       const int64_t *tokens, int64_t n, double *out, int32_t *idx, double *w,
                       float *logits) {
    if (fmt != OR_FMT_MXFP4 && fmt != OR_FMT_VQ13R8 && fmt != OR_FMT_VQ13) return -1;
    if (H % 256 != 0 || I % 32 != 0 || k < 1 || k > E) return -1;
    if (fmt != OR_FMT_MXFP4 && (I % 256 != 0 || E < 1)) return -1;
    layer_t L = {fmt, H, I, E, packed};
    if (tokens == NULL) n = T;
    double *xd = malloc(sizeof(double) * (size_t)H);
    double *h = malloc(sizeof(double) * (size_t)I);
    double *y = malloc(sizeof(double) * (size_t)H);
    if (!xd || !h || !y) { free(xd); free(h); free(y); return -2; }
    int rc = 0;
    for (int64_t q = 0; q < n && rc == 0; q++) {
        int64_t t = tokens ? tokens[q] : q;
        if (t < 0 || t >= T) { rc = -1; break; }
        const uint16_t *xt = x + t * H;
        rc = oracle_router_logits(xt, wr, 1, H, E, logits + q * E);
        if (rc == 0) rc = oracle_topk(logits + q * E, 1, E, k, routing, idx + q * k, w + q * k);
        if (rc != 0) break;
        for (int64_t kk = 0; kk < H; kk++) xd[kk] = oracle_bf16(xt[kk]);
        double *o = out + q * H;
        for (int64_t j = 0; j < H; j++) o[j] = 0.0;
        for (int64_t s = 0; s < k; s++) {
            expert_ffn(&L, idx[q * k + s], xd, h, y);
            double ws = w[q * k + s];
            for (int64_t j = 0; j < H; j++) o[j] += ws * y[j];
        }
    }
    free(xd); free(h); free(y);
    return rc;
}
