// route.hip -- router logits, top-k selection with softmax, and grouping of
// routes by expert (counting sort), for gfx950.
//
// The router is the F32 router the MiMo-V2.6-Flash-RL cards keep at full
// precision (savrn mixed-quant card, "Quantization targets"); each token is
// sent to its 8 highest-scoring experts out of 256 (TrevorJS GGUF card,
// "Architecture notes").  The logit sum order is fixed (see bqmoe.h) so that
// routing is reproducible bit for bit: lane c of a wave owns partial sum c,
// i.e. columns 4c..4c+3 of every 256-column group, accumulated with fused
// multiply-adds in ascending column order; the wave then adds partials with an
// xor butterfly, which forms exactly the pairwise tree of adjacent blocks.
#include "moe_internal.h"
#include "vq_common.h"

namespace bqmoe {

// ---------------------------------------------------------------------------
// router logits for large batches.  A block (4 waves) computes a TOK-token x
// 4*EXP-expert tile (32 x 16); wave w owns experts EXP*w..+EXP-1 of the tile
// for all TOK tokens (128 accumulators per lane).  Per 256-column group the
// block stages the token rows in LDS already widened to fp32 (32 KiB), so the
// FMA loop reads one 16-byte float4 per token and lane, four tokens ahead, and
// converts nothing, and each wave keeps its weight rows' float4s in registers;
// the next group's x and W loads are issued before the current group's FMAs.
// (2048 tokens x 256 experts x 4096: 89 -> 77 us against 16 x 16 tiles that
// widened bf16 inside the FMA loop; a 16 x 32 tile measured the same.)  Lane c holds columns
// 4c..4c+3 of every group, so each logit keeps the summation order described
// above.  Rows past T or E are clamped duplicates that are never stored.
//
// The 64 lane partials of the 128 logits are then added by a transposing
// butterfly: at stride m (1, 2, 4, ..., 32) lanes c and c^m exchange half of
// their remaining list and each adds the half it keeps, so after six strides
// every lane holds two finished logits.  Each addition joins the sums of two
// adjacent blocks of 2m lanes' partials -- the same pairwise tree as adding
// every logit's partials with an xor butterfly (IEEE addition commutes, so
// which of the two lanes adds is immaterial) -- with 126 exchanges per lane
// instead of 6 per logit.
// ---------------------------------------------------------------------------
constexpr int kRtTok = 32;  // tokens per block
constexpr int kRtExp = 4;   // experts per wave

template <int TOK, int EXP>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t *__restrict__ x,
                                                     const float *__restrict__ wr, int T, int H,
                                                     int E, float *__restrict__ logits) {
    constexpr int NACC = TOK * EXP;  // accumulators per lane (a power of two)
    static_assert(NACC == 128, "the butterfly below leaves two logits per lane");
    __shared__ __align__(16) float4 xs[2][TOK][64];  // [buffer][token][lane]: 2 x 32 KiB
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * TOK;
    const int e0 = (blockIdx.y * 4 + wave) * EXP;
    float acc[NACC];  // [token t][expert e] at t * EXP + e
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = 0.0f;
    // element offsets (32-bit: H * max(T, E) stays far below 2^32 here)
    const float *wbase = wr + (lane << 2);
    uint32_t woff[EXP];
#pragma unroll
    for (int e = 0; e < EXP; ++e) woff[e] = (uint32_t)min(e0 + e, E - 1) * (uint32_t)H;
    // x staging: piece i of thread tid is 8 columns (16 bytes) of one token:
    // p = tid + 256 i, token p / 32, columns 8 (p % 32) .. +7 of the group
    constexpr int XP = TOK * 32 / 256;  // pieces per thread
    uint32_t xoff[XP];
#pragma unroll
    for (int i = 0; i < XP; ++i) {
        const int pc = tid + 256 * i;
        xoff[i] = (uint32_t)min(t0 + (pc >> 5), T - 1) * (uint32_t)H + 8 * (pc & 31);
    }
    float4 wv[2][EXP];
    uint4 xn[XP];
    auto load_x = [&](int j) {
#pragma unroll
        for (int i = 0; i < XP; ++i) xn[i] = *reinterpret_cast<const uint4 *>(x + xoff[i] + (j << 8));
    };
    auto load_w = [&](int buf, int j) {
#pragma unroll
        for (int e = 0; e < EXP; ++e) wv[buf][e] = *reinterpret_cast<const float4 *>(wbase + woff[e] + (j << 8));
    };
    auto store_x = [&](int buf) {  // widened to fp32: 32 bytes per piece
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int pc = tid + 256 * i;
            float4 *d = &xs[buf][pc >> 5][2 * (pc & 31)];
            d[0] = make_float4(bf16_to_f32(xn[i].x & 0xFFFFu), bf16_to_f32(xn[i].x >> 16),
                               bf16_to_f32(xn[i].y & 0xFFFFu), bf16_to_f32(xn[i].y >> 16));
            d[1] = make_float4(bf16_to_f32(xn[i].z & 0xFFFFu), bf16_to_f32(xn[i].z >> 16),
                               bf16_to_f32(xn[i].w & 0xFFFFu), bf16_to_f32(xn[i].w >> 16));
        }
    };
    // the token rows' float4s are read from LDS kRtBatch tokens ahead of
    // their FMAs, so the LDS latency is covered by a batch of FMAs
    constexpr int kRtBatch = 4;
    auto fma_group = [&](int buf) {
        float4 v[2][kRtBatch];
#pragma unroll
        for (int u = 0; u < kRtBatch; ++u) v[0][u] = xs[buf][u][lane];
#pragma unroll
        for (int tb = 0; tb < TOK / kRtBatch; ++tb) {
            const int cur = tb & 1;
            if (tb + 1 < TOK / kRtBatch) {
#pragma unroll
                for (int u = 0; u < kRtBatch; ++u)
                    v[cur ^ 1][u] = xs[buf][(tb + 1) * kRtBatch + u][lane];
            }
#pragma unroll
            for (int u = 0; u < kRtBatch; ++u) {
                const int t = tb * kRtBatch + u;
#pragma unroll
                for (int e = 0; e < EXP; ++e) {
                    float a = acc[t * EXP + e];
                    a = __builtin_fmaf(v[cur][u].x, wv[buf][e].x, a);
                    a = __builtin_fmaf(v[cur][u].y, wv[buf][e].y, a);
                    a = __builtin_fmaf(v[cur][u].z, wv[buf][e].z, a);
                    a = __builtin_fmaf(v[cur][u].w, wv[buf][e].w, a);
                    acc[t * EXP + e] = a;
                }
            }
        }
    };
    const int groups = H >> 8;
    load_x(0);
    load_w(0, 0);
    store_x(0);  // waits for the x loads only
    lds_barrier();
    for (int j = 0; j < groups; j += 2) {
        // group j (buffer 0) while group j+1 loads; then group j+1 (buffer 1)
        load_x(min(j + 1, groups - 1));
        load_w(1, min(j + 1, groups - 1));
        fma_group(0);
        store_x(1);
        lds_barrier();
        load_x(min(j + 2, groups - 1));
        load_w(0, min(j + 2, groups - 1));
        if (j + 1 < groups) fma_group(1);
        store_x(0);
        lds_barrier();
    }
    // transposing butterfly: after stride m = 2^k the lane keeps list entries
    // [0, n/2) of the previous list (n = 128 >> k), namely the upper half if
    // its lane bit k is set; entry i ends as logit index i + 2 * rev6(lane)
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        const int m = 1 << k, half = (NACC / 2) >> k;
        const bool up = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = up ? acc[i] : acc[i + half];
            const float keep = up ? acc[i + half] : acc[i];
            acc[i] = keep + __shfl_xor(send, m, 64);
        }
    }
    const int rv = (int)(__builtin_bitreverse32((uint32_t)lane) >> 26);  // rev6(lane)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = i + 2 * rv, t = idx / EXP, e = idx % EXP;
        if (t0 + t < T && e0 + e < E) logits[(size_t)(t0 + t) * E + e0 + e] = acc[i];
    }
}

// ---------------------------------------------------------------------------
// block-wide exclusive scan of one int per thread (blockDim = 256 or 1024)
// ---------------------------------------------------------------------------
__device__ int block_exclusive_scan(int v, int *total, int *lds /* >= 16 ints */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int incl = v;
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    if (lane == 63) lds[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int q = 0; q < nw; ++q) {
        const int c = lds[q];
        if (q < wave) base += c;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// ---------------------------------------------------------------------------
// Small batches (T <= 16): router logits, then the whole routing in one block.
//
// router_small_kernel: each wave computes one expert's logits for up to TT
// tokens, with every load (MAXG 256-column groups of W and x) issued before the
// first FMA, in the same summation order as router_kernel.  With xexp (VQ
// layers) the wave of expert 0 also writes each token's fp16 row exponent
// (its largest |x| scaled into [2^14, 2^15)), which the batch-1 VQ gate/up
// kernel needs before its first barrier.
//
// route_small_kernel (one block of 16 waves): top-k and weights, one wave per
// token; a 16-bit mask per expert of the tokens routed to it (LDS atomic or);
// counts as mask popcounts, offsets and the active list as block scans; and
// the stable grouping, in which route r of token t takes position
// offsets[e] + popcount(mask[e] below bit t).  A separate launch costs less than
// publishing the logits across the XCDs from inside the router kernel (a
// device-scope release per block plus an arrival counter).
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 1024;

__global__ __launch_bounds__(kRouteThreads) void route_small_kernel(
    const float *__restrict__ logits, int T, int E, int K, int32_t *__restrict__ idx_out,
    float *__restrict__ w_out, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ active, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    bool sigmoid) {
    __shared__ int s_idx[kDecodeMaxTokens * kMaxTopK];
    __shared__ uint32_t s_mask[kMaxExperts];  // bit t: token t routes to the expert
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_scan[kRouteThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int R = T * K;
    if (tid < kMaxExperts) s_mask[tid] = 0;
    for (int t = wave; t < T; t += nw) {
        int idx[kMaxTopK];
        float w[kMaxTopK];
        wave_topk(logits + (size_t)t * E, E, K, sigmoid, idx, w);
        if (lane < K) {
            int iv = idx[0];
            float wv = w[0];
#pragma unroll
            for (int s = 1; s < kMaxTopK; ++s)
                if (s < K && lane == s) { iv = idx[s]; wv = w[s]; }
            idx_out[t * K + lane] = iv;
            w_out[t * K + lane] = wv;
            s_idx[t * K + lane] = iv;
        }
    }
    __syncthreads();
    // which tokens route to each expert (a token's k experts are distinct)
    if (tid < R) atomicOr(&s_mask[s_idx[tid]], 1u << (tid / K));
    __syncthreads();
    // counts, and offsets as their exclusive scan; the active list in
    // ascending expert order (threads of the first four waves hold experts)
    const int e = tid;
    const int cnt = e < E ? __popc(s_mask[e]) : 0;
    int total;
    const int off = block_exclusive_scan(cnt, &total, s_scan);
    int n_act;
    const int apos = block_exclusive_scan(cnt > 0 ? 1 : 0, &n_act, s_scan);
    if (e < E) {
        s_off[e] = off;
        counts[e] = cnt;
        offsets[e] = off;
        if (cnt > 0) active[1 + apos] = e;
    }
    if (tid == 0) {
        offsets[E] = total;
        active[0] = n_act;
    }
    __syncthreads();
    // route r = t*K + s goes to position offsets[e] + (number of earlier tokens
    // routed to e): the stable grouping by (expert, token)
    if (tid < R) {
        const int er = s_idx[tid], t = tid / K;
        const int pos = s_off[er] + __popc(s_mask[er] & ((1u << t) - 1u));
        perm[pos] = tid;
        inv[tid] = pos;
    }
}

constexpr int kRsWaves = 2;  // waves (experts) per block of the small-batch router

template <int TT, int MAXG>
__global__ __launch_bounds__(64 * kRsWaves) void router_small_kernel(const uint16_t *__restrict__ x,
                                                           const float *__restrict__ wr, int T,
                                                           int H, int E,
                                                           float *__restrict__ logits,
                                                           int32_t *__restrict__ xexp) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.y * kRsWaves + (threadIdx.x >> 6);
    const int t0 = blockIdx.x * TT;
    if (e >= E) return;
    const int groups = H >> 8;
    float4 wv[MAXG];
    uint2 xb[TT][MAXG];
#pragma unroll
    for (int j = 0; j < MAXG; ++j)
        if (j < groups)
            wv[j] = *reinterpret_cast<const float4 *>(wr + (size_t)e * H + (j << 8) + (lane << 2));
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int j = 0; j < MAXG; ++j)
            if (j < groups && t0 + t < T)
                xb[t][j] = *reinterpret_cast<const uint2 *>(x + (size_t)(t0 + t) * H + (j << 8) + (lane << 2));
    if (xexp != nullptr && e == 0) {  // wave-uniform; x arrives before the W row
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t0 + t >= T) break;
            uint32_t mb = 0;  // largest |x| as fp32 bits (bf16 bits shifted up)
#pragma unroll
            for (int j = 0; j < MAXG; ++j) {
                if (j < groups) {
                    mb = max(mb, (xb[t][j].x & 0x7FFFu) << 16);
                    mb = max(mb, xb[t][j].x & 0x7FFF0000u);
                    mb = max(mb, (xb[t][j].y & 0x7FFFu) << 16);
                    mb = max(mb, xb[t][j].y & 0x7FFF0000u);
                }
            }
            const float xm = wave_max_f32(__uint_as_float(mb));
            if (lane == 0) xexp[t0 + t] = fp16_row_exponent(__float_as_uint(xm));
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        if (t0 + t >= T) break;
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < MAXG; ++j) {
            if (j < groups) {
                a = __builtin_fmaf(bf16_to_f32(xb[t][j].x & 0xFFFFu), wv[j].x, a);
                a = __builtin_fmaf(bf16_to_f32(xb[t][j].x >> 16), wv[j].y, a);
                a = __builtin_fmaf(bf16_to_f32(xb[t][j].y & 0xFFFFu), wv[j].z, a);
                a = __builtin_fmaf(bf16_to_f32(xb[t][j].y >> 16), wv[j].w, a);
            }
        }
        a = wave_sum_xor(a, 1);
        if (lane == 0) logits[(size_t)(t0 + t) * E + e] = a;
    }
}

template <int TT>
static void router_small_launch(const Shape &s, dim3 grid, hipStream_t st, const uint16_t *x,
                                const float *wr, int T, float *logits, int32_t *xexp) {
    const int g = s.H / 256;
    constexpr int nt = 64 * kRsWaves;
    if (g <= 1) router_small_kernel<TT, 1><<<grid, nt, 0, st>>>(x, wr, T, s.H, s.E, logits, xexp);
    else if (g <= 4) router_small_kernel<TT, 4><<<grid, nt, 0, st>>>(x, wr, T, s.H, s.E, logits, xexp);
    else if (g <= 16) router_small_kernel<TT, 16><<<grid, nt, 0, st>>>(x, wr, T, s.H, s.E, logits, xexp);
    else router_small_kernel<TT, 32><<<grid, nt, 0, st>>>(x, wr, T, s.H, s.E, logits, xexp);
}

hipError_t launch_router_route_small(const Shape &s, const uint16_t *x, const float *wr, int T,
                                     const Workspace &ws, hipStream_t st, bool route_single) {
    if (T < 1 || T > kDecodeMaxTokens || s.H / 256 > 32) return hipErrorInvalidValue;
    const int ey = (s.E + kRsWaves - 1) / kRsWaves;
    // the fp16 row exponents of x feed the batch-1 VQ kernels (a VQ workspace
    // has xexp; for larger VQ batches the x packing kernel rewrites them)
    int32_t *xexp = is_vq_format(s.fmt) ? ws.xexp : nullptr;
    if (T == 1)
        router_small_launch<1>(s, dim3(1, ey), st, x, wr, T, ws.logits, xexp);
    else
        router_small_launch<4>(s, dim3((T + 3) / 4, ey), st, x, wr, T, ws.logits, xexp);
    hipError_t e = hipGetLastError();
    // a single token is routed by the batch-1 gate/up kernel unless route_single
    if (e != hipSuccess || (T == 1 && !route_single)) return e;
    route_small_kernel<<<1, kRouteThreads, 0, st>>>(ws.logits, T, s.E, s.K, ws.idx, ws.w,
                                                    ws.counts, ws.offsets, ws.active, ws.perm,
                                                    ws.inv, s.routing == MOE_ROUTE_SIGMOID);
    return hipGetLastError();
}

hipError_t launch_router(const Shape &s, const uint16_t *x, const float *wr, int T, float *logits,
                         hipStream_t st) {
    dim3 grid((T + kRtTok - 1) / kRtTok, (s.E + 4 * kRtExp - 1) / (4 * kRtExp));
    router_kernel<kRtTok, kRtExp><<<grid, 256, 0, st>>>(x, wr, T, s.H, s.E, logits);
    return hipGetLastError();
}

// one wave per token (prefill)
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int K, int32_t *__restrict__ idx_out,
                                                   float *__restrict__ w_out, bool sigmoid) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int idx[kMaxTopK];
    float w[kMaxTopK];
    wave_topk(logits + (size_t)t * E, E, K, sigmoid, idx, w);
    const int lane = threadIdx.x & 63;
    if (lane < K) {
        int iv = idx[0];
        float wv = w[0];
#pragma unroll
        for (int s = 1; s < kMaxTopK; ++s)
            if (s < K && lane == s) { iv = idx[s]; wv = w[s]; }
        idx_out[(size_t)t * K + lane] = iv;
        w_out[(size_t)t * K + lane] = wv;
    }
}

hipError_t launch_topk(const Shape &s, int T, const Workspace &ws, hipStream_t st) {
    topk_kernel<<<(T + 3) / 4, 256, 0, st>>>(ws.logits, T, s.E, s.K, ws.idx, ws.w,
                                             s.routing == MOE_ROUTE_SIGMOID);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// large batches: one block per expert.  Thread t owns a contiguous run of
// kPermPer routes (per pass of 256 * kPermPer), so a block-wide exclusive scan
// of the per-thread match counts gives every route of expert e its place in
// route order (a stable counting sort split by expert).  The expert's offset
// is the number of routes with a smaller expert index, counted the same way;
// block 0 also builds the histogram (counts, offsets, the active list).  With
// R <= 256 * kPermPer (2048 tokens at k = 8) the routes are read once, into
// registers, with all loads in flight together.
// ---------------------------------------------------------------------------
constexpr int kPermPer = 64;
constexpr int kPermPass = 256 * kPermPer;

// the pass's expert indices of thread tid: routes [r0, r0 + kPermPer), padded with E
__device__ __forceinline__ void perm_load(const int32_t *__restrict__ idx, int R, int E, int r0,
                                          int (&v)[kPermPer]) {
#pragma unroll
    for (int i = 0; i < kPermPer; i += 4) {
        const int r = r0 + i;
        if (r + 3 < R) {
            const int4 q = *reinterpret_cast<const int4 *>(idx + r);
            v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) v[i + k] = r + k < R ? idx[r + k] : E;
        }
    }
}

__global__ __launch_bounds__(256) void permute_kernel(const int32_t *__restrict__ idx, int R, int E,
                                                      int32_t *__restrict__ counts,
                                                      int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ active,
                                                      int32_t *__restrict__ perm,
                                                      int32_t *__restrict__ inv) {
    __shared__ int hist[kMaxExperts];
    __shared__ int s_scan[16];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    if (e == 0) {
        for (int i = tid; i < kMaxExperts; i += blockDim.x) hist[i] = 0;
        __syncthreads();
    }
    int v[kPermPer];
    const bool one = R <= kPermPass;
    // offset of expert e: routes with a smaller expert index (block 0 also
    // counts every expert)
    int below = 0;
    for (int b = 0; b < R; b += kPermPass) {
        perm_load(idx, R, E, b + tid * kPermPer, v);
#pragma unroll
        for (int i = 0; i < kPermPer; ++i) {
            below += v[i] < e;
            if (e == 0 && v[i] < E) atomicAdd(&hist[v[i]], 1);
        }
    }
    int base;
    {
        int tot;
        block_exclusive_scan(below, &tot, s_scan);
        base = tot;
    }
    if (e == 0) {
        __syncthreads();
        int total;
        const int my = (tid < E) ? hist[tid] : 0;
        const int excl = block_exclusive_scan(my, &total, s_scan);
        if (tid < E) { counts[tid] = my; offsets[tid] = excl; }
        if (tid == 0) offsets[E] = total;
        int n_active;
        const int flag = (tid < E && my > 0) ? 1 : 0;
        const int apos = block_exclusive_scan(flag, &n_active, s_scan);
        if (flag) active[1 + apos] = tid;
        if (tid == 0) active[0] = n_active;
    }
    // compaction: this thread's matches, in route order
    int running = base;
    for (int b = 0; b < R; b += kPermPass) {
        const int r0 = b + tid * kPermPer;
        if (!one) perm_load(idx, R, E, r0, v);
        uint64_t m = 0;
#pragma unroll
        for (int i = 0; i < kPermPer; ++i) m |= (uint64_t)(v[i] == e) << i;
        int tot;
        int pos = block_exclusive_scan(__popcll(m), &tot, s_scan) + running;
        while (m) {
            const int i = __builtin_ctzll(m);
            m &= m - 1;
            perm[pos] = r0 + i;
            inv[r0 + i] = pos;
            ++pos;
        }
        running += tot;
    }
}

hipError_t launch_permute(const Shape &s, int T, const Workspace &ws, hipStream_t st) {
    permute_kernel<<<s.E, 256, 0, st>>>(ws.idx, T * s.K, s.E, ws.counts, ws.offsets, ws.active,
                                        ws.perm, ws.inv);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// combine: out[t] = sum_s w[t,s] * y[inv[t*K+s]], slots in order.  The
// per-route outputs are fp16 with an exponent per GW columns (16 for MXFP4,
// 4 for the VQ formats): y[p][j] = y16[p][j] * 2^yexp[p][j/GW], exact in fp32,
// then one fused multiply-add per slot.  A thread takes 8 columns.
// ---------------------------------------------------------------------------
template <int GW>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ y16,
                                                      const int8_t *__restrict__ yexp,
                                                      const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv, int H, int K,
                                                      float *__restrict__ out) {
    static_assert(GW == 4 || GW == 16, "exponent group width");
    const int t = blockIdx.x;
    float wk[kMaxTopK];
    int pk[kMaxTopK];
    for (int s = 0; s < K; ++s) {
        wk[s] = w[(size_t)t * K + s];
        pk[s] = inv[(size_t)t * K + s];
    }
    for (int j = threadIdx.x * 8; j < H; j += blockDim.x * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < K; ++s) {
            union { uint4 u; _Float16 h[8]; } v;
            v.u = *reinterpret_cast<const uint4 *>(y16 + (size_t)pk[s] * H + j);
            const int8_t *ep = yexp + (size_t)pk[s] * (H / GW) + j / GW;
            const int e0 = ep[0], e1 = GW == 4 ? ep[1] : e0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = __builtin_fmaf(wk[s], ldexpf((float)v.h[i], i < 4 ? e0 : e1), acc[i]);
        }
        float4 *o = reinterpret_cast<float4 *>(out + (size_t)t * H + j);
        o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

hipError_t launch_combine(const Shape &s, int T, const Workspace &ws, float *out, hipStream_t st) {
    if (is_vq_format(s.fmt))
        combine_kernel<4><<<T, 256, 0, st>>>(ws.y16, ws.yexp, ws.w, ws.inv, s.H, s.K, out);
    else
        combine_kernel<16><<<T, 256, 0, st>>>(ws.y16, ws.yexp, ws.w, ws.inv, s.H, s.K, out);
    return hipGetLastError();
}

}  // namespace bqmoe
