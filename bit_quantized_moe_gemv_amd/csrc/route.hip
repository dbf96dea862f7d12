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

namespace bqmoe {

// ---------------------------------------------------------------------------
// router logits: one wave computes a TT-token x TE-expert tile
// ---------------------------------------------------------------------------
template <int TT, int TE>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t *__restrict__ x,
                                                     const float *__restrict__ wr, int T, int H,
                                                     int E, float *__restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * TT;
    const int e0 = (blockIdx.y * 4 + wave) * TE;
    if (e0 >= E) return;
    float acc[TT][TE];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int e = 0; e < TE; ++e) acc[t][e] = 0.0f;

    const int groups = H >> 8;
    for (int j = 0; j < groups; ++j) {
        const int k0 = (j << 8) + (lane << 2);
        float4 wv[TE];
#pragma unroll
        for (int e = 0; e < TE; ++e)
            wv[e] = (e0 + e < E) ? *reinterpret_cast<const float4 *>(wr + (size_t)(e0 + e) * H + k0)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            uint2 xb = make_uint2(0u, 0u);
            if (t0 + t < T) xb = *reinterpret_cast<const uint2 *>(x + (size_t)(t0 + t) * H + k0);
            const float x0 = bf16_to_f32(xb.x & 0xFFFFu), x1 = bf16_to_f32(xb.x >> 16);
            const float x2 = bf16_to_f32(xb.y & 0xFFFFu), x3 = bf16_to_f32(xb.y >> 16);
#pragma unroll
            for (int e = 0; e < TE; ++e) {
                float a = acc[t][e];
                a = __builtin_fmaf(x0, wv[e].x, a);
                a = __builtin_fmaf(x1, wv[e].y, a);
                a = __builtin_fmaf(x2, wv[e].z, a);
                a = __builtin_fmaf(x3, wv[e].w, a);
                acc[t][e] = a;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int e = 0; e < TE; ++e) acc[t][e] = wave_sum_xor(acc[t][e], 1);
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int e = 0; e < TE; ++e)
            if (lane == ((t * TE + e) & 63) && t0 + t < T && e0 + e < E)
                logits[(size_t)(t0 + t) * E + e0 + e] = acc[t][e];
}

hipError_t launch_router(const Shape &s, const uint16_t *x, const float *wr, int T, float *logits,
                         hipStream_t st) {
    if (T == 1) {
        dim3 grid(1, (s.E + 3) / 4);
        router_kernel<1, 1><<<grid, 256, 0, st>>>(x, wr, T, s.H, s.E, logits);
    } else if (T <= 16) {
        dim3 grid(1, (s.E + 3) / 4);
        router_kernel<16, 1><<<grid, 256, 0, st>>>(x, wr, T, s.H, s.E, logits);
    } else {
        dim3 grid((T + 7) / 8, (s.E + 31) / 32);
        router_kernel<8, 8><<<grid, 256, 0, st>>>(x, wr, T, s.H, s.E, logits);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// top-k of one token by one wave
// ---------------------------------------------------------------------------

// (value, index) key: a beats b if its value is larger, or equal with a lower
// index.  Comparing floats makes -0 and +0 equal, so they tie to the index.
__device__ __forceinline__ bool key_beats(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Selects the k best experts of `l` (E <= 256 logits) and their softmax
// weights.  Every lane returns the same idx[]/val[]; lanes own experts
// lane, lane+64, lane+128, lane+192.
__device__ void wave_topk(const float *__restrict__ l, int E, int K, int *idx, float *w) {
    const int lane = threadIdx.x & 63;
    float v[4];
    int id[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        id[q] = e;
        v[q] = (e < E) ? l[e] : -INFINITY;
    }
    bool taken[4] = {false, false, false, false};
    float val[kMaxTopK];
    for (int s = 0; s < K; ++s) {
        // best candidate of this lane
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (!taken[q] && id[q] < E && key_beats(v[q], id[q], bv, bi)) { bv = v[q]; bi = id[q]; }
        // wave arg-best
        for (int m = 1; m < 64; m <<= 1) {
            const float ov = __shfl_xor(bv, m, 64);
            const int oi = __shfl_xor(bi, m, 64);
            if (key_beats(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (id[q] == bi) taken[q] = true;
        idx[s] = bi;
        val[s] = bv;
    }
    // softmax over the selected logits (val[0] is the largest)
    float sum = 0.0f;
    for (int s = 0; s < K; ++s) {
        w[s] = __expf(val[s] - val[0]);
        sum += w[s];
    }
    const float inv = 1.0f / sum;
    for (int s = 0; s < K; ++s) w[s] *= inv;
}

// one wave per token (prefill)
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int K, int32_t *__restrict__ idx_out,
                                                   float *__restrict__ w_out) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int idx[kMaxTopK];
    float w[kMaxTopK];
    wave_topk(logits + (size_t)t * E, E, K, idx, w);
    const int lane = threadIdx.x & 63;
    if (lane < K) {
        int iv = idx[0];
        float wv = w[0];
        for (int s = 1; s < K; ++s)
            if (lane == s) { iv = idx[s]; wv = w[s]; }
        idx_out[(size_t)t * K + lane] = iv;
        w_out[(size_t)t * K + lane] = wv;
    }
}

hipError_t launch_topk(const Shape &s, int T, const Workspace &ws, hipStream_t st) {
    topk_kernel<<<(T + 3) / 4, 256, 0, st>>>(ws.logits, T, s.E, s.K, ws.idx, ws.w);
    return hipGetLastError();
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
// small batches (T <= 16): top-k, grouping and active-expert list in one block
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void route_small_kernel(const float *__restrict__ logits, int T,
                                                           int E, int K, int32_t *__restrict__ idx_out,
                                                           float *__restrict__ w_out,
                                                           int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ active,
                                                           int32_t *__restrict__ perm,
                                                           int32_t *__restrict__ inv,
                                                           uint32_t *__restrict__ sync, int n_sync) {
    __shared__ int s_idx[kDecodeMaxTokens * kMaxTopK];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_scan[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = T * K;

    for (int i = tid; i < n_sync; i += blockDim.x) sync[i] = 0u;

    if (wave < T) {
        int idx[kMaxTopK];
        float w[kMaxTopK];
        wave_topk(logits + (size_t)wave * E, E, K, idx, w);
        if (lane < K) {
            int iv = idx[0];
            float wv = w[0];
            for (int s = 1; s < K; ++s)
                if (lane == s) { iv = idx[s]; wv = w[s]; }
            idx_out[wave * K + lane] = iv;
            w_out[wave * K + lane] = wv;
            s_idx[wave * K + lane] = iv;
        }
    }
    __syncthreads();
    // counts
    int c = 0;
    if (tid < E)
        for (int r = 0; r < R; ++r) c += (s_idx[r] == tid);
    int total;
    const int off = block_exclusive_scan(tid < E ? c : 0, &total, s_scan);
    if (tid < E) {
        s_cnt[tid] = c;
        s_off[tid] = off;
        counts[tid] = c;
        offsets[tid] = off;
    }
    if (tid == 0) offsets[E] = total;
    // active experts, ascending
    const int flag = (tid < E && c > 0) ? 1 : 0;
    int n_active;
    const int apos = block_exclusive_scan(flag, &n_active, s_scan);
    if (flag) active[1 + apos] = tid;
    if (tid == 0) active[0] = n_active;
    __syncthreads();
    // stable scatter: rank of route r among earlier routes of the same expert
    if (tid < R) {
        const int e = s_idx[tid];
        int rank = 0;
        for (int r = 0; r < tid; ++r) rank += (s_idx[r] == e);
        const int p = s_off[e] + rank;
        perm[p] = tid;
        inv[tid] = p;
    }
}

hipError_t launch_route_small(const Shape &s, int T, const Workspace &ws, hipStream_t st) {
    route_small_kernel<<<1, 1024, 0, st>>>(ws.logits, T, s.E, s.K, ws.idx, ws.w, ws.counts,
                                           ws.offsets, ws.active, ws.perm, ws.inv, ws.sync,
                                           s.H / 16);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// large batches: one block per expert.  Each block builds the full expert
// histogram, takes its own offset, then compacts its routes in route order
// (a stable counting sort split by expert; no inter-block communication).
// ---------------------------------------------------------------------------
constexpr int kPermPerThread = 8;

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
    for (int i = tid; i < kMaxExperts; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int r = tid; r < R; r += blockDim.x) atomicAdd(&hist[idx[r]], 1);
    __syncthreads();
    int total;
    const int my = (tid < E) ? hist[tid] : 0;
    const int excl = block_exclusive_scan(my, &total, s_scan);
    __shared__ int s_base;
    if (tid == e) s_base = excl;
    if (e == 0) {
        if (tid < E) { counts[tid] = my; offsets[tid] = excl; }
        if (tid == 0) offsets[E] = total;
    }
    if (e == 0) {
        int n_active;
        const int flag = (tid < E && my > 0) ? 1 : 0;
        const int apos = block_exclusive_scan(flag, &n_active, s_scan);
        if (flag) active[1 + apos] = tid;
        if (tid == 0) active[0] = n_active;
    }
    __syncthreads();
    const int base = s_base;
    int running = 0;
    const int chunk = blockDim.x * kPermPerThread;
    for (int b = 0; b < R; b += chunk) {
        const int r0 = b + tid * kPermPerThread;
        int flags = 0, n = 0;
#pragma unroll
        for (int q = 0; q < kPermPerThread; ++q) {
            const int r = r0 + q;
            if (r < R && idx[r] == e) { flags |= 1 << q; ++n; }
        }
        int tot;
        int pos = block_exclusive_scan(n, &tot, s_scan) + running + base;
#pragma unroll
        for (int q = 0; q < kPermPerThread; ++q)
            if (flags & (1 << q)) {
                perm[pos] = r0 + q;
                inv[r0 + q] = pos;
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
// combine: out[t] = sum_s w[t,s] * y[inv[t*K+s]], slots in order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv, int H, int K,
                                                      float *__restrict__ out) {
    const int t = blockIdx.x;
    float wk[kMaxTopK];
    int pk[kMaxTopK];
    for (int s = 0; s < K; ++s) {
        wk[s] = w[(size_t)t * K + s];
        pk[s] = inv[(size_t)t * K + s];
    }
    for (int j = threadIdx.x * 4; j < H; j += blockDim.x * 4) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < K; ++s) {
            const float4 v = *reinterpret_cast<const float4 *>(y + (size_t)pk[s] * H + j);
            acc.x = __builtin_fmaf(wk[s], v.x, acc.x);
            acc.y = __builtin_fmaf(wk[s], v.y, acc.y);
            acc.z = __builtin_fmaf(wk[s], v.z, acc.z);
            acc.w = __builtin_fmaf(wk[s], v.w, acc.w);
        }
        *reinterpret_cast<float4 *>(out + (size_t)t * H + j) = acc;
    }
}

hipError_t launch_combine(const Shape &s, int T, const Workspace &ws, float *out, hipStream_t st) {
    combine_kernel<<<T, 256, 0, st>>>(ws.y, ws.w, ws.inv, s.H, s.K, out);
    return hipGetLastError();
}

}  // namespace bqmoe
