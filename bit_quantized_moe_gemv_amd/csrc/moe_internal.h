// moe_internal.h -- shared definitions of the gfx950 MoE layer library:
// workspace carving, launcher declarations and small device helpers.
#pragma once

#include <hip/hip_runtime.h>

#include "bqmoe.h"
#include <stddef.h>
#include <stdint.h>

namespace bqmoe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;
constexpr int kDecodeMaxTokens = 16;
constexpr int kMaxHidden = 8192;
constexpr int kVqEntries = 8192;
constexpr int kVqResEntries = 256;
constexpr size_t kVqBooksBytes = (size_t)(kVqEntries + kVqResEntries) * 8 * 2;  // VQ13R8
constexpr size_t kVq13BooksBytes = (size_t)kVqEntries * 8 * 2;                     // VQ13

__host__ __device__ constexpr bool is_vq_format(int fmt) {
    return fmt == MOE_FMT_VQ13R8 || fmt == MOE_FMT_VQ13;
}

// Shapes of one layer.
struct Shape {
    int H, I, E, K;      // hidden, intermediate, experts, top-k
    int fmt;
    int routing;         // MOE_ROUTE_*
    size_t expert_bytes;  // bytes of one expert in the packed buffer
    size_t books_bytes;   // bytes before expert 0 (VQ books)
};

// Device pointers carved out of the caller's workspace.
struct Workspace {
    float *logits;     // [Tmax][E]
    int32_t *idx;      // [Tmax][K]
    float *w;          // [Tmax][K]
    int32_t *counts;   // [E]
    int32_t *offsets;  // [E+1]
    int32_t *active;   // [1 + E]: n_active, then active experts ascending
    int32_t *perm;     // [Rmax]
    int32_t *inv;      // [Rmax]
    void *h;           // [Rmax][I] fp32
    // per-route expert outputs, fp16 times a power of two per 16 (MXFP4) or
    // 4 (VQ) output rows: y = y16 * 2^yexp
    uint16_t *y16;     // [Rmax][H]
    int8_t *yexp;      // [Rmax][H/16] or [Rmax][H/4], after y16
    // fp16 rows with a power-of-two exponent each: h16/hexp feed the down GEMM
    // of both formats, x16/xexp (VQ only, null otherwise) the VQ gate/up GEMM
    uint16_t *x16;     // [Tmax][H]
    int32_t *xexp;     // [Tmax]
    uint16_t *h16;     // [Rmax][I]
    int32_t *hexp;     // [Rmax]
    // VQ only (null otherwise): the largest |h| of each 64-column piece of a
    // route's h row, written by the batch-1 VQ gate/up blocks for the down kernel
    float *hpmax;      // [Rmax][I/64]
};

size_t workspace_bytes(const Shape &s, int tmax);
void carve_workspace(const Shape &s, int tmax, void *base, Workspace *ws);

// ---- launchers (each returns hipSuccess or the launch error) ----
hipError_t launch_router(const Shape &s, const uint16_t *x, const float *wr, int T, float *logits,
                         hipStream_t st);
// Small batches (T <= 16): logits, then the routing kernel -- except for a
// single token when route_single is false (the batch-1 decode gate/up kernel
// routes it).
hipError_t launch_router_route_small(const Shape &s, const uint16_t *x, const float *wr, int T,
                                     const Workspace &ws, hipStream_t st, bool route_single);
hipError_t launch_topk(const Shape &s, int T, const Workspace &ws, hipStream_t st);
hipError_t launch_permute(const Shape &s, int T, const Workspace &ws, hipStream_t st);
bool decode_supported(const Shape &s);
int decode_max_tokens(const Shape &s);  // largest T the decode kernels take
bool vq_decode_supported(const Shape &s);
hipError_t launch_vq_decode_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                   const Workspace &ws, hipStream_t st);
hipError_t launch_vq_decode_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                                 float *out, hipStream_t st);
hipError_t launch_decode_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                const Workspace &ws, hipStream_t st);
hipError_t launch_decode_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                              float *out, hipStream_t st);
hipError_t launch_prefill_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                 const Workspace &ws, hipStream_t st);
hipError_t launch_prefill_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                               hipStream_t st);
// h (fp32, R rows) -> h16 and hexp
hipError_t launch_hpack(const Shape &s, int R, const Workspace &ws, hipStream_t st);
hipError_t launch_vq_prefill_gateup(const Shape &s, int T, const uint16_t *x,
                                    const uint8_t *packed, const Workspace &ws, hipStream_t st);
hipError_t launch_vq_prefill_down(const Shape &s, int T, const uint8_t *packed,
                                  const Workspace &ws, hipStream_t st);
hipError_t launch_combine(const Shape &s, int T, const Workspace &ws, float *out, hipStream_t st);
// measurement aid: one streaming read of `bytes` (a multiple of 16) at buf
hipError_t launch_read_probe(const uint8_t *buf, size_t bytes, uint32_t *sink, hipStream_t st);

// ---- device helpers ----
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// E8M0 exponent byte (1..254) as the fp32 scale 2^(e-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) { return __uint_as_float(e << 23); }

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// Four packed fp4 bytes (one dword) -> eight bf16, each times `scale`.
// Byte b of the dword holds columns 2b (low nibble) and 2b+1 (high nibble).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t v, float scale) {
    union { bf16x8 v8; bf16x2 v2[4]; } r;
    r.v2[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
    r.v2[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
    r.v2[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
    r.v2[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
    return r.v8;
}

// Workgroup barrier that orders LDS only.  Unlike __syncthreads() it does not
// wait for outstanding global loads, so weight streams stay in flight across
// it.  Use only where the barrier protects LDS data.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders one wave's own LDS writes before its later LDS reads.
__device__ __forceinline__ void lds_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// DPP lane moves (gfx9 encodings).
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// v from lane (per CTRL), or `old` where the lane has no source / is masked.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_or_old(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}

// Exact wave-wide maximum of a float (returned to every lane).  Lane i of each
// row takes the max of lanes i-1, i-2, i-4, i-8 (so lane 15 holds its row's
// max), then row broadcasts carry rows 0..3 into lane 63.  Max is exact and
// order-free, so this equals any other reduction order.
__device__ __forceinline__ float wave_max_f32(float v) {
    int b = __float_as_int(v);
    b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_or_old<kDppRowShr1>(b, b))));
    b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_or_old<kDppRowShr2>(b, b))));
    b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_or_old<kDppRowShr4>(b, b))));
    b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_or_old<kDppRowShr8>(b, b))));
    b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_or_old<kDppRowBcast15, 0xA>(b, b))));
    b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(dpp_or_old<kDppRowBcast31, 0xC>(b, b))));
    return __int_as_float(__builtin_amdgcn_readlane(b, 63));
}

// Wave-wide minimum of an int (returned to every lane); same lane pattern.
__device__ __forceinline__ int wave_min_i32(int v) {
    v = min(v, dpp_or_old<kDppRowShr1>(v, v));
    v = min(v, dpp_or_old<kDppRowShr2>(v, v));
    v = min(v, dpp_or_old<kDppRowShr4>(v, v));
    v = min(v, dpp_or_old<kDppRowShr8>(v, v));
    v = min(v, dpp_or_old<kDppRowBcast15, 0xA>(v, v));
    v = min(v, dpp_or_old<kDppRowBcast31, 0xC>(v, v));
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_sum_xor(float v, int from_mask) {
    for (int m = from_mask; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// ---------------------------------------------------------------------------
// top-k of one token by one wave
// ---------------------------------------------------------------------------

// (value, index) key: a beats b if its value is larger, or equal with a lower
// index.  Comparing floats makes -0 and +0 equal, so they tie to the index.
__device__ __forceinline__ bool key_beats(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Selects the k best experts of `l` (E <= 256 logits) and their routing
// weights (softmax, or normalised sigmoids).  Every lane returns the same
// idx[]/w[]; lane l owns experts l, l+64, l+128, l+192, sorted once by key.  Each round reduces the lanes' heads
// to the wave maximum, then to the lowest expert index holding it (both
// reductions are exact, so the winner does not depend on reduction order); the
// winning lane pops its head.
__device__ __forceinline__ void cswap(float &va, int &ia, float &vb, int &ib) {
    // after the call (va, ia) beats or equals (vb, ib)
    const bool sw = key_beats(vb, ib, va, ia);
    const float tv = sw ? vb : va;
    const int ti = sw ? ib : ia;
    vb = sw ? va : vb;
    ib = sw ? ia : ib;
    va = tv;
    ia = ti;
}

// The value a logit is ranked by.  A NaN logit (reachable only from
// non-finite inputs, e.g. inf - inf inside a router sum of huge activations)
// ranks as -inf, below every number: both selections below then compare
// ordinary floats, agree, and never pick an index outside [0, E).
__host__ __device__ constexpr float selection_value(float v) { return v != v ? -INFINITY : v; }

// Order-preserving unsigned key of a ranked value (after selection_value):
// a > b as floats iff key(a) > key(b); -0 is first turned into +0, so the two
// zeros tie (and the index decides), as in key_beats.
__host__ __device__ constexpr uint32_t f32_order_key(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The lane's four ranked logits (experts lane + 64j), -inf past E.  Issued as
// unconditional loads (clamped index) so a caller can count them.
__device__ __forceinline__ void topk_load(const float *__restrict__ l, int E, float (&v)[4]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = selection_value(l[min(lane + 64 * j, E - 1)]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (lane + 64 * j >= E) v[j] = -INFINITY;
}

__device__ inline void wave_topk_vals(const float (&lv)[4], int E, int K, bool sigmoid,
                                      int *idx, float *w) {
    const int lane = threadIdx.x & 63;
    float v0 = lv[0], v1 = lv[1], v2 = lv[2], v3 = lv[3];
    int i0 = lane, i1 = lane + 64, i2 = lane + 128, i3 = lane + 192;
    if (i0 >= E) i0 = 0x7FFFFFFF;
    if (i1 >= E) i1 = 0x7FFFFFFF;
    if (i2 >= E) i2 = 0x7FFFFFFF;
    if (i3 >= E) i3 = 0x7FFFFFFF;
    // sorting network for 4 keys
    cswap(v0, i0, v1, i1);
    cswap(v2, i2, v3, i3);
    cswap(v0, i0, v2, i2);
    cswap(v1, i1, v3, i3);
    cswap(v1, i1, v2, i2);
    float val[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (s < K) {
            const float m = wave_max_f32(v0);
            const uint64_t hit = __ballot(v0 == m);
            int gi;
            if (__popcll(hit) == 1)  // usual case: one lane holds the maximum
                gi = __builtin_amdgcn_readlane(i0, __ffsll((unsigned long long)hit) - 1);
            else                     // equal logits: lowest expert index wins
                gi = wave_min_i32(v0 == m ? i0 : 0x7FFFFFFF);
            idx[s] = min(gi, E - 1);  // gi < E whenever k <= E; kept in range regardless
            val[s] = m;
            if (i0 == gi) {  // pop the head
                v0 = v1; i0 = i1;
                v1 = v2; i1 = i2;
                v2 = v3; i2 = i3;
                v3 = -INFINITY; i3 = 0x7FFFFFFF;
            }
        }
    }
    // weights over the selected logits (val[0] is the largest), each first
    // relative to slot 0's: softmax exp(l_s - l_0); sigmoid
    // sigma(l_s)/sigma(l_0), as (1 + e^-l0)/(1 + e^-ls) when l_0 > 0 and as
    // e^(l_s - l_0) (1 + e^l0)/(1 + e^ls) otherwise, so that no exponential
    // overflows into inf/inf; the ratio of slot 0 is 1, so the sum is >= 1.
    float sum = 0.0f;
    const float e0n = __expf(-val[0]), e0p = __expf(val[0]);
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (s < K) {
            const float d = __expf(val[s] - val[0]);
            float r = d;
            if (sigmoid)
                r = val[0] > 0.0f ? (1.0f + e0n) / (1.0f + __expf(-val[s]))
                                  : d * (1.0f + e0p) / (1.0f + __expf(val[s]));
            w[s] = s == 0 ? 1.0f : r;
            sum += w[s];
        }
    }
    const float inv = 1.0f / sum;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
        if (s < K) w[s] *= inv;
}

__device__ inline void wave_topk(const float *__restrict__ l, int E, int K, bool sigmoid, int *idx,
                                 float *w) {
    float v[4];
    topk_load(l, E, v);
    wave_topk_vals(v, E, K, sigmoid, idx, w);
}

// ---------------------------------------------------------------------------
// The selected set alone (no order, no weights), for kernels that only need to
// know which experts a single token uses.  Same selection as wave_topk: the K
// best by (logit descending, expert index ascending).  The K-th largest key t
// comes from a bitwise binary search whose counts are wave ballots; the set is
// every key above t plus the lowest-index experts equal to t.  The search stops
// as soon as a prefix of t has exactly K keys at or above it (the usual case
// after the sign, exponent and a few mantissa bits).  Wave-uniform
// scalar work only: no cross-lane data movement besides the ballots.
// ---------------------------------------------------------------------------

// Bit l of m[j] is set when expert l + 64j is among the K selected (E <= 256).
__device__ inline void wave_topk_set(const float (&lv)[4], int E, int K, uint64_t (&m)[4]) {
    const int lane = threadIdx.x & 63;
    uint32_t k[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)  // past E: key 0, below every finite logit's key
        k[j] = lane + 64 * j < E ? f32_order_key(lv[j]) : 0u;
    uint32_t t = 0;  // the largest t with at least K keys >= t: the K-th largest key
    // unrolled: each step's threshold is t | constant, with t and the counts
    // in scalar registers
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        const uint32_t c = t | (1u << b);
        int n = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) n += __popcll(__ballot(k[j] >= c));
        if (n >= K) {
            t = c;
            // exactly K keys >= c: they are the selection, and no tie can
            // straddle it (n is wave-uniform, so is the early exit)
            if (n == K) {
#pragma unroll
                for (int j = 0; j < 4; ++j) m[j] = __ballot(k[j] >= c);
                return;
            }
        }
    }
    int need = K;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        m[j] = __ballot(k[j] > t);
        need -= __popcll(m[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // ties at t: lowest expert indices first
        uint64_t eq = __ballot(k[j] == t && lane + 64 * j < E);
        while (need > 0 && eq) {
            const uint64_t low = eq & (~eq + 1);
            m[j] |= low;
            eq ^= low;
            --need;
        }
    }
}

// The r-th (from 0) selected expert in ascending index order, i.e. the expert
// the counting sort puts at route position r of a single token.
__device__ inline int topk_set_nth(const uint64_t (&m)[4], int r) {
    int e = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = __popcll(m[j]);
        if (!found && r < c) {
            uint64_t x = m[j];
            for (int i = 0; i < r; ++i) x &= x - 1;
            e = 64 * j + __builtin_ctzll(x);
            found = true;
        }
        r -= found ? 0 : c;
    }
    return e;
}

// Route positions of a single token: slot s goes to position pos[s], the rank
// of its expert among the selected ones (ascending), which is the order the
// counting sort gives.
__device__ __forceinline__ void single_token_positions(const int *sel, int K, int *pos) {
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        pos[s] = 0;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
            if (s < K && j < K) pos[s] += sel[j] < sel[s];
    }
}

// Writes a single token's routing, computed identically by every lane of one
// wave, in the layout the routing kernels produce: idx/w in slot order,
// perm/inv between route ids and positions, the active expert list, and
// counts/offsets over all E experts.
__device__ inline void publish_single_token(const int *sel, const float *wt, const int *pos, int E,
                                            int K, int32_t *idx_out, float *w_out, int32_t *perm,
                                            int32_t *inv, int32_t *active, int32_t *counts,
                                            int32_t *offsets) {
    const int ln = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
        if (s < K && ln == s) {
            idx_out[s] = sel[s];
            w_out[s] = wt[s];
            perm[pos[s]] = s;
            inv[s] = pos[s];
            active[1 + pos[s]] = sel[s];
        }
    if (ln == 0) {
        active[0] = K;
        offsets[E] = K;
    }
    for (int ee = ln; ee < E; ee += 64) {
        int c = 0, below = 0;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
            if (j < K) {
                c += sel[j] == ee;
                below += sel[j] < ee;
            }
        counts[ee] = c;
        offsets[ee] = below;
    }
}

}  // namespace bqmoe
