// decode.hip -- small-batch (T <= 16) expert kernels for MXFP4 experts on
// gfx950: stream each selected expert's packed weights from HBM once with
// 128-bit loads, dequantise in registers and accumulate in fp32 on the vector
// ALUs (the work is bandwidth-bound, so no matrix cores are used).
//
// Formats: E2M1 codes two per byte with one E8M0 exponent per 32 weights of a
// row (TrevorJS GGUF card, "Architecture notes"); tiles of 16 rows x 32
// columns (see bqmoe.h).  A lane (n = lane%16, q = lane/16) of a wave reads,
// at super-step J, the 16 code bytes of tile column 4J+q for tile row n: the
// 64 lanes cover one contiguous 1 KiB block, and each lane's 16 bytes are one
// scale block of 32 weights.
//
// Accumulation stays in fp32 from the dot products through SwiGLU to the
// down projection: the pages report expert intermediates above fp16's range
// (TrevorJS card, "Recipe"; benthecarman EXL3 card, "Bitrate").
#include "moe_internal.h"

namespace bqmoe {

constexpr int kDecTC = 4;  // routes (tokens) per pass through the staged operand
// row groups a gate/up block streams one after another: one token / up to 16 tokens
constexpr int kDecRS1 = 2;
constexpr int kDecRS = 4;
// K slices per matrix in a gate/up block (the block has 2 * KW waves): one token
// / up to 16 tokens
constexpr int kDecKW1 = 4;
constexpr int kDecKW = 2;

// bf16 pairs of a 16-byte fp4 block: out[b] = columns (2b, 2b+1) * scale.
__device__ __forceinline__ void fp4x32_to_bf16(const uint4 v, float scale, bf16x2 *out) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], scale, 0);
        out[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], scale, 1);
        out[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], scale, 2);
        out[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], scale, 3);
    }
}

constexpr int kRing = 4;  // 1 KiB wave loads kept in flight per wave

// Global loads below never sit under a divergent branch: predicated loads make
// the compiler fall back to waiting for every outstanding load at the branch
// joins, which serialises the weight stream.  Shapes are template parameters
// and out-of-range staging loads are clamped duplicates instead of skipped.
// Weights are read once per step: non-temporal loads, so they do not displace
// the cached x, h and routing rows.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const uint8_t *base, uint32_t off) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + off));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Empty asm register fences: the value becomes opaque at this point of the
// program, so the compiler can neither hoist its consumers above it (e.g. all
// conversions above the staging barrier) nor sink it.  Used to keep the ring's
// per-super-step order and register footprint.
__device__ __forceinline__ void reg_fence(uint32_t &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void reg_fence(uint4 &v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Grid: (expert slots, I/(16*RS)).  Block: 2*KW waves
// owning the 16 gate rows and the 16 matching up rows of RS row groups of one
// active expert: wave w streams matrix w/KW (gate, up) over K slice w%KW, per
// row group a contiguous run of NW = 2*NJ/KW super-steps of 1 KiB (NJ = H/256),
// with kRing loads in flight.  The x rows of up to TC routes are fetched first
// and staged in LDS behind an LDS-only barrier, so the weight stream is never
// stalled by them.  h is written in fp32, in route-position order.  One token
// takes four K slices (eight waves): twice the loads in flight per CU, 16.6 ->
// 16.0 us for the 4096 x 2048 experts; wider batches keep two, their dot
// products being four times the work per byte.
// ---------------------------------------------------------------------------
// With R1 (a single token) the blocks route the token themselves, which
// replaces a separate routing launch: every wave of a streaming block finds the
// selected set of experts (wave_topk_set: ballots only, no ordering or
// weights) and takes the slot-th selected expert in ascending order; one block
// of an extra row runs the full ordered selection with its weights (the same
// one-wave selection as the routing kernel) and publishes the routing for the
// down kernel and moe_layer_routing.
template <int NJ, int TC, bool R1, int RS, int KW>
__global__ __launch_bounds__(128 * KW) void decode_gateup_mxfp4(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed, size_t expert_bytes,
    int H, int I, int E, int K, int32_t *__restrict__ active, int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm, float *__restrict__ h, const float *__restrict__ logits,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out, int32_t *__restrict__ counts,
    int32_t *__restrict__ inv, bool sigmoid) {
    extern __shared__ __align__(16) uint16_t xs[];  // [TC][H]
    __shared__ float red[RS][2 * KW][TC][64];  // [row group][wave][token][lane]: lanes 0..15 used
    const int slot = blockIdx.x;
    int e, p0, ne;
    if (R1) {
        if (blockIdx.y == gridDim.y - 1) {
            // the extra row (dispatched after the streaming blocks, which keep
            // their even spread over the XCDs): block (0, last) publishes the
            // ordered routing and its weights for the down kernel and
            // moe_layer_routing while the other blocks stream
            if (slot == 0 && threadIdx.x < 64) {
                int sel[kMaxTopK];
                float wt[kMaxTopK];
                wave_topk(logits, E, K, sigmoid, sel, wt);
                int pos[kMaxTopK];
                single_token_positions(sel, K, pos);
                publish_single_token(sel, wt, pos, E, K, idx_out, w_out, perm, inv, active,
                                     counts, offsets);
            }
            return;
        }
        // which expert: every wave finds it itself (the selected set only,
        // ballots), so no wave waits on a barrier before its weight stream
        float lv[4];
        topk_load(logits, E, lv);
        uint64_t m[4];
        wave_topk_set(lv, E, K, m);
        e = __builtin_amdgcn_readfirstlane(topk_set_nth(m, slot));
        p0 = slot;
        ne = 1;
    } else {
        // routing reads through the vector unit, the lanes' loads together:
        // lane 0 the active count, lane 1 the slot's expert, then lanes 0 and 1
        // its route range
        const int l = threadIdx.x & 63;
        const int av = active[l == 0 ? 0 : 1 + min(slot, E - 1)];
        if (slot >= __builtin_amdgcn_readlane(av, 0)) return;
        e = __builtin_amdgcn_readlane(av, 1);
        const int ov = offsets[e + (l & 1)];
        p0 = __builtin_amdgcn_readlane(ov, 0);
        ne = __builtin_amdgcn_readlane(ov, 1) - p0;
    }
    const int rg0 = blockIdx.y * RS;  // first of the block's RS row groups
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int mat = wave / KW, kh = wave % KW;
    constexpr int NT = 128 * KW;     // threads
    constexpr int NW = 2 * NJ / KW;  // super-steps of one K slice
    static_assert(NW * KW == 2 * NJ, "K slices must split the row evenly");

    const size_t kt = (size_t)(H / 32);  // tiles along K per row group
    const size_t grp = (size_t)(mat ? I / 16 + rg0 : rg0);
    const uint8_t *ex = packed + (size_t)e * expert_bytes;
    const uint8_t *cbase = ex + (grp * kt + (size_t)kh * NW * 4) * 256;          // wave's first tile
    const uint8_t *sbase = ex + (size_t)I * H + (grp * kt + (size_t)kh * NW * 4) * 16;
    const uint32_t coff = (uint32_t)(q * 256 + n * 16);
    const uint32_t soff = (uint32_t)(q * 16 + n);
    const int per_row = H / 8;                   // uint4 per x row
    constexpr int XN = (TC * NJ * 32 + NT - 1) / NT;  // uint4 per thread for TC rows (H = 256*NJ)

    for (int c0 = 0; c0 < ne; c0 += TC) {
        const int nt = min(TC, ne - c0);
        if (c0 > 0) lds_barrier();  // previous chunk's readers are done with xs and red
        // token of each staged row: uniform values, read through the scalar unit
        // so that they do not queue behind the vector loads
        int trow[TC];
#pragma unroll
        for (int r = 0; r < TC; ++r) trow[r] = R1 ? 0 : perm[p0 + c0 + min(r, nt - 1)] / K;
        uint4 xv[XN];
#pragma unroll
        for (int i = 0; i < XN; ++i) {
            const int idx = min(tid + NT * i, TC * per_row - 1);
            const int r = idx / per_row, c = idx - r * per_row;
            int t = trow[0];
#pragma unroll
            for (int rr = 1; rr < TC; ++rr) t = (r == rr) ? trow[rr] : t;
            xv[i] = reinterpret_cast<const uint4 *>(x + (size_t)t * H)[c];
        }
        __builtin_amdgcn_sched_barrier(0);  // x loads first, then the weight ring
        // The wave's stream: RS row groups one after another, NW super-steps
        // each; row group r starts r*rstride bytes (r*sstride scale bytes)
        // further on.  The ring runs across row-group boundaries.
        constexpr int JJ = RS * NW;
        const uint32_t rstride = (uint32_t)(kt * 256), sstride = (uint32_t)(kt * 16);
        uint4 ring[kRing];
        uint32_t sring[kRing];
#pragma unroll
        for (int j = 0; j < kRing && j < JJ; ++j) {
            ring[j] = ld16(cbase, (j / NW) * rstride + coff + (j % NW) * 1024);
            sring[j] = sbase[(j / NW) * sstride + soff + (j % NW) * 64];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < XN; ++i)
            reinterpret_cast<uint4 *>(xs)[min(tid + NT * i, TC * per_row - 1)] = xv[i];
        lds_barrier();

        float acc[TC];
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            const int r = jj / NW, j = jj % NW;
            if (j == 0) {
#pragma unroll
                for (int tt = 0; tt < TC; ++tt) acc[tt] = 0.f;
            }
            uint4 wv = ring[jj % kRing];
            uint32_t sv = sring[jj % kRing];
            reg_fence(wv);
            reg_fence(sv);
            const float sc = e8m0_to_f32(sv);
            if (jj + kRing < JJ) {
                const int jn = jj + kRing;
                uint32_t o = (jn / NW) * rstride + coff + (jn % NW) * 1024;
                uint32_t so = (jn / NW) * sstride + soff + (jn % NW) * 64;
                reg_fence(o);
                reg_fence(so);
                ring[jj % kRing] = ld16(cbase, o);
                sring[jj % kRing] = sbase[so];
            }
            bf16x2 w2[16];
            fp4x32_to_bf16(wv, sc, w2);
            const int J = kh * NW + j;
#pragma unroll
            for (int tt = 0; tt < TC; ++tt) {
                if (tt < nt) {
                    const uint4 *xr = reinterpret_cast<const uint4 *>(xs + tt * H + 128 * J + 32 * q);
                    union { uint4 u[4]; bf16x2 p[16]; } xx;
#pragma unroll
                    for (int m = 0; m < 4; ++m) xx.u[m] = xr[m];
                    float a = acc[tt];
#pragma unroll
                    for (int b = 0; b < 16; ++b)
                        a = __builtin_amdgcn_fdot2_f32_bf16(w2[b], xx.p[b], a, false);
                    acc[tt] = a;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (j == NW - 1) {  // row group r done: the wave's partial sums to LDS
#pragma unroll
                for (int tt = 0; tt < TC; ++tt) {
                    acc[tt] += __shfl_xor(acc[tt], 16, 64);
                    acc[tt] += __shfl_xor(acc[tt], 32, 64);
                    red[r][wave][tt][lane] = acc[tt];  // every lane: no branch in the stream
                }
            }
        }
        // one barrier after the whole stream (a barrier or a global store
        // inside it would make the compiler drain the weight ring), then
        // SwiGLU and h for the block's RS row groups
        lds_barrier();
        for (int i = tid; i < RS * nt * 16; i += NT) {
            const int r = i / (nt * 16), tt = (i >> 4) % nt, nn = i & 15;
            float g = red[r][0][tt][nn], u = red[r][KW][tt][nn];
#pragma unroll
            for (int w = 1; w < KW; ++w) {
                g += red[r][w][tt][nn];
                u += red[r][KW + w][tt][nn];
            }
            h[(size_t)(p0 + c0 + tt) * I + 16 * (rg0 + r) + nn] = silu_f32(g) * u;
        }
    }
}

// ---------------------------------------------------------------------------
// down projection + weighted combine.  Grid: H/16 blocks (one 16-row group of
// the output each) of 16 waves.  The block covers every active expert: wave w
// takes active slots w/2, w/2+8, ... and K half w%2 of their 16 down rows
// (NJ = I/256 super-steps; with I = 128 the second half is empty).  Per slot
// it fetches its half of the route's h row into its own LDS area, then its
// packed bytes (kept in registers while the expert's further routes are
// processed), computing each super-step as it arrives.  Route outputs
// y[p][16] (two K halves) stay in LDS; after one barrier the block forms
// out[t][j] = sum_s w[t,s] * y[inv[t,s]][j] in slot order.  No atomics and no
// cross-block traffic: the result is bitwise reproducible.
// ---------------------------------------------------------------------------
constexpr int kDnWaves = 16;
constexpr int kDnMaxI = 2048;
constexpr int kDnMaxR = kDecodeMaxTokens * kMaxTopK;

template <int NJ>
__global__ __launch_bounds__(kDnWaves * 64) void decode_down_mxfp4(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int K, int T,
    const int32_t *__restrict__ active, const int32_t *__restrict__ offsets,
    const float *__restrict__ h, const float *__restrict__ wts, const int32_t *__restrict__ inv,
    float *__restrict__ out) {
    __shared__ __align__(16) float hs[kDnWaves][kDnMaxI / 2];
    __shared__ float ys[2][kDnMaxR][16];
    __shared__ float s_w[kDnMaxR];
    __shared__ int s_inv[kDnMaxR];
    const int a = blockIdx.x;  // output row group
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int kh = wave & 1;
    // a single token has K distinct experts, and the counting sort puts the
    // q-th of them (ascending) at route position q: no routing reads are
    // needed before the h rows can be fetched
    const bool single = T == 1;
    const int n_active = single ? K : active[0];
    const int R = T * K;
    // routing weights of the combine, fetched now so their latency is hidden
    const int rr = min(tid, R - 1);
    const float my_w = wts[rr];
    const int my_inv = inv[rr];
    const bool live = kh * NJ * 128 < I;  // false only for the empty second half when I = 128
    const size_t kt = (size_t)(I / 32);
    const uint32_t coff = (uint32_t)(q * 256 + n * 16);
    const uint32_t soff = (uint32_t)(q * 16 + n);
    float *hw = hs[wave];

    // the wave's slots qs = wave/2 + 8i (at most 32): lane i fetches slot i's
    // expert and route range up front, so no slot waits on routing reads
    const int qsl = (wave >> 1) + (kDnWaves / 2) * lane;
    const int el = active[1 + min(qsl, n_active - 1)];
    const int p0l = single ? qsl : offsets[el];
    const int nel = single ? 1 : offsets[el + 1] - p0l;
    for (int qs = wave >> 1, i = 0; qs < n_active; qs += kDnWaves / 2, ++i) {
        const int e = __builtin_amdgcn_readlane(el, i);
        const int p0 = __builtin_amdgcn_readlane(p0l, i);
        const int ne = __builtin_amdgcn_readlane(nel, i);
        if (!live) {
            for (int r = 0; r < ne; ++r)
                if (q == 0) ys[kh][p0 + r][n] = 0.f;
            continue;
        }
        const uint8_t *ex = packed + (size_t)e * expert_bytes;
        const uint8_t *dcode = ex + (size_t)I * H + (size_t)I * H / 16;
        const uint8_t *dscl = dcode + (size_t)H * I / 2;
        const uint8_t *cbase = dcode + ((size_t)a * kt + (size_t)kh * NJ * 4) * 256;
        const uint8_t *sbase = dscl + ((size_t)a * kt + (size_t)kh * NJ * 4) * 16;

        uint4 cv[NJ];
        uint32_t cs[NJ];
        for (int r = 0; r < ne; ++r) {
            // this wave's half of h[p]: floats [128*NJ*kh, 128*NJ*(kh+1)), two per lane per step
            const float2 *hrow =
                reinterpret_cast<const float2 *>(h + (size_t)(p0 + r) * I + 128 * NJ * kh);
            float2 hv[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) hv[j] = hrow[64 * j + lane];
            if (r == 0) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    cv[j] = ld16(cbase, coff + j * 1024);
                    cs[j] = sbase[soff + j * 64];
                }
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) reinterpret_cast<float2 *>(hw)[64 * j + lane] = hv[j];
            lds_wave_sync();
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                uint4 wv = cv[j];
                uint32_t sv = cs[j];
                reg_fence(wv);
                reg_fence(sv);
                const float sc = e8m0_to_f32(sv);
                const uint32_t d[4] = {wv.x, wv.y, wv.z, wv.w};
                const float4 *hr = reinterpret_cast<const float4 *>(hw + 128 * j + 32 * q);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], sc, 0);
                    const f32x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], sc, 1);
                    const f32x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], sc, 2);
                    const f32x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], sc, 3);
                    const float4 v0 = hr[2 * i], v1 = hr[2 * i + 1];
                    acc = __builtin_fmaf(w0.x, v0.x, acc);
                    acc = __builtin_fmaf(w0.y, v0.y, acc);
                    acc = __builtin_fmaf(w1.x, v0.z, acc);
                    acc = __builtin_fmaf(w1.y, v0.w, acc);
                    acc = __builtin_fmaf(w2.x, v1.x, acc);
                    acc = __builtin_fmaf(w2.y, v1.y, acc);
                    acc = __builtin_fmaf(w3.x, v1.z, acc);
                    acc = __builtin_fmaf(w3.y, v1.w, acc);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            acc += __shfl_xor(acc, 16, 64);
            acc += __shfl_xor(acc, 32, 64);
            if (q == 0) ys[kh][p0 + r][n] = acc;
            lds_wave_sync();
        }
    }
    if (tid < R) {
        s_w[tid] = my_w;
        s_inv[tid] = my_inv;
    }
    lds_barrier();
    for (int i = tid; i < T * 16; i += kDnWaves * 64) {
        const int t = i >> 4, nn = i & 15;
        float acc = 0.f;
        for (int s = 0; s < K; ++s) {
            const int p = s_inv[t * K + s];
            acc = __builtin_fmaf(s_w[t * K + s], ys[0][p][nn] + ys[1][p][nn], acc);
        }
        out[(size_t)t * H + 16 * a + nn] = acc;
    }
}

template <int NJ, int TC, bool R1, int RS, int KW>
static hipError_t gateup_launch(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                const Workspace &ws, hipStream_t st) {
    // a single token gets one more row of blocks: its block (0, last) publishes the routing
    const int slots = min(s.E, T * s.K);
    dim3 grid(slots, s.I / (16 * RS) + (R1 ? 1 : 0));
    decode_gateup_mxfp4<NJ, TC, R1, RS, KW><<<grid, 128 * KW, (size_t)TC * s.H * 2, st>>>(
        x, packed, s.expert_bytes, s.H, s.I, s.E, s.K, ws.active, ws.offsets, ws.perm,
        static_cast<float *>(ws.h), ws.logits, ws.idx, ws.w, ws.counts, ws.inv,
        s.routing == MOE_ROUTE_SIGMOID);
    return hipGetLastError();
}

template <int NJ>
static hipError_t gateup_launch_tc(const Shape &s, int T, const uint16_t *x,
                                   const uint8_t *packed, const Workspace &ws, hipStream_t st) {
    // (the unrolled stream grows with RS * NJ)
    constexpr int RS1 = NJ >= 32 ? 1 : kDecRS1, RS = NJ >= 32 ? 1 : kDecRS;
    constexpr int KW1 = kDecKW1 < 2 * NJ ? kDecKW1 : 2 * NJ;  // a slice is at least one super-step
    constexpr int KW = kDecKW < 2 * NJ ? kDecKW : 2 * NJ;
    return T == 1 ? gateup_launch<NJ, 1, true, RS1, KW1>(s, T, x, packed, ws, st)
                  : gateup_launch<NJ, kDecTC, false, RS, KW>(s, T, x, packed, ws, st);
}

bool decode_supported(const Shape &s) {
    if (is_vq_format(s.fmt)) return vq_decode_supported(s);
    const int nj = s.H / 256;
    const bool h_ok = nj == 1 || nj == 2 || nj == 4 || nj == 8 || nj == 16 || nj == 32;
    const bool i_ok = s.I == 128 || s.I == 256 || s.I == 512 || s.I == 1024 || s.I == 2048;
    return s.fmt == MOE_FMT_MXFP4 && h_ok && i_ok;
}

int decode_max_tokens(const Shape &s) { return is_vq_format(s.fmt) ? 1 : kDecodeMaxTokens; }

hipError_t launch_decode_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                const Workspace &ws, hipStream_t st) {
    if (is_vq_format(s.fmt)) return launch_vq_decode_gateup(s, T, x, packed, ws, st);
    switch (s.H / 256) {
        case 1: return gateup_launch_tc<1>(s, T, x, packed, ws, st);
        case 2: return gateup_launch_tc<2>(s, T, x, packed, ws, st);
        case 4: return gateup_launch_tc<4>(s, T, x, packed, ws, st);
        case 8: return gateup_launch_tc<8>(s, T, x, packed, ws, st);
        case 16: return gateup_launch_tc<16>(s, T, x, packed, ws, st);
        case 32: return gateup_launch_tc<32>(s, T, x, packed, ws, st);
        default: return hipErrorInvalidValue;
    }
}

template <int NJ>
static hipError_t down_launch(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                              float *out, hipStream_t st) {
    decode_down_mxfp4<NJ><<<s.H / 16, kDnWaves * 64, 0, st>>>(
        packed, s.expert_bytes, s.H, s.I, s.K, T, ws.active, ws.offsets,
        static_cast<const float *>(ws.h), ws.w, ws.inv, out);
    return hipGetLastError();
}

hipError_t launch_decode_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                              float *out, hipStream_t st) {
    if (is_vq_format(s.fmt)) return launch_vq_decode_down(s, T, packed, ws, out, st);
    if (s.I > kDnMaxI || T * s.K > kDnMaxR) return hipErrorInvalidValue;
    switch (s.I) {
        case 128:
        case 256: return down_launch<1>(s, T, packed, ws, out, st);
        case 512: return down_launch<2>(s, T, packed, ws, out, st);
        case 1024: return down_launch<4>(s, T, packed, ws, out, st);
        case 2048: return down_launch<8>(s, T, packed, ws, out, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bqmoe
