// vq_decode.hip -- batch-1 expert kernels for VQ13R8 experts on gfx950.
//
// At one token the layer streams the k selected experts' index bytes once
// (21 bits per 8 weights, Baekpica VQ card, "Recipe") and every weight vector
// is rebuilt from the two books -- the pages' decode case of expanding each
// selected expert with the books kept on chip.  Both books (128 KiB + 4 KiB of
// fp16) are copied into LDS by every block at its start (from L2 after the
// first block), so a gather is two 16-byte LDS reads.
//
// The dot products run on the matrix core with the gathered vectors as the A
// operand (16 weight rows x 32 K, lane (n, q): row n, vectors 8q..8q+7 of a
// 256-column tile, exactly a lane's contiguous run of index bytes) and the
// activation as B, the same in all 16 columns: lanes (n, q) all read the one
// 16-byte piece of x or h that K step s needs, an LDS broadcast, and column 0
// of the result is the dot product.  As in the large-batch kernels the A
// operand is Cb + Rb rounded once to fp16 and the activations enter as fp16
// rows scaled by an exact power of two.
//
// Kernels (one token, k routes):
//  * vq_dec_gateup: block = 4 (gate, up) row-group pairs of one route (8
//    groups of 16 rows).  Each wave streams GW groups over TJ tiles of K; the
//    partial dot products meet in LDS and the block applies the row gains,
//    2^s_x and SwiGLU, writing h (fp32, route-position order).  Every block
//    selects the top-k from the router logits itself; block 0 publishes the
//    routing.
//  * vq_dec_down: block = one output row group (16 rows) for all k routes.
//    Each wave streams one route's tiles over a quarter of K; the routes go
//    through in two phases of four, h of the phase's routes staged in LDS as
//    fp16 with a per-route exponent (the books leave room for four).  The
//    block sums the weighted contributions in a fixed order and stores out.
#include "vq_common.h"

namespace bqmoe {

constexpr int kVdWaves = 16;
constexpr int kVdThreads = kVdWaves * 64;
constexpr int kVdPairs = 4;                       // gate/up pairs per gate/up block
constexpr int kVdGroups = 2 * kVdPairs;           // row groups per gate/up block
constexpr int kVdMaxH = 4096;
constexpr int kVdMaxI = 2048;

struct VdBooks {
    uint4 cb[kVqEntries];     // 128 KiB
    uint4 rb[kVqResEntries];  // 4 KiB, directly after cb (one contiguous copy)
};

struct VdGuLds {
    VdBooks bk;
    uint4 x16[kVdMaxH / 8];   // fp16 x * 2^-s, piece (J, s, q) at (8J + s)*4 + q
    float red[kVdWaves][kVdGroups][16];  // [K slice][group][row]
    float wmax[kVdWaves];
};

struct VdDnLds {
    VdBooks bk;
    uint4 h16[4][kVdMaxI / 8];  // one phase's 4 routes, fp16 h * 2^-s, same piece order
    float red[kVdWaves][16];    // [wave][row]
    float wmax[kVdWaves][4];
};

// The books reach LDS through registers: a thread loads kBookLoads 16-byte
// pieces (the last repeats for threads past the end, rewriting the same bytes)
// early, and stores them once its own routing-dependent loads are issued.
// (An LDS-direct copy would leave the compiler unable to count the vector
// loads behind it, so every later wait would be for all loads in flight.)
constexpr int kBookPieces = kVqEntries + kVqResEntries;  // 16-byte pieces
constexpr int kBookLoads = (kBookPieces + kVdThreads - 1) / kVdThreads;

__device__ __forceinline__ void load_books(const uint8_t *packed, int tid, uint4 (&bv)[kBookLoads]) {
    const uint4 *src = reinterpret_cast<const uint4 *>(packed);
#pragma unroll
    for (int j = 0; j < kBookLoads; ++j) bv[j] = src[min(tid + kVdThreads * j, kBookPieces - 1)];
}

__device__ __forceinline__ void store_books(VdBooks &bk, int tid, const uint4 (&bv)[kBookLoads]) {
    uint4 *dst = reinterpret_cast<uint4 *>(&bk);
#pragma unroll
    for (int j = 0; j < kBookLoads; ++j) dst[min(tid + kVdThreads * j, kBookPieces - 1)] = bv[j];
}

// One K step (vector S of the lane's runs) for G groups against B piece b.
template <int S, int G>
__device__ __forceinline__ void vd_kstep(const uint32_t (&cr)[G][6], const VdBooks &bk, uint4 b,
                                         f32x4 (&acc)[G]) {
    uint4 cbv[G], rbv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        uint32_t i13, i8;
        vq_indices<S>(cr[g], i13, i8);
        cbv[g] = bk.cb[i13];
        rbv[g] = bk.rb[i8];
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(add_f16x8(cbv[g], rbv[g]),
                                                        __builtin_bit_cast(f16x8, b), acc[g], 0,
                                                        0, 0);
}

template <int G>
__device__ __forceinline__ void vd_tile(const uint32_t (&cr)[G][6], const VdBooks &bk,
                                        const uint4 *bpieces, int q, f32x4 (&acc)[G]) {
    vd_kstep<0, G>(cr, bk, bpieces[0 * 4 + q], acc);
    vd_kstep<1, G>(cr, bk, bpieces[1 * 4 + q], acc);
    vd_kstep<2, G>(cr, bk, bpieces[2 * 4 + q], acc);
    vd_kstep<3, G>(cr, bk, bpieces[3 * 4 + q], acc);
    vd_kstep<4, G>(cr, bk, bpieces[4 * 4 + q], acc);
    vd_kstep<5, G>(cr, bk, bpieces[5 * 4 + q], acc);
    vd_kstep<6, G>(cr, bk, bpieces[6 * 4 + q], acc);
    vd_kstep<7, G>(cr, bk, bpieces[7 * 4 + q], acc);
}

// Index into the (J, s, q) piece order of the column c (a multiple of 4) of a
// 256-column-tiled row, in fp16 elements.
__device__ __forceinline__ int piece_elem(int c) {
    const int J = c >> 8, r = c & 255;
    return (((J * 8 + ((r & 63) >> 3)) * 4 + (r >> 6)) << 3) + (r & 7);
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Wave = (group set of GW groups, K slice of TJ tiles);
// NSL slices of TJ tiles cover H / 256.  With fewer than kVdWaves such pairs
// the spare waves repeat the last one's loads and discard the result.
// ---------------------------------------------------------------------------
template <int GW, int TJ, int NSL>
__global__ __launch_bounds__(kVdThreads) void vq_dec_gateup(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed, size_t expert_bytes, int H,
    int I, int E, int K, const float *__restrict__ logits, int32_t *__restrict__ idx_out,
    float *__restrict__ w_out, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ active, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    float *__restrict__ h) {
    constexpr int NJ = NSL * TJ;
    constexpr int NWA = NSL * (kVdGroups / GW);  // waves with work
    static_assert(kVdGroups % GW == 0 && NWA <= kVdWaves, "wave split");
    __shared__ __align__(16) VdGuLds lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, n = lane & 15;
    const int wa = min(wave, NWA - 1);
    const int gset = wa / NSL, js = wa % NSL;  // groups [gset*GW, +GW), tiles [js*TJ, +TJ)

    float lv[4];
    topk_load(logits, E, lv);
    const int nx = H / 8;
    const uint4 xv = reinterpret_cast<const uint4 *>(x)[min(tid, nx - 1)];

    int sel[kMaxTopK], pos[kMaxTopK];
    float wt[kMaxTopK];
    wave_topk_vals(lv, E, K, sel, wt);
    single_token_positions(sel, K, pos);

    const int ipg = I / 16;                       // gate row groups
    const int p = (kVdPairs * blockIdx.x) / ipg;  // route position of this block
    const int i0 = (kVdPairs * blockIdx.x) % ipg;
    int e = sel[0];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
        if (s < K && pos[s] == p) e = sel[s];
    e = __builtin_amdgcn_readfirstlane(e);

    // the books (L2-resident after the first blocks) go out first, then the
    // weight indices; compute starts once both are in
    uint4 bv[kBookLoads];
    load_books(packed, tid, bv);
    __builtin_amdgcn_sched_barrier(0);
    const VqMatrix m(packed + kVqBooksBytes + (size_t)e * expert_bytes, (size_t)2 * I, (size_t)H);
    uint32_t cr[TJ][GW][6];
#pragma unroll
    for (int u = 0; u < TJ; ++u)
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            const int gi = gset * GW + g;  // pair gi>>1, gate (even) or up (odd)
            const size_t grp = (size_t)((gi & 1) ? ipg : 0) + i0 + (gi >> 1);
            m.load(grp * NJ + js * TJ + u, lane, cr[u][g]);
        }
    // the row gains of the epilogue (thread t < 64: pair t/16, row t%16)
    const int grow = 16 * (i0 + ((tid >> 4) & (kVdPairs - 1))) + (tid & 15);
    const uint32_t gg = m.gain[grow], gu = m.gain[I + grow];

    store_books(lds.bk, tid, bv);

    // x -> fp16 * 2^-s_x, s_x from the row's largest magnitude
    uint32_t mb = 0;
    {
        const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mb = max(mb, (w4[k] & 0x7FFFu) << 16);
            mb = max(mb, w4[k] & 0x7FFF0000u);
        }
    }
    const float wm = wave_max_f32(__uint_as_float(mb));
    if (lane == 0) lds.wmax[wave] = wm;
    __syncthreads();
    float xm = lds.wmax[0];
#pragma unroll
    for (int w2 = 1; w2 < kVdWaves; ++w2) xm = fmaxf(xm, lds.wmax[w2]);
    const int xs = fp16_row_exponent(__float_as_uint(xm));
    if (tid < nx) {
        const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const _Float16 lo = (_Float16)ldexpf(bf16_to_f32(w4[k] & 0xFFFFu), -xs);
            const _Float16 hi = (_Float16)ldexpf(bf16_to_f32(w4[k] >> 16), -xs);
            o[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(lds.x16) + piece_elem(8 * tid))[0] =
            make_uint4(o[0], o[1], o[2], o[3]);
    }
    __syncthreads();

    f32x4 acc[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < TJ; ++u) vd_tile<GW>(cr[u], lds.bk, &lds.x16[32 * (js * TJ + u)], q, acc);

    if (n == 0 && wave < NWA) {
#pragma unroll
        for (int g = 0; g < GW; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) lds.red[js][gset * GW + g][4 * q + j] = acc[g][j];
    }
    __syncthreads();
    if (tid < 16 * kVdPairs) {
        const int pr = tid >> 4, r = tid & 15;
        float gs = lds.red[0][2 * pr][r], us = lds.red[0][2 * pr + 1][r];
#pragma unroll
        for (int j = 1; j < NSL; ++j) {
            gs += lds.red[j][2 * pr][r];
            us += lds.red[j][2 * pr + 1][r];
        }
        const float gv = ldexpf(gs * f16_bits_to_f32(gg), xs);
        const float uv = ldexpf(us * f16_bits_to_f32(gu), xs);
        h[(size_t)p * I + grow] = silu_f32(gv) * uv;
    }
    if (blockIdx.x == 0 && wave == 0)  // after the weight stream, so its stores do not delay it
        publish_single_token(sel, wt, pos, E, K, idx_out, w_out, perm, inv, active, counts, offsets);
}

// ---------------------------------------------------------------------------
// down + weighted combine.  Block = output row group blockIdx.x; wave w =
// (route slot r4 = w & 3, K quarter jq = w >> 2): phase f streams route 4f+r4
// over tiles [jq * TJ, +TJ).  NJD = I / 256 is 4 * TJ, or less with TJ = 1
// (then the upper quarters repeat the last tiles' loads and contribute
// nothing); routes past k likewise.
// ---------------------------------------------------------------------------
template <int TJ>
__global__ __launch_bounds__(kVdThreads) void vq_dec_down(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int K,
    const int32_t *__restrict__ active, const int32_t *__restrict__ perm,
    const float *__restrict__ wts, const float *__restrict__ h, float *__restrict__ out) {
    __shared__ __align__(16) VdDnLds lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, n = lane & 15;
    const int rg = blockIdx.x;
    const int NJD = I / 256;
    const int r4 = wave & 3, jq = wave >> 2;
    const bool jlive = jq * TJ < NJD;
    const int j0 = min(jq * TJ, NJD - TJ);  // clamped for loads

    uint4 bv[kBookLoads];
    load_books(packed, tid, bv);
    int ex[2];
    float wgt[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {  // uniform: scalar loads
        const int pc = min(4 * f + r4, K - 1);
        ex[f] = active[1 + pc];
        wgt[f] = wts[perm[pc]];
    }
    // h: thread t holds columns 4c..4c+3 (c = t mod I/4) of the routes of
    // phase hh = (t / (I/4)) & 1; threads past the first 2 * I/4 repeat them
    const int ncg = I / 4;
    const int cg = tid & (ncg - 1), hh = (tid / ncg) & 1;
    float4 hv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        hv[k] = reinterpret_cast<const float4 *>(h + (size_t)min(4 * hh + k, K - 1) * I)[cg];

    const size_t dn_off = vq_down_offset((size_t)H, (size_t)I);
    uint32_t cr[2][TJ][1][6];
    uint2 gn[2];  // gains of rows 16rg + 4q .. +3
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const VqMatrix m(packed + kVqBooksBytes + (size_t)ex[f] * expert_bytes + dn_off,
                         (size_t)H, (size_t)I);
#pragma unroll
        for (int u = 0; u < TJ; ++u) m.load((size_t)rg * NJD + j0 + u, lane, cr[f][u][0]);
        gn[f] = *reinterpret_cast<const uint2 *>(m.gain + 16 * rg + 4 * q);
    }

    store_books(lds.bk, tid, bv);
    // per-route exponents: wave maxima of the four routes it holds
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a = fmaxf(fmaxf(fabsf(hv[k].x), fabsf(hv[k].y)),
                              fmaxf(fabsf(hv[k].z), fabsf(hv[k].w)));
        const float mx = wave_max_f32(a);
        if (lane == 0) lds.wmax[wave][k] = mx;
    }
    __syncthreads();
    int hs[2][4];
    {
        float rm[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) rm[r] = 0.f;
        for (int w2 = 0; w2 < kVdWaves; ++w2) {
            const int h2 = ((w2 * 64) / ncg) & 1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float v = lds.wmax[w2][k];
                rm[k] = h2 == 0 ? fmaxf(rm[k], v) : rm[k];
                rm[4 + k] = h2 == 1 ? fmaxf(rm[4 + k], v) : rm[4 + k];
            }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) hs[r >> 2][r & 3] = fp16_row_exponent(__float_as_uint(rm[r]));
    }

    f32x4 acc[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        if (f > 0) __syncthreads();  // phase 0's readers are done with h16
        if (hh == f) {
            const int pe = piece_elem(4 * cg);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int s2 = hs[f][k];
                const _Float16 a = (_Float16)ldexpf(hv[k].x, -s2), b = (_Float16)ldexpf(hv[k].y, -s2);
                const _Float16 c = (_Float16)ldexpf(hv[k].z, -s2), d = (_Float16)ldexpf(hv[k].w, -s2);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(lds.h16[k]) + pe) =
                    make_uint2((uint32_t)__builtin_bit_cast(uint16_t, a) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16),
                               (uint32_t)__builtin_bit_cast(uint16_t, c) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, d) << 16));
            }
        }
        __syncthreads();
        f32x4 a1[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int u = 0; u < TJ; ++u) vd_tile<1>(cr[f][u], lds.bk, &lds.h16[r4][32 * (j0 + u)], q, a1);
        acc[f] = a1[0];
    }

    if (n == 0) {
        const bool l0 = jlive && r4 < K, l1 = jlive && 4 + r4 < K;
        const float s0 = ldexpf(wgt[0], hs[0][r4]), s1 = ldexpf(wgt[1], hs[1][r4]);
        const uint32_t g0[4] = {gn[0].x & 0xFFFFu, gn[0].x >> 16, gn[0].y & 0xFFFFu, gn[0].y >> 16};
        const uint32_t g1[4] = {gn[1].x & 0xFFFFu, gn[1].x >> 16, gn[1].y & 0xFFFFu, gn[1].y >> 16};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float c0 = l0 ? acc[0][j] * f16_bits_to_f32(g0[j]) * s0 : 0.f;
            const float c1 = l1 ? acc[1][j] * f16_bits_to_f32(g1[j]) * s1 : 0.f;
            lds.red[wave][4 * q + j] = c0 + c1;
        }
    }
    __syncthreads();
    if (tid < 16) {
        float v = lds.red[0][tid];
#pragma unroll
        for (int w2 = 1; w2 < kVdWaves; ++w2) v += lds.red[w2][tid];
        out[16 * rg + tid] = v;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool vq_decode_supported(const Shape &s) {
    const int nj = s.H / 256;
    const bool h_ok = nj == 1 || nj == 2 || nj == 4 || nj == 8 || nj == 16;
    const bool i_ok = s.I == 256 || s.I == 512 || s.I == 1024 || s.I == 2048;
    return s.fmt == MOE_FMT_VQ13R8 && h_ok && i_ok;
}

template <int GW, int TJ, int NSL>
static hipError_t vd_gateup_launch(const Shape &s, const uint16_t *x, const uint8_t *packed,
                                   const Workspace &ws, hipStream_t st) {
    const int grid = s.K * (s.I / 16) / kVdPairs;
    vq_dec_gateup<GW, TJ, NSL><<<grid, kVdThreads, 0, st>>>(
        x, packed, s.expert_bytes, s.H, s.I, s.E, s.K, ws.logits, ws.idx, ws.w, ws.counts,
        ws.offsets, ws.active, ws.perm, ws.inv, static_cast<float *>(ws.h));
    return hipGetLastError();
}

hipError_t launch_vq_decode_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                   const Workspace &ws, hipStream_t st) {
    if (T != 1 || !vq_decode_supported(s)) return hipErrorInvalidValue;
    switch (s.H / 256) {
        case 1: return vd_gateup_launch<1, 1, 1>(s, x, packed, ws, st);
        case 2: return vd_gateup_launch<1, 1, 2>(s, x, packed, ws, st);
        case 4: return vd_gateup_launch<2, 1, 4>(s, x, packed, ws, st);
        case 8: return vd_gateup_launch<4, 1, 8>(s, x, packed, ws, st);
        default: return vd_gateup_launch<4, 2, 8>(s, x, packed, ws, st);
    }
}

template <int TJ>
static hipError_t vd_down_launch(const Shape &s, const uint8_t *packed, const Workspace &ws,
                                 float *out, hipStream_t st) {
    vq_dec_down<TJ><<<s.H / 16, kVdThreads, 0, st>>>(packed, s.expert_bytes, s.H, s.I, s.K,
                                                     ws.active, ws.perm, ws.w,
                                                     static_cast<const float *>(ws.h), out);
    return hipGetLastError();
}

hipError_t launch_vq_decode_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                                 float *out, hipStream_t st) {
    if (T != 1 || !vq_decode_supported(s)) return hipErrorInvalidValue;
    switch (s.I / 256) {
        case 1:
        case 2:
        case 4: return vd_down_launch<1>(s, packed, ws, out, st);
        default: return vd_down_launch<2>(s, packed, ws, out, st);
    }
}

}  // namespace bqmoe
