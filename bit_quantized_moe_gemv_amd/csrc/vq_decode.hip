// vq_decode.hip -- batch-1 expert kernels for VQ13R8 experts on gfx950.
//
// At one token the layer streams the k selected experts' index bytes once
// (21 bits per 8 weights, Baekpica VQ card, "Recipe") and every weight vector
// is rebuilt from the two books -- the pages' decode case of expanding each
// selected expert with the books kept on chip.  Both books (128 KiB + 4 KiB of
// fp16) are copied into LDS by every block at its start (from L2 after the
// first block), so a gather is two 16-byte LDS reads.
//
// Lane (n, q) of a wave owns, in each 16-row x 256-column tile, row n's
// vectors 8q..8q+7 -- exactly its contiguous run of index bytes.  At K step s
// it gathers Cb[i13] and Rb[i8] of vector 8q+s and takes both dot products
// with the matching 16-byte piece of the activation (lanes of one q read the
// same piece: an LDS broadcast) on the vector ALU (v_dot2_f32_f16: fp16 pairs,
// exact products, fp32 sums); the four lanes of a row add up at the end.  The
// books' values enter unrounded; the activations enter as fp16 rows scaled by
// an exact power of two, as in the large-batch kernels.  (At one token the
// matrix core would waste 15 of its 16 columns.)
//
// Every barrier in these kernels orders LDS only (lds_barrier): a full
// __syncthreads() would also wait for every global load in flight, i.e. the
// block's whole index stream, before the first gather.  Index loads are
// issued after the last barrier that precedes the gathers: issuing them
// stalls while the HBM stream is saturated, so a barrier behind them would
// hold every wave's gathers until the slowest wave had issued all of its
// loads.
//
// Kernels (one token, k routes):
//  * vq_dec_gateup: block = 4 (gate, up) row-group pairs of one route (8
//    groups of 16 rows).  Each wave streams GW groups over TJ tiles of K; the
//    partial dot products meet in LDS and the block applies the row gains,
//    2^s_x and SwiGLU, writing h (fp32, route-position order).  Every block
//    finds its expert from the router logits itself (one wave, the selected
//    set only); block 0 runs the ordered top-k with its weights and publishes
//    the routing.  The activation's fp16 exponent s_x comes from the router
//    kernel, so x16 is staged in LDS before the block's first barrier.
//  * vq_dec_down: block = one output row group (16 rows) for all k routes.
//    Each wave streams one route's tiles over a quarter of K; the routes go
//    through in two phases of four, h of the phase's routes staged in LDS as
//    fp16 with a per-route exponent (the books leave room for four), taken
//    from the largest |h| of each 64-column piece that the gate/up blocks
//    leave beside h.  The block sums the weighted contributions in a fixed
//    order and stores out.
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
    int expert;
};

struct VdDnLds {
    VdBooks bk;
    uint4 h16[4][kVdMaxI / 8];  // one phase's 4 routes, fp16 h * 2^-s, same piece order
    float red[kVdWaves][16];    // [wave][row]
};

// The books reach LDS through registers: each of NT threads loads kBookLoads
// 16-byte pieces (the last repeats for threads past the end, rewriting the
// same bytes).  (An LDS-direct copy would leave the compiler unable to count
// the vector loads behind it, so every later wait would be for all loads in
// flight.)
template <bool RES>
constexpr int book_pieces() {  // 16-byte pieces: Cb, then Rb with the residual stage
    return RES ? kVqEntries + kVqResEntries : kVqEntries;
}
constexpr int kBookLoads = (kVqEntries + kVqResEntries + kVdThreads - 65) / (kVdThreads - 64);

template <int NT, bool RES>
__device__ __forceinline__ void load_books(const uint8_t *packed, int t, uint4 (&bv)[kBookLoads]) {
    constexpr int P = book_pieces<RES>();
    static_assert(NT * kBookLoads >= P, "book split");
    const uint4 *src = reinterpret_cast<const uint4 *>(packed);
#pragma unroll
    for (int j = 0; j < kBookLoads; ++j) bv[j] = src[min(t + NT * j, P - 1)];
}

template <int NT, bool RES>
__device__ __forceinline__ void store_books(VdBooks &bk, int t, const uint4 (&bv)[kBookLoads]) {
    constexpr int P = book_pieces<RES>();
    uint4 *dst = reinterpret_cast<uint4 *>(&bk);
#pragma unroll
    for (int j = 0; j < kBookLoads; ++j) dst[min(t + NT * j, P - 1)] = bv[j];
}

// One K step (vector S of the lane's runs) for G groups against the
// activation piece b: two fp32 dot products per group, Cb[i13] . b and
// Rb[i8] . b, each over the eight fp16 pairs with exact products.  Random
// 16-byte reads are what bound these kernels: from LDS they cost about 5 ns
// per wave instruction on a CU (bank conflicts), and from the 4 KiB residual
// book in global memory, which stays in the L1 cache, about 14 ns, but on the
// vector-memory path, in parallel with LDS.  So odd K steps read Rb from
// global memory (rbg) and even ones from LDS: about 8 ns per vector pair
// against 10.5 with both from LDS (measured on a random-gather probe).
template <int S, int G, bool RES>
__device__ __forceinline__ void vd_kstep(const uint32_t (&cr)[G][6], const VdBooks &bk,
                                         const uint4 *__restrict__ rbg, uint4 b,
                                         float (&acc)[G][2]) {
    uint4 cbv[G], rbv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        uint32_t i13, i8;
        vq_indices<S>(cr[g], i13, i8);
        cbv[g] = bk.cb[i13];
        if (RES) rbv[g] = (S & 1) ? rbg[i8] : bk.rb[i8];
    }
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint32_t cw[4] = {cbv[g].x, cbv[g].y, cbv[g].z, cbv[g].w};
        const uint32_t rw[4] = {RES ? rbv[g].x : 0u, RES ? rbv[g].y : 0u, RES ? rbv[g].z : 0u,
                                RES ? rbv[g].w : 0u};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc[g][0] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, cw[w]),
                                               __builtin_bit_cast(f16x2, bw[w]), acc[g][0], false);
            if (RES)
                acc[g][1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, rw[w]),
                                                   __builtin_bit_cast(f16x2, bw[w]), acc[g][1],
                                                   false);
        }
    }
    // The sums leave every step through an empty asm: left free, the compiler
    // defers all the dot products to the end of the tile and keeps every
    // gathered vector alive until then.
#pragma unroll
    for (int g = 0; g < G; ++g) asm volatile("" : "+v"(acc[g][0]), "+v"(acc[g][1]));
}

template <int G, bool RES>
__device__ __forceinline__ void vd_tile(const uint32_t (&cr)[G][6], const VdBooks &bk,
                                        const uint4 *__restrict__ rbg,
                                        const uint4 *bpieces, int q, float (&acc)[G][2]) {
    vd_kstep<0, G, RES>(cr, bk, rbg, bpieces[0 * 4 + q], acc);
    vd_kstep<1, G, RES>(cr, bk, rbg, bpieces[1 * 4 + q], acc);
    vd_kstep<2, G, RES>(cr, bk, rbg, bpieces[2 * 4 + q], acc);
    vd_kstep<3, G, RES>(cr, bk, rbg, bpieces[3 * 4 + q], acc);
    vd_kstep<4, G, RES>(cr, bk, rbg, bpieces[4 * 4 + q], acc);
    vd_kstep<5, G, RES>(cr, bk, rbg, bpieces[5 * 4 + q], acc);
    vd_kstep<6, G, RES>(cr, bk, rbg, bpieces[6 * 4 + q], acc);
    vd_kstep<7, G, RES>(cr, bk, rbg, bpieces[7 * 4 + q], acc);
}

// A row's dot product from its four lanes (n, q = 0..3): every lane of row n
// gets the sum.
__device__ __forceinline__ float row_sum(const float (&a)[2]) {
    float v = a[0] + a[1];
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    return v;
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
template <int GW, int TJ, int NSL, bool RES>
__global__ __launch_bounds__(kVdThreads) void vq_dec_gateup(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ xexp,
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H,
    int I, int E, int K, const float *__restrict__ logits, int32_t *__restrict__ idx_out,
    float *__restrict__ w_out, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ active, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    float *__restrict__ h, float *__restrict__ hpmax, bool sigmoid) {
    constexpr int NJ = NSL * TJ;
    constexpr int NWA = NSL * (kVdGroups / GW);  // waves with work
    static_assert(kVdGroups % GW == 0 && NWA <= kVdWaves, "wave split");
    __shared__ __align__(16) VdGuLds lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, n = lane & 15;
    const uint4 *rbg = reinterpret_cast<const uint4 *>(packed) + kVqEntries;  // Rb in memory
    const int wa = min(wave, NWA - 1);
    const int gset = wa / NSL, js = wa % NSL;  // groups [gset*GW, +GW), tiles [js*TJ, +TJ)

    // Wave 0 selects the routes while the other waves copy the books, which
    // do not depend on the routing, into LDS.
    const int ipg = I / 16;                       // gate row groups
    const int p = (kVdPairs * blockIdx.x) / ipg;  // route position of this block
    const int i0 = (kVdPairs * blockIdx.x) % ipg;
    const int nx = H / 8;
    const uint4 xv = reinterpret_cast<const uint4 *>(x)[min(tid, nx - 1)];
    // x's fp16 row exponent s_x (largest |x| scaled into [2^14, 2^15)), written
    // by the router kernel: x16 is staged before the first barrier, so no
    // barrier separates the index loads from the gathers
    const int xs = __builtin_amdgcn_readfirstlane(xexp[0]);
    if (wave == 0) {
        float lv[4];
        topk_load(logits, E, lv);
        if (blockIdx.x == 0) {  // the ordered selection with its weights, published
            int sel[kMaxTopK], pos[kMaxTopK];
            float wt[kMaxTopK];
            wave_topk_vals(lv, E, K, sigmoid, sel, wt);
            single_token_positions(sel, K, pos);
            int e0 = sel[0];
#pragma unroll
            for (int s = 0; s < kMaxTopK; ++s)
                if (s < K && pos[s] == p) e0 = sel[s];
            if (lane == 0) lds.expert = e0;
            publish_single_token(sel, wt, pos, E, K, idx_out, w_out, perm, inv, active, counts,
                                 offsets);
        } else {  // the set only: route position p holds its p-th expert in index order
            uint64_t m[4];
            wave_topk_set(lv, E, K, m);
            if (lane == 0) lds.expert = topk_set_nth(m, p);
        }
    } else {
        uint4 bv[kBookLoads];
        load_books<kVdThreads - 64, RES>(packed, tid - 64, bv);
        store_books<kVdThreads - 64, RES>(lds.bk, tid - 64, bv);
    }
    // x -> fp16 * 2^-s_x
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
    lds_barrier();
    const int e = __builtin_amdgcn_readfirstlane(lds.expert);

    const VqMatrix<RES> m(packed + vq_books_bytes<RES>() + (size_t)e * expert_bytes, (size_t)2 * I,
                          (size_t)H);
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

    float acc[GW][2];
#pragma unroll
    for (int g = 0; g < GW; ++g) acc[g][0] = acc[g][1] = 0.f;
#pragma unroll
    for (int u = 0; u < TJ; ++u)
        vd_tile<GW, RES>(cr[u], lds.bk, rbg, &lds.x16[32 * (js * TJ + u)], q, acc);

#pragma unroll
    for (int g = 0; g < GW; ++g) {
        const float v = row_sum(acc[g]);
        if (q == 0 && wave < NWA) lds.red[js][gset * GW + g][n] = v;
    }
    lds_barrier();
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
        const float hv = silu_f32(gv) * uv;
        h[(size_t)p * I + grow] = hv;
        // the block's 64 h values are one 64-column piece of the route's row:
        // its largest |h| lets the down kernel pick the row's fp16 exponent
        // without a block-wide reduction (threads 0..63 are wave 0)
        const float hm = wave_max_f32(fabsf(hv));
        if (tid == 0) hpmax[(size_t)p * (I / 64) + i0 / 4] = hm;
    }
}

// ---------------------------------------------------------------------------
// down + weighted combine.  Block = output row group blockIdx.x; wave w =
// (route slot r4 = w & 3, K quarter jq = w >> 2): phase f streams route 4f+r4
// over tiles [jq * TJ, +TJ).  NJD = I / 256 is 4 * TJ, or less with TJ = 1
// (then the upper quarters repeat the last tiles' loads and contribute
// nothing); routes past k likewise.
// ---------------------------------------------------------------------------
template <int TJ, bool RES>
__global__ __launch_bounds__(kVdThreads) void vq_dec_down(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int K,
    const int32_t *__restrict__ active, const int32_t *__restrict__ perm,
    const float *__restrict__ wts, const float *__restrict__ h, const float *__restrict__ hpmax,
    float *__restrict__ out) {
    __shared__ __align__(16) VdDnLds lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, n = lane & 15;
    const uint4 *rbg = reinterpret_cast<const uint4 *>(packed) + kVqEntries;  // Rb in memory
    const int rg = blockIdx.x;
    const int NJD = I / 256;
    const int r4 = wave & 3, jq = wave >> 2;
    const bool jlive = jq * TJ < NJD;
    const int j0 = min(jq * TJ, NJD - TJ);  // clamped for loads

    uint4 bv[kBookLoads];
    load_books<kVdThreads, RES>(packed, tid, bv);
    // the routes' experts and weights: lane l (< 8) fetches route l's, each
    // wave takes its two with readlane
    const int pcl = min(lane, K - 1);
    const int exl = active[1 + pcl];
    const float wgl = wts[perm[pcl]];
    int ex[2];
    float wgt[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int pc = min(4 * f + r4, K - 1);
        ex[f] = __builtin_amdgcn_readlane(exl, pc);
        wgt[f] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wgl), pc));
    }
    // h: thread t holds columns 4c..4c+3 (c = t mod I/4) of the routes of
    // phase hh = (t / (I/4)) & 1; threads past the first 2 * I/4 repeat them
    const int ncg = I / 4;
    const int cg = tid & (ncg - 1), hh = (tid / ncg) & 1;
    float4 hv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        hv[k] = reinterpret_cast<const float4 *>(h + (size_t)min(4 * hh + k, K - 1) * I)[cg];
    // per-route exponents from the largest |h|: the gate/up blocks left the
    // maxima of the NP = I/64 pieces of each route's row, [route][piece]; lane
    // l takes pieces 4l..4l+3 of the flattened array (one route: NP is a
    // multiple of 4), the lanes of a route combine by xor steps, and lane
    // r*NP/4 ends with route r's maximum (max is exact in any order)
    const int NP = I / 64, LPR = NP / 4;  // lanes per route
    const int pl = min(4 * lane, K * NP - 4);
    const float4 pm = *reinterpret_cast<const float4 *>(hpmax + pl);
    float rm = fmaxf(fmaxf(pm.x, pm.y), fmaxf(pm.z, pm.w));
    for (int o = 1; o < LPR; o <<= 1) rm = fmaxf(rm, __shfl_xor(rm, o, kWave));
    int hs[2][4];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        hs[r >> 2][r & 3] = fp16_row_exponent(
            __float_as_uint(__shfl(rm, min(r, K - 1) * LPR, kWave)));
    uint32_t gn[2];  // gain of row 16rg + n
    const size_t dn_off = vq_down_offset((size_t)H, (size_t)I, RES);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const VqMatrix<RES> m(packed + vq_books_bytes<RES>() + (size_t)ex[f] * expert_bytes + dn_off,
                              (size_t)H, (size_t)I);
        gn[f] = m.gain[16 * rg + n];
    }

    auto stage_h16 = [&](int f) {  // the phase's 4 routes of h as fp16 * 2^-s
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
    };
    store_books<kVdThreads, RES>(lds.bk, tid, bv);
    stage_h16(0);
    lds_barrier();  // books and phase 0's h16

    // the index streams of both phases, issued after the barrier (see above)
    uint32_t cr[2][TJ][1][6];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const VqMatrix<RES> m(packed + vq_books_bytes<RES>() + (size_t)ex[f] * expert_bytes + dn_off,
                              (size_t)H, (size_t)I);
#pragma unroll
        for (int u = 0; u < TJ; ++u) m.load((size_t)rg * NJD + j0 + u, lane, cr[f][u][0]);
    }

    float acc[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        if (f > 0) {
            lds_barrier();  // phase 0's readers are done with h16
            stage_h16(1);
            lds_barrier();
        }
        float a1[1][2] = {{0.f, 0.f}};
#pragma unroll
        for (int u = 0; u < TJ; ++u)
            vd_tile<1, RES>(cr[f][u], lds.bk, rbg, &lds.h16[r4][32 * (j0 + u)], q, a1);
        acc[f] = row_sum(a1[0]);
    }

    if (q == 0) {
        const bool l0 = jlive && r4 < K, l1 = jlive && 4 + r4 < K;
        const float c0 = l0 ? acc[0] * f16_bits_to_f32(gn[0]) * ldexpf(wgt[0], hs[0][r4]) : 0.f;
        const float c1 = l1 ? acc[1] * f16_bits_to_f32(gn[1]) * ldexpf(wgt[1], hs[1][r4]) : 0.f;
        lds.red[wave][n] = c0 + c1;
    }
    lds_barrier();
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
    return (s.fmt == MOE_FMT_VQ13R8 || s.fmt == MOE_FMT_VQ13) && h_ok && i_ok;
}

template <int GW, int TJ, int NSL, bool RES>
static hipError_t vd_gateup_launch(const Shape &s, const uint16_t *x, const uint8_t *packed,
                                   const Workspace &ws, hipStream_t st) {
    const int grid = s.K * (s.I / 16) / kVdPairs;
    vq_dec_gateup<GW, TJ, NSL, RES><<<grid, kVdThreads, 0, st>>>(
        x, ws.xexp, packed, s.expert_bytes, s.H, s.I, s.E, s.K, ws.logits, ws.idx, ws.w, ws.counts,
        ws.offsets, ws.active, ws.perm, ws.inv, static_cast<float *>(ws.h), ws.hpmax,
        s.routing == MOE_ROUTE_SIGMOID);
    return hipGetLastError();
}

template <bool RES>
static hipError_t vd_gateup_res(const Shape &s, const uint16_t *x, const uint8_t *packed,
                                const Workspace &ws, hipStream_t st) {
    switch (s.H / 256) {
        case 1: return vd_gateup_launch<1, 1, 1, RES>(s, x, packed, ws, st);
        case 2: return vd_gateup_launch<1, 1, 2, RES>(s, x, packed, ws, st);
        case 4: return vd_gateup_launch<2, 1, 4, RES>(s, x, packed, ws, st);
        case 8: return vd_gateup_launch<4, 1, 8, RES>(s, x, packed, ws, st);
        default: return vd_gateup_launch<4, 2, 8, RES>(s, x, packed, ws, st);
    }
}

hipError_t launch_vq_decode_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                   const Workspace &ws, hipStream_t st) {
    if (T != 1 || !vq_decode_supported(s)) return hipErrorInvalidValue;
    return s.fmt == MOE_FMT_VQ13R8 ? vd_gateup_res<true>(s, x, packed, ws, st)
                                   : vd_gateup_res<false>(s, x, packed, ws, st);
}

template <int TJ, bool RES>
static hipError_t vd_down_launch(const Shape &s, const uint8_t *packed, const Workspace &ws,
                                 float *out, hipStream_t st) {
    vq_dec_down<TJ, RES><<<s.H / 16, kVdThreads, 0, st>>>(packed, s.expert_bytes, s.H, s.I, s.K,
                                                          ws.active, ws.perm, ws.w,
                                                          static_cast<const float *>(ws.h),
                                                          ws.hpmax, out);
    return hipGetLastError();
}

template <bool RES>
static hipError_t vd_down_res(const Shape &s, const uint8_t *packed, const Workspace &ws,
                              float *out, hipStream_t st) {
    return s.I / 256 <= 4 ? vd_down_launch<1, RES>(s, packed, ws, out, st)
                          : vd_down_launch<2, RES>(s, packed, ws, out, st);
}

hipError_t launch_vq_decode_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                                 float *out, hipStream_t st) {
    if (T != 1 || !vq_decode_supported(s)) return hipErrorInvalidValue;
    return s.fmt == MOE_FMT_VQ13R8 ? vd_down_res<true>(s, packed, ws, out, st)
                                   : vd_down_res<false>(s, packed, ws, out, st);
}

}  // namespace bqmoe
