// vq_prefill.hip -- large-batch expert kernels for VQ13R8 and VQ13 experts on
// gfx950 (VQ13 layers have no residual stage: the A operand is Cb itself, and
// everything below that concerns Rb drops out).
//
// A VQ13R8 weight is w[n][8v+d] = gain[n] * (Cb[i13][d] + Rb[i8][d]): an
// 8-wide codeword from a per-layer book of 8192 entries (13-bit index: a
// 12-bit stream plus a 1-bit plane) plus a codeword from a 256-entry residual
// book (8-bit index), times an fp16 gain per output row (Baekpica VQ card,
// "Recipe" and "Why 13 bits plus an 8-bit residual").  Both books are fp16.
//
// Design.  The gain is a per-row factor, so it moves out of the dot product
// into the epilogue; what the matrix core multiplies is Cb + Rb.  That sum is
// formed in fp16 (one packed add per two weights, rounding once: relative
// error at most 2^-11, an order of magnitude inside the layer's tolerance),
// so both GEMMs run as single v_mfma_f32_16x16x32_f16 passes with fp32
// accumulation.  The activations reach fp16 through an exact power-of-two
// scale per row: x[t] * 2^-s_t and h[r] * 2^-s_r put each row's largest
// magnitude in [2^14, 2^15), inside fp16's range whatever the data, and the
// epilogue multiplies 2^s back in.  bf16 x values are exact in fp16 there;
// fp32 h values round once to fp16 (relative 2^-11).
//
// Both books (128 KiB + 4 KiB) live in LDS for the whole kernel: blocks are
// persistent (one per CU) and loop over (expert, row slice, token chunk)
// items, so the books are loaded once per CU.  A lane gathers its A operand
// with two 16-byte LDS reads per K step.  The B operand (64 tokens) streams
// through a 3-deep LDS ring of 64-column sub-steps (8 KiB each) with
// global_load_lds; the index streams of a 256-column super-step go straight
// to registers one super-step ahead.
//
// Lane roles.  A = 16 weight rows x 32 K of fp16 (lane l: row l%16, K slice
// 8*(l/16)..+7).  In a VQ tile (16 rows x 256 columns) lane (n, q) owns the
// eight vectors of row n in columns 64q..64q+63 -- 12 contiguous code12 bytes,
// 8 res bytes and one plane byte at lane-contiguous offsets -- and K step s
// (0..7) of the super-step uses its vector s, i.e. columns 64q+8s..+7.  The B
// operand of lane (m, q) at K step s is therefore x[m][256J+64q+8s..+7];
// sub-step u holds K steps 2u and 2u+1.
#include "vq_common.h"

namespace bqmoe {

constexpr int kVqWaves = 8;  // two per SIMD, sharing the books
constexpr int kVqThreads = kVqWaves * 64;
constexpr int kVqGroups = 4;  // row groups (16 rows) per wave; 512 rows per block item
constexpr int kVqRing = 3;    // B sub-stages in LDS
constexpr int kVqChunkLanes = 2;  // an expert's 64-token chunks are dealt to 2 items

struct VqLds {
    uint4 cb[kVqEntries];     // 128 KiB
    uint4 rb[kVqResEntries];  // 4 KiB
    uint8_t b[kVqRing][2][4][64][16];  // [slot][K step parity][q][token][8 fp16]
};

template <int N>
__device__ __forceinline__ void vq_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void vq_stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only: loads stay in flight
    __builtin_amdgcn_s_barrier();
}

// ---------------------------------------------------------------------------
// x (bf16) -> fp16 rows scaled by 2^-s_t.  One block per token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void vq_xpack_kernel(const uint16_t *__restrict__ x, int H,
                                                       uint16_t *__restrict__ x16,
                                                       int32_t *__restrict__ xexp) {
    __shared__ uint32_t smax;
    if (threadIdx.x == 0) smax = 0;
    __syncthreads();
    const uint16_t *row = x + (size_t)blockIdx.x * H;
    uint32_t m = 0;
    for (int i = threadIdx.x * 8; i < H; i += 256 * 8) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m = max(m, (w[k] & 0x7FFFu) << 16);
            m = max(m, w[k] & 0x7FFF0000u);
        }
    }
    const int s = fp16_row_exponent(block_max_bits(m, &smax));
    uint16_t *dst = x16 + (size_t)blockIdx.x * H;
    for (int i = threadIdx.x * 8; i < H; i += 256 * 8) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const _Float16 lo = (_Float16)ldexpf(bf16_to_f32(w[k] & 0xFFFFu), -s);
            const _Float16 hi = (_Float16)ldexpf(bf16_to_f32(w[k] >> 16), -s);
            o[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *reinterpret_cast<uint4 *>(dst + i) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (threadIdx.x == 0) xexp[blockIdx.x] = s;
}

// ---------------------------------------------------------------------------
// h (fp32) -> fp16 rows scaled by 2^-s_r, the B operand of both formats' down
// GEMM.  One wave per route row, four rows per block; with NV > 0 the lane
// keeps its NV float4 (I = 256 * NV) in registers between the maximum and the
// conversion, otherwise it reads the row twice.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint2 f32x4_to_f16x4(float4 v, int s) {
    const _Float16 a = (_Float16)ldexpf(v.x, -s), b = (_Float16)ldexpf(v.y, -s);
    const _Float16 c = (_Float16)ldexpf(v.z, -s), d = (_Float16)ldexpf(v.w, -s);
    return make_uint2((uint32_t)__builtin_bit_cast(uint16_t, a) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16),
                      (uint32_t)__builtin_bit_cast(uint16_t, c) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, d) << 16));
}

__device__ __forceinline__ uint32_t abs_max_bits(float4 v, uint32_t m) {
    m = max(m, __float_as_uint(v.x) & 0x7FFFFFFFu);
    m = max(m, __float_as_uint(v.y) & 0x7FFFFFFFu);
    m = max(m, __float_as_uint(v.z) & 0x7FFFFFFFu);
    return max(m, __float_as_uint(v.w) & 0x7FFFFFFFu);
}

template <int NV>
__global__ __launch_bounds__(256) void hpack_kernel(const float *__restrict__ h, int I, int R,
                                                    uint16_t *__restrict__ h16,
                                                    int32_t *__restrict__ hexp) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= R) return;
    const float4 *row = reinterpret_cast<const float4 *>(h + (size_t)r * I);
    uint2 *dst = reinterpret_cast<uint2 *>(h16 + (size_t)r * I);
    uint32_t m = 0;
    if constexpr (NV > 0) {
        float4 v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = row[64 * i + lane];
#pragma unroll
        for (int i = 0; i < NV; ++i) m = abs_max_bits(v[i], m);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
        const int s = fp16_row_exponent(m);
#pragma unroll
        for (int i = 0; i < NV; ++i) dst[64 * i + lane] = f32x4_to_f16x4(v[i], s);
        if (lane == 0) hexp[r] = s;
    } else {
        for (int i = lane; i < I / 4; i += 64) m = abs_max_bits(row[i], m);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
        const int s = fp16_row_exponent(m);
        for (int i = lane; i < I / 4; i += 64) dst[i] = f32x4_to_f16x4(row[i], s);
        if (lane == 0) hexp[r] = s;
    }
}

// Book rows of K step S for one row group: Cb[i13] and (with the residual
// stage) Rb[i8].  c[0..2] code12, c[3..4] res, c[5] plane byte.
template <int S, bool RES>
__device__ __forceinline__ void gather_a(const uint32_t (&c)[6], const VqLds &lds, uint4 &cbv,
                                         uint4 &rbv) {
    uint32_t i13, i8;
    vq_indices<S>(c, i13, i8);
    cbv = lds.cb[i13];
    if (RES) rbv = lds.rb[i8];
}

// The A operand: Cb + Rb rounded once to fp16, or Cb alone.
template <bool RES>
__device__ __forceinline__ f16x8 a_operand(uint4 cbv, uint4 rbv) {
    return RES ? add_f16x8(cbv, rbv) : __builtin_bit_cast(f16x8, cbv);
}

// One sub-step (two K steps) of a wave: 2 x 4 groups x NTT token tiles MFMAs.
template <int U, int NTT, bool RES>
__device__ __forceinline__ void vq_substep(const uint32_t (&cr)[kVqGroups][6], const VqLds &lds,
                                           int slot, int lane, f32x4 (&acc)[kVqGroups][NTT]) {
    const int q = lane >> 4, n = lane & 15;
    uint4 cb0[kVqGroups], rb0[kVqGroups], cb1[kVqGroups], rb1[kVqGroups];
    uint4 b0[NTT], b1[NTT];
#pragma unroll
    for (int g = 0; g < kVqGroups; ++g) gather_a<2 * U, RES>(cr[g], lds, cb0[g], rb0[g]);
#pragma unroll
    for (int t = 0; t < NTT; ++t)
        b0[t] = *reinterpret_cast<const uint4 *>(lds.b[slot][0][q][16 * t + n]);
#pragma unroll
    for (int g = 0; g < kVqGroups; ++g) gather_a<2 * U + 1, RES>(cr[g], lds, cb1[g], rb1[g]);
#pragma unroll
    for (int t = 0; t < NTT; ++t)
        b1[t] = *reinterpret_cast<const uint4 *>(lds.b[slot][1][q][16 * t + n]);
    f16x8 a0[kVqGroups];
#pragma unroll
    for (int g = 0; g < kVqGroups; ++g) a0[g] = a_operand<RES>(cb0[g], rb0[g]);
#pragma unroll
    for (int t = 0; t < NTT; ++t)
#pragma unroll
        for (int g = 0; g < kVqGroups; ++g)
            acc[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a0[g], __builtin_bit_cast(f16x8, b0[t]), acc[g][t], 0, 0, 0);
    f16x8 a1[kVqGroups];
#pragma unroll
    for (int g = 0; g < kVqGroups; ++g) a1[g] = a_operand<RES>(cb1[g], rb1[g]);
#pragma unroll
    for (int t = 0; t < NTT; ++t)
#pragma unroll
        for (int g = 0; g < kVqGroups; ++g)
            acc[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a1[g], __builtin_bit_cast(f16x8, b1[t]), acc[g][t], 0, 0, 0);
}

// ---------------------------------------------------------------------------
// The grouped GEMM.  MODE 0: gate/up + SwiGLU, B = x16 (gathered through
// perm), out = h (fp32, [route position][I]).  MODE 1: down, B = h16 (route
// rows), out = y (fp32, [route position][H]).  Item = (expert, slice, chunk
// lane); MODE 0 slices are 256 gate rows with their up partners (wave w: gate
// groups 16b+2w, +1 and the two up partners), MODE 1 slices are 512 output
// rows (wave w: groups 32b+4w..+3, clamped past the end and never stored).
// NTT = 4: 64-token chunks over all E experts.  NTT = 1 (batches of at most
// 16 tokens, so at most 16 routes per expert): one 16-token chunk per item,
// and the items run over the active experts only (the list the small-batch
// routing writes), so no MFMA works on absent tokens or experts.  RES: the
// layer has the residual stage (VQ13R8) or not (VQ13).
// ---------------------------------------------------------------------------
template <int MODE, int NTT, bool RES>
__global__ __launch_bounds__(kVqThreads) void vq_prefill_kernel(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int K, int E,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ active, const uint16_t *__restrict__ bsrc,
    const int32_t *__restrict__ bexp, float *__restrict__ out) {
    constexpr bool kSmall = NTT == 1;
    constexpr int kChunk = 16 * NTT;                   // tokens per chunk
    constexpr int kLanes = kSmall ? 1 : kVqChunkLanes;  // items per (expert, slice)
    __shared__ __align__(16) VqLds lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;

    {  // both books -> LDS, once per block
        const uint4 *books = reinterpret_cast<const uint4 *>(packed);
        for (int i = tid; i < kVqEntries; i += kVqThreads) lds.cb[i] = books[i];
        if (RES)
            for (int i = tid; i < kVqResEntries; i += kVqThreads) lds.rb[i] = books[kVqEntries + i];
    }
    __syncthreads();

    const int NK = MODE == 0 ? H : I;        // reduction length
    const int NROW = MODE == 0 ? 2 * I : H;  // matrix rows
    const int NJ = NK / 256;                 // super-steps
    const int NS = 4 * NJ;                   // sub-steps
    const int nslice = MODE == 0 ? I / 256 : (H + 511) / 512;
    const int per_e = nslice * kLanes;
    const size_t nvec = (size_t)NROW * NK / 8;
    const size_t mat_off = MODE == 1 ? vq_down_offset((size_t)H, (size_t)I, RES) : 0;
    constexpr int kCodeLoads = (RES ? 3 : 2) * kVqGroups;  // loads per wave per super-step

    // blockIdx -> items: with E and the grid multiples of 8, the blocks of one
    // XCD (the dispatcher deals blocks round-robin over the 8 XCDs) take the
    // experts e = xcd (mod 8), so an expert's token rows stay in one L2.
    const bool by_xcd = !kSmall && (E & 7) == 0 && (gridDim.x & 7) == 0;
    const int xcd = by_xcd ? (int)(blockIdx.x & 7) : 0;
    const int first = by_xcd ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
    const int stride = by_xcd ? (int)(gridDim.x >> 3) : (int)gridDim.x;
    const int items = kSmall ? active[0] * per_e : by_xcd ? (E >> 3) * per_e : E * per_e;

    for (int it = first; it < items; it += stride) {
        const int e = kSmall ? active[1 + it / per_e] : by_xcd ? xcd + 8 * (it / per_e) : it / per_e;
        const int rest = it % per_e;
        const int slice = rest / kLanes, chl = rest % kLanes;
        const int p0 = offsets[e];
        const int ne = offsets[e + 1] - p0;
        const uint8_t *mat = packed + vq_books_bytes<RES>() + (size_t)e * expert_bytes + mat_off;
        const uint8_t *c12 = mat;
        const uint8_t *pln = c12 + nvec * 3 / 2;
        const uint8_t *res = pln + nvec / 8;
        const uint16_t *gain = reinterpret_cast<const uint16_t *>(res + (RES ? nvec : 0));

        int grp[kVqGroups];
#pragma unroll
        for (int g = 0; g < kVqGroups; ++g) {
            if (MODE == 0)
                grp[g] = (g < 2 ? 0 : I / 16) + 16 * slice + 2 * wave + (g & 1);
            else
                grp[g] = min(32 * slice + 4 * wave + g, H / 16 - 1);
        }

        for (int c0 = kChunk * chl; c0 < ne; c0 += kChunk * kLanes) {
            const int nt = min(kChunk, ne - c0);
            const int pr = p0 + c0 + min(lane, nt - 1);
            const uint16_t *brow =
                MODE == 0 ? bsrc + (size_t)(perm[pr] / K) * H : bsrc + (size_t)pr * I;

            f32x4 acc[kVqGroups][NTT];
#pragma unroll
            for (int g = 0; g < kVqGroups; ++g)
#pragma unroll
                for (int t = 0; t < NTT; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

            uint32_t cr[2][kVqGroups][6];
            auto issue_codes = [&](int slot, int J) {
#pragma unroll
                for (int g = 0; g < kVqGroups; ++g) {
                    const size_t tile = (size_t)grp[g] * NJ + J;
                    const u32x3 c = *reinterpret_cast<const u32x3 *>(c12 + tile * 768 + lane * 12);
                    uint2 r = make_uint2(0u, 0u);
                    if (RES) r = *reinterpret_cast<const uint2 *>(res + tile * 512 + lane * 8);
                    const uint32_t p = pln[tile * 64 + lane];
                    cr[slot][g][0] = c.x;
                    cr[slot][g][1] = c.y;
                    cr[slot][g][2] = c.z;
                    cr[slot][g][3] = r.x;
                    cr[slot][g][4] = r.y;
                    cr[slot][g][5] = p;
                }
            };
            // Wave w stages the (K step parity w/4, q = w%4) 1 KiB piece of each
            // sub-step: a 16-byte register load per lane, written to the LDS ring
            // one sub-step later.  (Register staging instead of global_load_lds:
            // the compiler cannot tell an LDS DMA target from the books and would
            // wait for every such copy in flight before each LDS read.)
            uint4 bstage;
            auto load_b = [&](int S) {
                const int J = S >> 2, u = S & 3, sb = wave >> 2, qq = wave & 3;
                bstage = *reinterpret_cast<const uint4 *>(brow + 256 * J + 64 * qq + 16 * u + 8 * sb);
            };
            auto store_b = [&](int S) {
                const int sb = wave >> 2, qq = wave & 3;
                *reinterpret_cast<uint4 *>(lds.b[S % kVqRing][sb][qq][lane]) = bstage;
            };

            vq_stage_barrier();  // the previous chunk's readers are done with the ring
            const int lastS = NS - 1, lastJ = NJ - 1;
            issue_codes(0, 0);
            load_b(0);
            vq_wait_vmcnt<0>();
            store_b(0);
            load_b(min(1, lastS));
            // Per sub-step S = 4J+u: the load of B(S+1) (issued at S-1, followed
            // by the 12 code loads when S-1 began a super-step) lands and goes to
            // LDS; the barrier publishes B(S); then B(S+2) and, at u = 0, the
            // codes of super-step J+1 are issued.  Loads are issued every step
            // (indices clamped past the end), so the wait counts are exact.
            for (int J0 = 0; J0 < NJ; J0 += 2) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int J = J0 + jj;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int S = 4 * J + u;
                        if (u == 1)
                            vq_wait_vmcnt<kCodeLoads>();
                        else
                            vq_wait_vmcnt<0>();
                        store_b(min(S + 1, lastS));
                        vq_stage_barrier();
                        load_b(min(S + 2, lastS));
                        if (u == 0) issue_codes(jj ^ 1, min(J + 1, lastJ));
                        if (J < NJ) {
                            const int slot = S % kVqRing;
                            if (u == 0) vq_substep<0, NTT, RES>(cr[jj], lds, slot, lane, acc);
                            if (u == 1) vq_substep<1, NTT, RES>(cr[jj], lds, slot, lane, acc);
                            if (u == 2) vq_substep<2, NTT, RES>(cr[jj], lds, slot, lane, acc);
                            if (u == 3) vq_substep<3, NTT, RES>(cr[jj], lds, slot, lane, acc);
                        }
                    }
                }
            }
            vq_wait_vmcnt<0>();  // the repeated tail loads land before the ring is reused

            // epilogue: lane holds rows 4q..4q+3 of each group for token 16t+n
#pragma unroll
            for (int t = 0; t < NTT; ++t) {
                const int m = 16 * t + n;
                if (m >= nt) continue;
                const int p = p0 + c0 + m;
                if (MODE == 0) {
                    const int xs = bexp[perm[p] / K];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int gg = grp[i], ug = grp[2 + i];
                        const uint2 gw = *reinterpret_cast<const uint2 *>(gain + 16 * gg + 4 * q);
                        const uint2 uw = *reinterpret_cast<const uint2 *>(gain + 16 * ug + 4 * q);
                        const uint32_t gb[4] = {gw.x & 0xFFFFu, gw.x >> 16, gw.y & 0xFFFFu, gw.y >> 16};
                        const uint32_t ub[4] = {uw.x & 0xFFFFu, uw.x >> 16, uw.y & 0xFFFFu, uw.y >> 16};
                        float hv[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float gv = ldexpf(acc[i][t][j] * f16_bits_to_f32(gb[j]), xs);
                            const float uv = ldexpf(acc[2 + i][t][j] * f16_bits_to_f32(ub[j]), xs);
                            hv[j] = silu_f32(gv) * uv;
                        }
                        *reinterpret_cast<float4 *>(out + (size_t)p * I + 16 * gg + 4 * q) =
                            make_float4(hv[0], hv[1], hv[2], hv[3]);
                    }
                } else {
                    const int hs = bexp[p];
#pragma unroll
                    for (int g = 0; g < kVqGroups; ++g) {
                        const int gg = 32 * slice + 4 * wave + g;
                        if (gg >= H / 16) continue;
                        const uint2 gw = *reinterpret_cast<const uint2 *>(gain + 16 * gg + 4 * q);
                        const uint32_t gb[4] = {gw.x & 0xFFFFu, gw.x >> 16, gw.y & 0xFFFFu, gw.y >> 16};
                        float yv[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            yv[j] = ldexpf(acc[g][t][j] * f16_bits_to_f32(gb[j]), hs);
                        *reinterpret_cast<float4 *>(out + (size_t)p * H + 16 * gg + 4 * q) =
                            make_float4(yv[0], yv[1], yv[2], yv[3]);
                    }
                }
            }
        }
    }
}

// Persistent grid: one block per CU (the books fill most of the LDS), a
// multiple of 8 when there is enough work so every XCD gets the same share.
static int vq_grid(int items) {
    int g = min(items, device_cu_count());
    if (g >= 8) g &= ~7;
    return max(g, 1);
}

template <int MODE, int NTT, bool RES>
static void vq_launch3(const Shape &s, int items, const uint8_t *packed, const Workspace &ws,
                       const uint16_t *bsrc, const int32_t *bexp, float *out, hipStream_t st) {
    vq_prefill_kernel<MODE, NTT, RES><<<vq_grid(items), kVqThreads, 0, st>>>(
        packed, s.expert_bytes, s.H, s.I, s.K, s.E, ws.offsets, ws.perm, ws.active, bsrc, bexp,
        out);
}

template <int MODE, int NTT>
static void vq_launch(const Shape &s, int items, const uint8_t *packed, const Workspace &ws,
                      const uint16_t *bsrc, const int32_t *bexp, float *out, hipStream_t st) {
    if (s.fmt == MOE_FMT_VQ13R8)
        vq_launch3<MODE, NTT, true>(s, items, packed, ws, bsrc, bexp, out, st);
    else
        vq_launch3<MODE, NTT, false>(s, items, packed, ws, bsrc, bexp, out, st);
}

hipError_t launch_hpack(const Shape &s, int R, const Workspace &ws, hipStream_t st) {
    const float *h = static_cast<const float *>(ws.h);
    const int nb = (R + 3) / 4;
    switch (s.I % 256 ? 0 : s.I / 256) {
        case 1: hpack_kernel<1><<<nb, 256, 0, st>>>(h, s.I, R, ws.h16, ws.hexp); break;
        case 2: hpack_kernel<2><<<nb, 256, 0, st>>>(h, s.I, R, ws.h16, ws.hexp); break;
        case 4: hpack_kernel<4><<<nb, 256, 0, st>>>(h, s.I, R, ws.h16, ws.hexp); break;
        case 8: hpack_kernel<8><<<nb, 256, 0, st>>>(h, s.I, R, ws.h16, ws.hexp); break;
        default: hpack_kernel<0><<<nb, 256, 0, st>>>(h, s.I, R, ws.h16, ws.hexp); break;
    }
    return hipGetLastError();
}

// Batches of at most kDecodeMaxTokens tokens (routed by the small-batch
// routing, which lists the active experts) take the one-tile variant.
hipError_t launch_vq_prefill_gateup(const Shape &s, int T, const uint16_t *x,
                                    const uint8_t *packed, const Workspace &ws, hipStream_t st) {
    vq_xpack_kernel<<<T, 256, 0, st>>>(x, s.H, ws.x16, ws.xexp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ns = s.I / 256;
    float *h = static_cast<float *>(ws.h);
    if (T <= kDecodeMaxTokens)
        vq_launch<0, 1>(s, min(T * s.K, s.E) * ns, packed, ws, ws.x16, ws.xexp, h, st);
    else
        vq_launch<0, 4>(s, s.E * ns * kVqChunkLanes, packed, ws, ws.x16, ws.xexp, h, st);
    return hipGetLastError();
}

hipError_t launch_vq_prefill_down(const Shape &s, int T, const uint8_t *packed,
                                  const Workspace &ws, hipStream_t st) {
    hipError_t e = launch_hpack(s, T * s.K, ws, st);
    if (e != hipSuccess) return e;
    const int ns = (s.H + 511) / 512;
    if (T <= kDecodeMaxTokens)
        vq_launch<1, 1>(s, min(T * s.K, s.E) * ns, packed, ws, ws.h16, ws.hexp, ws.y, st);
    else
        vq_launch<1, 4>(s, s.E * ns * kVqChunkLanes, packed, ws, ws.h16, ws.hexp, ws.y, st);
    return hipGetLastError();
}

}  // namespace bqmoe
