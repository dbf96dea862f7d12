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
// persistent (one per CU) and loop over (expert, row slice) items, so the
// books are loaded once per CU.  A lane gathers its A operand with two
// 16-byte LDS reads per K step.  Batches of more than 16 tokens run
// vq_grouped_kernel: an item covers 256 weight rows and all of the expert's
// tokens, 128 per pass (up to 8 token tiles per gathered A fragment), with
// the B operand streaming through an LDS ring of two 14 KiB slots (two K
// steps of up to 112 tokens each), and the index streams of a 256-column
// super-step going straight to registers one super-step ahead.  Batches of at
// most 16 tokens run vq_small_kernel over the active experts only: one
// 16-token tile per MFMA, index streams two super-steps ahead, B one
// super-step per LDS slot.
//
// Lane roles.  A = 16 weight rows x 32 K of fp16 (lane l: row l%16, K slice
// 8*(l/16)..+7).  In a VQ tile (16 rows x 256 columns) lane (n, q) owns the
// eight vectors of row n in columns 64q..64q+63 -- 12 contiguous code12 bytes,
// 8 res bytes and one plane byte at lane-contiguous offsets -- and K step s
// (0..7) of the super-step uses its vector s, i.e. columns 64q+8s..+7.  The B
// operand of lane (m, q) at K step s is therefore x[m][256J+64q+8s..+7].
#include <type_traits>

#include "vq_common.h"

namespace bqmoe {

constexpr int kVqWaves = 8;  // two per SIMD, sharing the books
constexpr int kVqThreads = kVqWaves * 64;

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

// ---------------------------------------------------------------------------
// The grouped GEMM for batches of more than 16 tokens.  Item = (expert,
// slice); a block covers 256 weight rows of its slice (wave w: row groups
// grp[0], grp[1]) for all of the expert's tokens, 128 per pass, so each
// gathered A fragment feeds up to 8 token tiles and an expert of up to 128
// tokens gathers its weights once.  MODE 0: slice = 128 gate rows and their
// up partners (wave w: gate group 8*slice + w and its up partner), B = x16
// gathered through perm, out = h; MODE 1: slice = 256 output rows (wave w:
// groups 16*slice + 2w, +1), B = h16 (route rows), out = y.  MT: the pass's
// 16-token tiles (a compile-time count, dispatched per pass; a lone tile runs
// as two).  B goes through an LDS ring of two 14 KiB slots, each two K steps
// of up to 112 tokens (4 pieces of 8 columns per K step and token) or one K
// step of 128; with both books that fills the 160 KiB.
// ---------------------------------------------------------------------------
constexpr int kVgGroups = 2;
constexpr int kVgChunk = 128;
constexpr int kVgPair = 112;              // tokens of a two-K-step slot
constexpr int kVgSlot = 2 * 4 * kVgPair;  // uint4 per slot: 14 KiB

struct VgLds {
    uint4 cb[kVqEntries];     // 128 KiB
    uint4 rb[kVqResEntries];  // 4 KiB
    uint4 b[2][kVgSlot];      // B ring: [K step][q][token] or [q][token], 8 fp16 each
};
static_assert(sizeof(VgLds) <= 160 * 1024, "the block's LDS");

// Book rows of K step S for the wave's G groups (issued, not waited for).
template <int S, bool RES, int G, class L>
__device__ __forceinline__ void vg_gather(const uint32_t (&cr)[G][6], const L &lds, uint4 (&cbv)[G],
                                          uint4 (&rbv)[G]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        uint32_t i13, i8;
        vq_indices<S>(cr[g], i13, i8);
        cbv[g] = lds.cb[i13];
        if (RES) rbv[g] = lds.rb[i8];
    }
}

template <bool RES, int G>
__device__ __forceinline__ void vg_form_a(const uint4 (&cbv)[G], const uint4 (&rbv)[G],
                                          f16x8 (&a)[G]) {
#pragma unroll
    for (int g = 0; g < G; ++g)
        a[g] = RES ? add_f16x8(cbv[g], rbv[g]) : __builtin_bit_cast(f16x8, cbv[g]);
}

// One K step of a wave: G groups x MT token tiles with the A operands a
// (gathered one K step earlier) and B from the LDS row bq (the step's piece
// q = lane/16, indexed by token).  The step's B reads go first, then the book
// gathers of the next K step SN (codes crn), then the MFMAs, which wait for
// the B reads only (LDS reads complete in order), so the gathers' latency
// hides under the MFMAs; a then becomes the next step's A.
template <int SN, int MT, bool RES, int G, class L>
__device__ __forceinline__ void vg_kstep(const uint32_t (&crn)[G][6], const L &lds, const uint4 *bq,
                                         int lane, f16x8 (&a)[G], f32x4 (&acc)[G][MT]) {
    const int n = lane & 15;
    uint4 bv[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) bv[t] = bq[16 * t + n];  // token 16t + n of the lane's piece
    uint4 cbv[G], rbv[G];
    vg_gather<SN, RES>(crn, lds, cbv, rbv);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int g = 0; g < G; ++g)
            acc[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[g], __builtin_bit_cast(f16x8, bv[t]),
                                                               acc[g][t], 0, 0, 0);
    vg_form_a<RES>(cbv, rbv, a);
}

// The same K step with its B operands already in registers (bv, read one K
// step earlier): it reads the next step's B from bqn into bv and gathers the
// next step's book rows before its MFMAs, which therefore wait for nothing.
template <int SN, int MT, bool RES, int G, class L>
__device__ __forceinline__ void vg_kstep_pf(const uint32_t (&crn)[G][6], const L &lds,
                                            const uint4 *bqn, int lane, f16x8 (&a)[G],
                                            uint4 (&bv)[MT], f32x4 (&acc)[G][MT]) {
    const int n = lane & 15;
    uint4 bvn[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) bvn[t] = bqn[16 * t + n];
    uint4 cbv[G], rbv[G];
    vg_gather<SN, RES>(crn, lds, cbv, rbv);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int g = 0; g < G; ++g)
            acc[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[g], __builtin_bit_cast(f16x8, bv[t]),
                                                               acc[g][t], 0, 0, 0);
    vg_form_a<RES>(cbv, rbv, a);
#pragma unroll
    for (int t = 0; t < MT; ++t) bv[t] = bvn[t];
}

// The index streams of one item's rows: the code12, plane and residual
// regions of its matrix and the wave's row groups.
struct VgCodes {
    const uint8_t *c12, *pln, *res;
    int grp[kVgGroups];
};

// One pass (at most 128 tokens from route position pc) over the item's rows
// (codes cur).  cr holds the codes of two super-steps; with have_first the
// previous pass already loaded this pass's super-step 0 into cr[0].  The code
// loads of the last super-step fetch the next pass's super-step 0 (codes nxt,
// when has_next) instead of repeating the last one, so no pass starts with a
// wait on HBM for its first codes.
template <int MODE, int MT, bool RES>
__device__ __forceinline__ void vg_pass(VgLds &lds, const VgCodes &cur, const uint16_t *gain,
                                        const VgCodes &nxt, bool has_next, bool have_first,
                                        uint32_t (&cr)[2][kVgGroups][6], int NJ, int H, int I,
                                        int K, int pc, int nt, int wave, int lane,
                                        const int32_t *__restrict__ perm,
                                        const uint16_t *__restrict__ bsrc,
                                        const int32_t *__restrict__ bexp,
                                        float *__restrict__ out, int8_t *__restrict__ yexp) {
    const int(&grp)[kVgGroups] = cur.grp;
    const int q = lane >> 4, n = lane & 15;
    // An LDS slot holds two K steps of up to 112 tokens ([K step][piece
    // q][token]) or, for passes of more tokens, one K step of 128 ([q][token]),
    // so most passes meet a barrier every two K steps.
    constexpr int KPS = MT <= 7 ? 2 : 1;            // K steps per slot
    constexpr int SPS = 8 / KPS;                    // slot steps per super-step
    constexpr int NL = KPS == 2 && MT > 4 ? 2 : 1;  // B loads per lane and slot step
    // B staging: wave w moves piece w%4 (columns 64q + 8s..+7 of K step s) of
    // K step w/4 of the slot for tokens lane and, with NL = 2, 64 + lane (two
    // K steps per slot), or of tokens 64(w/4) + lane (one); 16-byte register
    // loads, clamped to the pass's last token
    const int sq = wave & 3;
    const int kw = KPS == 2 ? wave >> 2 : 0;
    auto token_row = [&](int tok) {
        tok = min(tok, nt - 1);
        return MODE == 0 ? bsrc + (size_t)(perm[pc + tok] / K) * H : bsrc + (size_t)(pc + tok) * I;
    };
    const uint16_t *brow0 = token_row((KPS == 2 ? 0 : 64 * (wave >> 2)) + lane);
    const uint16_t *brow1 = NL == 2 ? token_row(64 + lane) : brow0;
    f32x4 acc[kVgGroups][MT];
#pragma unroll
    for (int g = 0; g < kVgGroups; ++g)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // super-step J's codes into cr[slot]; past the last super-step they are
    // the next pass's super-step 0 (or a repeat of the last one), chosen by
    // uniform selects, so every call issues the same loads
    auto issue_codes = [&](int slot, int J) {
        const bool to_next = J >= NJ && has_next;
        const VgCodes &src = to_next ? nxt : cur;
        const int Js = to_next ? 0 : min(J, NJ - 1);
#pragma unroll
        for (int g = 0; g < kVgGroups; ++g) {
            const size_t tile = (size_t)src.grp[g] * NJ + Js;
            vq_load_run<RES>(src.c12, src.res, src.pln, tile, lane, cr[slot][g]);
        }
    };
    auto slot_base = [&](int P) { return &lds.b[P & 1][0]; };
    auto load_to = [&](int P, uint4 &r0, uint4 &r1) {  // slot step P; K step S = KPS*P + kw
        const int S = KPS * P + kw;
        const int off = 256 * (S >> 3) + 64 * sq + 8 * (S & 7);
        r0 = *reinterpret_cast<const uint4 *>(brow0 + off);
        if constexpr (NL == 2) r1 = *reinterpret_cast<const uint4 *>(brow1 + off);
    };
    auto store_from = [&](int P, const uint4 &r0, const uint4 &r1) {
        uint4 *base = slot_base(P);
        if constexpr (KPS == 2) {
            base[(kw * 4 + sq) * kVgPair + lane] = r0;
            if constexpr (NL == 2)
                if (64 + lane < kVgPair) base[(kw * 4 + sq) * kVgPair + 64 + lane] = r1;
        } else {
            base[sq * kVgChunk + 64 * (wave >> 2) + lane] = r0;
        }
    };
    uint4 bst0, bst1;
    auto load_b = [&](int P) { load_to(P, bst0, bst1); };
    auto store_b = [&](int P) { store_from(P, bst0, bst1); };
    auto b_row = [&](int P, int kk) -> const uint4 * {  // K step kk of slot step P, piece q
        return slot_base(P) + (KPS == 2 ? (kk * 4 + q) * kVgPair : q * kVgChunk);
    };
    constexpr int kCodeLoads = (RES ? 3 : 2) * kVgGroups;

    vq_stage_barrier();  // the previous pass's readers are done with the ring
    const int NP = SPS * NJ, lastP = NP - 1;
    if (!have_first) issue_codes(0, 0);
    uint4 b00, b01, b10, b11;  // B of slot steps 0 and 1
    load_to(0, b00, b01);
    load_to(min(1, lastP), b10, b11);
    // The epilogue's operands travel with the first B rows: the gains of the
    // wave's two groups (rows 4q..4q+3) and, per token tile, the exponent of
    // the lane's token (MODE 0: through perm, so the exponent loads follow
    // once perm has landed; the first step's full wait covers them).
    const uint2 gw0 = *reinterpret_cast<const uint2 *>(gain + 16 * grp[0] + 4 * q);
    const uint2 gw1 = *reinterpret_cast<const uint2 *>(gain + 16 * grp[1] + 4 * q);
    int ex[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int pt = pc + min(16 * t + n, nt - 1);
        ex[t] = MODE == 0 ? perm[pt] : bexp[pt];
    }
    vq_wait_vmcnt<0>();
    if (MODE == 0)
#pragma unroll
        for (int t = 0; t < MT; ++t) ex[t] = bexp[ex[t] / K];
    store_from(0, b00, b01);
    store_from(1, b10, b11);
    load_b(min(2, lastP));
    vq_stage_barrier();  // slots 0 and 1 published
    f16x8 a[kVgGroups];  // the A operands of the current K step
    uint4 bv[MT];        // its B operands
    {
        const uint4 *bq = b_row(0, 0);
#pragma unroll
        for (int t = 0; t < MT; ++t) bv[t] = bq[16 * t + n];
        uint4 cbv[kVgGroups], rbv[kVgGroups];
        vg_gather<0, RES>(cr[0], lds, cbv, rbv);
        vg_form_a<RES>(cbv, rbv, a);
    }
    // Per slot step P = SPS*J + p, before its last K step: a barrier publishes
    // slot step P+1 (stored at P-1) and, every wave having read all of slot
    // step P's B (each K step reads the next one's), frees slot P's buffer,
    // where B(P+2) (issued at P-1, followed by the code loads of super-step
    // J+1 when P-1 began super-step J) goes once it lands; then B(P+3) and, at
    // p = 0, the codes of super-step J+1 are issued, and the last K step reads
    // slot step P+1's first B.  Loads are issued every step (indices clamped
    // past the end), so the wait counts are exact.
    for (int J0 = 0; J0 < NJ; J0 += 2) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int J = J0 + jj;
#pragma unroll
            for (int p = 0; p < SPS; ++p) {
                const int P = SPS * J + p;
#pragma unroll
                for (int kk = 0; kk < KPS; ++kk) {
                    if (kk == KPS - 1) {
                        vq_stage_barrier();
                        if (p == 1)
                            vq_wait_vmcnt<kCodeLoads>();
                        else
                            vq_wait_vmcnt<0>();
                        store_b(min(P + 2, lastP));
                        load_b(min(P + 3, lastP));
                        if (p == 0) issue_codes(jj ^ 1, J + 1);
                    }
                    if (J < NJ) {
                        // K step s; the next one's B: this slot step's, or
                        // after the last the next slot step's first; its
                        // codes: this super-step's, or at s = 7 the next
                        // super-step's (issued at p = 0, landed by p = 2;
                        // past the end they repeat the last)
                        const int s = KPS * p + kk;
                        const uint4 *bqn = kk < KPS - 1 ? b_row(P, kk + 1) : b_row(P + 1, 0);
                        if (s == 0) vg_kstep_pf<1, MT, RES>(cr[jj], lds, bqn, lane, a, bv, acc);
                        if (s == 1) vg_kstep_pf<2, MT, RES>(cr[jj], lds, bqn, lane, a, bv, acc);
                        if (s == 2) vg_kstep_pf<3, MT, RES>(cr[jj], lds, bqn, lane, a, bv, acc);
                        if (s == 3) vg_kstep_pf<4, MT, RES>(cr[jj], lds, bqn, lane, a, bv, acc);
                        if (s == 4) vg_kstep_pf<5, MT, RES>(cr[jj], lds, bqn, lane, a, bv, acc);
                        if (s == 5) vg_kstep_pf<6, MT, RES>(cr[jj], lds, bqn, lane, a, bv, acc);
                        if (s == 6) vg_kstep_pf<7, MT, RES>(cr[jj], lds, bqn, lane, a, bv, acc);
                        if (s == 7) vg_kstep_pf<0, MT, RES>(cr[jj ^ 1], lds, bqn, lane, a, bv, acc);
                    }
                }
            }
        }
    }
    vq_wait_vmcnt<0>();  // the repeated tail loads land before the ring is reused

    // epilogue: lane holds rows 4q..4q+3 of each group for token 16t+n
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int m = 16 * t + n;
        if (m >= nt) continue;
        const int p = pc + m;
        if (MODE == 0) {
            const int xs = ex[t];
            const int gg = grp[0];
            const uint2 gw = gw0, uw = gw1;
            const uint32_t gb[4] = {gw.x & 0xFFFFu, gw.x >> 16, gw.y & 0xFFFFu, gw.y >> 16};
            const uint32_t ub[4] = {uw.x & 0xFFFFu, uw.x >> 16, uw.y & 0xFFFFu, uw.y >> 16};
            float hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float gv = ldexpf(acc[0][t][j] * f16_bits_to_f32(gb[j]), xs);
                const float uv = ldexpf(acc[1][t][j] * f16_bits_to_f32(ub[j]), xs);
                hv[j] = silu_f32(gv) * uv;
            }
            *reinterpret_cast<float4 *>(out + (size_t)p * I + 16 * gg + 4 * q) =
                make_float4(hv[0], hv[1], hv[2], hv[3]);
        } else {
            const int hs = ex[t];
#pragma unroll
            for (int g = 0; g < kVgGroups; ++g) {
                const int gg = grp[g];
                if (gg >= H / 16) continue;  // clamped duplicate past the last group
                if (g == 1 && grp[1] == grp[0]) continue;
                const uint2 gw = g == 0 ? gw0 : gw1;
                const uint32_t gb[4] = {gw.x & 0xFFFFu, gw.x >> 16, gw.y & 0xFFFFu, gw.y >> 16};
                float yv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) yv[j] = ldexpf(acc[g][t][j] * f16_bits_to_f32(gb[j]), hs);
                store_y16x4(reinterpret_cast<uint16_t *>(out), yexp, (size_t)p, H, 16 * gg + 4 * q, yv);
            }
        }
    }
}

template <int MODE, bool RES>
__global__ __launch_bounds__(kVqThreads) void vq_grouped_kernel(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int K, int E,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const uint16_t *__restrict__ bsrc, const int32_t *__restrict__ bexp,
    float *__restrict__ out, int8_t *__restrict__ yexp) {
    __shared__ __align__(16) VgLds lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int nslice = MODE == 0 ? I / 128 : (H + 255) / 256;
    const size_t nvec = (size_t)NROW * NK / 8;
    const size_t mat_off = MODE == 1 ? vq_down_offset((size_t)H, (size_t)I, RES) : 0;
    // blockIdx -> items: with E and the grid multiples of 8, the blocks of one
    // XCD take the experts e = xcd (mod 8), so an expert's rows stay in one L2
    const bool by_xcd = (E & 7) == 0 && (gridDim.x & 7) == 0;
    const int xcd = by_xcd ? (int)(blockIdx.x & 7) : 0;
    const int first = by_xcd ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
    const int stride = by_xcd ? (int)(gridDim.x >> 3) : (int)gridDim.x;
    const int items = by_xcd ? (E >> 3) * nslice : E * nslice;

    // The block's passes in order: items it = first, first + stride, ...
    // (empty experts skipped), chunks of kVgChunk tokens within an item.  Each
    // pass is told the next one's index streams, whose first codes it loads.
    struct Item {
        int p0, ne;
        const uint16_t *gain;
        VgCodes codes;
    };
    auto item_at = [&](int it, Item &o) {  // false for an empty expert
        const int e = by_xcd ? xcd + 8 * (it / nslice) : it / nslice;
        const int slice = it % nslice;
        o.p0 = offsets[e];
        o.ne = offsets[e + 1] - o.p0;
        const uint8_t *mat = packed + vq_books_bytes<RES>() + (size_t)e * expert_bytes + mat_off;
        o.codes.c12 = mat;
        o.codes.pln = mat + nvec * 3 / 2;
        o.codes.res = o.codes.pln + nvec / 8;
        o.gain = reinterpret_cast<const uint16_t *>(o.codes.res + (RES ? nvec : 0));
        if (MODE == 0) {
            o.codes.grp[0] = 8 * slice + wave;          // gate group
            o.codes.grp[1] = I / 16 + 8 * slice + wave;  // its up partner
        } else {
            o.codes.grp[0] = min(16 * slice + 2 * wave, H / 16 - 1);
            o.codes.grp[1] = min(16 * slice + 2 * wave + 1, H / 16 - 1);
        }
        return o.ne > 0;
    };
    uint32_t cr[2][kVgGroups][6];
    Item cur, nxt;
    int it = first;
    while (it < items && !item_at(it, cur)) it += stride;
    int c0 = 0;
    bool have_first = false;
    while (it < items) {
        int it2 = it, c2 = c0 + kVgChunk;
        bool has_next = true;
        if (c2 < cur.ne) {
            nxt = cur;
        } else {
            c2 = 0;
            it2 = it + stride;
            while (it2 < items && !item_at(it2, nxt)) it2 += stride;
            has_next = it2 < items;
            if (!has_next) nxt = cur;
        }
        const int nt = min(kVgChunk, cur.ne - c0);
        const int mt = (nt + 15) / 16;
        auto pass = [&](auto mtc) {
            vg_pass<MODE, decltype(mtc)::value, RES>(lds, cur.codes, cur.gain, nxt.codes, has_next,
                                                     have_first, cr, NJ, H, I, K, cur.p0 + c0, nt,
                                                     wave, lane, perm, bsrc, bexp, out, yexp);
        };
        switch (mt) {
            case 1:
            case 2: pass(std::integral_constant<int, 2>{}); break;
            case 3: pass(std::integral_constant<int, 3>{}); break;
            case 4: pass(std::integral_constant<int, 4>{}); break;
            case 5: pass(std::integral_constant<int, 5>{}); break;
            case 6: pass(std::integral_constant<int, 6>{}); break;
            case 7: pass(std::integral_constant<int, 7>{}); break;
            default: pass(std::integral_constant<int, 8>{}); break;
        }
        have_first = has_next;
        it = it2;
        c0 = c2;
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// Batches of at most 16 tokens (so at most 16 routes per expert), over the
// active experts that the small-batch routing lists.  Each wave owns G row
// groups: 4 for VQ13 layers, 2 with the residual stage (whose index streams
// and gathers would not fit in registers for 4).  Item = (active expert,
// slice): MODE 0 slice = 64G gate rows and their up partners (wave w: gate
// groups (G/2)(8*slice + w) + i, i < G/2, and their up partners), MODE 1 slice
// = 128G output rows (wave w: groups G(8*slice + w) + g, clamped past the end
// and never stored).  One 16-token tile, so the index streams carry the kernel:
// they go to registers two super-steps ahead (a ring of four, so a pass's
// last two super-steps can load the next pass's first two), and B, one
// super-step of 16 tokens (8 KiB), goes through two LDS slots, so a pass
// meets one barrier per super-step.  The K steps run as in the grouped GEMM
// (the next step's book rows gathered under the current step's MFMAs).
// ---------------------------------------------------------------------------
template <bool RES>
constexpr int vs_groups() { return RES ? 2 : 4; }

struct VsLds {
    uint4 cb[kVqEntries];     // 128 KiB
    uint4 rb[kVqResEntries];  // 4 KiB
    uint4 b[2][8][4][16];     // [slot][K step][piece q][token]: 8 fp16 each
};

template <int MODE, bool RES>
__global__ __launch_bounds__(kVqThreads) void vq_small_kernel(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int K,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ active, const uint16_t *__restrict__ bsrc,
    const int32_t *__restrict__ bexp, float *__restrict__ out, int8_t *__restrict__ yexp) {
    constexpr int G = vs_groups<RES>();
    constexpr int GG = G / 2;  // gate groups per wave (MODE 0)
    __shared__ __align__(16) VsLds lds;
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
    const int nslice = MODE == 0 ? I / (128 * GG) : (H + 128 * G - 1) / (128 * G);
    const size_t nvec = (size_t)NROW * NK / 8;
    const size_t mat_off = MODE == 1 ? vq_down_offset((size_t)H, (size_t)I, RES) : 0;
    constexpr int kCodeLoads = (RES ? 3 : 2) * G;  // loads per wave per super-step
    const int items = active[0] * nslice;

    // The block's passes in order: items it = blockIdx.x, +gridDim.x, ...
    // (every listed expert has tokens), chunks of 16 tokens within an item.
    struct Item {
        int p0, ne, slice;
        const uint16_t *gain;
        const uint8_t *c12, *pln, *res;
        int grp[G];
    };
    auto item_at = [&](int it, Item &o) {
        const int e = active[1 + it / nslice];
        const int slice = it % nslice;
        o.slice = slice;
        o.p0 = offsets[e];
        o.ne = offsets[e + 1] - o.p0;
        o.c12 = packed + vq_books_bytes<RES>() + (size_t)e * expert_bytes + mat_off;
        o.pln = o.c12 + nvec * 3 / 2;
        o.res = o.pln + nvec / 8;
        o.gain = reinterpret_cast<const uint16_t *>(o.res + (RES ? nvec : 0));
#pragma unroll
        for (int g = 0; g < G; ++g)
            o.grp[g] = MODE == 0 ? (g < GG ? 0 : I / 16) + GG * (8 * slice + wave) + g % GG
                                 : min(G * (8 * slice + wave) + g, H / 16 - 1);
    };
    // super-step J's codes sit in cr[J % 4]; when NJ is a multiple of 4 the
    // last two super-steps of a pass load the next pass's first two into
    // slots 0 and 1
    const bool chain = (NJ & 3) == 0;
    uint32_t cr[4][G][6];
    int it = (int)blockIdx.x;
    if (it >= items) return;
    Item cur, nxt;
    item_at(it, cur);
    int c0 = 0;
    bool have_first = false;
    while (true) {
        int it2 = it, c2 = c0 + 16;
        bool has_next = true;
        if (c2 < cur.ne) {
            nxt = cur;
        } else {
            c2 = 0;
            it2 = it + (int)gridDim.x;
            has_next = it2 < items;
            if (has_next) item_at(it2, nxt);
            else nxt = cur;
        }
        const bool pf = has_next && chain;
        {
            const int(&grp)[G] = cur.grp;
            const uint16_t *gain = cur.gain;
            const int nt = min(16, cur.ne - c0);
            const int pc = cur.p0 + c0;
            // lane (n, q) stages piece q of token n (clamped to the pass) for
            // K step `wave` of each super-step, and its epilogue covers token n
            const int tok = min(n, nt - 1);
            const uint16_t *brow = MODE == 0 ? bsrc + (size_t)(perm[pc + tok] / K) * H
                                             : bsrc + (size_t)(pc + tok) * I;
            // super-step J's codes into cr[slot]; past the last super-step
            // they are the next pass's (with pf) or the last one again, chosen
            // by uniform selects, so every call issues the same loads
            auto issue_codes = [&](int slot, int J) {
                const bool to_next = J >= NJ && pf;
                const Item &src = to_next ? nxt : cur;
                const int Js = to_next ? J - NJ : min(J, NJ - 1);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const size_t tile = (size_t)src.grp[g] * NJ + Js;
                    vq_load_run<RES>(src.c12, src.res, src.pln, tile, lane, cr[slot][g]);
                }
            };
            uint4 bst;
            auto load_b = [&](int J) {
                bst = *reinterpret_cast<const uint4 *>(brow + 256 * min(J, NJ - 1) + 64 * q + 8 * wave);
            };
            auto store_b = [&](int J) { lds.b[J & 1][wave][q][n] = bst; };
            f32x4 acc[G][1];
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g][0] = f32x4{0.f, 0.f, 0.f, 0.f};

            vq_stage_barrier();  // the previous pass's readers are done with the ring
            if (!have_first) {
                issue_codes(0, 0);
                issue_codes(1, 1);
            }
            load_b(0);
            // the epilogue's operands: the groups' gains (rows 4q..4q+3) and
            // the exponent of token n (MODE 0: through perm)
            uint2 gw[G];
#pragma unroll
            for (int g = 0; g < G; ++g)
                gw[g] = *reinterpret_cast<const uint2 *>(gain + 16 * grp[g] + 4 * q);
            int ex = MODE == 0 ? perm[pc + tok] : bexp[pc + tok];
            vq_wait_vmcnt<0>();
            if (MODE == 0) ex = bexp[ex / K];
            store_b(0);
            load_b(1);
            f16x8 a[G];  // the A operands of the current K step
            {
                uint4 cbv[G], rbv[G];
                vg_gather<0, RES>(cr[0], lds, cbv, rbv);
                vg_form_a<RES>(cbv, rbv, a);
            }
            // Per super-step J: the barrier publishes B(J) (stored at J-1) and,
            // every wave being done with step J-1, frees the other slot; B(J+1)
            // (issued at J-1, ahead of the codes of J+1) lands and goes there;
            // then B(J+2) and the codes of J+2 are issued.  The codes of J+1
            // are first needed by the gathers of the step's last K step.
            for (int J0 = 0; J0 < NJ; J0 += 4) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int J = J0 + jj;
                    vq_stage_barrier();
                    vq_wait_vmcnt<kCodeLoads>();
                    store_b(J + 1);
                    load_b(J + 2);
                    issue_codes((jj + 2) & 3, J + 2);
                    if (J < NJ) {
                        const uint4 *bs = &lds.b[J & 1][0][q][0];  // K step s at bs + 64 s
                        const uint32_t(&c)[G][6] = cr[jj];
                        vg_kstep<1, 1, RES>(c, lds, bs, lane, a, acc);
                        vg_kstep<2, 1, RES>(c, lds, bs + 64, lane, a, acc);
                        vg_kstep<3, 1, RES>(c, lds, bs + 128, lane, a, acc);
                        vg_kstep<4, 1, RES>(c, lds, bs + 192, lane, a, acc);
                        vg_kstep<5, 1, RES>(c, lds, bs + 256, lane, a, acc);
                        vg_kstep<6, 1, RES>(c, lds, bs + 320, lane, a, acc);
                        vg_kstep<7, 1, RES>(c, lds, bs + 384, lane, a, acc);
                        vg_kstep<0, 1, RES>(cr[(jj + 1) & 3], lds, bs + 448, lane, a, acc);
                    }
                }
            }
            // the B loads past the end have landed; the codes issued last (the
            // next pass's, with pf) may stay in flight through the epilogue
            vq_wait_vmcnt<kCodeLoads>();

            // epilogue: lane holds rows 4q..4q+3 of each group for token n
            if (n < nt) {
                const int p = pc + n;
                if (MODE == 0) {
#pragma unroll
                    for (int i = 0; i < GG; ++i) {
                        const uint2 g2 = gw[i], u2 = gw[GG + i];
                        const uint32_t gb[4] = {g2.x & 0xFFFFu, g2.x >> 16, g2.y & 0xFFFFu, g2.y >> 16};
                        const uint32_t ub[4] = {u2.x & 0xFFFFu, u2.x >> 16, u2.y & 0xFFFFu, u2.y >> 16};
                        float hv[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float gv = ldexpf(acc[i][0][j] * f16_bits_to_f32(gb[j]), ex);
                            const float uv = ldexpf(acc[GG + i][0][j] * f16_bits_to_f32(ub[j]), ex);
                            hv[j] = silu_f32(gv) * uv;
                        }
                        *reinterpret_cast<float4 *>(out + (size_t)p * I + 16 * grp[i] + 4 * q) =
                            make_float4(hv[0], hv[1], hv[2], hv[3]);
                    }
                } else {
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const int gg = G * (8 * cur.slice + wave) + g;
                        if (gg >= H / 16) continue;  // clamped duplicate past the last group
                        const uint2 g2 = gw[g];
                        const uint32_t gb[4] = {g2.x & 0xFFFFu, g2.x >> 16, g2.y & 0xFFFFu, g2.y >> 16};
                        float yv[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            yv[j] = ldexpf(acc[g][0][j] * f16_bits_to_f32(gb[j]), ex);
                        store_y16x4(reinterpret_cast<uint16_t *>(out), yexp, (size_t)p, H,
                                    16 * gg + 4 * q, yv);
                    }
                }
            }
        }
        if (!has_next) break;
        have_first = pf;
        it = it2;
        c0 = c2;
        cur = nxt;
    }
}

// Persistent grid: one block per CU (the books fill most of the LDS), a
// multiple of 8 when there is enough work so every XCD gets the same share.
static int vq_grid(int items) {
    int g = min(items, device_cu_count());
    if (g >= 8) g &= ~7;
    return max(g, 1);
}

template <int MODE>
static void vg_launch(const Shape &s, const uint8_t *packed, const Workspace &ws,
                      const uint16_t *bsrc, const int32_t *bexp, float *out, hipStream_t st) {
    const int nslice = MODE == 0 ? s.I / 128 : (s.H + 255) / 256;
    const int grid = vq_grid(s.E * nslice);
    if (s.fmt == MOE_FMT_VQ13R8)
        vq_grouped_kernel<MODE, true><<<grid, kVqThreads, 0, st>>>(
            packed, s.expert_bytes, s.H, s.I, s.K, s.E, ws.offsets, ws.perm, bsrc, bexp, out,
            ws.yexp);
    else
        vq_grouped_kernel<MODE, false><<<grid, kVqThreads, 0, st>>>(
            packed, s.expert_bytes, s.H, s.I, s.K, s.E, ws.offsets, ws.perm, bsrc, bexp, out,
            ws.yexp);
}

// items: at most min(T*K, E) active experts times the slices per expert
template <int MODE, bool RES>
static void vs_launch(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                      const uint16_t *bsrc, const int32_t *bexp, float *out, hipStream_t st) {
    constexpr int G = vs_groups<RES>();
    const int ns = MODE == 0 ? s.I / (64 * G) : (s.H + 128 * G - 1) / (128 * G);
    vq_small_kernel<MODE, RES><<<vq_grid(min(T * s.K, s.E) * ns), kVqThreads, 0, st>>>(
        packed, s.expert_bytes, s.H, s.I, s.K, ws.offsets, ws.perm, ws.active, bsrc, bexp, out,
        ws.yexp);
}

template <int MODE>
static void vs_launch(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                      const uint16_t *bsrc, const int32_t *bexp, float *out, hipStream_t st) {
    if (s.fmt == MOE_FMT_VQ13R8)
        vs_launch<MODE, true>(s, T, packed, ws, bsrc, bexp, out, st);
    else
        vs_launch<MODE, false>(s, T, packed, ws, bsrc, bexp, out, st);
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
// routing, which lists the active experts) take vq_small_kernel.
hipError_t launch_vq_prefill_gateup(const Shape &s, int T, const uint16_t *x,
                                    const uint8_t *packed, const Workspace &ws, hipStream_t st) {
    vq_xpack_kernel<<<T, 256, 0, st>>>(x, s.H, ws.x16, ws.xexp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    float *h = static_cast<float *>(ws.h);
    if (T <= kDecodeMaxTokens)
        vs_launch<0>(s, T, packed, ws, ws.x16, ws.xexp, h, st);
    else
        vg_launch<0>(s, packed, ws, ws.x16, ws.xexp, h, st);
    return hipGetLastError();
}

hipError_t launch_vq_prefill_down(const Shape &s, int T, const uint8_t *packed,
                                  const Workspace &ws, hipStream_t st) {
    hipError_t e = launch_hpack(s, T * s.K, ws, st);
    if (e != hipSuccess) return e;
    if (T <= kDecodeMaxTokens)
        vs_launch<1>(s, T, packed, ws, ws.h16, ws.hexp, reinterpret_cast<float *>(ws.y16), st);
    else
        vg_launch<1>(s, packed, ws, ws.h16, ws.hexp, reinterpret_cast<float *>(ws.y16), st);
    return hipGetLastError();
}

}  // namespace bqmoe
