// prefill.hip -- large-batch expert kernels for MXFP4 experts on gfx950: a
// grouped GEMM per expert on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulators.
//
// The micro-batch matters (a 512-token micro-batch leaves much of prefill
// unused because each of the 256 experts then sees too few tokens per matmul
// -- TrevorJS GGUF card, "Speed"): a block owns one slice of one expert's
// weights and multiplies it with every token routed to that expert, so the
// weights leave HBM once.
//
// Pipeline of a block (four waves, one per SIMD, one block per CU): the
// kernel is bound by streaming weights from HBM, so what matters is the number
// of weight bytes in flight.  Each step (one K super-step of 128 columns) every
// wave issues, in a fixed order, its share of the B operand stage and of the
// scales (global_load_lds straight into a 4-deep LDS ring) and then its own 8
// row groups of packed code tiles (1 KiB wave loads into a 4-deep register
// ring).  Because a wave's load counter completes in issue order, waiting
// until no more than "the loads of the steps after J" are outstanding means
// step J has landed; one barrier then publishes the B stage.  Waves are wide
// (8 row groups x 128 tokens, 256 fp32 accumulators in AGPRs, using the
// 512-register budget of one wave per SIMD) so that a step's MFMA work covers
// the memory latency three steps deep.  Weights are dequantised to bf16 in
// registers (every E2M1 value times an in-range E8M0 scale is a bf16 value, so
// the A operand and the products are exact) and accumulated in fp32.
//
// MFMA roles: A = 16 weight rows x 32 K (lane l: row l%16, K slice
// 8*(l/16)..+7), B = 32 K x 16 tokens, D[row][token].  Lane (n, q) of a wave
// holds the 16 code bytes of tile column 4J+q of its row n: K columns
// 128J+32q .. +31; MFMA step s uses bytes 4s..4s+3 (columns 128J+32q+8s..+7),
// and the B operand of lane (m, q) at step s is x[m][128J+32q+8s..+7].
//
// SwiGLU is fused into the gate/up epilogue in fp32.  Expert intermediates
// exceed fp16's range (TrevorJS card, "Recipe"; benthecarman EXL3 card,
// "Bitrate") and a single bf16 is too coarse for the down projection, so h is
// stored as hi = bf16(h), lo = bf16(h - hi) and the down GEMM runs both
// halves through the MFMA into the same fp32 accumulators.
#include "moe_internal.h"

namespace bqmoe {

constexpr int kPfWaves = 4;    // one per SIMD; each owns 8 weight row groups
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kPfRing = 3;     // steps in flight (register code ring, LDS B ring)
constexpr int kPfGroups = 8;   // row groups per wave
constexpr int kPfBlockGroups = kPfWaves * kPfGroups;

// B operand stage: [s][q][m][8 bf16] for a 128-column super-step, m = token.
template <int TOK>
struct BStage {
    uint8_t b[4][4][TOK][16];
};

// Scales of a block's 32 row groups for one super-step: [group][tile q][row n].
struct ScaleStage {
    uint8_t s[kPfBlockGroups][64];
};

// Wait until at most N vector-memory loads of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, other counters open).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier publishing a B stage.  Each wave has waited (on its own load count)
// for its copies into that stage; the barrier also needs its LDS reads of the
// stage about to be refilled to be done.  An LDS fence here would wait for
// every load still in flight and collapse the pipeline.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt open
    __builtin_amdgcn_s_barrier();
}

// One 1 KiB wave copy global -> LDS: lane l moves 16 bytes from src (its own
// address) to dst + 16*l.
__device__ __forceinline__ void copy_lds16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// blockIdx -> (expert, block): the blocks of one expert land on one XCD (the
// dispatcher deals workgroups round-robin over the 8 XCDs), so the expert's
// token rows and shared weight slices are re-read from that XCD's L2.
__device__ __forceinline__ void map_expert_block(int bid, int E, int NB, int *e, int *blk) {
    if ((E & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        *e = xcd + 8 * (slot / NB);
        *blk = slot % NB;
    } else {
        *e = bid / NB;
        *blk = bid % NB;
    }
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// This wave's copies into one B stage (64 tokens): (s, q) slices wave,
// wave+4, wave+8, wave+12, 1 KiB each.  row: the lane's token row (element
// pointer into a [*, K] bf16 matrix).
__device__ __forceinline__ void load_bstage(BStage<64> *dst, const uint16_t *row, int J, int wave) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = wave + 4 * i;
        const int s = c >> 2, q = c & 3;
        copy_lds16(row + 128 * J + 32 * q + 8 * s, dst->b[s][q][0]);
    }
}

// Row groups of a block.  A block owns 32 row groups; group index i of the
// block maps to a row group of the matrix through BlockGroups::at(i).
struct BlockGroups {
    int mode;   // 0: gate/up (i < 16 gate 16b+i, else up partner), 1: down (32b+i)
    int blk;
    int limit;  // gate groups (mode 0) or row groups (mode 1)
    __device__ __forceinline__ int at(int i) const {
        if (mode == 0) {
            const int g = min(16 * blk + (i & 15), limit - 1);
            return i < 16 ? g : limit + g;
        }
        return min(32 * blk + i, limit - 1);
    }
};

// Block group index of the wave's group g: gate/up waves take gate 4w..4w+3
// and their up partners 16+4w..; down waves take 8w..8w+7.
__device__ __forceinline__ int wave_group(int mode, int wave, int g) {
    return mode == 0 ? (g < 4 ? 4 * wave + g : 16 + 4 * wave + (g - 4)) : 8 * wave + g;
}

// Scales of step J for the block's 32 groups: waves 0 and 1 copy 16 groups each
// (lane l: block group 16*wave + l/4, tile 4J + l%4).
__device__ __forceinline__ void load_scales(ScaleStage *dst, const uint8_t *scales,
                                            const BlockGroups &bg, size_t kt, int J, int wave,
                                            int lane) {
    const int g = bg.at(16 * wave + (lane >> 2));
    copy_lds16(scales + ((size_t)g * kt + 4 * J + (lane & 3)) * 16, dst->s[16 * wave]);
}

// MFMAs of one super-step for a wave: 4 K steps x 8 row groups x 4 token
// tiles; NB B operands per tile (1: x, 2: h hi and lo).  Operands are double
// buffered: while the MFMAs of K step s run, the wave reads step s+1's B
// operands from LDS and dequantises its A operands, interleaved one VALU op
// per MFMA (or per two for NB = 2) so the matrix core never waits for them.
// Token tiles past the chunk's tokens multiply clamped duplicate rows whose
// results are never stored; a branch per tile would expose an LDS round trip.
template <int NB>
__device__ __forceinline__ void mfma_step(const uint4 (&code)[kPfGroups], const ScaleStage *sc,
                                          const BStage<64> *b0, const BStage<64> *b1, int mode,
                                          int wave, int lane, f32x4 (&acc)[kPfGroups][4]) {
    const int q = lane >> 4, n = lane & 15;
    float scale[kPfGroups];
#pragma unroll
    for (int g = 0; g < kPfGroups; ++g)
        scale[g] = e8m0_to_f32(sc->s[wave_group(mode, wave, g)][q * 16 + n]);
    bf16x8 a[2][kPfGroups];
    bf16x8 bv[2][NB][4];
    auto load_b = [&](int buf, int s) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bv[buf][0][t] = *reinterpret_cast<const bf16x8 *>(b0->b[s][q][16 * t + n]);
            if (NB == 2) bv[buf][NB - 1][t] = *reinterpret_cast<const bf16x8 *>(b1->b[s][q][16 * t + n]);
        }
    };
    auto dequant = [&](int buf, int s) {
#pragma unroll
        for (int g = 0; g < kPfGroups; ++g) {
            const uint4 c = code[g];
            const uint32_t d = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
            a[buf][g] = fp4x8_to_bf16x8(d, scale[g]);
        }
    };
    load_b(0, 0);
    dequant(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int cur = s & 1;
        if (s < 3) {
            load_b(cur ^ 1, s + 1);
            dequant(cur ^ 1, s + 1);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int g = 0; g < kPfGroups; ++g)
                    acc[g][t] = mfma_bf16(a[cur][g], bv[cur][nb][t], acc[g][t]);
        if (s < 3) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * NB, 0);  // LDS reads first
#pragma unroll
            for (int i = 0; i < 4 * kPfGroups; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // dequant op
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The pipeline: per step J, every wave issues [its B copies, its scale copy
// (waves 0-1), its 8 code loads]; steps run kPfRing-1 ahead.  C = loads per
// step of this wave, NB = B operands per step (1: x, 2: h hi and lo).
//
// The loop is branch-free around loads: past the last step the issue repeats
// the last step's addresses (cache hits, never consumed), so every wave always
// has exactly kPfRing-1 steps in flight at a wait and the compiler's own
// load-counter tracking stays exact.  A conditional issue makes it fall back
// to waiting for every load in flight, which serialises the stream.
template <int C, int NB>
__device__ __forceinline__ void pipeline(const uint8_t *codes, const uint8_t *scales, size_t kt,
                                         int nsuper, const BlockGroups &bg, int mode,
                                         BStage<64> (*bring)[2], ScaleStage *scring,
                                         const uint16_t *row0, const uint16_t *row1,
                                         int wave, int lane, f32x4 (&acc)[kPfGroups][4]) {
    uint4 ring[kPfRing][kPfGroups];
    uint32_t goff[kPfGroups];  // byte offset of the wave's group g, tile 0, this lane
#pragma unroll
    for (int g = 0; g < kPfGroups; ++g)
        goff[g] = (uint32_t)((size_t)bg.at(wave_group(mode, wave, g)) * kt * 256) + lane * 16;
    auto issue = [&](int slot, int J) {
        load_bstage(&bring[slot][0], row0, J, wave);
        if (NB == 2) load_bstage(&bring[slot][1], row1, J, wave);
        if (wave < 2) load_scales(&scring[slot], scales, bg, kt, J, wave, lane);
#pragma unroll
        for (int g = 0; g < kPfGroups; ++g)
            ring[slot][g] = *reinterpret_cast<const uint4 *>(codes + goff[g] + (size_t)J * 1024);
    };
    const int last = nsuper - 1;
#pragma unroll
    for (int j = 0; j < kPfRing - 1; ++j) issue(j, min(j, last));
    for (int J0 = 0; J0 < nsuper; J0 += kPfRing) {
#pragma unroll
        for (int jj = 0; jj < kPfRing; ++jj) {
            const int J = J0 + jj;
            wait_vmcnt<(kPfRing - 2) * C>();  // step J has landed
            stage_barrier();
            issue((jj + kPfRing - 1) % kPfRing, min(J + kPfRing - 1, last));
            if (J < nsuper)
                mfma_step<NB>(ring[jj], &scring[jj], &bring[jj][0], &bring[jj][1], mode, wave,
                              lane, acc);
        }
    }
    wait_vmcnt<0>();  // the repeated tail loads land before the rings are reused
}

// Dispatch on the per-step load count of this wave (compile-time wait counts).
template <int NB>
__device__ __forceinline__ void run_pipeline(const uint8_t *codes, const uint8_t *scales,
                                             size_t kt, int nsuper, const BlockGroups &bg,
                                             int mode, BStage<64> (*bring)[2],
                                             ScaleStage *scring, const uint16_t *row0,
                                             const uint16_t *row1, int wave, int lane,
                                             f32x4 (&acc)[kPfGroups][4]) {
    constexpr int CB = 4 * NB;  // B copies per step
    if (wave < 2)
        pipeline<CB + 1 + kPfGroups, NB>(codes, scales, kt, nsuper, bg, mode, bring, scring, row0,
                                         row1, wave, lane, acc);
    else
        pipeline<CB + kPfGroups, NB>(codes, scales, kt, nsuper, bg, mode, bring, scring, row0,
                                     row1, wave, lane, acc);
}

struct PrefillLds {
    BStage<64> b[kPfRing][2];  // x (slot 0) or h hi, lo: up to 128 KiB
    ScaleStage sc[kPfRing];    // 8 KiB
};

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Grid: E * I/128 * 2 blocks of 4 waves; two blocks share
// a CU (51 KiB of LDS and at most 256 registers per wave each), so every SIMD
// runs two independent waves that hide each other's stalls.  Block (b, half
// th) of expert e owns gate row groups 8b..8b+7 and their up partners and the
// expert's tokens in 64-token chunks th, th+2, ...; wave w computes gate
// groups 8b+2w, +1 and their up partners.  The two halves of a slice are
// neighbouring blocks on one XCD, so the second one's weights mostly come
// from that XCD's L2.  Per 128-column step every wave issues its four 1 KiB
// pieces of the B stage, the scales of its 4 groups, then its 4 code loads,
// kGuRing-1 steps ahead, branch-free so the wait counts stay exact.
// ---------------------------------------------------------------------------
constexpr int kGuWaves = 4;
constexpr int kGuThreads = kGuWaves * 64;
constexpr int kGuGroups = 4;  // row groups per wave
constexpr int kGuRing = 3;

// B stage of one 128-column step: [chunk group cg][token m][4 x 16 B], the
// 16-byte chunk c = 4cg + p (columns 8c..8c+7) of token m kept at position
// p ^ ((m/4) % 4).  A copy instruction moves 64 contiguous bytes of each of 16
// token rows (lane l: token 16w + l/4, position l%4), and the MFMA reads of
// 16 tokens touch 16 distinct bank groups.
// Scales: each wave copies those of its own 4 groups (4 replicas of 256 B:
// [replica][group][tile q][row]), so every wave issues the same loads per step.
struct GuLds {
    uint8_t b[kGuRing][4][64][64];          // 16 KiB per slot
    uint8_t sc[kGuRing][kGuWaves][4][256];  // 4 KiB per slot
};

// MFMAs of one step for one wave: 4 K steps x 4 groups x mt token tiles.  The
// next K step's B operands and dequantised A operands are prepared before the
// current K step's MFMAs (double buffering).  Every step dequantises, even
// with no token tile, so no load is left in flight on a ring register.
__device__ __forceinline__ void gu_step(const uint4 (&code)[kGuGroups], const GuLds &lds,
                                        int slot, int wave, int mt, int lane,
                                        f32x4 (&acc)[kGuGroups][4]) {
    const int q = lane >> 4, n = lane & 15;
    float scale[kGuGroups];
#pragma unroll
    for (int g = 0; g < kGuGroups; ++g)
        scale[g] = e8m0_to_f32(lds.sc[slot][wave][0][64 * g + 16 * q + n]);
    bf16x8 a[2][kGuGroups];
    bf16x8 bv[2][4];
    auto load_b = [&](int buf, int ks) {  // token 16t + n, chunk 4q + ks
#pragma unroll
        for (int t = 0; t < 4; ++t)
            bv[buf][t] = *reinterpret_cast<const bf16x8 *>(
                &lds.b[slot][q][16 * t + n][16 * (ks ^ ((n >> 2) & 3))]);
    };
    auto dequant = [&](int buf, int ks) {
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g) {
            const uint4 c = code[g];
            const uint32_t d = ks == 0 ? c.x : ks == 1 ? c.y : ks == 2 ? c.z : c.w;
            a[buf][g] = fp4x8_to_bf16x8(d, scale[g]);
        }
    };
    load_b(0, 0);
    dequant(0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int cur = ks & 1;
        if (ks < 3) {
            load_b(cur ^ 1, ks + 1);
            dequant(cur ^ 1, ks + 1);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (t < mt) {
#pragma unroll
                for (int g = 0; g < kGuGroups; ++g)
                    acc[g][t] = mfma_bf16(a[cur][g], bv[cur][t], acc[g][t]);
            }
    }
}

__device__ __forceinline__ void gu_pipeline(const uint8_t *codes, const uint8_t *scales, size_t kt,
                                            int nsuper, const int (&grp)[kGuGroups], int sgrp,
                                            GuLds &lds, const uint16_t *brow, int wave, int lane,
                                            int mt, f32x4 (&acc)[kGuGroups][4]) {
    constexpr int C = 4 + 1 + kGuGroups;  // loads per wave per step
    uint4 ring[kGuRing][kGuGroups];
    uint32_t goff[kGuGroups];
#pragma unroll
    for (int g = 0; g < kGuGroups; ++g)
        goff[g] = (uint32_t)((size_t)grp[g] * kt * 256) + lane * 16;
    auto issue = [&](int slot, int J) {
        // B: copy i of this wave moves chunk group i of tokens 16w..16w+15;
        // lane l (token 16w + l/4) fills position l%4
        const int swz = (lane & 3) ^ ((lane >> 4) & 3);  // chunk within the group
#pragma unroll
        for (int i = 0; i < 4; ++i)
            copy_lds16(brow + 128 * J + 8 * (4 * i + swz), lds.b[slot][i][16 * wave]);
        // scales: lane l copies group (l/4)%4 (row group sgrp), tile 4J + l%4
        copy_lds16(scales + ((size_t)sgrp * kt + 4 * J + (lane & 3)) * 16, lds.sc[slot][wave][0]);
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g)
            ring[slot][g] = *reinterpret_cast<const uint4 *>(codes + goff[g] + (size_t)J * 1024);
    };
    const int last = nsuper - 1;
#pragma unroll
    for (int j = 0; j < kGuRing - 1; ++j) issue(j, min(j, last));
    for (int J0 = 0; J0 < nsuper; J0 += kGuRing) {
#pragma unroll
        for (int jj = 0; jj < kGuRing; ++jj) {
            const int J = J0 + jj;
            wait_vmcnt<(kGuRing - 2) * C>();  // step J has landed
            stage_barrier();
            issue((jj + kGuRing - 1) % kGuRing, min(J + kGuRing - 1, last));
            if (J < nsuper) gu_step(ring[jj], lds, jj, wave, mt, lane, acc);
        }
    }
    wait_vmcnt<0>();  // the repeated tail loads land before the rings are reused
}

__global__ __launch_bounds__(kGuThreads, 2) void prefill_gateup_mxfp4(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed, size_t expert_bytes,
    int H, int I, int K, int E, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ perm, uint16_t *__restrict__ h_hi, uint16_t *__restrict__ h_lo) {
    __shared__ __align__(16) GuLds lds;
    int e, part;
    map_expert_block(blockIdx.x, E, (I / 128) * 2, &e, &part);
    const int b = part >> 1, th = part & 1;
    const int p0 = offsets[e];
    const int ne = offsets[e + 1] - p0;
    if (64 * th >= ne) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const int ngate = I / 16;
    const uint8_t *ex = packed + (size_t)e * expert_bytes;
    const size_t kt = (size_t)(H / 32);
    int grp[kGuGroups];
#pragma unroll
    for (int g = 0; g < kGuGroups; ++g) grp[g] = (g < 2 ? 0 : ngate) + 8 * b + 2 * wave + (g & 1);
    // the scale copy's lane l covers the wave's group (l/4)%4
    const int sg = (lane >> 2) & 3;
    const int sgrp = (sg < 2 ? 0 : ngate) + 8 * b + 2 * wave + (sg & 1);

    for (int c0 = 64 * th; c0 < ne; c0 += 128) {
        const int nt = min(64, ne - c0);
        const int mt = (nt + 15) / 16;
        // the token row this lane copies: token 16w + l/4 of the chunk
        const uint16_t *brow =
            x + (size_t)(perm[p0 + c0 + min(16 * wave + (lane >> 2), nt - 1)] / K) * H;
        f32x4 acc[kGuGroups][4];
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c0 > 64 * th) stage_barrier();  // previous chunk's readers are done with the rings
        gu_pipeline(ex, ex + (size_t)I * H, kt, H / 128, grp, sgrp, lds, brow, wave, lane, mt,
                    acc);
        // epilogue: lane holds rows 4q..4q+3 of each group for token 16t + n;
        // gate group i pairs with up group 2 + i
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int m = 16 * t + n;
            if (m < nt) {
                const size_t p = (size_t)(p0 + c0 + m);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int gg = 8 * b + 2 * wave + i;  // gate group
                    uint32_t hi[4], lo[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float hv = silu_f32(acc[i][t][jj]) * acc[2 + i][t][jj];
                        hi[jj] = f32_to_bf16_rne(hv);
                        lo[jj] = f32_to_bf16_rne(hv - bf16_to_f32(hi[jj]));
                    }
                    const size_t col = (size_t)16 * gg + 4 * q;
                    *reinterpret_cast<uint2 *>(h_hi + p * I + col) =
                        make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                    *reinterpret_cast<uint2 *>(h_lo + p * I + col) =
                        make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down.  Grid: E * ceil(H/512) * 2 blocks.  Block (b, half th) owns output row
// groups 32b..32b+31 (wave w: groups 32b+8w..+7) and the expert's tokens in
// 64-token chunks th, th+2, ...; h rows are contiguous (route-position order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPfThreads) void prefill_down_mxfp4(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int E,
    const int32_t *__restrict__ offsets, const uint16_t *__restrict__ h_hi,
    const uint16_t *__restrict__ h_lo, float *__restrict__ y) {
    __shared__ __align__(16) PrefillLds lds;
    const int nrow = H / 16;
    int e, part;
    map_expert_block(blockIdx.x, E, ((H + 511) / 512) * 2, &e, &part);
    const int blk = part >> 1, th = part & 1;
    const int p0 = offsets[e];
    const int ne = offsets[e + 1] - p0;
    if (64 * th >= ne) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, q = lane >> 4;
    const uint8_t *codes = packed + (size_t)e * expert_bytes + (size_t)I * H + (size_t)I * H / 16;
    const BlockGroups bg{1, blk, nrow};

    for (int c0 = 64 * th; c0 < ne; c0 += 128) {
        const int nt = min(64, ne - c0);
        const size_t r = (size_t)(p0 + c0 + min(lane, nt - 1)) * I;
        f32x4 acc[kPfGroups][4];
#pragma unroll
        for (int g = 0; g < kPfGroups; ++g)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c0 > 64 * th) stage_barrier();
        run_pipeline<2>(codes, codes + (size_t)H * I / 2, (size_t)(I / 32), I / 128, bg, 1, lds.b,
                        lds.sc, h_hi + r, h_lo + r, wave, lane, acc);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int m = 16 * t + n;
            if (m < nt) {
                const size_t p = (size_t)(p0 + c0 + m);
#pragma unroll
                for (int g = 0; g < kPfGroups; ++g) {
                    const int gg = 32 * blk + 8 * wave + g;
                    if (gg < nrow)
                        *reinterpret_cast<float4 *>(y + p * H + 16 * gg + 4 * q) =
                            make_float4(acc[g][t][0], acc[g][t][1], acc[g][t][2], acc[g][t][3]);
                }
            }
        }
    }
}

hipError_t launch_prefill_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                 const Workspace &ws, hipStream_t st) {
    uint16_t *hh = static_cast<uint16_t *>(ws.h);
    uint16_t *hl = hh + (size_t)T * s.K * s.I;
    prefill_gateup_mxfp4<<<s.E * (s.I / 128) * 2, kGuThreads, 0, st>>>(
        x, packed, s.expert_bytes, s.H, s.I, s.K, s.E, ws.offsets, ws.perm, hh, hl);
    return hipGetLastError();
}

hipError_t launch_prefill_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                               hipStream_t st) {
    const uint16_t *hh = static_cast<const uint16_t *>(ws.h);
    const uint16_t *hl = hh + (size_t)T * s.K * s.I;
    prefill_down_mxfp4<<<s.E * ((s.H + 511) / 512) * 2, kPfThreads, 0, st>>>(
        packed, s.expert_bytes, s.H, s.I, s.E, ws.offsets, hh, hl, ws.y);
    return hipGetLastError();
}

}  // namespace bqmoe
