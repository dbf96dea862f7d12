// prefill.hip -- large-batch expert kernels for MXFP4 experts on gfx950: a
// grouped GEMM per expert on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulators.
//
// The micro-batch matters (a 512-token micro-batch leaves much of prefill
// unused because each of the 256 experts then sees too few tokens per matmul
// -- TrevorJS GGUF card, "Speed"): a block owns one slice of one expert's
// weights and multiplies it with the expert's tokens, 64 at a time.
//
// Shape of a kernel: blocks of four waves with 4 row groups (16 weight rows
// each) per wave, at most 256 registers and 51 KiB of LDS per block,
// so two independent blocks share each CU and every SIMD runs two waves that
// hide each other's memory and barrier stalls.  Per K step of 128 columns each
// wave issues, in a fixed order, its copies of the B stage and of its groups'
// scales (global_load_lds into an LDS ring) and its 4 code loads (1 KiB wave
// loads into a register ring), a fixed number of steps ahead.  Loads are
// issued unconditionally (past the end they repeat the last step's
// addresses) so the wait counts are compile-time constants that the compiler
// tracks exactly; a conditional issue makes it wait for every load in flight.
//
// Weights are dequantised to bf16 in registers: every E2M1 value times an
// in-range E8M0 scale is a bf16 value, so the A operand and the products are
// exact, and the dequantisation of K step s+1 runs while the MFMAs of step s
// issue.
//
// MFMA roles: A = 16 weight rows x 32 K (lane l: row l%16, K slice
// 8*(l/16)..+7), B = 32 K x 16 tokens, D[row][token].  Lane (n, q) of a wave
// holds the 16 code bytes of tile column 4J+q of its row n: K columns
// 128J+32q .. +31; K step s uses bytes 4s..4s+3 (columns 128J+32q+8s..+7),
// and the B operand of lane (m, q) at step s is x[m][128J+32q+8s..+7].
//
// SwiGLU is fused into the gate/up epilogue in fp32, and h is written in
// fp32.  Expert intermediates exceed fp16's range (TrevorJS card, "Recipe";
// benthecarman EXL3 card, "Bitrate") and a single bf16 is too coarse for the
// down projection, so a packing pass stores each h row as fp16 times a power
// of two of its own (h16 = h * 2^-s_r, 11 significant bits), and the down GEMM
// runs on the fp16 matrix cores (v_mfma_f32_16x16x32_f16): one pass, where a
// bf16 hi + lo split of h would take two.  Its A operand is the weight times
// 2^(e - b_g), e the block's E8M0 exponent and b_g the largest exponent of the
// 16-row group, which is exact in fp16 while a group's exponents span at most
// 13 (further below b_g the products only lose bits that sit 2^-14 under the
// group's largest weights); the epilogue multiplies by 2^(b_g - 127 + s_r).
#include <type_traits>

#include "moe_internal.h"
#include "vq_common.h"

namespace bqmoe {

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
// The same with 4 bytes per lane (256 B per wave).
__device__ __forceinline__ void copy_lds4(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
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

__device__ __forceinline__ f32x4 mfma_op(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_op(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Four packed fp4 bytes -> eight fp16, each times `scale` (byte b: columns 2b, 2b+1).
__device__ __forceinline__ f16x8 fp4x8_to_f16x8(uint32_t v, float scale) {
    union { f16x8 v8; f16x2 v2[4]; } r;
    r.v2[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, 0);
    r.v2[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, 1);
    r.v2[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, 2);
    r.v2[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, 3);
    return r.v8;
}

// 2^(e - b) for an E8M0 exponent e at most b, 0 below 2^-126.
__device__ __forceinline__ float e8m0_rel_f32(uint32_t e, int b) {
    const int d = (int)e + 127 - b;
    return d > 0 ? __uint_as_float((uint32_t)d << 23) : 0.f;
}

// Token chunks of block half th of an expert with ne tokens: chunk i of the
// expert (64 tokens) belongs to half i%2.  For 64 < ne <= 128 the two halves
// take an even split in 16-token tiles instead (the first half gets the odd
// tile), so the sibling blocks that stream the same weight slice run at the
// same pace and the second one finds the slice in L2.
struct ChunkPlan {
    int c0, nt0;  // first chunk's start and size (nt0 < 0: 64-token chunks throughout)
};
__device__ __forceinline__ ChunkPlan chunk_plan(int ne, int th) {
    if (ne > 64 && ne <= 128) {
        const int split = 16 * (((ne + 15) / 16 + 1) / 2);
        return {th ? split : 0, th ? ne - split : split};
    }
    return {64 * th, -1};
}

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
// Scales: each wave copies those of its own 4 groups, 256 B per step laid out
// [group][tile q][row] (lane l moves rows 4(l%4)..+3 of tile (l/4)%4 of group
// l/16), so every wave issues the same loads per step.
struct GuLds {
    uint8_t b[kGuRing][4][64][64];          // 16 KiB per slot
    uint8_t sc[kGuRing][kGuWaves][256];     // 1 KiB per slot
};

// MFMAs of one step for one wave: 4 K steps x 4 groups x MT token tiles.  MT
// is a template parameter (the chunk's tile count, dispatched once per
// chunk): with a run-time count every tile's MFMAs sat in a basic block of
// their own, and the compiler could not interleave them with the next K
// step's LDS reads and conversions (measured: 7% slower).  The
// next K step's B operands and dequantised A operands are prepared before the
// current K step's MFMAs (double buffering).  Every step dequantises, even
// with no token tile, so no load is left in flight on a ring register.
// F16: fp16 operands, the weights scaled relative to the group exponents b[g].
template <bool F16, int MT>
__device__ __forceinline__ void gu_step(const uint4 (&code)[kGuGroups], const GuLds &lds,
                                        int slot, int wave, int lane,
                                        const int (&b)[kGuGroups], f32x4 (&acc)[kGuGroups][4]) {
    using V8 = std::conditional_t<F16, f16x8, bf16x8>;
    const int q = lane >> 4, n = lane & 15;
    float scale[kGuGroups];
#pragma unroll
    for (int g = 0; g < kGuGroups; ++g) {
        const uint32_t e = lds.sc[slot][wave][64 * g + 16 * q + n];
        scale[g] = F16 ? e8m0_rel_f32(e, b[g]) : e8m0_to_f32(e);
    }
    V8 a[2][kGuGroups];
    V8 bv[2][4];
    auto load_b = [&](int buf, int ks) {  // token 16t + n, chunk 4q + ks
#pragma unroll
        for (int t = 0; t < 4; ++t)
            bv[buf][t] = *reinterpret_cast<const V8 *>(
                &lds.b[slot][q][16 * t + n][16 * (ks ^ ((n >> 2) & 3))]);
    };
    auto dequant = [&](int buf, int ks) {
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g) {
            const uint4 c = code[g];
            const uint32_t d = ks == 0 ? c.x : ks == 1 ? c.y : ks == 2 ? c.z : c.w;
            if constexpr (F16)
                a[buf][g] = fp4x8_to_f16x8(d, scale[g]);
            else
                a[buf][g] = fp4x8_to_bf16x8(d, scale[g]);
        }
    };
    load_b(0, 0);
    dequant(0, 0);
    // raised issue priority while this wave has MFMAs to issue, so the
    // co-resident block's waves, busy with loads and barriers, yield to it
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int cur = ks & 1;
        if (ks < 3) {
            load_b(cur ^ 1, ks + 1);
            dequant(cur ^ 1, ks + 1);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (t < MT) {
#pragma unroll
                for (int g = 0; g < kGuGroups; ++g)
                    acc[g][t] = mfma_op(a[cur][g], bv[cur][t], acc[g][t]);
            }
    }
    __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ uint32_t byte_max(uint32_t w) {
    return max(max(w & 0xFFu, (w >> 8) & 0xFFu), max((w >> 16) & 0xFFu, w >> 24));
}

template <bool F16, int MT>
__device__ __forceinline__ void gu_pipeline(const uint8_t *codes, const uint8_t *scales, size_t kt,
                                            int nsuper, const int (&grp)[kGuGroups],
                                            GuLds &lds, const uint16_t *brow, int wave, int lane,
                                            f32x4 (&acc)[kGuGroups][4],
                                            int (&b)[kGuGroups]) {
    constexpr int C = 4 + 1 + kGuGroups;  // loads per wave per step
    uint4 ring[kGuRing][kGuGroups];
    uint32_t goff[kGuGroups];
    const uint32_t soff =
        (uint32_t)(((size_t)grp[lane >> 4] * kt + ((lane >> 2) & 3)) * 16) + 4 * (lane & 3);
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
        // scales: lane l copies rows 4(l%4)..+3 of tile 4J + (l/4)%4 of group l/16
        copy_lds4(scales + soff + (size_t)J * 64, lds.sc[slot][wave]);
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g)
            ring[slot][g] = *reinterpret_cast<const uint4 *>(codes + goff[g] + (size_t)J * 1024);
    };
    const int last = nsuper - 1;
#pragma unroll
    for (int j = 0; j < kGuRing - 1; ++j) issue(j, min(j, last));
    if constexpr (F16) {
        // b[g] = the largest E8M0 exponent of row group grp[g] (kt tiles of 16
        // bytes), read while the first steps are in flight
        // (the four groups' loads of a pass are issued together; past the
        // last tile lanes repeat it)
        uint32_t m[kGuGroups] = {0, 0, 0, 0};
        for (size_t c0 = 0; c0 < kt; c0 += 64) {
            const size_t c = min(c0 + (size_t)lane, kt - 1);
            uint4 v[kGuGroups];
#pragma unroll
            for (int g = 0; g < kGuGroups; ++g)
                v[g] = *reinterpret_cast<const uint4 *>(scales + ((size_t)grp[g] * kt + c) * 16);
#pragma unroll
            for (int g = 0; g < kGuGroups; ++g)
                m[g] = max(m[g], max(max(byte_max(v[g].x), byte_max(v[g].y)),
                                     max(byte_max(v[g].z), byte_max(v[g].w))));
        }
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                m[g] = max(m[g], (uint32_t)__shfl_xor((int)m[g], o, 64));
            b[g] = __builtin_amdgcn_readfirstlane((int)m[g]);
        }
    }
    for (int J0 = 0; J0 < nsuper; J0 += kGuRing) {
#pragma unroll
        for (int jj = 0; jj < kGuRing; ++jj) {
            const int J = J0 + jj;
            wait_vmcnt<(kGuRing - 2) * C>();  // step J has landed
            stage_barrier();
            issue((jj + kGuRing - 1) % kGuRing, min(J + kGuRing - 1, last));
            if (J < nsuper) gu_step<F16, MT>(ring[jj], lds, jj, wave, lane, b, acc);
        }
    }
    wait_vmcnt<0>();  // the repeated tail loads land before the rings are reused
}

__global__ __launch_bounds__(kGuThreads, 2) void prefill_gateup_mxfp4(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed, size_t expert_bytes,
    int H, int I, int K, int E, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ perm, float *__restrict__ h) {
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

    const ChunkPlan plan = chunk_plan(ne, th);
    for (int c0 = plan.c0; c0 < ne; c0 += 128) {
        const int nt = plan.nt0 >= 0 ? plan.nt0 : min(64, ne - c0);
        const int mt = (nt + 15) / 16;
        // the token row this lane copies: token 16w + l/4 of the chunk
        const uint16_t *brow =
            x + (size_t)(perm[p0 + c0 + min(16 * wave + (lane >> 2), nt - 1)] / K) * H;
        f32x4 acc[kGuGroups][4];
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c0 > plan.c0) stage_barrier();  // previous chunk's readers are done with the rings
        int unused[kGuGroups];
        auto run = [&](auto mtc) {
            gu_pipeline<false, decltype(mtc)::value>(ex, ex + (size_t)I * H, kt, H / 128, grp, lds,
                                                     brow, wave, lane, acc, unused);
        };
        switch (mt) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
        }
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
                    float hv[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        hv[jj] = silu_f32(acc[i][t][jj]) * acc[2 + i][t][jj];
                    *reinterpret_cast<float4 *>(h + p * I + (size_t)16 * gg + 4 * q) =
                        make_float4(hv[0], hv[1], hv[2], hv[3]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down.  Grid: E * H/256 * 2 blocks of 4 waves, two blocks per CU as in
// gate/up, on the same pipeline with fp16 operands.  Block (b, half th) owns
// output row groups 16b..16b+15 (wave w: 16b+4w..+3) and the expert's tokens
// in 64-token chunks th, th+2, ...; the h16 rows are contiguous (route-position
// order).  y[p][row] = acc * 2^(b_g - 127 + s_p).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGuThreads, 2) void prefill_down_mxfp4(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int E,
    const int32_t *__restrict__ offsets, const uint16_t *__restrict__ h16,
    const int32_t *__restrict__ hexp, float *__restrict__ y) {
    __shared__ __align__(16) GuLds lds;
    int e, part;
    map_expert_block(blockIdx.x, E, (H / 256) * 2, &e, &part);
    const int b = part >> 1, th = part & 1;
    const int p0 = offsets[e];
    const int ne = offsets[e + 1] - p0;
    if (64 * th >= ne) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const uint8_t *codes = packed + (size_t)e * expert_bytes + (size_t)I * H + (size_t)I * H / 16;
    const size_t kt = (size_t)(I / 32);
    int grp[kGuGroups];
#pragma unroll
    for (int g = 0; g < kGuGroups; ++g) grp[g] = 16 * b + 4 * wave + g;

    const ChunkPlan plan = chunk_plan(ne, th);
    for (int c0 = plan.c0; c0 < ne; c0 += 128) {
        const int nt = plan.nt0 >= 0 ? plan.nt0 : min(64, ne - c0);
        const int mt = (nt + 15) / 16;
        const uint16_t *brow = h16 + (size_t)(p0 + c0 + min(16 * wave + (lane >> 2), nt - 1)) * I;
        f32x4 acc[kGuGroups][4];
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c0 > plan.c0) stage_barrier();
        int bexp[kGuGroups];
        auto run = [&](auto mtc) {
            gu_pipeline<true, decltype(mtc)::value>(codes, codes + (size_t)H * I / 2, kt, I / 128,
                                                    grp, lds, brow, wave, lane, acc, bexp);
        };
        switch (mt) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
        }
        int hs[4];  // row exponents of the lane's tokens, fetched together
#pragma unroll
        for (int t = 0; t < 4; ++t) hs[t] = hexp[p0 + c0 + min(16 * t + n, nt - 1)] - 127;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int m = 16 * t + n;
            if (m < nt) {
                const size_t p = (size_t)(p0 + c0 + m);
#pragma unroll
                for (int g = 0; g < kGuGroups; ++g) {
                    const int sc = bexp[g] + hs[t];
                    *reinterpret_cast<float4 *>(y + p * H + 16 * grp[g] + 4 * q) =
                        make_float4(ldexpf(acc[g][t][0], sc), ldexpf(acc[g][t][1], sc),
                                    ldexpf(acc[g][t][2], sc), ldexpf(acc[g][t][3], sc));
                }
            }
        }
    }
}

hipError_t launch_prefill_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                 const Workspace &ws, hipStream_t st) {
    prefill_gateup_mxfp4<<<s.E * (s.I / 128) * 2, kGuThreads, 0, st>>>(
        x, packed, s.expert_bytes, s.H, s.I, s.K, s.E, ws.offsets, ws.perm,
        static_cast<float *>(ws.h));
    return hipGetLastError();
}

hipError_t launch_prefill_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                               hipStream_t st) {
    hipError_t e = launch_hpack(s, T * s.K, ws, st);
    if (e != hipSuccess) return e;
    prefill_down_mxfp4<<<s.E * (s.H / 256) * 2, kGuThreads, 0, st>>>(
        packed, s.expert_bytes, s.H, s.I, s.E, ws.offsets, ws.h16, ws.hexp, ws.y);
    return hipGetLastError();
}

}  // namespace bqmoe
