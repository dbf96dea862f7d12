// prefill.hip -- large-batch expert kernels for MXFP4 experts on gfx950: a
// grouped GEMM per expert on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulators.
//
// The micro-batch matters (a 512-token micro-batch leaves much of prefill
// unused because each of the 256 experts then sees too few tokens per matmul
// -- TrevorJS GGUF card, "Speed"): a block owns one slice of one expert's
// weights and multiplies it with all of the expert's tokens, up to 128 of them
// per pass over the slice, so the slice leaves HBM once.
//
// Shape of a kernel: one persistent block of eight waves per CU, at most 256
// registers per wave and 136 KiB of LDS.  Each wave owns 2 row groups (16 weight rows
// each; for gate/up a gate group and its up partner) and all of the pass's
// 16-token tiles, so no two waves load or dequantise the same weights.  Per K
// step of 128 columns each wave issues, in a fixed order, its copies of the B
// stage (only waves whose token rows hold tokens of the pass) and of its
// groups' scales (global_load_lds into a 4-slot LDS ring) and its 2 code loads
// (1 KiB wave loads into a register ring), three steps ahead, at a barrier in
// the middle of each step.  Loads are issued unconditionally (past the end
// they repeat the last step's addresses) so the wait counts are compile-time
// constants that the compiler tracks exactly; a conditional issue makes it
// wait for every load in flight.
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

// item -> (expert, block): the items of one expert go to blocks of one XCD
// (the dispatcher deals workgroups round-robin over the 8 XCDs, and a block
// takes the items congruent to its index mod 8), so the expert's token rows
// and shared weight slices are re-read from that XCD's L2.
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

// 16 bytes per lane of a weight stream read once per forward: a non-temporal
// load, so the codes do not displace the token rows re-read from L2.
typedef uint32_t u32x4nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const uint8_t *p) {
    const u32x4nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4nt *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
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

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Persistent blocks of 8 waves, one per CU, loop over the
// E * I/128 items; item (e, b) owns gate row groups 8b..8b+7 of expert e and
// their up partners and all of the expert's tokens, 128 per pass; wave w
// computes gate group 8b+w and its up partner for every 16-token tile of the
// pass.  Per 128-column step every
// wave issues its four 1 KiB pieces of the B stage, the scales of its 2
// groups, then its 2 code loads, for the step three ahead, at a barrier in the
// middle of the current step; branch-free, so the wait counts stay exact.
// ---------------------------------------------------------------------------
constexpr int kGuWaves = 8;
constexpr int kGuThreads = kGuWaves * 64;
constexpr int kGuGroups = 2;   // row groups per wave
constexpr int kGuRing = 4;
constexpr int kGuChunk = 128;  // tokens per pass over the weight slice
constexpr int kGuTiles = kGuChunk / 16;

// B stage of one 128-column step: [chunk group cg][token m][4 x 16 B], the
// 16-byte chunk c = 4cg + p (columns 8c..8c+7) of token m kept at position
// p ^ ((m/4) % 4).  A copy instruction moves 64 contiguous bytes of each of 16
// token rows (lane l: token 16w + l/4, position l%4), and the MFMA reads of
// 16 tokens touch 16 distinct bank groups.
// Scales: each wave copies those of its own 2 groups, 128 B per step laid out
// [group][tile q][row] (lane l < 32 moves rows 4(l%4)..+3 of tile (l/4)%4 of
// group l/16; lanes 32-63 repeat that into the unused upper half).
struct GuLds {
    uint8_t b[kGuRing][4][kGuChunk][64];    // 32 KiB per slot
    uint8_t sc[kGuRing][kGuWaves][256];     // 2 KiB per slot
};

__device__ __forceinline__ uint32_t byte_max(uint32_t w) {
    return max(max(w & 0xFFu, (w >> 8) & 0xFFu), max((w >> 16) & 0xFFu, w >> 24));
}

// The pipeline of one pass for one wave.  Per step (128 columns): 4 K steps x
// 2 groups x MT token tiles of MFMAs.  MT is a template parameter (the pass's
// tile count): with a run-time count every tile's MFMAs sat in a basic block
// of their own, and the compiler could not interleave them with the next K
// step's LDS reads and conversions.  The next K step's B operands and
// dequantised A operands are prepared before the current K step's MFMAs
// (double buffering), across step boundaries too: the barrier that publishes
// step J+1 sits between K steps 1 and 2 of step J, and the first operands of
// step J+1 are prepared under the MFMAs of step J's last K step, so no step
// starts with the matrix cores idle.  Four LDS slots: step J being read, J+1
// published, J+2 landing, J+3 issued at that barrier (two steps ahead).
// BCOPY: this wave copies its 16 token rows of the B stage (waves whose rows
// lie past the pass's last token copy nothing; their count of loads per step
// is a compile-time constant too).
// F16: fp16 operands, the weights scaled relative to the group exponents b[g].
template <bool F16, int MT, bool BCOPY>
__device__ __forceinline__ void gu_pipeline(const uint8_t *codes, const uint8_t *scales, size_t kt,
                                            int nsuper, const int (&grp)[kGuGroups],
                                            GuLds &lds, const uint16_t *brow, int wave, int lane,
                                            f32x4 (&acc)[kGuGroups][kGuTiles],
                                            int (&b)[kGuGroups]) {
    using V8 = std::conditional_t<F16, f16x8, bf16x8>;
    static_assert(kGuRing == 4, "slot arithmetic below");
    constexpr int C = (BCOPY ? 4 : 0) + 1 + kGuGroups;  // loads per wave per step
    const int q = lane >> 4, n = lane & 15;
    uint4 ring[kGuRing][kGuGroups];
    uint32_t goff[kGuGroups];
    const uint32_t soff =
        (uint32_t)(((size_t)grp[(lane >> 4) & 1] * kt + ((lane >> 2) & 3)) * 16) + 4 * (lane & 3);
#pragma unroll
    for (int g = 0; g < kGuGroups; ++g)
        goff[g] = (uint32_t)((size_t)grp[g] * kt * 256) + lane * 16;
    auto issue = [&](int slot, int J) {
        // B: copy i of this wave moves chunk group i of tokens 16w..16w+15;
        // lane l (token 16w + l/4) fills position l%4
        const int swz = (lane & 3) ^ ((lane >> 4) & 3);  // chunk within the group
        if constexpr (BCOPY) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                copy_lds16(brow + 128 * J + 8 * (4 * i + swz), lds.b[slot][i][16 * wave]);
        }
        // scales: lane l copies rows 4(l%4)..+3 of tile 4J + (l/4)%4 of group (l/16)%2
        copy_lds4(scales + soff + (size_t)J * 64, lds.sc[slot][wave]);
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g)
            ring[slot][g] = ld16_nt(codes + goff[g] + (size_t)J * 1024);
    };
    const int last = nsuper - 1;
    issue(0, 0);
    issue(1, min(1, last));
    issue(2, min(2, last));
    if constexpr (F16) {
        // b[g] = the largest E8M0 exponent of row group grp[g] (kt tiles of 16
        // bytes), read while the first steps are in flight (past the last
        // tile lanes repeat it)
        uint32_t m[kGuGroups] = {0, 0};
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

    float scale[kGuGroups];
    V8 a[2][kGuGroups];
    V8 bv[2][MT];
    auto read_scales = [&](int slot) {
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g) {
            const uint32_t e = lds.sc[slot][wave][64 * g + 16 * q + n];
            scale[g] = F16 ? e8m0_rel_f32(e, b[g]) : e8m0_to_f32(e);
        }
    };
    auto load_b = [&](int buf, int slot, int ks) {  // token 16t + n, chunk 4q + ks
#pragma unroll
        for (int t = 0; t < MT; ++t)
            bv[buf][t] = *reinterpret_cast<const V8 *>(
                &lds.b[slot][q][16 * t + n][16 * (ks ^ ((n >> 2) & 3))]);
    };
    auto dequant = [&](int buf, const uint4 (&code)[kGuGroups], int ks) {
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
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int g = 0; g < kGuGroups; ++g)
                acc[g][t] = mfma_op(a[buf][g], bv[buf][t], acc[g][t]);
    };

    wait_vmcnt<2 * C>();  // step 0 has landed
    stage_barrier();
    read_scales(0);
    load_b(0, 0, 0);
    dequant(0, ring[0], 0);
    for (int J0 = 0; J0 < nsuper; J0 += kGuRing) {
#pragma unroll
        for (int jj = 0; jj < kGuRing; ++jj) {
            const int J = J0 + jj;
            const int nx = (jj + 1) % kGuRing;  // slot of step J+1
            __builtin_amdgcn_s_setprio(1);
            if (J < nsuper) {
                load_b(1, jj, 1);
                dequant(1, ring[jj], 1);
                mfmas(0);  // K step 0
                load_b(0, jj, 2);
                dequant(0, ring[jj], 2);
                mfmas(1);  // K step 1
            }
            __builtin_amdgcn_s_setprio(0);
            wait_vmcnt<C>();  // step J+1 has landed (step J+2 may be in flight)
            stage_barrier();  // publishes step J+1; every wave is done with step J-1
            issue((jj + 3) % kGuRing, min(J + 3, last));
            __builtin_amdgcn_s_setprio(1);
            if (J < nsuper) {
                load_b(1, jj, 3);
                dequant(1, ring[jj], 3);
                mfmas(0);  // K step 2
                read_scales(nx);
                load_b(0, nx, 0);
                dequant(0, ring[nx], 0);
                mfmas(1);  // K step 3
            }
            __builtin_amdgcn_s_setprio(0);
        }
    }
    wait_vmcnt<0>();  // the repeated tail loads land before the rings are reused
}

// Runs f(integral_constant<int, mt>, integral_constant<bool, copies>) for a
// tile count mt in 1..kGuTiles; `copies` is whether this wave's token rows
// (16w..16w+15) hold any of the pass's tokens.
template <typename F>
__device__ __forceinline__ void with_tiles(int mt, int wave, F &&f) {
    auto g = [&](auto mtc) {
        if (wave < decltype(mtc)::value)
            f(mtc, std::true_type{});
        else
            f(mtc, std::false_type{});
    };
    switch (mt) {
        case 1: g(std::integral_constant<int, 1>{}); break;
        case 2: g(std::integral_constant<int, 2>{}); break;
        case 3: g(std::integral_constant<int, 3>{}); break;
        case 4: g(std::integral_constant<int, 4>{}); break;
        case 5: g(std::integral_constant<int, 5>{}); break;
        case 6: g(std::integral_constant<int, 6>{}); break;
        case 7: g(std::integral_constant<int, 7>{}); break;
        default: f(std::integral_constant<int, 8>{}, std::true_type{}); break;
    }
}

__global__ __launch_bounds__(kGuThreads, 1) void prefill_gateup_mxfp4(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed, size_t expert_bytes,
    int H, int I, int K, int E, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ perm, float *__restrict__ h) {
    __shared__ __align__(16) GuLds lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const int ngate = I / 16;
    const size_t kt = (size_t)(H / 32);
    const int nitems = E * (I / 128);
    bool first = true;
    for (int item = (int)blockIdx.x; item < nitems; item += (int)gridDim.x) {
    int e, b;
    map_expert_block(item, E, I / 128, &e, &b);
    const int p0 = offsets[e];
    const int ne = offsets[e + 1] - p0;
    if (ne == 0) continue;
    const uint8_t *ex = packed + (size_t)e * expert_bytes;
    const int gg = 8 * b + wave;  // this wave's gate group
    const int grp[kGuGroups] = {gg, ngate + gg};

    for (int c0 = 0; c0 < ne; c0 += kGuChunk) {
        const int nt = min(kGuChunk, ne - c0);
        const int mt = (nt + 15) / 16;
        // the token row this lane copies: token 16w + l/4 of the chunk
        const uint16_t *brow =
            x + (size_t)(perm[p0 + c0 + min(16 * wave + (lane >> 2), nt - 1)] / K) * H;
        f32x4 acc[kGuGroups][kGuTiles];
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g)
#pragma unroll
            for (int t = 0; t < kGuTiles; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!first) stage_barrier();  // previous pass's readers are done with the rings
        first = false;
        int unused[kGuGroups];
        with_tiles(mt, wave, [&](auto mtc, auto copies) {
            gu_pipeline<false, decltype(mtc)::value, decltype(copies)::value>(
                ex, ex + (size_t)I * H, kt, H / 128, grp, lds, brow, wave, lane, acc, unused);
        });
        // epilogue: lane holds rows 4q..4q+3 of the gate group (acc[0]) and of
        // its up partner (acc[1]) for token 16t + n
#pragma unroll
        for (int t = 0; t < kGuTiles; ++t) {
            const int m = 16 * t + n;
            if (t < mt && m < nt) {
                const size_t p = (size_t)(p0 + c0 + m);
                float hv[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) hv[jj] = silu_f32(acc[0][t][jj]) * acc[1][t][jj];
                *reinterpret_cast<float4 *>(h + p * I + (size_t)16 * gg + 4 * q) =
                    make_float4(hv[0], hv[1], hv[2], hv[3]);
            }
        }
    }
    }
}

// ---------------------------------------------------------------------------
// down.  Persistent blocks of 8 waves, one per CU, over the E * H/256 items,
// on the same pipeline with fp16 operands.  Item (e, b) owns output row groups
// 16b..16b+15 (wave w: 16b+2w, +1) and all of the expert's tokens, 128 per
// pass; the h16 rows are contiguous (route-position order).  y[p][row] = acc * 2^(b_g - 127 + s_p),
// written as fp16 rows with an exponent per 16 rows (y16, yexp).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGuThreads, 1) void prefill_down_mxfp4(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int E,
    const int32_t *__restrict__ offsets, const uint16_t *__restrict__ h16,
    const int32_t *__restrict__ hexp, int ysh, uint16_t *__restrict__ y16,
    int8_t *__restrict__ yexp) {
    __shared__ __align__(16) GuLds lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const int nitems = E * (H / 256);
    bool first = true;
    for (int item = (int)blockIdx.x; item < nitems; item += (int)gridDim.x) {
    int e, b;
    map_expert_block(item, E, H / 256, &e, &b);
    const int p0 = offsets[e];
    const int ne = offsets[e + 1] - p0;
    if (ne == 0) continue;
    const uint8_t *codes = packed + (size_t)e * expert_bytes + (size_t)I * H + (size_t)I * H / 16;
    const size_t kt = (size_t)(I / 32);
    const int grp[kGuGroups] = {16 * b + 2 * wave, 16 * b + 2 * wave + 1};

    for (int c0 = 0; c0 < ne; c0 += kGuChunk) {
        const int nt = min(kGuChunk, ne - c0);
        const int mt = (nt + 15) / 16;
        const uint16_t *brow = h16 + (size_t)(p0 + c0 + min(16 * wave + (lane >> 2), nt - 1)) * I;
        f32x4 acc[kGuGroups][kGuTiles];
#pragma unroll
        for (int g = 0; g < kGuGroups; ++g)
#pragma unroll
            for (int t = 0; t < kGuTiles; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!first) stage_barrier();
        first = false;
        int bexp[kGuGroups];
        with_tiles(mt, wave, [&](auto mtc, auto copies) {
            gu_pipeline<true, decltype(mtc)::value, decltype(copies)::value>(
                codes, codes + (size_t)H * I / 2, kt, I / 128, grp, lds, brow, wave, lane, acc,
                bexp);
        });
        int hs[kGuTiles];  // row exponents of the lane's tokens, fetched together
#pragma unroll
        for (int t = 0; t < kGuTiles; ++t) hs[t] = hexp[p0 + c0 + min(16 * t + n, nt - 1)] - 127;
        // y = acc * 2^(b_g + s_r), stored as fp16 times 2^ey per 16 output
        // rows of a route, ey = b_g + s_r + ysh.  |acc| <= I * 6 * 2^15 (the
        // A operand is at most 6 in magnitude, an h16 row's largest is below
        // 2^15), so acc * 2^-ysh with ysh = ceil(log2(6 I)) stays below 2^15
        // and every value at most 2^29 under that bound keeps fp16's 11
        // significant bits.
#pragma unroll
        for (int t = 0; t < kGuTiles; ++t) {
            const int m = 16 * t + n;
            if (t < mt && m < nt) {
                const size_t p = (size_t)(p0 + c0 + m);
#pragma unroll
                for (int g = 0; g < kGuGroups; ++g) {
                    const int ey = min(max(bexp[g] + hs[t] + ysh, -128), 127);
                    const int sh = bexp[g] + hs[t] - ey;  // -ysh unless ey was clamped
                    union { _Float16 h[4]; uint2 u; } r;
#pragma unroll
                    for (int i = 0; i < 4; ++i) r.h[i] = (_Float16)ldexpf(acc[g][t][i], sh);
                    *reinterpret_cast<uint2 *>(y16 + p * H + 16 * grp[g] + 4 * q) = r.u;
                    if (q == 0) yexp[p * (H / 16) + grp[g]] = (int8_t)ey;
                }
            }
        }
    }
    }
}

// Persistent grid: one block per CU, a multiple of 8 when there is enough
// work, so block b stays on XCD b % 8 and deals the items of that XCD.
static int gu_grid(int items) {
    int g = min(items, device_cu_count());
    if (g >= 8) g &= ~7;
    return max(g, 1);
}

hipError_t launch_prefill_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                 const Workspace &ws, hipStream_t st) {
    prefill_gateup_mxfp4<<<gu_grid(s.E * (s.I / 128)), kGuThreads, 0, st>>>(
        x, packed, s.expert_bytes, s.H, s.I, s.K, s.E, ws.offsets, ws.perm,
        static_cast<float *>(ws.h));
    return hipGetLastError();
}

hipError_t launch_prefill_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                               hipStream_t st) {
    hipError_t e = launch_hpack(s, T * s.K, ws, st);
    if (e != hipSuccess) return e;
    int ysh = 0;  // ceil(log2(6 I))
    while ((1 << ysh) < 6 * s.I) ++ysh;
    prefill_down_mxfp4<<<gu_grid(s.E * (s.H / 256)), kGuThreads, 0, st>>>(
        packed, s.expert_bytes, s.H, s.I, s.E, ws.offsets, ws.h16, ws.hexp, ysh, ws.y16, ws.yexp);
    return hipGetLastError();
}

}  // namespace bqmoe
