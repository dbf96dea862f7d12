// prefill.hip -- large-batch expert kernels for MXFP4 experts on gfx950:
// a grouped GEMM per expert on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulators.
//
// Roles: the MFMA A operand is a 16-row weight tile, the B operand is 16
// tokens.  Lane l of A supplies row l%16 and 8 consecutive K values of
// sub-block l/16; with the 16x32 tile layout of the packed format, lane
// (n, q) loads the 16 code bytes of tile column 4J+q (32 weights, one E8M0
// block) and converts them to bf16 in registers with the block scale; these
// feed four MFMAs (K slices 8s..8s+7, s = 0..3).  Every E2M1 value times an
// in-range E8M0 scale is a bf16 value, so the dequantised operand is exact and
// the products are exact; only the fp32 accumulation rounds.
//
// SwiGLU is fused into the gate/up epilogue in fp32.  Because expert
// intermediates exceed fp16's range (TrevorJS GGUF card, "Recipe"; benthecarman
// EXL3 card, "Bitrate") and a single bf16 is too coarse for the down
// projection, h is written as an error-free-enough pair hi = bf16(h),
// lo = bf16(h - hi), and the down GEMM runs both halves through the MFMA.
//
// The micro-batch matters on the pages (a 512-token micro-batch "leaves ~45%
// of prefill" unused because each of the 256 experts sees too few tokens per
// matmul -- TrevorJS card, "Speed"): each workgroup owns one expert's weight
// slice and walks every token of that expert, so weights leave HBM once.
#include "moe_internal.h"

namespace bqmoe {

constexpr int kPfM = 64;        // tokens per chunk (4 MFMA column tiles)
constexpr int kPfLd = 128 + 8;  // LDS row pitch in bf16 (pad against bank conflicts)

// blockIdx -> (expert, block): the blocks of one expert land on one XCD (the
// dispatcher deals workgroups to the 8 XCDs round-robin), so its tokens are
// re-read from that XCD's L2.
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

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Grid: E * (I/64) blocks of 4 waves.  Wave w owns gate rows
// 16*(4*blk+w) .. +16 and the same up rows; the block walks the expert's
// tokens kPfM at a time, K in super-steps of 128 (x staged in LDS, double
// buffered).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_gateup_mxfp4(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed, size_t expert_bytes,
    int H, int I, int K, int E, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ perm, uint16_t *__restrict__ h_hi, uint16_t *__restrict__ h_lo) {
    __shared__ __align__(16) uint16_t xs[2][kPfM][kPfLd];
    int e, blk;
    map_expert_block(blockIdx.x, E, I / 64, &e, &blk);
    const int p0 = offsets[e];
    const int ne = offsets[e + 1] - p0;
    if (ne == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int ag = blk * 4 + wave;  // gate row group; up row group is I/16 + ag

    const uint8_t *ex = packed + (size_t)e * expert_bytes;
    const size_t kt = (size_t)(H / 32);
    const uint8_t *gcode = ex + (size_t)ag * kt * 256 + n * 16;
    const uint8_t *ucode = ex + (size_t)(I / 16 + ag) * kt * 256 + n * 16;
    const uint8_t *scl = ex + (size_t)I * H;
    const uint8_t *gscl = scl + (size_t)ag * kt * 16 + n;
    const uint8_t *uscl = scl + (size_t)(I / 16 + ag) * kt * 16 + n;
    const int nsuper = H / 128;

    // staging: thread -> (token row r = tid/4, 32-column part tid%4)
    const int sr = tid >> 2, sp = tid & 3;

    for (int c0 = 0; c0 < ne; c0 += kPfM) {
        const int nt = min(kPfM, ne - c0);
        const uint16_t *xrow = nullptr;
        if (sr < nt) xrow = x + (size_t)(perm[p0 + c0 + sr] / K) * H + sp * 32;
        uint4 stage[4];
        auto gload = [&](int J) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                stage[m] = xrow ? reinterpret_cast<const uint4 *>(xrow + 128 * J)[m]
                                : make_uint4(0u, 0u, 0u, 0u);
        };
        auto sstore = [&](int buf) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                *reinterpret_cast<uint4 *>(&xs[buf][sr][sp * 32 + 8 * m]) = stage[m];
        };
        f32x4 accg[4], accu[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            accg[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();  // previous chunk's readers are done with xs
        gload(0);
        sstore(0);
        __syncthreads();
        for (int J = 0; J < nsuper; ++J) {
            const int buf = J & 1;
            if (J + 1 < nsuper) gload(J + 1);
            const size_t tile = (size_t)(4 * J + q);
            const uint4 gv = *reinterpret_cast<const uint4 *>(gcode + tile * 256);
            const uint4 uv = *reinterpret_cast<const uint4 *>(ucode + tile * 256);
            const float gsc = e8m0_to_f32(gscl[tile * 16]);
            const float usc = e8m0_to_f32(uscl[tile * 16]);
            const uint32_t gd[4] = {gv.x, gv.y, gv.z, gv.w};
            const uint32_t ud[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 ag8 = fp4x8_to_bf16x8(gd[s], gsc);
                const bf16x8 au8 = fp4x8_to_bf16x8(ud[s], usc);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8 *>(&xs[buf][16 * t + n][32 * q + 8 * s]);
                    accg[t] = mfma_bf16(ag8, b, accg[t]);
                    accu[t] = mfma_bf16(au8, b, accu[t]);
                }
            }
            if (J + 1 < nsuper) sstore(buf ^ 1);
            __syncthreads();
        }
        // epilogue: lane holds rows 4q..4q+3 of the wave's 16-row group for token 16t+n
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int m = 16 * t + n;
            if (m < nt) {
                const size_t p = (size_t)(p0 + c0 + m);
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float hv = silu_f32(accg[t][jj]) * accu[t][jj];
                    hi[jj] = f32_to_bf16_rne(hv);
                    lo[jj] = f32_to_bf16_rne(hv - bf16_to_f32(hi[jj]));
                }
                const size_t col = (size_t)16 * ag + 4 * q;
                *reinterpret_cast<uint2 *>(h_hi + p * I + col) =
                    make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                *reinterpret_cast<uint2 *>(h_lo + p * I + col) =
                    make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down.  Grid: E * (H/64) blocks of 4 waves; wave w owns output rows
// 16*(4*blk+w) .. +16.  The h rows of an expert are contiguous (route-position
// order), staged hi and lo in LDS per 128-column super-step.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_down_mxfp4(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int E,
    const int32_t *__restrict__ offsets, const uint16_t *__restrict__ h_hi,
    const uint16_t *__restrict__ h_lo, float *__restrict__ y) {
    __shared__ __align__(16) uint16_t hs[2][2][kPfM][kPfLd];  // [buf][hi/lo][token][col]
    int e, blk;
    map_expert_block(blockIdx.x, E, H / 64, &e, &blk);
    const int p0 = offsets[e];
    const int ne = offsets[e + 1] - p0;
    if (ne == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int a = blk * 4 + wave;

    const uint8_t *ex = packed + (size_t)e * expert_bytes;
    const uint8_t *dcode = ex + (size_t)I * H + (size_t)I * H / 16;
    const uint8_t *dscl = dcode + (size_t)H * I / 2;
    const size_t kt = (size_t)(I / 32);
    const uint8_t *code = dcode + (size_t)a * kt * 256 + n * 16;
    const uint8_t *scal = dscl + (size_t)a * kt * 16 + n;
    const int nsuper = I / 128;
    const int sr = tid >> 2, sp = tid & 3;

    for (int c0 = 0; c0 < ne; c0 += kPfM) {
        const int nt = min(kPfM, ne - c0);
        const bool valid = sr < nt;
        const size_t rowoff = (size_t)(p0 + c0 + sr) * I + sp * 32;
        uint4 sh[4], sl[4];
        auto gload = [&](int J) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                sh[m] = valid ? reinterpret_cast<const uint4 *>(h_hi + rowoff + 128 * J)[m]
                              : make_uint4(0u, 0u, 0u, 0u);
                sl[m] = valid ? reinterpret_cast<const uint4 *>(h_lo + rowoff + 128 * J)[m]
                              : make_uint4(0u, 0u, 0u, 0u);
            }
        };
        auto sstore = [&](int buf) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                *reinterpret_cast<uint4 *>(&hs[buf][0][sr][sp * 32 + 8 * m]) = sh[m];
                *reinterpret_cast<uint4 *>(&hs[buf][1][sr][sp * 32 + 8 * m]) = sl[m];
            }
        };
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
        gload(0);
        sstore(0);
        __syncthreads();
        for (int J = 0; J < nsuper; ++J) {
            const int buf = J & 1;
            if (J + 1 < nsuper) gload(J + 1);
            const size_t tile = (size_t)(4 * J + q);
            const uint4 cv = *reinterpret_cast<const uint4 *>(code + tile * 256);
            const float sc = e8m0_to_f32(scal[tile * 16]);
            const uint32_t cd[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 a8 = fp4x8_to_bf16x8(cd[s], sc);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(&hs[buf][0][16 * t + n][32 * q + 8 * s]);
                    const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(&hs[buf][1][16 * t + n][32 * q + 8 * s]);
                    acc[t] = mfma_bf16(a8, bh, acc[t]);
                    acc[t] = mfma_bf16(a8, bl, acc[t]);
                }
            }
            if (J + 1 < nsuper) sstore(buf ^ 1);
            __syncthreads();
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int m = 16 * t + n;
            if (m < nt) {
                const size_t p = (size_t)(p0 + c0 + m);
                *reinterpret_cast<float4 *>(y + p * H + 16 * a + 4 * q) =
                    make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
            }
        }
    }
}

hipError_t launch_prefill_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                 const Workspace &ws, hipStream_t st) {
    (void)T;
    uint16_t *hh = static_cast<uint16_t *>(ws.h);
    uint16_t *hl = hh + (size_t)T * s.K * s.I;
    prefill_gateup_mxfp4<<<s.E * (s.I / 64), 256, 0, st>>>(x, packed, s.expert_bytes, s.H, s.I,
                                                           s.K, s.E, ws.offsets, ws.perm, hh, hl);
    return hipGetLastError();
}

hipError_t launch_prefill_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                               hipStream_t st) {
    const uint16_t *hh = static_cast<const uint16_t *>(ws.h);
    const uint16_t *hl = hh + (size_t)T * s.K * s.I;
    prefill_down_mxfp4<<<s.E * (s.H / 64), 256, 0, st>>>(packed, s.expert_bytes, s.H, s.I, s.E,
                                                         ws.offsets, hh, hl, ws.y);
    return hipGetLastError();
}

}  // namespace bqmoe
