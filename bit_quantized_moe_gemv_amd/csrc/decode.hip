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

// fp32 pairs of a 16-byte fp4 block: out[b] = columns (2b, 2b+1) * scale.
__device__ __forceinline__ void fp4x32_to_f32(const uint4 v, float scale, f32x2 *out) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], scale, 0);
        out[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], scale, 1);
        out[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], scale, 2);
        out[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], scale, 3);
    }
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Grid: (expert slots, I/16).  Block: 4 waves; the block
// owns 16 gate rows and the matching 16 up rows of one active expert, the
// waves split the K super-steps (J = wave, wave+4, ...).  Each wave loads all
// of its packed bytes up front (MAXJ super-steps), then sweeps the expert's
// routes kDecTC at a time with x staged in LDS.  h is written in fp32, in
// route-position order: h[p][i].
// ---------------------------------------------------------------------------
template <int MAXJ>
__global__ __launch_bounds__(256) void decode_gateup_mxfp4(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed, size_t expert_bytes,
    int H, int I, int K, const int32_t *__restrict__ active, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ perm, float *__restrict__ h) {
    extern __shared__ __align__(16) uint16_t xs[];  // [kDecTC][H]
    __shared__ float red[4][kDecTC][16][2];
    const int slot = blockIdx.x;
    if (slot >= active[0]) return;
    const int e = active[1 + slot];
    const int p0 = offsets[e];
    const int ne = offsets[e + 1] - p0;
    const int rg = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, q = lane >> 4;

    const uint8_t *ex = packed + (size_t)e * expert_bytes;
    const size_t kt = (size_t)(H / 32);  // tiles along K per row group
    const uint8_t *gcode = ex + (size_t)rg * kt * 256;
    const uint8_t *ucode = ex + (size_t)(I / 16 + rg) * kt * 256;
    const uint8_t *scl = ex + (size_t)I * H;  // gate/up scale region
    const uint8_t *gscl = scl + (size_t)rg * kt * 16;
    const uint8_t *uscl = scl + (size_t)(I / 16 + rg) * kt * 16;
    const int nsuper = H / 128;

    uint4 gv[MAXJ], uv[MAXJ];
    uint32_t gs[MAXJ], us[MAXJ];
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
        const int J = wave + 4 * j;
        if (J < nsuper) {
            const size_t tile = (size_t)(4 * J + q);
            gv[j] = *reinterpret_cast<const uint4 *>(gcode + tile * 256 + n * 16);
            uv[j] = *reinterpret_cast<const uint4 *>(ucode + tile * 256 + n * 16);
            gs[j] = gscl[tile * 16 + n];
            us[j] = uscl[tile * 16 + n];
        }
    }

    for (int c0 = 0; c0 < ne; c0 += kDecTC) {
        const int nt = min(kDecTC, ne - c0);
        __syncthreads();
        const int per_row = H / 8;  // uint4 per x row
        for (int i = tid; i < nt * per_row; i += 256) {
            const int r = i / per_row, c = i - r * per_row;
            const int t = perm[p0 + c0 + r] / K;
            reinterpret_cast<uint4 *>(xs)[r * per_row + c] =
                reinterpret_cast<const uint4 *>(x + (size_t)t * H)[c];
        }
        __syncthreads();
        float ga[kDecTC], ua[kDecTC];
#pragma unroll
        for (int tt = 0; tt < kDecTC; ++tt) { ga[tt] = 0.f; ua[tt] = 0.f; }
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            const int J = wave + 4 * j;
            if (J < nsuper) {
                bf16x2 gw[16], uw[16];
                fp4x32_to_bf16(gv[j], e8m0_to_f32(gs[j]), gw);
                fp4x32_to_bf16(uv[j], e8m0_to_f32(us[j]), uw);
#pragma unroll
                for (int tt = 0; tt < kDecTC; ++tt) {
                    if (tt < nt) {
                        const uint4 *xr =
                            reinterpret_cast<const uint4 *>(xs + tt * H + 128 * J + 32 * q);
                        union { uint4 u[4]; bf16x2 p[16]; } xv;
#pragma unroll
                        for (int m = 0; m < 4; ++m) xv.u[m] = xr[m];
                        float g = ga[tt], u = ua[tt];
#pragma unroll
                        for (int b = 0; b < 16; ++b) {
                            g = __builtin_amdgcn_fdot2_f32_bf16(gw[b], xv.p[b], g, false);
                            u = __builtin_amdgcn_fdot2_f32_bf16(uw[b], xv.p[b], u, false);
                        }
                        ga[tt] = g;
                        ua[tt] = u;
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < kDecTC; ++tt) {
            ga[tt] += __shfl_xor(ga[tt], 16, 64);
            ga[tt] += __shfl_xor(ga[tt], 32, 64);
            ua[tt] += __shfl_xor(ua[tt], 16, 64);
            ua[tt] += __shfl_xor(ua[tt], 32, 64);
            if (q == 0) {
                red[wave][tt][n][0] = ga[tt];
                red[wave][tt][n][1] = ua[tt];
            }
        }
        __syncthreads();
        if (tid < nt * 16) {
            const int tt = tid >> 4, nn = tid & 15;
            const float g = ((red[0][tt][nn][0] + red[1][tt][nn][0]) + red[2][tt][nn][0]) + red[3][tt][nn][0];
            const float u = ((red[0][tt][nn][1] + red[1][tt][nn][1]) + red[2][tt][nn][1]) + red[3][tt][nn][1];
            h[(size_t)(p0 + c0 + tt) * I + 16 * rg + nn] = silu_f32(g) * u;
        }
    }
}

// ---------------------------------------------------------------------------
// down projection + weighted combine.  Grid: (expert slots, H/64).  Block: 4
// waves, wave w owns output row group 4*blockIdx.y + w (16 rows) and sweeps all
// I/128 super-steps itself.  y[p][j] is written per route position; the last
// block to finish a 64-row block (counted with a device-scope atomic) forms
// out[t][j] = sum_s w[t,s] * y[inv[t,s]][j] in slot order, so the result does
// not depend on block timing.
// ---------------------------------------------------------------------------
template <int MAXJ>
__global__ __launch_bounds__(256) void decode_down_mxfp4(
    const uint8_t *__restrict__ packed, size_t expert_bytes, int H, int I, int K, int T,
    const int32_t *__restrict__ active, const int32_t *__restrict__ offsets,
    const float *__restrict__ h, float *__restrict__ y, const float *__restrict__ wts,
    const int32_t *__restrict__ inv, uint32_t *__restrict__ sync, float *__restrict__ out) {
    extern __shared__ __align__(16) float hs[];  // [kDecTC][I]
    __shared__ int s_last;
    const int slot = blockIdx.x;
    const int n_active = active[0];
    if (slot >= n_active) return;
    const int e = active[1 + slot];
    const int p0 = offsets[e];
    const int ne = offsets[e + 1] - p0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int a = blockIdx.y * 4 + wave;  // output row group

    const uint8_t *ex = packed + (size_t)e * expert_bytes;
    const uint8_t *dcode = ex + (size_t)I * H + (size_t)I * H / 16;
    const uint8_t *dscl = dcode + (size_t)H * I / 2;
    const size_t kt = (size_t)(I / 32);
    const int nsuper = I / 128;

    uint4 cv[MAXJ];
    uint32_t cs[MAXJ];
#pragma unroll
    for (int J = 0; J < MAXJ; ++J) {
        if (J < nsuper) {
            const size_t tile = (size_t)a * kt + 4 * J + q;
            cv[J] = *reinterpret_cast<const uint4 *>(dcode + tile * 256 + n * 16);
            cs[J] = dscl[tile * 16 + n];
        }
    }

    for (int c0 = 0; c0 < ne; c0 += kDecTC) {
        const int nt = min(kDecTC, ne - c0);
        __syncthreads();
        const int per_row = I / 4;  // float4 per h row
        for (int i = tid; i < nt * per_row; i += 256)
            reinterpret_cast<float4 *>(hs)[i] =
                reinterpret_cast<const float4 *>(h + (size_t)(p0 + c0) * I)[i];
        __syncthreads();
        float acc[kDecTC];
#pragma unroll
        for (int tt = 0; tt < kDecTC; ++tt) acc[tt] = 0.f;
#pragma unroll
        for (int J = 0; J < MAXJ; ++J) {
            if (J < nsuper) {
                f32x2 wv[16];
                fp4x32_to_f32(cv[J], e8m0_to_f32(cs[J]), wv);
#pragma unroll
                for (int tt = 0; tt < kDecTC; ++tt) {
                    if (tt < nt) {
                        const float4 *hr =
                            reinterpret_cast<const float4 *>(hs + tt * I + 128 * J + 32 * q);
                        float s = acc[tt];
#pragma unroll
                        for (int m = 0; m < 8; ++m) {
                            const float4 hv = hr[m];
                            s = __builtin_fmaf(wv[2 * m].x, hv.x, s);
                            s = __builtin_fmaf(wv[2 * m].y, hv.y, s);
                            s = __builtin_fmaf(wv[2 * m + 1].x, hv.z, s);
                            s = __builtin_fmaf(wv[2 * m + 1].y, hv.w, s);
                        }
                        acc[tt] = s;
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < kDecTC; ++tt) {
            acc[tt] += __shfl_xor(acc[tt], 16, 64);
            acc[tt] += __shfl_xor(acc[tt], 32, 64);
            if (q == 0 && tt < nt) y[(size_t)(p0 + c0 + tt) * H + 16 * a + n] = acc[tt];
        }
    }

    // publish y, then count arrivals for this 64-row block
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&sync[blockIdx.y], 1u);
        s_last = (prev == (uint32_t)(n_active - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const int j0 = blockIdx.y * 64;
    for (int i = tid; i < T * 64; i += 256) {
        const int t = i >> 6, j = j0 + (i & 63);
        float acc = 0.f;
        for (int s = 0; s < K; ++s)
            acc = __builtin_fmaf(wts[t * K + s], y[(size_t)inv[t * K + s] * H + j], acc);
        out[(size_t)t * H + j] = acc;
    }
}

template <int MAXJ>
static hipError_t gateup_launch(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                const Workspace &ws, hipStream_t st) {
    const int slots = min(s.E, T * s.K);
    dim3 grid(slots, s.I / 16);
    const size_t lds = (size_t)kDecTC * s.H * 2;
    decode_gateup_mxfp4<MAXJ><<<grid, 256, lds, st>>>(x, packed, s.expert_bytes, s.H, s.I, s.K,
                                                      ws.active, ws.offsets, ws.perm,
                                                      static_cast<float *>(ws.h));
    return hipGetLastError();
}

hipError_t launch_decode_gateup(const Shape &s, int T, const uint16_t *x, const uint8_t *packed,
                                const Workspace &ws, hipStream_t st) {
    const int per_wave = (s.H / 128 + 3) / 4;
    if (per_wave <= 1) return gateup_launch<1>(s, T, x, packed, ws, st);
    if (per_wave <= 2) return gateup_launch<2>(s, T, x, packed, ws, st);
    if (per_wave <= 4) return gateup_launch<4>(s, T, x, packed, ws, st);
    if (per_wave <= 8) return gateup_launch<8>(s, T, x, packed, ws, st);
    if (per_wave <= 16) return gateup_launch<16>(s, T, x, packed, ws, st);
    return hipErrorInvalidValue;
}

template <int MAXJ>
static hipError_t down_launch(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                              float *out, hipStream_t st) {
    const int slots = min(s.E, T * s.K);
    dim3 grid(slots, s.H / 64);
    const size_t lds = (size_t)kDecTC * s.I * 4;
    decode_down_mxfp4<MAXJ><<<grid, 256, lds, st>>>(packed, s.expert_bytes, s.H, s.I, s.K, T,
                                                    ws.active, ws.offsets,
                                                    static_cast<const float *>(ws.h), ws.y, ws.w,
                                                    ws.inv, ws.sync, out);
    return hipGetLastError();
}

hipError_t launch_decode_down(const Shape &s, int T, const uint8_t *packed, const Workspace &ws,
                              float *out, hipStream_t st) {
    const int nsuper = s.I / 128;
    if (nsuper <= 1) return down_launch<1>(s, T, packed, ws, out, st);
    if (nsuper <= 2) return down_launch<2>(s, T, packed, ws, out, st);
    if (nsuper <= 4) return down_launch<4>(s, T, packed, ws, out, st);
    if (nsuper <= 8) return down_launch<8>(s, T, packed, ws, out, st);
    if (nsuper <= 16) return down_launch<16>(s, T, packed, ws, out, st);
    return hipErrorInvalidValue;
}

}  // namespace bqmoe
