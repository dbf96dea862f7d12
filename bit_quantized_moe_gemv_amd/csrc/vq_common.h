// vq_common.h -- device helpers shared by the VQ kernels (the packed formats
// are described with MOE_FMT_VQ13R8 and MOE_FMT_VQ13 in bqmoe.h).
#pragma once

#include "moe_internal.h"

namespace bqmoe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Exponent s with max * 2^-s in [2^14, 2^15), from the fp32 bits of a row's
// largest magnitude (0 for an all-zero row).
__device__ __forceinline__ int fp16_row_exponent(uint32_t maxbits) {
    if (maxbits == 0) return 0;
    const int e = (int)(maxbits >> 23);
    return (e == 0 ? -126 : e - 127) - 14;
}

// Four consecutive values of a per-route output row -> fp16 times 2^ey, ey
// putting their largest magnitude in [2^14, 2^15): y16[p][c..c+3] and
// yexp[p][c/4] (c a multiple of 4).
__device__ __forceinline__ void store_y16x4(uint16_t *__restrict__ y16, int8_t *__restrict__ yexp,
                                            size_t p, int H, int c, const float (&v)[4]) {
    const float mx = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    const int ey = max((int)((__float_as_uint(mx) >> 23) & 0xFFu) - 141, -128);
    union { _Float16 h[4]; uint2 u; } r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.h[i] = (_Float16)ldexpf(v[i], -ey);
    *reinterpret_cast<uint2 *>(y16 + p * H + c) = r.u;
    yexp[p * (H / 4) + c / 4] = (int8_t)ey;
}

// Block-wide maximum of non-negative fp32 bit patterns, compared as integers
// (the same order as the magnitudes, subnormals included).  *slot must be 0
// and visible to the block before the call.
__device__ __forceinline__ uint32_t block_max_bits(uint32_t v, uint32_t *slot) {
    atomicMax(slot, v);
    __syncthreads();
    return *slot;
}

// 12-bit index s (0..7) of a lane's 96-bit code12 run (little-endian stream).
template <int S>
__device__ __forceinline__ uint32_t code12_at(const uint32_t (&c)[6]) {
    constexpr int b = 12 * S, k = b / 32, sh = b % 32;
    if (sh + 12 <= 32 || k == 2) return (c[k] >> sh) & 0xFFFu;
    return __builtin_amdgcn_alignbit(c[k + 1], c[k], sh) & 0xFFFu;
}

// Book rows of vector s of a lane's run: c[0..2] code12, c[3..4] res, c[5]
// plane byte; i13 = code12 | plane << 12.
template <int S>
__device__ __forceinline__ void vq_indices(const uint32_t (&c)[6], uint32_t &i13, uint32_t &i8) {
    i13 = code12_at<S>(c) | (((c[5] >> S) & 1u) << 12);
    i8 = (c[3 + S / 4] >> (8 * (S % 4))) & 0xFFu;
}

__device__ __forceinline__ f16x8 add_f16x8(uint4 a, uint4 b) {
    return __builtin_bit_cast(f16x8, a) + __builtin_bit_cast(f16x8, b);
}

// A lane's index run of one 16 x 256 tile (12 code12 bytes, 8 res bytes or
// zero, 1 plane byte), read with non-temporal loads: every index byte is read
// once per forward, so it need not displace the cached rows and books.
typedef uint32_t u32x2nt __attribute__((ext_vector_type(2)));
template <bool RES>
__device__ __forceinline__ void vq_load_run(const uint8_t *c12, const uint8_t *res,
                                            const uint8_t *pln, size_t tile, int lane,
                                            uint32_t (&c)[6]) {
    const u32x3 a = __builtin_nontemporal_load(reinterpret_cast<const u32x3 *>(c12 + tile * 768 + lane * 12));
    c[0] = a.x;
    c[1] = a.y;
    c[2] = a.z;
    if (RES) {
        const u32x2nt r = __builtin_nontemporal_load(reinterpret_cast<const u32x2nt *>(res + tile * 512 + lane * 8));
        c[3] = r.x;
        c[4] = r.y;
    } else {
        c[3] = c[4] = 0;
    }
    c[5] = __builtin_nontemporal_load(pln + tile * 64 + lane);
}

// Byte regions of one VQ matrix of N rows and K columns; RES: the matrix
// carries the residual index region (VQ13R8) or not (VQ13).
template <bool RES>
struct VqMatrix {
    const uint8_t *c12, *pln, *res;
    const uint16_t *gain;
    __device__ __forceinline__ VqMatrix(const uint8_t *base, size_t N, size_t K) {
        const size_t nvec = N * K / 8;
        c12 = base;
        pln = c12 + nvec * 3 / 2;
        res = pln + nvec / 8;
        gain = reinterpret_cast<const uint16_t *>(res + (RES ? nvec : 0));
    }
    // lane's run of tile `tile`: 12 code12 bytes, 8 res bytes (zero without
    // the residual stage), 1 plane byte
    __device__ __forceinline__ void load(size_t tile, int lane, uint32_t (&c)[6]) const {
        vq_load_run<RES>(c12, res, pln, tile, lane, c);
    }
};

// Byte offset of the down matrix inside a VQ expert.
__host__ __device__ __forceinline__ size_t vq_down_offset(size_t H, size_t I, bool res) {
    const size_t nv0 = 2 * I * H / 8;
    return nv0 * 3 / 2 + nv0 / 8 + (res ? nv0 : 0) + 2 * (2 * I);
}

// Bytes of the layer's books in front of the experts.
template <bool RES>
__host__ __device__ constexpr size_t vq_books_bytes() {
    return RES ? kVqBooksBytes : kVq13BooksBytes;
}

// Compute units of the current device (persistent grids), 256 if unknown.
inline int device_cu_count() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        ncu < 1)
        ncu = 256;
    return ncu;
}

}  // namespace bqmoe
