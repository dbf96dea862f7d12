// measure.hip -- measurement aid: a plain streaming read of device memory,
// the attainable-read-bandwidth reference that the weight-streaming kernels'
// HBM rates are compared with.  Each thread reads 16-byte words with a
// grid-wide stride (consecutive lanes read consecutive words, so every wave
// load is one contiguous 1 KiB block, as in the decode kernels), with
// kProbeUnroll loads in flight; nothing is written.
#include "moe_internal.h"

namespace bqmoe {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocksPerCu = 8;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4 *__restrict__ buf,
                                                                   size_t n16,
                                                                   uint32_t *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = buf[i + u * stride];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // the loads feed acc, so they stay; the store almost never happens
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_read_probe(const uint8_t *buf, size_t bytes, uint32_t *sink, hipStream_t st) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    read_probe_kernel<<<cus * kProbeBlocksPerCu, kProbeThreads, 0, st>>>(
        reinterpret_cast<const uint4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace bqmoe
