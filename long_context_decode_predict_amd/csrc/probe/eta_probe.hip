// eta_probe.hip -- streaming read probes (see include/eta_probe.h): the HBM read
// bandwidth plain kernels sustain with the ETA kernels' 16-byte loads, from one
// buffer, or from two buffers read chunk by chunk together as the attention
// reads K and V.
#include "eta_probe.h"

#include "../eta_device.hpp"

namespace {

constexpr int kProbeThreads = 256;
constexpr size_t kChunkBytes = 32768;
constexpr int kLoadsPerThread = kChunkBytes / (16 * kProbeThreads);  // 8
constexpr uint32_t kNeverValue = 0x9e3779b9u;

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4 *__restrict__ p,
                                                                    uint32_t *__restrict__ sink) {
    const uint4 *q = p + (size_t)blockIdx.x * (kChunkBytes / 16) + threadIdx.x;
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
        const uint4 v = NT ? eta::ld_stream(q + i * kProbeThreads) : q[i * kProbeThreads];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kNeverValue) sink[threadIdx.x] = acc;
}

constexpr size_t kPairChunkBytes = 16384;
constexpr int kPairLoads = kPairChunkBytes / (16 * kProbeThreads);  // 4 per buffer

__global__ __launch_bounds__(kProbeThreads) void pair_read_kernel(const uint4 *__restrict__ a,
                                                                  const uint4 *__restrict__ b,
                                                                  uint32_t *__restrict__ sink) {
    const size_t off = (size_t)blockIdx.x * (kPairChunkBytes / 16) + threadIdx.x;
    uint4 v[2 * kPairLoads];
#pragma unroll
    for (int i = 0; i < kPairLoads; ++i) v[i] = eta::ld_stream(a + off + i * kProbeThreads);
#pragma unroll
    for (int i = 0; i < kPairLoads; ++i) v[kPairLoads + i] = eta::ld_stream(b + off + i * kProbeThreads);
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 2 * kPairLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == kNeverValue) sink[threadIdx.x] = acc;
}

}  // namespace

extern "C" int eta_probe_pair_read(const void *a, const void *b, size_t bytes, uint32_t *sink,
                                   hipStream_t stream) {
    if (a == nullptr || b == nullptr || sink == nullptr || bytes == 0 || bytes % kPairChunkBytes != 0)
        return -1;
    if (reinterpret_cast<uintptr_t>(a) % 16 != 0 || reinterpret_cast<uintptr_t>(b) % 16 != 0) return -1;
    const size_t chunks = bytes / kPairChunkBytes;
    if (chunks > 0x7fffffffull) return -1;
    hipLaunchKernelGGL(pair_read_kernel, dim3((unsigned)chunks), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4 *>(a), static_cast<const uint4 *>(b), sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int eta_probe_stream_read(const void *buf, size_t bytes, int nontemporal,
                                     uint32_t *sink, hipStream_t stream) {
    if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % kChunkBytes != 0) return -1;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return -1;
    const size_t chunks = bytes / kChunkBytes;
    if (chunks > 0x7fffffffull) return -1;
    const uint4 *p = static_cast<const uint4 *>(buf);
    if (nontemporal) {
        hipLaunchKernelGGL(stream_read_kernel<true>, dim3((unsigned)chunks), dim3(kProbeThreads), 0,
                           stream, p, sink);
    } else {
        hipLaunchKernelGGL(stream_read_kernel<false>, dim3((unsigned)chunks), dim3(kProbeThreads),
                           0, stream, p, sink);
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
