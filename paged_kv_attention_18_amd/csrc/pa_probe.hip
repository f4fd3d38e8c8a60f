// pa_probe.hip -- a plain streaming read of device memory.  It measures the
// read rate the device sustains on one large contiguous buffer, which the
// attention kernels' achieved HBM bandwidth is reported beside (next to the
// nominal peak).  It is measurement support, not part of the forward pass.
#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;   // 16-byte loads in flight per thread

// Workgroup w reads the w-th contiguous share of the buffer; every lane keeps
// kProbeUnroll loads in flight.  One word per workgroup is written so the
// loads are kept.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *src, long long n16,
                                                                   uint32_t *sink)
{
    const long long per = (n16 + gridDim.x - 1) / gridDim.x;
    const long long lo = (long long)blockIdx.x * per;
    const long long hi = lo + per < n16 ? lo + per : n16;
    uint32_t acc = 0;
    for (long long i = lo + threadIdx.x; i < hi; i += (long long)kProbeThreads * kProbeUnroll) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const long long j = i + (long long)u * kProbeThreads;
            v[u] = j < hi ? src[j] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int o = 32; o > 0; o >>= 1)
        acc += __shfl_xor(acc, o);
    __shared__ uint32_t s_acc[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0)
        s_acc[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kProbeThreads / 64; ++w)
            t += s_acc[w];
        sink[blockIdx.x] = t;
    }
}

}  // namespace

hipError_t launch_read_probe(const void *src, long long bytes, uint32_t *sink, int workgroups, hipStream_t s)
{
    if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || workgroups <= 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, s, (const u32x4 *)src,
                       bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace pa
