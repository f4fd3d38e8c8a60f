// pa_noalloc.hip -- pa_forward_noalloc, the entry point for callers that
// cannot allocate device memory: its workspace is a static device array that
// each GPU the library runs on holds for the life of the process.
#include <hip/hip_runtime.h>

#include <cstring>
#include <functional>
#include <mutex>

#include "pa.h"
#include "pa_internal.h"

// The workspace of pa_forward_noalloc, one copy per GPU.  In host code this
// name stands for a host-side shadow, not for device memory: host code only
// uses the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    pa_status status = PA_ERR_HIP;
    void *ptr = nullptr;   // this device's copy of `scratch`
    int num_cus = 256;
};

DeviceScratch g_device[kMaxDevices];

// Once per device, with that device current: its copy of the array, its
// architecture and its compute units.
void setup_device(DeviceScratch &d, int dev)
{
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        d.status = PA_ERR_HIP;
        return;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        d.status = PA_ERR_UNSUPPORTED;
        return;
    }
    void *ptr = nullptr;
    if (hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
        d.status = PA_ERR_HIP;
        return;
    }
    d.ptr = ptr;
    d.num_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
    d.status = PA_OK;
}

constexpr int kZeroThreads = 256;

__global__ __launch_bounds__(kZeroThreads) void zero_words_kernel(uint32_t *p, long long n)
{
    for (long long i = (long long)blockIdx.x * kZeroThreads + threadIdx.x; i < n;
         i += (long long)gridDim.x * kZeroThreads)
        p[i] = 0u;
}

}  // namespace

namespace pa {

hipError_t launch_zero_words(uint32_t *p, long long n, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    long long wgs = (n + kZeroThreads - 1) / kZeroThreads;
    if (wgs > 1024)
        wgs = 1024;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)wgs), dim3(kZeroThreads), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace pa

extern "C" pa_status pa_forward_noalloc(const pa_config *cfg, const void *query, const void *key_cache,
                                        const void *value_cache, const int32_t *block_tables,
                                        const int32_t *context_lens, const int32_t *q_seq_lens, int32_t batch,
                                        int32_t num_q_tokens, int32_t max_q_seq_len, void *out, float *lse,
                                        void *stream)
{
    const pa_status cst = pa::validate_config(cfg);   // before any HIP call
    if (cst != PA_OK)
        return cst;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return PA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return PA_ERR_UNSUPPORTED;
    DeviceScratch &d = g_device[dev];
    std::call_once(d.once, setup_device, std::ref(d), dev);
    if (d.status != PA_OK)
        return d.status;
    return pa::forward_in_buffer(cfg, d.num_cus, d.ptr, (size_t)PA_NOALLOC_SCRATCH_BYTES, query, key_cache,
                                 value_cache, block_tables, context_lens, q_seq_lens, batch, num_q_tokens,
                                 max_q_seq_len, out, lse, stream);
}
