// pa_tile.hip -- the matrix-core kernels without the band mask, and the host
// side of their selection, occupancy and launch.  The kernels themselves are
// described in pa_tile_kernels.h.
#include "pa_tile_kernels.h"

namespace pa {

const void *tile_kernel_plain(int dtype, int dk, int dv, int variant, bool shared, TileShape *t)
{
    return kernel_select<false>(dtype, dk, dv, variant, shared, t);
}

namespace {

const void *tile_kernel_ptr(int dtype, int dk, int dv, int variant, bool shared, TileShape *t, bool band = false)
{
    return band ? tile_kernel_band(dtype, dk, dv, variant, shared, t)
                : tile_kernel_plain(dtype, dk, dv, variant, shared, t);
}

}  // namespace

bool tile_supported(int dk, int dv, int variant)
{
    TileShape t;
    return tile_kernel_ptr(0, dk, dv, variant, false, &t) != nullptr;
}

int tile_chunk(int dk, int dv, int variant, bool shared)
{
    TileShape t;
    return tile_kernel_ptr(0, dk, dv, variant, shared, &t) ? t.kt : 0;
}

int tile_rows(int dk, int dv, int variant, bool shared)
{
    TileShape t;
    return tile_kernel_ptr(0, dk, dv, variant, shared, &t) ? 16 * t.mb * (t.nw / t.cs) : 0;
}

bool tile_streaming(int dk, int dv, int variant)
{
    TileShape t;
    return tile_kernel_ptr(0, dk, dv, variant, false, &t) && t.nw == 1;
}

int tile_workers_per_cu(int dtype, int dk, int dv, int variant, bool shared, bool band)
{
    TileShape t;
    const void *k = tile_kernel_ptr(dtype, dk, dv, variant, shared, &t, band);
    int n = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, t.threads, 0) != hipSuccess || n < 1)
        return 1;
    return n;
}

hipError_t launch_tile(const Params &p, int dtype, int variant, hipStream_t s)
{
    TileShape t;
    const void *k = tile_kernel_ptr(dtype, p.head_size_k, p.head_size_v, variant, p.shared_kv != 0, &t, p.band != 0);
    if (!k)
        return hipErrorInvalidValue;
    void *args[] = {(void *)&p};
    return hipLaunchKernel(k, dim3(p.partitions), dim3(t.threads), args, 0, s);
}

}  // namespace pa
