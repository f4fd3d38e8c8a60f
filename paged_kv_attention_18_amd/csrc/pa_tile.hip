// pa_tile.hip -- the matrix-core kernels without the band mask, and the host
// side of their selection, occupancy and launch.  The kernels themselves are
// described in pa_tile_kernels.h.
#include "pa_tile_kernels.h"

namespace pa {

const void *tile_kernel_plain(int dtype, int dk, int dv, int variant, bool shared, TileShape *t)
{
    return kernel_select<MODE_PLAIN>(dtype, dk, dv, variant, shared, t);
}

namespace {

const void *tile_kernel_ptr(int dtype, int dk, int dv, int variant, bool shared, TileShape *t, int mode = MODE_PLAIN)
{
    if (mode == MODE_BAND)
        return tile_kernel_band(dtype, dk, dv, variant, shared, t);
    if (mode == MODE_TENSOR)
        return tile_kernel_tensor(dtype, dk, dv, variant, shared, t);
    if (mode == MODE_SPARSE)
        return tile_kernel_sparse(dtype, dk, dv, variant, shared, t);
    return tile_kernel_plain(dtype, dk, dv, variant, shared, t);
}

}  // namespace

bool tile_supported(int dk, int dv, int variant)
{
    TileShape t;
    return tile_kernel_ptr(0, dk, dv, variant, false, &t) != nullptr;
}

int tile_chunk(int dk, int dv, int variant, bool shared, int mode)
{
    TileShape t;
    return tile_kernel_ptr(0, dk, dv, variant, shared, &t, mode) ? t.kt : 0;
}

int tile_rows(int dk, int dv, int variant, bool shared, int mode)
{
    TileShape t;
    return tile_kernel_ptr(0, dk, dv, variant, shared, &t, mode) ? 16 * t.mb * (t.nw / t.cs) : 0;
}

bool tile_streaming(int dk, int dv, int variant)
{
    TileShape t;
    return tile_kernel_ptr(0, dk, dv, variant, false, &t) && t.nw == 1;
}

int tile_workers_per_cu(int dtype, int dk, int dv, int variant, bool shared, int mode)
{
    TileShape t;
    const void *k = tile_kernel_ptr(dtype, dk, dv, variant, shared, &t, mode);
    int n = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, t.threads, 0) != hipSuccess || n < 1)
        return 1;
    return n;
}

hipError_t launch_tile(const Params &p, int dtype, int variant, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    TileShape t;
    const int mode = p.band ? MODE_BAND : (p.tmask ? MODE_TENSOR : (p.sparse ? MODE_SPARSE : MODE_PLAIN));
    const void *k = tile_kernel_ptr(dtype, p.head_size_k, p.head_size_v, variant, p.shared_kv != 0, &t, mode);
    // the plan was made for this kernel's chunk and tile sizes
    if (!k || t.kt != p.chunk || 16 * t.mb * (t.nw / t.cs) != p.rows_per_tile)
        return hipErrorInvalidValue;
    // only the streaming kernel's variants 3 and 4 (6 and 7 on head pairs)
    // and the 576/512 kernel's variant 8 plan for themselves, for at most
    // kSelfPlanMaxBatch sequences, one static piece per workgroup (variants 4
    // and 7 may add claimed pieces) or, without split, one whole unit per
    // workgroup: the streaming kernel for at most 16 query tokens per
    // sequence, variant 8 for one row tile per (sequence, KV head) and no
    // whole-tile tasks
    const bool self_var = variant == 3 || variant == 4 || variant == 6 || variant == 7 || variant == 8;
    const bool tail_var = variant == 4 || variant == 7;
    if ((p.self_plan != 0) != self_var || (p.tail_min > 0) != tail_var ||
        (p.self_plan && (p.batch > kSelfPlanMaxBatch || (!p.no_split && p.pieces != p.partitions) ||
                         (t.nw == 1 ? p.max_q > 16 : (p.max_tiles != 1 || p.tile_order != 0)))))
        return hipErrorInvalidValue;
    void *args[] = {(void *)&p};
    return launch_kernel(k, dim3(p.partitions), dim3(t.threads), args, s, e0, e1);
}

}  // namespace pa
