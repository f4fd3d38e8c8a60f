// pa_tile_sparse.hip -- the matrix-core kernels for sparse lists (each query
// token attends over the cache tokens its list selects), instantiated in a
// translation unit of their own.
#include "pa_tile_kernels.h"

namespace pa {

const void *tile_kernel_sparse(int dtype, int dk, int dv, int variant, bool shared, TileShape *t)
{
    return kernel_select<MODE_SPARSE>(dtype, dk, dv, variant, shared, t);
}

}  // namespace pa
