// pa_tile_band.hip -- the matrix-core kernels with the band mask (a lower
// visibility bound per row), instantiated in a translation unit of their own.
#include "pa_tile_kernels.h"

namespace pa {

const void *tile_kernel_band(int dtype, int dk, int dv, int variant, bool shared, TileShape *t)
{
    return kernel_select<MODE_BAND>(dtype, dk, dv, variant, shared, t);
}

}  // namespace pa
