// pa_tile_tensor.hip -- the matrix-core kernels with the tensor mask (the
// shared mask matrix added to the scaled scores), instantiated in a
// translation unit of their own.
#include "pa_tile_kernels.h"

namespace pa {

const void *tile_kernel_tensor(int dtype, int dk, int dv, int variant, bool shared, TileShape *t)
{
    return kernel_select<MODE_TENSOR>(dtype, dk, dv, variant, shared, t);
}

}  // namespace pa
