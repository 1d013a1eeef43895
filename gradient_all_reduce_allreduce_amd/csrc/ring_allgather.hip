// Ring all-gather kernels (see ring_reduce_impl.h), by element size.
#include "ring_reduce_impl.h"

namespace ddp {

const void* ring_ag_kernel(int elem_bytes, int P, int scalar) {
    if (elem_bytes == 2) return scalar ? rr::ring_ag_kernel_for<2, true>(P) : rr::ring_ag_kernel_for<2, false>(P);
    return scalar ? rr::ring_ag_kernel_for<4, true>(P) : rr::ring_ag_kernel_for<4, false>(P);
}

}  // namespace ddp
