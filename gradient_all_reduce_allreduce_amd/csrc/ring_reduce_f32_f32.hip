// Ring all-reduce kernels with f32 inputs and f32 outputs (see ring_reduce_impl.h).
#include "ring_reduce_impl.h"

DDP_RING_TYPE_PAIR(f32_f32, false, false)
