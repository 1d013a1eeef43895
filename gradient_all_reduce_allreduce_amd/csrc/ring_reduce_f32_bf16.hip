// Ring all-reduce kernels with f32 inputs and bf16 outputs (see ring_reduce_impl.h).
#include "ring_reduce_impl.h"

DDP_RING_TYPE_PAIR(f32_bf16, false, true)
