// Ring all-reduce kernels with bf16 inputs and f32 outputs (see ring_reduce_impl.h).
#include "ring_reduce_impl.h"

DDP_RING_TYPE_PAIR(bf16_f32, true, false)
