// Ring all-reduce kernels with bf16 inputs and bf16 outputs (see ring_reduce_impl.h).
#include "ring_reduce_impl.h"

DDP_RING_TYPE_PAIR(bf16_bf16, true, true)
