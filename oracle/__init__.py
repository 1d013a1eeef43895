"""CPU oracle for the data-parallel gradient all-reduce.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct statement of what the hot path computes.  It exists so that the HIP
path can be checked against something written from the pages rather than
from the kernels.  Only the test suite, the package-level ``smoke()`` check
and the CPU-baseline leg of the benchmark may import it; the product path
(the C-ABI library and its Python binding) never does, and fails loudly
when its native library is missing instead of falling back here.

It shares no code with the HIP path: no kernels, headers, helpers, tables
or constant generators.  It is NumPy only (plus ``fractions`` in a few
exact checks), single-threaded, and each function cites the passage of the
pages it follows:

* "Burn collective" blog post (cielbird.github.io/blog/burn-distributed),
  section "Methods" (Centralized / Tree / Ring).
* Burn distributed-computing guide (pgsm.cn/news/420861), section on the
  reduction configuration (ReduceOperation Sum / Mean, all_reduce returning
  the result to every device).
* "Distributed Training" (computervisiononline.com/explains/
  distributed-training), sections "Data parallelism and all-reduce",
  "Sharded data parallelism", "Communication costs" and "How to Apply It".
* CS336 "Lecture 8 - Parallelism" (rd.me/cs336/lec8), "Collective
  Operations" and "Data Parallelism (DDP)".

Modules:
    ring    -- the chunked ring all-reduce simulated step by step, and its
               two halves (reduce-scatter, all-gather) on their own
    bf16    -- bfloat16 <-> float32 conversions by definition
    sgd     -- SGD with momentum on fp32 master weights
    bucket  -- reverse-order gradient bucketing, pack and unpack
    tree    -- the centralized and b-ary tree all-reduce
    hierarchical -- the two-level (local / global) all-reduce
    zero    -- ZeRO stage 1: reduce-scatter, the owner's optimizer step,
               all-gather of the updated parameters

Parity status of each function is stated in its module header.
"""

from .ring import (SUM, MEAN, chunk_length, chunk_owners, chunk_start_ranks,
                   chunk_start_ranks_at, ring_all_gather, ring_allreduce,
                   ring_allreduce_sampled, ring_reduce_scatter)
from .tree import tree_allreduce, tree_parents
from .hierarchical import hierarchical_allreduce
from .zero import zero1_sgd_step
from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from .sgd import sgd_momentum
from .bucket import bucket_plan, pack, unpack

__all__ = [
    "SUM", "MEAN", "chunk_length", "chunk_owners", "chunk_start_ranks",
    "chunk_start_ranks_at", "ring_all_gather", "ring_allreduce", "ring_reduce_scatter",
    "ring_allreduce_sampled", "bf16_bits_to_f32", "f32_to_bf16_bits",
    "sgd_momentum", "bucket_plan", "pack", "unpack", "tree_allreduce", "tree_parents",
    "hierarchical_allreduce", "zero1_sgd_step",
]
