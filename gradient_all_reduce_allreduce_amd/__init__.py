"""MI355X-native gradient all-reduce for data-parallel training.

P ranks' gradient buffers are combined elementwise with Sum or Mean in the
order of a chunked ring (reduce-scatter then all-gather), every rank ending
with the same result; on one GPU the ranks are P buffers in HBM.  The work
runs in the HIP library ``libddp_allreduce.so`` (C ABI in
include/ddp_allreduce.h); this package is its Python binding.
"""

from .api import (SUM, MEAN, F32, BF16, MAX_RANKS, DdpError, ddp_bucket_plan, ddp_bucket_pack,
                  ddp_bucket_unpack, allreduce_ring_emulated, allreduce_fused_sgd,
                  reducescatter_ring_emulated, allgather_ring_emulated, allreduce_ring_stepwise,
                  allreduce_tree_emulated, ddp_multi_plan, ddp_multi_block_map,
                  allreduce_multi_ring_emulated,
                  allreduce, allreduce_stepwise, allreduce_tree, MultiAllReduce,
                  allreduce_sgd, reduce_scatter, all_gather, allreduce_hierarchical_emulated,
                  allreduce_hierarchical, zero1_sgd_step_emulated, zero1_sgd_step,
                  allreduce_multi_fused_sgd, allreduce_multi_ring_noalloc, ddp_set_wg_per_cu, KERNEL_FAMILIES,
                  allreduce_ring_buckets, allreduce_fused_sgd_buckets, zero1_sgd_step_buckets,
                  ddp_buckets_launch_count, reducescatter_ring_buckets, allgather_ring_buckets,
                  allreduce_ring_stepwise_buckets, allreduce_hierarchical_buckets)
from .bucketer import GradBucketer

__all__ = [
    "SUM", "MEAN", "F32", "BF16", "MAX_RANKS", "DdpError", "ddp_bucket_plan", "ddp_bucket_pack",
    "ddp_bucket_unpack", "allreduce_ring_emulated", "allreduce_fused_sgd",
    "reducescatter_ring_emulated", "allgather_ring_emulated", "allreduce_ring_stepwise",
    "allreduce_tree_emulated", "ddp_multi_plan", "ddp_multi_block_map", "allreduce_multi_ring_emulated",
    "allreduce",
    "allreduce_stepwise", "allreduce_tree", "MultiAllReduce",
    "allreduce_sgd",
    "reduce_scatter", "all_gather", "GradBucketer", "allreduce_hierarchical_emulated",
    "allreduce_hierarchical", "zero1_sgd_step_emulated", "zero1_sgd_step",
    "allreduce_multi_fused_sgd", "allreduce_multi_ring_noalloc", "ddp_set_wg_per_cu", "KERNEL_FAMILIES",
    "allreduce_ring_buckets", "allreduce_fused_sgd_buckets", "zero1_sgd_step_buckets",
    "ddp_buckets_launch_count", "reducescatter_ring_buckets", "allgather_ring_buckets",
    "allreduce_ring_stepwise_buckets", "allreduce_hierarchical_buckets",
]
