"""ZeRO stage 1: the optimizer state sharded over the ranks, simulated phase
by phase.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("Distributed Training", "Sharded data parallelism: ZeRO
and FSDP"):
* Stage 1 partitions the optimizer states -- the 32-bit master weights and
  the optimizer's moments -- across the data-parallel ranks, so that each
  rank updates only its partition.
* In PyTorch's ZeroRedundancyOptimizer (stage 1 in DeepSpeed's terms) each
  parameter belongs to one rank, whose local optimizer updates it, and the
  updated parameters are then sent to all ranks.
* The model's parameters are 16-bit and the master copy 32-bit (mixed
  precision, same section and "Mixed-Precision Training").

Readings where the pages are silent (listed in the design notes):
* The partition is the ring's own: element i belongs to the owner of its
  chunk, the rank where the chunk's reduce-scatter ends, so the reduced
  gradient arrives exactly where it is used.  The reduce-scatter then
  replaces the all-reduce of replicated data parallelism.
* The owner's update is the momentum step of ``oracle.sgd`` on the reduced
  float32 gradient (after Mean), with one rounding per operation.
* The owner rounds its updated master weights to the parameter dtype (bf16:
  nearest even) and the ring's all-gather delivers them to every rank.
* Every shard of the master weights and of the momentum lives at its owner;
  the (n,) arrays here are the union of the P shards, element i held by its
  owner.

Parity status: pinned by the tests against replicated data parallelism
(all-reduce, then the same step on every replica: stage 1 partitions the
state without changing the update, so the bits must agree), the closed form
of the first step from zero momentum, every element updated exactly once,
and the traffic of the two halves (together the all-reduce's).
"""

import numpy as np

from .bf16 import f32_to_bf16_bits
from .ring import MEAN, SUM, ring_all_gather, ring_reduce_scatter
from .sgd import sgd_momentum


def zero1_sgd_step(X, w, v, lr, mu, op=MEAN, chunking=None, in_dtype="f32", param_dtype="f32"):
    """One stage-1 step over P ranks' gradients X (P, n).

    w, v: the (n,) float32 master weights and momentum (all shards).
    Returns (params, w_new, v_new, sent): params (P, n) every rank's updated
    parameters in ``param_dtype`` ("f32", or "bf16" as uint16 bit patterns),
    the new master weights and momentum, and the elements each rank sent
    over both phases.
    """
    if op not in (SUM, MEAN):
        raise ValueError(f"unknown op {op!r}")
    # 1. Reduce-scatter: the owner of element i holds its reduced gradient.
    R, owner, sent_rs = ring_reduce_scatter(X, op, chunking, in_dtype=in_dtype, out_dtype="f32")
    P, n = R.shape
    w = np.asarray(w, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    w_new = np.empty(n, dtype=np.float32)
    v_new = np.empty(n, dtype=np.float32)
    B = np.zeros((P, n), dtype=np.float32 if param_dtype == "f32" else np.uint16)
    # 2. Each rank steps its own shard and rounds it to the parameter dtype.
    for r in range(P):
        mine = np.flatnonzero(owner == r)
        w_new[mine], v_new[mine] = sgd_momentum(R[r, mine], w[mine], v[mine], lr, mu)
        if param_dtype == "f32":
            B[r, mine] = w_new[mine]
        elif param_dtype == "bf16":
            B[r, mine] = f32_to_bf16_bits(w_new[mine])
        else:
            raise ValueError(f"unknown parameter dtype {param_dtype!r}")
    # 3. All-gather of the updated parameters from their owners.
    params, sent_ag = ring_all_gather(B, chunking)
    return params, w_new, v_new, sent_rs + sent_ag
