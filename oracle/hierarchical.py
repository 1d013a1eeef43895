"""Two-level (local / global) all-reduce, simulated phase by phase.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (Burn collective blog, "Local strategy and global
strategy" and "Local ring downfall"):
* The all-reduce is split over two levels: a local (intra-node) level and a
  global (inter-node) level, and each level may use its own strategy
  (Centralized, Tree or Ring, section "Methods").
* Centralized and Tree split into a reduce and a broadcast, so with either
  of them locally the steps are: local reduce, then the global all-reduce,
  then a local broadcast.
* A ring cannot be split that way, so with Ring locally the steps are:
  local all-reduce, then the global all-reduce, then a local broadcast.

Readings where the pages are silent (listed in the design notes):
* P = G * Lr ranks in G nodes of Lr peers each, numbered node-major: rank
  g * Lr + l is local peer l of node g.
* Local peer 0 of every node is the node's root: it takes part in the
  global all-reduce and broadcasts the result to its node.  After a local
  ring all-reduce every peer holds the node's sum, so the choice does not
  change any value.
* Each level runs the single-level strategy of this package over its
  members: the chunked ring (``ring_allreduce``, with that level's chunk
  count) or the b-ary heap tree (``tree_allreduce``; Centralized is the
  tree whose root has every other member as a child).  At the global level
  the members are the node roots in node order.
* Both levels sum; Mean divides the global sum once, by P (every rank, not
  the number of nodes), with a correctly rounded division, before the
  broadcast.  Partial sums stay in the accumulation type across both levels.

Parity status: pinned by the tests against hand-worked values that tell
the two levels' orders apart from the flat ring (tests/golden), every
association written out for small shapes, exact integer sums, the
recursive-summation error bound, and the reductions to the single-level
strategies when G = 1 or Lr = 1.
"""

import numpy as np

from .ring import MEAN, SUM, _narrow, _widen, ring_allreduce
from .tree import tree_allreduce

RING = "ring"
TREE = "tree"
CENTRALIZED = "centralized"


def _level_sum(M, strategy, param, acc_dtype):
    """Sum the members' buffers M (m, n) with one level's strategy; returns
    the value every member holds afterwards, shape (m, n)."""
    m = M.shape[0]
    if strategy == RING:
        Y, _ = ring_allreduce(M, SUM, chunking=param if param else m, in_dtype=acc_dtype)
    elif strategy == TREE:
        Y, _ = tree_allreduce(M, SUM, branching=param, in_dtype=acc_dtype)
    elif strategy == CENTRALIZED:
        Y, _ = tree_allreduce(M, SUM, branching=max(1, m - 1), in_dtype=acc_dtype)
    else:
        raise ValueError(f"unknown strategy {strategy!r}")
    return Y


def hierarchical_allreduce(X, op=SUM, nodes=1, local=(RING, None), global_=(RING, None),
                           in_dtype="f32", out_dtype=None):
    """All-reduce P rank buffers over G = ``nodes`` nodes of P / G peers.

    local, global_: (strategy, parameter) with strategy ``"ring"``
    (parameter: the chunk count, default the level's member count),
    ``"tree"`` (parameter: the branching factor) or ``"centralized"``
    (parameter ignored).  Returns Y of shape (P, n) in ``out_dtype``
    (default: the input dtype), every rank's result.
    """
    A = _widen(X, in_dtype)
    if A.ndim != 2 or A.shape[0] < 1:
        raise ValueError("X must have shape (P, n)")
    if op not in (SUM, MEAN):
        raise ValueError(f"unknown op {op!r}")
    P, n = A.shape
    G = int(nodes)
    if G < 1 or P % G != 0:
        raise ValueError("nodes must divide the rank count")
    Lr = P // G
    acc = "f64" if A.dtype == np.float64 else "f32"

    # 1. Local phase in every node: a reduce to local peer 0 (Centralized,
    #    Tree) or an all-reduce (Ring); local peer 0 then holds the node sum.
    roots = np.empty((G, n), dtype=A.dtype)
    for g in range(G):
        Y = _level_sum(A[g * Lr:(g + 1) * Lr], local[0], local[1], acc)
        roots[g] = Y[0]

    # 2. Global all-reduce among the node roots.
    total = _level_sum(roots, global_[0], global_[1], acc)[0]

    # 3. Mean over all P ranks, once.
    if op == MEAN:
        total = total / A.dtype.type(P)

    # 4. Local broadcast: every peer of every node receives its root's value.
    out = np.empty_like(A)
    out[:] = total
    return _narrow(out, out_dtype or in_dtype)
