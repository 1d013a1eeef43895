"""Centralized and tree all-reduce, simulated level by level on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (Burn collective blog, "Methods"): in the Centralized
strategy all peers send their tensors to a root, which aggregates them and
broadcasts the result back; in the Tree strategy peers are arranged in a
b-tree and reduce in parallel, in O(log_b N) time.  Both split into a
reduce followed by a broadcast (same page, "Local ring downfall").

Readings where the pages are silent (listed in the design notes):
* The tree is a b-ary heap over the ranks: rank 0 is the root and the
  children of rank i are ranks b*i + 1 ... b*i + b (those below P).
* The reduce runs level by level from the deepest: every node adds its
  children's partial sums to its own value in increasing child order, after
  all of them have arrived (a fixed order, independent of arrival times).
* Mean divides once, at the root, after the full sum; the broadcast then
  copies the root's value down the tree.
* With b >= P - 1 every peer is a child of the root: that is the
  Centralized strategy, the root adding the peers' tensors in rank order.
* Partial sums are float32 for fp32 and bf16 inputs (bf16 widened exactly).

Parity status: pinned by the tests against brute force on tiny inputs
(every association written out by hand for P = 4 and 5), exact integer
sums, the identity centralized == ring with one chunk (both start at rank 0
and add the ranks in order), and the traffic of the two phases.
"""

import numpy as np

from .ring import MEAN, SUM, _narrow, _widen


def tree_parents(P, branching):
    """parent[c] of every rank c >= 1 in the b-ary heap (parent[0] = -1)."""
    if branching < 1:
        raise ValueError("branching must be >= 1")
    return [-1] + [(c - 1) // branching for c in range(1, P)]


def tree_allreduce(X, op=SUM, branching=2, in_dtype="f32", out_dtype=None):
    """All-reduce P rank buffers along a b-ary tree: reduce to rank 0, then
    broadcast.  Returns (Y, sent) like ``ring_allreduce``."""
    A = _widen(X, in_dtype)
    if A.ndim != 2 or A.shape[0] < 1:
        raise ValueError("X must have shape (P, n)")
    if op not in (SUM, MEAN):
        raise ValueError(f"unknown op {op!r}")
    P, n = A.shape
    parent = tree_parents(P, branching)
    depth = [0] * P
    for c in range(1, P):
        depth[c] = depth[parent[c]] + 1
    children = [[c for c in range(1, P) if parent[c] == p] for p in range(P)]
    sent = np.zeros(P, dtype=np.int64)

    # Reduce: deepest level first; each node adds its children in order.
    for d in range(max(depth), -1, -1):
        for p in range(P):
            if depth[p] != d:
                continue
            for c in children[p]:
                A[p] = A[p] + A[c]
                sent[c] += n
    if op == MEAN:
        A[0] = A[0] / A.dtype.type(P)
    # Broadcast: level by level from the root.
    for d in range(0, max(depth) + 1):
        for p in range(P):
            if depth[p] != d:
                continue
            for c in children[p]:
                A[c] = A[p]
                sent[p] += n
    return _narrow(A, out_dtype or in_dtype), sent
