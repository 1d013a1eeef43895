"""Pins for the tree / centralized oracle."""

import numpy as np
import pytest

import oracle
import workloads


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def test_parents_of_the_heap():
    assert oracle.tree_parents(8, 2) == [-1, 0, 0, 1, 1, 2, 2, 3]
    assert oracle.tree_parents(5, 4) == [-1, 0, 0, 0, 0]
    assert oracle.tree_parents(4, 1) == [-1, 0, 1, 2]


def test_binary_tree_p5_written_out():
    """P = 5, b = 2: node 1 holds (x1 + x3) + x4, node 2 holds x2, the root
    ((x0 + p1) + x2)."""
    X = workloads.rank_buffers(5, 300, dist="wide", seed=1)
    x = [X[r] for r in range(5)]
    p1 = (x[1] + x[3]) + x[4]
    want = (x[0] + p1) + x[2]
    Y, sent = oracle.tree_allreduce(X, "sum", 2)
    for r in range(5):
        assert np.array_equal(bits(Y[r]), bits(want))
    # up: every non-root sends once; down: nodes 0 and 1 send to 2 children each
    assert sent.tolist() == [2 * 300, 3 * 300, 300, 300, 300]


def test_chain_p4_written_out():
    """b = 1: a chain 0 <- 1 <- 2 <- 3 summed from the far end."""
    X = workloads.rank_buffers(4, 200, dist="wide", seed=2)
    want = X[0] + (X[1] + (X[2] + X[3]))
    Y, _ = oracle.tree_allreduce(X, "sum", 1)
    assert np.array_equal(bits(Y[0]), bits(want))


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 16])
def test_centralized_is_the_one_chunk_ring(P):
    """b >= P-1: the root adds the peers' tensors in rank order, the same
    association as a ring with a single chunk (started at rank 0)."""
    X = workloads.rank_buffers(P, 257, dist="wide", seed=P)
    for op in ("sum", "mean"):
        T, _ = oracle.tree_allreduce(X, op, max(1, P - 1))
        R, _ = oracle.ring_allreduce(X, op, 1)
        assert np.array_equal(bits(T), bits(R))


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_tree_integer_sums_exact_and_ranks_identical(b):
    P = 16
    X = workloads.rank_buffers(P, 500, "int", 1024, seed=b)
    Y, sent = oracle.tree_allreduce(X, "sum", b)
    assert np.array_equal(Y[0].astype(np.int64), X.astype(np.int64).sum(0))
    for r in range(1, P):
        assert np.array_equal(bits(Y[r]), bits(Y[0]))
    assert sent.sum() == 2 * (P - 1) * 500     # every edge carries n up and n down
    Ym, _ = oracle.tree_allreduce(X, "mean", b)
    assert np.array_equal(bits(Ym[0]), bits(Y[0] / np.float32(P)))


def test_tree_order_differs_from_ring():
    X = workloads.rank_buffers(8, 1000, dist="wide", seed=3)
    T, _ = oracle.tree_allreduce(X, "sum", 2)
    R, _ = oracle.ring_allreduce(X, "sum", 8)
    assert np.count_nonzero(bits(T[0]) != bits(R[0])) > 100
