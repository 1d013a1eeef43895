"""Pins for the ZeRO stage 1 oracle (sharded optimizer state)."""

import numpy as np
import pytest

import oracle
import workloads


def bits(a):
    a = np.ascontiguousarray(a)
    return a if a.dtype == np.uint16 else a.view(np.uint32)


def inputs(P, n, seed, in_dtype):
    X = workloads.rank_buffers(P, n, "normal", 1e-3, seed=seed)
    if in_dtype == "bf16":
        X = workloads.to_bf16_bits(X)
    w = workloads.rank_buffers(1, n, "normal", 0.02, seed=seed + 1)[0]
    v = workloads.rank_buffers(1, n, "normal", 1e-3, seed=seed + 2)[0]
    return X, w, v


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("in_dtype,param_dtype", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_stage1_equals_replicated_data_parallelism(P, in_dtype, param_dtype):
    """Stage 1 only partitions the optimizer state: the update equals the
    replicated one (all-reduce, then the same step on every replica) bit
    for bit, and every rank ends with the same parameters."""
    for n, C in ((1, 1), (37, P), (1000, 2 * P), (999, 3)):
        X, w, v = inputs(P, n, seed=P * 10 + n, in_dtype=in_dtype)
        for op in ("mean", "sum"):
            params, w1, v1, _ = oracle.zero1_sgd_step(X, w, v, 1e-3, 0.9, op, C, in_dtype, param_dtype)
            G, _ = oracle.ring_allreduce(X, op, C, in_dtype=in_dtype, out_dtype="f32")
            w2, v2 = oracle.sgd_momentum(G[0], w, v, 1e-3, 0.9)
            assert np.array_equal(bits(w1), bits(w2))
            assert np.array_equal(bits(v1), bits(v2))
            want = w2 if param_dtype == "f32" else oracle.f32_to_bf16_bits(w2)
            for r in range(P):
                assert np.array_equal(bits(params[r]), bits(want)), (r, n, C, op)


def test_first_step_from_zero_momentum():
    """v0 = 0: v = g and w = w0 - fl(lr * g), with g the ring Mean."""
    P, n = 4, 300
    X, w, _ = inputs(P, n, seed=3, in_dtype="f32")
    v0 = np.zeros(n, np.float32)
    _, w1, v1, _ = oracle.zero1_sgd_step(X, w, v0, 0.5, 0.9, "mean", P)
    g, _ = oracle.ring_allreduce(X, "mean", P)
    assert np.array_equal(bits(v1), bits(g[0]))
    assert np.array_equal(bits(w1), bits(w - np.float32(0.5) * g[0]))


def test_every_element_is_updated_exactly_once():
    """With mu = 1, lr = 1 and integer data every operation is exact: an
    element stepped twice, or not at all, would show."""
    P, n = 5, 203
    X = workloads.rank_buffers(P, n, "int", 8, seed=4)
    w = np.zeros(n, np.float32)
    v = workloads.rank_buffers(1, n, "int", 8, seed=5)[0]
    params, w1, v1, _ = oracle.zero1_sgd_step(X, w, v, 1.0, 1.0, "sum", 3)
    g = X.astype(np.int64).sum(0)
    assert np.array_equal(v1.astype(np.int64), v.astype(np.int64) + g)
    assert np.array_equal(w1.astype(np.int64), -(v.astype(np.int64) + g))
    assert np.array_equal(params[2].astype(np.int64), -(v.astype(np.int64) + g))


@pytest.mark.parametrize("P", [2, 4, 8])
def test_traffic_equals_the_all_reduce(P):
    """Reduce-scatter + all-gather move 2(P-1)/P of the tensor per rank, the
    same as the replicated ring all-reduce: stage 1 costs no extra
    communication."""
    n = 64 * P
    X, w, v = inputs(P, n, seed=P, in_dtype="f32")
    _, _, _, sent = oracle.zero1_sgd_step(X, w, v, 1e-3, 0.9, "mean", P)
    _, sent_ar = oracle.ring_allreduce(X, "mean", P)
    assert sent.tolist() == sent_ar.tolist()
    assert np.all(sent == 2 * (P - 1) * n // P)


def test_rejects_unknown_arguments():
    X, w, v = inputs(2, 8, seed=0, in_dtype="f32")
    with pytest.raises(ValueError):
        oracle.zero1_sgd_step(X, w, v, 1e-3, 0.9, "max")
    with pytest.raises(ValueError):
        oracle.zero1_sgd_step(X, w, v, 1e-3, 0.9, "mean", 2, "f32", "f16")
