"""Pins for the ring oracle: it is checked against things other than itself.

* a closed-form fold derived by hand from the ring reading (a different
  formulation: no steps, no snapshots);
* hand-worked examples (tests/golden/ring_hand_examples.json);
* exact integer sums, exact power-of-two means, correctly rounded means
  checked with exact rational arithmetic;
* the recursive-summation error bound against exact sums;
* the per-device traffic the pages print for the replicated case;
* invariants: every rank ends with the same bits, Mean == fl(Sum / P).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def fold_closed_form(X, C):
    """out[i] = (((x_s[i] + x_{s+1}[i]) + x_{s+2}[i]) + ...), s = (i // L) % P.

    Derived from the ring: the chunk holding element i leaves its start rank
    s at step 0 and picks up one more rank's value per step.
    """
    X = np.asarray(X)
    P, n = X.shape
    if n == 0:
        return np.zeros((0,), X.dtype)
    L = -(-n // C)
    s = (np.arange(n) // L) % P
    cols = np.arange(n)
    acc = X[s, cols].copy()
    for k in range(1, P):
        acc = acc + X[(s + k) % P, cols]
    return acc


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint64)


@pytest.mark.parametrize("P", list(range(1, 9)))
def test_stepwise_equals_closed_form(P):
    for n in (0, 1, 3, 37, 64, 257):
        for C in sorted({1, 2, P, 2 * P, 3}):
            X = workloads.rank_buffers(P, n, dist="wide", seed=100 * P + n + C)
            Y, _ = oracle.ring_allreduce(X, "sum", C)
            ref = fold_closed_form(X, C)
            for r in range(P):
                assert np.array_equal(bits(Y[r]), bits(ref)), (P, n, C, r)


def test_order_is_observable():
    """The test data above is sensitive to the order of additions: summing in
    plain rank order 0..P-1 gives different bits in many elements."""
    P, n = 8, 1000
    X = workloads.rank_buffers(P, n, dist="wide", seed=7)
    Y, _ = oracle.ring_allreduce(X, "sum", P)
    naive = X[0].copy()
    for r in range(1, P):
        naive = naive + X[r]
    differ = np.count_nonzero(bits(Y[0]) != bits(naive))
    assert differ > 100


def test_hand_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "ring_hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        X = np.array(c["inputs"], dtype=np.float32)
        Y, sent = oracle.ring_allreduce(X, "sum", c["chunking"])
        for r in range(c["P"]):
            assert Y[r].tolist() == c["sum"], c["name"]
        assert sent.tolist() == c["sent_per_rank"], c["name"]
        Ym, _ = oracle.ring_allreduce(X, "mean", c["chunking"])
        want = np.array([int(h, 16) for h in c["mean_f32_bits"]], np.uint32)
        for r in range(c["P"]):
            assert np.array_equal(bits(Ym[r]), want), c["name"]


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 7, 8, 11, 16])
def test_integer_valued_sum_is_exact(P):
    """Integers in [-2^10, 2^10] with P <= 16: every partial sum is an integer
    below 2^24 in magnitude, exactly representable, so any order gives the
    exact sum."""
    for n, C in ((1, 1), (100, P), (257, 3), (1000, 2 * P)):
        X = workloads.rank_buffers(P, n, dist="int", scale=1024, seed=P * n)
        exact = X.astype(np.int64).sum(axis=0)
        Y, _ = oracle.ring_allreduce(X, "sum", C)
        for r in range(P):
            assert np.array_equal(Y[r].astype(np.int64), exact)
        if P & (P - 1) == 0:
            Ym, _ = oracle.ring_allreduce(X, "mean", C)
            for r in range(P):
                for i in range(0, n, max(1, n // 50)):
                    assert Fraction(float(Ym[r, i])) == Fraction(int(exact[i]), P)


def _correctly_rounded(q: Fraction, y: np.float32) -> bool:
    """y is the float32 nearest q (ties to even)."""
    fy = Fraction(float(y))
    err = abs(fy - q)
    for nb in (np.nextafter(y, np.float32(np.inf)), np.nextafter(y, np.float32(-np.inf))):
        e2 = abs(Fraction(float(nb)) - q)
        if e2 < err:
            return False
        if e2 == err and (int(np.float32(y).view(np.uint32)) & 1):
            return False
    return True


@pytest.mark.parametrize("P", [3, 5, 6, 7, 9, 12])
def test_mean_correctly_rounded_non_power_of_two(P):
    X = workloads.rank_buffers(P, 200, dist="int", scale=1024, seed=P)
    exact = X.astype(np.int64).sum(axis=0)
    Ym, _ = oracle.ring_allreduce(X, "mean", P)
    for i in range(200):
        assert _correctly_rounded(Fraction(int(exact[i]), P), Ym[0, i]), i


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 6, 7, 8, 13, 16])
def test_mean_is_sum_divided_by_P(P):
    X = workloads.rank_buffers(P, 500, dist="wide", seed=11 * P)
    for C in (1, P, 3 * P):
        Ys, _ = oracle.ring_allreduce(X, "sum", C)
        Ym, _ = oracle.ring_allreduce(X, "mean", C)
        assert np.array_equal(bits(Ym), bits(Ys / np.float32(P)))


@pytest.mark.parametrize("P", [2, 3, 4, 8, 16])
def test_all_ranks_identical(P):
    X = workloads.rank_buffers(P, 333, dist="normal", seed=P)
    for op in ("sum", "mean"):
        Y, _ = oracle.ring_allreduce(X, op, P + 1)
        for r in range(1, P):
            assert np.array_equal(bits(Y[r]), bits(Y[0]))


@pytest.mark.parametrize("P", [2, 4, 8, 16])
def test_error_bound_against_exact_sum(P):
    """|ring - exact| <= gamma_{P-1} * sum_k |x_k| with gamma_m = m u/(1-m u),
    u = 2^-24: the bound for recursive summation of P terms (Higham, Accuracy
    and Stability of Numerical Algorithms, chapter 4)."""
    n = 300
    X = workloads.rank_buffers(P, n, dist="normal", seed=P + 1000)
    Y, _ = oracle.ring_allreduce(X, "sum", P)
    u = Fraction(1, 2 ** 24)
    m = P - 1
    gamma = m * u / (1 - m * u)
    for i in range(n):
        exact = sum(Fraction(float(X[k, i])) for k in range(P))
        absum = sum(abs(Fraction(float(X[k, i]))) for k in range(P))
        assert abs(Fraction(float(Y[0, i])) - exact) <= gamma * absum


def test_traffic_matches_pages(golden_dir):
    """Per-device traffic of the replicated all-reduce is 2(W-1)/W model
    sizes; the pages print 1.750 at W=8 and 1.969 at W=64."""
    with open(os.path.join(golden_dir, "pages_printed.json")) as f:
        printed = json.load(f)["ring_traffic_replicated"]["model_sizes_per_device"]
    for W in (8, 64):
        n = W * 6
        X = np.zeros((W, n), np.float32)
        _, sent = oracle.ring_allreduce(X, "sum", W)
        per_rank = sent / n
        assert np.all(per_rank == per_rank[0])
        assert f"{per_rank[0]:.3f}" == printed[str(W)]
        assert sent[0] * W == 2 * (W - 1) * n


def test_traffic_pipelined_chunks():
    """With C = kP chunks every rank still sends 2(P-1)/P of the buffer."""
    P, k = 4, 3
    n = P * k * 5
    _, sent = oracle.ring_allreduce(np.ones((P, n), np.float32), "sum", k * P)
    assert np.all(sent * P == 2 * (P - 1) * n)


def test_sampled_equals_full():
    P, n, C = 8, 1001, 8
    X = workloads.rank_buffers(P, n, dist="wide", seed=5)
    for op in ("sum", "mean"):
        Y, _ = oracle.ring_allreduce(X, op, C)
        idx = np.array([0, 1, 125, 126, 127, 500, 999, 1000])
        start = oracle.chunk_start_ranks(n, C, P)[idx]
        Ys = oracle.ring_allreduce_sampled(X[:, idx], start, op)
        assert np.array_equal(bits(Ys), bits(Y[:, idx]))


def test_p1_is_identity():
    X = workloads.rank_buffers(1, 100, dist="wide", seed=3)
    for op in ("sum", "mean"):
        Y, sent = oracle.ring_allreduce(X, op, 4)
        assert np.array_equal(bits(Y), bits(X))
        assert sent.tolist() == [0]


def test_empty_and_trailing_empty_chunks():
    Y, sent = oracle.ring_allreduce(np.zeros((4, 0), np.float32), "sum", 4)
    assert Y.shape == (4, 0) and sent.tolist() == [0, 0, 0, 0]
    # n = 5, C = 4 -> L = 2: chunks [0,2) [2,4) [4,5) and an empty [5,5)
    X = workloads.rank_buffers(4, 5, dist="wide", seed=9)
    Y, _ = oracle.ring_allreduce(X, "sum", 4)
    assert np.array_equal(bits(Y[0]), bits(fold_closed_form(X, 4)))


def test_non_finite_values_propagate():
    X = np.array([[np.inf, np.inf, 1.0, np.nan],
                  [1.0, -np.inf, 2.0, 1.0]], np.float32)
    Y, _ = oracle.ring_allreduce(X, "sum", 2)
    assert Y[0, 0] == np.inf and np.isnan(Y[0, 1]) and Y[0, 2] == 3.0
    assert np.isnan(Y[0, 3])


def test_subnormals_are_kept():
    tiny = np.float32(2.0 ** -140)           # subnormal in float32
    X = np.full((4, 8), tiny, np.float32)
    Y, _ = oracle.ring_allreduce(X, "sum", 4)
    assert np.all(Y == np.float32(2.0 ** -138))
    Ym, _ = oracle.ring_allreduce(X, "mean", 4)
    assert np.all(Ym == tiny)


def test_deterministic():
    X = workloads.rank_buffers(8, 4096, dist="wide", seed=1)
    a, _ = oracle.ring_allreduce(X, "mean", 8)
    b, _ = oracle.ring_allreduce(X, "mean", 8)
    assert np.array_equal(bits(a), bits(b))


def test_bf16_inputs_widen_exactly():
    P, n = 4, 777
    X = workloads.to_bf16_bits(workloads.rank_buffers(P, n, "normal", 1e-3, seed=4))
    widened = oracle.bf16_bits_to_f32(X)
    for op in ("sum", "mean"):
        Yb, _ = oracle.ring_allreduce(X, op, P, in_dtype="bf16", out_dtype="f32")
        Yf, _ = oracle.ring_allreduce(widened, op, P)
        assert np.array_equal(bits(Yb), bits(Yf))
        Yb16, _ = oracle.ring_allreduce(X, op, P, in_dtype="bf16")
        assert np.array_equal(Yb16, oracle.f32_to_bf16_bits(Yf))


def rel(a, b):
    """The pages' measure: normwise relative difference ||a - b|| / ||b||
    ("Distributed Training", How to Apply It)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_bf16_within_relative_tolerance_of_exact():
    """bf16 inputs, fp32 accumulation, bf16 output: within 1e-2 relative of
    the exact sum of the bf16 values."""
    P, n = 8, 2000
    X = workloads.to_bf16_bits(workloads.rank_buffers(P, n, "normal", 1e-3, seed=8))
    widened = oracle.bf16_bits_to_f32(X).astype(np.float64)
    exact = np.array([math.fsum(widened[:, i]) for i in range(n)]) / P
    Y, _ = oracle.ring_allreduce(X, "mean", P, in_dtype="bf16", out_dtype="bf16")
    got = oracle.bf16_bits_to_f32(Y[0])
    assert rel(got, exact) <= 1e-2
    Y32, _ = oracle.ring_allreduce(X, "mean", P, in_dtype="bf16", out_dtype="f32")
    assert rel(Y32[0], exact) <= 1e-6


def test_float64_accumulation():
    X = workloads.rank_buffers(4, 50, "normal", 1.0, seed=2, dtype=np.float64)
    Y, _ = oracle.ring_allreduce(X, "sum", 4, in_dtype="f64")
    assert Y.dtype == np.float64
    assert np.array_equal(Y[0], fold_closed_form(X, 4))


# ------------------------------------------------ the ring's two halves ----

@pytest.mark.parametrize("P", [1, 2, 3, 5, 8])
def test_reduce_scatter_then_all_gather_is_the_all_reduce(P):
    for n, C in ((37, P), (100, 2 * P + 1), (64, 1)):
        X = workloads.rank_buffers(P, n, dist="wide", seed=P + n)
        for op in ("sum", "mean"):
            R, owner, s1 = oracle.ring_reduce_scatter(X, op, C)
            G, s2 = oracle.ring_all_gather(R, C)
            Y, s = oracle.ring_allreduce(X, op, C)
            assert np.array_equal(bits(G), bits(Y))
            assert np.array_equal(s1 + s2, s)
            # the owner holds the finished value
            assert np.array_equal(bits(R[owner, np.arange(n)]), bits(Y[0]))


def test_reduce_scatter_owner_rule():
    """Chunk j starts at rank j mod P and ends at its owner, one rank
    before the start."""
    own = oracle.chunk_owners(12, 4, 4)
    assert own.tolist() == [3, 3, 3, 0, 0, 0, 1, 1, 1, 2, 2, 2]


def test_all_gather_copies_the_owner_values():
    P, n, C = 4, 20, 4
    B = np.arange(P * n, dtype=np.int64).reshape(P, n)
    G, sent = oracle.ring_all_gather(B, C)
    own = oracle.chunk_owners(n, C, P)
    for r in range(P):
        assert G[r].tolist() == B[own, np.arange(n)].tolist()
    assert np.all(sent * P == (P - 1) * n)


def test_fully_sharded_traffic_matches_pages(golden_dir):
    """Full sharding moves two all-gathers and a reduce-scatter per step,
    3(W-1)/W model sizes per device; the pages print 2.625 at W=8 and 2.953
    at W=64, 1.5 times the replicated ring all-reduce."""
    with open(os.path.join(golden_dir, "pages_printed.json")) as f:
        pr = json.load(f)
    full = pr["ring_traffic_fully_sharded"]["model_sizes_per_device"]
    for W in (8, 64):
        n = W * 3
        X = np.zeros((W, n), np.float32)
        _, _, rs = oracle.ring_reduce_scatter(X, "sum", W)
        _, ag = oracle.ring_all_gather(X, W)
        per_device = (2 * ag + rs) / n
        assert np.all(per_device == per_device[0])
        assert f"{per_device[0]:.3f}" == full[str(W)]
        rep = pr["ring_traffic_replicated"]["model_sizes_per_device"][str(W)]
        assert f"{per_device[0] / float(rep):.2f}" == "1.50"
