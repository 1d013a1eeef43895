"""Pins for the two-level (local / global) all-reduce oracle."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hierarchical_hand_examples.json")


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def load_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    X = np.array(case["inputs"], dtype=np.float32)
    Y = oracle.hierarchical_allreduce(X, case["op"], nodes=case["nodes"], local=tuple(case["local"]),
                                      global_=tuple(case["global"]))
    want = np.array(case["expected"], dtype=np.float32)
    for r in range(X.shape[0]):
        assert np.array_equal(bits(Y[r]), bits(want)), (r, Y[r], want)


def test_hand_examples_tell_the_two_levels_from_the_flat_ring():
    """The first case fails if the oracle ignored the node grouping."""
    case = load_cases()[0]
    X = np.array(case["inputs"], dtype=np.float32)
    flat, _ = oracle.ring_allreduce(X, "sum", 1)
    assert not np.array_equal(bits(flat[0]), bits(np.array(case["expected"], dtype=np.float32)))


# ---- every association written out, recursively ---------------------------
#
# An independent statement of the same reading: the value of a level is an
# expression over its members, built per element.  Ring: a left fold from the
# element's start member.  Tree: value(p) = (((x_p + value(c1)) + value(c2))
# ...), children in increasing order.  This evaluates the expression
# directly, element by element, instead of simulating the phases.

def fold_ring(vals, start):
    m = len(vals)
    acc = vals[start % m]
    for k in range(1, m):
        acc = np.float32(acc + vals[(start + k) % m])
    return acc


def fold_tree(vals, b):
    m = len(vals)

    def value(p):
        acc = vals[p]
        for c in range(b * p + 1, min(b * p + b, m - 1) + 1):
            acc = np.float32(acc + value(c))
        return acc

    return value(0)


def level_value(vals, strategy, param, i, n):
    m = len(vals)
    if strategy == "ring":
        C = param if param else m
        L = -(-n // C)
        return fold_ring(vals, (i // L) % m)
    if strategy == "tree":
        return fold_tree(vals, param)
    return fold_tree(vals, max(1, m - 1))


def written_out(X, nodes, local, glob):
    P, n = X.shape
    Lr = P // nodes
    out = np.empty(n, dtype=np.float32)
    for i in range(n):
        node_vals = [level_value([X[g * Lr + l, i] for l in range(Lr)], local[0], local[1], i, n)
                     for g in range(nodes)]
        out[i] = level_value(node_vals, glob[0], glob[1], i, n)
    return out


STRATEGIES = [("ring", None), ("ring", 1), ("ring", 2), ("ring", 3), ("tree", 1), ("tree", 2),
              ("centralized", None)]


def factorizations():
    out = []
    for P in (2, 4, 6, 8, 12):
        for G in range(1, P + 1):
            if P % G == 0:
                out.append((P, G))
    return out


@pytest.mark.parametrize("P,G", factorizations())
def test_every_association_written_out(P, G):
    n = 37
    X = workloads.rank_buffers(P, n, dist="wide", seed=P * 31 + G)
    for local in STRATEGIES:
        for glob in STRATEGIES:
            Y = oracle.hierarchical_allreduce(X, "sum", nodes=G, local=local, global_=glob)
            want = written_out(X, G, local, glob)
            assert np.array_equal(bits(Y[0]), bits(want)), (local, glob)
            for r in range(1, P):
                assert np.array_equal(bits(Y[r]), bits(Y[0]))


def test_the_data_makes_the_grouping_observable():
    """On the test data the two-level order differs from the flat ring in a
    good share of the elements, so a lost grouping could not pass."""
    X = workloads.rank_buffers(8, 1000, dist="wide", seed=5)
    H = oracle.hierarchical_allreduce(X, "sum", nodes=2, local=("ring", None), global_=("ring", None))
    F, _ = oracle.ring_allreduce(X, "sum", 8)
    assert np.mean(bits(H[0]) != bits(F[0])) > 0.2


# ---- reductions to one level ------------------------------------------------

@pytest.mark.parametrize("P", [1, 3, 4, 8])
def test_one_node_is_the_local_strategy_alone(P):
    X = workloads.rank_buffers(P, 257, dist="wide", seed=P)
    for op in ("sum", "mean"):
        H = oracle.hierarchical_allreduce(X, op, nodes=1, local=("ring", 2 * P), global_=("tree", 2))
        R, _ = oracle.ring_allreduce(X, op, 2 * P)
        assert np.array_equal(bits(H), bits(R))
        H = oracle.hierarchical_allreduce(X, op, nodes=1, local=("tree", 2), global_=("ring", None))
        T, _ = oracle.tree_allreduce(X, op, 2)
        assert np.array_equal(bits(H), bits(T))


@pytest.mark.parametrize("P", [2, 5, 8])
def test_one_peer_per_node_is_the_global_strategy_alone(P):
    X = workloads.rank_buffers(P, 257, dist="wide", seed=10 + P)
    for op in ("sum", "mean"):
        H = oracle.hierarchical_allreduce(X, op, nodes=P, local=("tree", 2), global_=("ring", 3))
        R, _ = oracle.ring_allreduce(X, op, 3)
        assert np.array_equal(bits(H), bits(R))
        H = oracle.hierarchical_allreduce(X, op, nodes=P, local=("ring", None), global_=("centralized", None))
        C, _ = oracle.tree_allreduce(X, op, max(1, P - 1))
        assert np.array_equal(bits(H), bits(C))


# ---- values ----------------------------------------------------------------

@pytest.mark.parametrize("local", STRATEGIES)
def test_integer_sums_are_exact(local):
    P, G = 16, 4
    X = workloads.rank_buffers(P, 300, "int", 1024, seed=3)
    Y = oracle.hierarchical_allreduce(X, "sum", nodes=G, local=local, global_=("ring", None))
    assert np.array_equal(Y[0].astype(np.int64), X.astype(np.int64).sum(0))


def test_error_within_the_recursive_summation_bound():
    """|computed - exact| <= gamma_{P-1} * sum |x| (Higham, "Accuracy and
    Stability of Numerical Algorithms", ch. 4): any order of P-1 additions."""
    P, G = 12, 3
    X = workloads.rank_buffers(P, 400, dist="wide", seed=8)
    Y = oracle.hierarchical_allreduce(X, "sum", nodes=G, local=("tree", 2), global_=("ring", 5))
    u = 2.0 ** -24
    gamma = (P - 1) * u / (1 - (P - 1) * u)
    for i in range(X.shape[1]):
        exact = sum(Fraction(float(X[r, i])) for r in range(P))
        mag = math.fsum(abs(float(X[r, i])) for r in range(P))
        assert abs(Fraction(float(Y[0, i])) - exact) <= Fraction(gamma * mag * (1 + 1e-12))


def test_mean_is_one_division_of_the_sum_by_every_rank():
    P, G = 6, 2
    X = workloads.rank_buffers(P, 500, dist="wide", seed=4)
    for local, glob in [(("ring", None), ("ring", None)), (("tree", 1), ("centralized", None))]:
        S = oracle.hierarchical_allreduce(X, "sum", nodes=G, local=local, global_=glob)
        M = oracle.hierarchical_allreduce(X, "mean", nodes=G, local=local, global_=glob)
        assert np.array_equal(bits(M[0]), bits(S[0] / np.float32(P)))


def test_bf16_inputs_equal_the_widened_f32_path():
    P, G = 8, 2
    X = workloads.rank_buffers(P, 300, dist="wide", seed=6)
    Xb = workloads.to_bf16_bits(X)
    Xw = oracle.bf16_bits_to_f32(Xb)
    for out in ("f32", "bf16"):
        A = oracle.hierarchical_allreduce(Xb, "mean", nodes=G, local=("tree", 2), global_=("ring", 4),
                                          in_dtype="bf16", out_dtype=out)
        B = oracle.hierarchical_allreduce(Xw, "mean", nodes=G, local=("tree", 2), global_=("ring", 4),
                                          in_dtype="f32", out_dtype=out)
        assert np.array_equal(A, B)


def test_rejects_a_node_count_that_does_not_divide_the_ranks():
    with pytest.raises(ValueError):
        oracle.hierarchical_allreduce(np.zeros((6, 3), np.float32), "sum", nodes=4)


def test_sampled_two_level_oracle_matches_the_whole_buffer():
    """The sampled form used by the full-size GPU test gives, for every
    element, the bits of the whole-buffer oracle."""
    from sampled_oracle import hierarchical_sampled
    rng = np.random.default_rng(7)
    for P, G in ((8, 2), (8, 4), (6, 3), (12, 4)):
        for local, glob in ((("ring", None), ("ring", None)), (("ring", 3), ("ring", 5)),
                            (("tree", 2), ("ring", None)), (("ring", None), ("centralized", None))):
            n = 257
            X = (rng.standard_normal((P, n)) * np.exp2(rng.integers(-20, 21, (P, n)))).astype(np.float32)
            for op in ("sum", "mean"):
                whole = oracle.hierarchical_allreduce(X, op, nodes=G, local=local, global_=glob)
                idx = np.arange(n)
                got = hierarchical_sampled(X, idx, n, op, G, local, glob)
                assert np.array_equal(got.view(np.uint32), whole.view(np.uint32)), (P, G, local, glob, op)
