"""GPU parity of the tree and centralized strategies against the oracle's
level-by-level simulation, bit for bit, and centralized == the one-chunk
ring."""

import pytest
import torch

import oracle
import workloads
from gpu_helpers import assert_same_bits, to_device, to_host, torch_dtype

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")


def draw(P, n, dtype, seed):
    X = workloads.rank_buffers(P, n, dist="wide", seed=seed)
    return workloads.to_bf16_bits(X) if dtype == "bf16" else X


@pytest.mark.parametrize("pair", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"),
                                  ("f32", "bf16")])
@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 16])
def test_tree_equals_oracle(pair, P):
    it, ot = pair
    for n in (1, 9, 4101, 70001):
        for b in sorted({1, 2, 3, 4, max(1, P - 1), 100}):
            for op in ("sum", "mean"):
                X = draw(P, n, it, seed=P * 7 + n + b)
                out = ddp.allreduce_tree(to_device(X, it), op, b, out_dtype=torch_dtype(ot))
                torch.cuda.synchronize()
                want, _ = oracle.tree_allreduce(X, op, b, in_dtype=it, out_dtype=ot)
                assert_same_bits(to_host(out), want, f"{it}->{ot} P={P} n={n} b={b} {op}")


@pytest.mark.parametrize("P", [2, 4, 8, 16])
def test_centralized_equals_one_chunk_ring(P):
    X = draw(P, 1_000_003, "f32", seed=P)
    cen = ddp.allreduce_tree(to_device(X, "f32"), "mean", P - 1)
    ring = ddp.allreduce(to_device(X, "f32"), "mean", 1)
    torch.cuda.synchronize()
    assert_same_bits(to_host(cen), to_host(ring), f"P={P}")
