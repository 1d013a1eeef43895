"""GPU parity of the stepwise ring (one launch per ring step): bit for bit
the oracle's stepwise ring, bit for bit the fused kernel, and the per-rank
counts of elements sent equal to the oracle's, which for C = P and n
divisible by P are the pages' 2(W-1)/W model sizes per device."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, assert_same_bits, to_device, to_host

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")


def stepwise(X, op, C):
    bufs = to_device(X, "f32")
    sent = torch.zeros(X.shape[0], dtype=torch.int64, device=DEV)
    ddp.allreduce_stepwise(bufs, op, C, sent=sent)
    torch.cuda.synchronize()
    return to_host(bufs), sent.cpu().numpy()


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16])
def test_stepwise_equals_oracle_including_traffic(P):
    for n in (1, 7, 4099, 70001):
        for C in sorted({1, P, 2 * P + 1, n}):
            for op in ("sum", "mean"):
                X = workloads.rank_buffers(P, n, dist="wide", seed=P * 101 + n + C)
                got, sent = stepwise(X, op, C)
                if C <= 64:
                    want, want_sent = oracle.ring_allreduce(X, op, C)
                    assert sent.tolist() == want_sent.tolist(), (P, n, C, op)
                else:
                    start = oracle.chunk_start_ranks(n, C, P)
                    want = oracle.ring_allreduce_sampled(X, start, op)
                    assert sent.sum() == 2 * (P - 1) * n
                assert_same_bits(got, want, f"P={P} n={n} C={C} {op}")


def test_stepwise_traffic_is_the_pages_ring_volume(golden_dir):
    with open(os.path.join(golden_dir, "pages_printed.json")) as f:
        printed = json.load(f)["ring_traffic_replicated"]["model_sizes_per_device"]
    P = 8
    n = P * 123_457
    X = workloads.rank_buffers(P, n, "normal", 1.0, seed=8)
    _, sent = stepwise(X, "sum", P)
    per_device = sent / n
    assert np.all(per_device == per_device[0])
    assert f"{per_device[0]:.3f}" == printed["8"]


def test_stepwise_equals_fused_at_bucket_size():
    P, n = 8, 6_553_600
    X = workloads.rank_buffers(P, n, "normal", 0.01, seed=2)
    got, sent = stepwise(X, "mean", P)
    fused = ddp.allreduce(to_device(X, "f32"), "mean", P)
    torch.cuda.synchronize()
    assert_same_bits(got, to_host(fused), "25 MiB bucket")
    assert np.all(sent * P == 2 * (P - 1) * n)


@pytest.mark.parametrize("P,C", [(8, 8), (4, 8), (3, 6)])
def test_full_buckets_as_one_call_equal_one_call_per_bucket(P, C):
    """With C a multiple of P and the bucket length a multiple of C,
    consecutive full buckets form one ring with chunking (buckets x C):
    every chunk keeps its start rank and length, so one stepwise call over
    three full buckets gives the bits of one call per bucket, and every rank
    sends the same number of elements."""
    E, nb = 4096 * C, 3
    n = nb * E
    X = workloads.rank_buffers(P, n, "normal", 0.01, seed=70 + P)
    per = to_device(X, "f32")
    one = to_device(X, "f32")
    sent_per = torch.zeros(P, dtype=torch.int64, device=DEV)
    sent_one = torch.zeros(P, dtype=torch.int64, device=DEV)
    for k in range(nb):
        ddp.allreduce_stepwise([x[k * E:(k + 1) * E] for x in per], "mean", C, sent=sent_per)
    ddp.allreduce_stepwise(one, "mean", nb * C, sent=sent_one)
    torch.cuda.synchronize()
    for r in range(P):
        assert torch.equal(per[r].view(torch.int32), one[r].view(torch.int32)), r
    assert torch.equal(sent_per, sent_one)
    for k in range(nb):
        want, _ = oracle.ring_allreduce(X[:, k * E:(k + 1) * E], "mean", C)
        assert_same_bits(to_host([t[k * E:(k + 1) * E] for t in one]), want, f"bucket {k}")


@pytest.mark.parametrize("P,C,E,n", [
    (8, 8, 4096 * 8, 3 * 4096 * 8 + 5_001),   # full buckets merged, a partial tail
    (3, 4, 10_000, 35_555),                   # C not a multiple of P: bucket by bucket
    (4, 4, 8_192, 8_192),                     # one full bucket
    (2, 2, 4_096, 5),                         # one partial bucket
])
def test_stepwise_buckets_equal_one_call_per_bucket(P, C, E, n):
    """allreduce_ring_stepwise_buckets: the bits and the per-rank send counts
    of one stepwise call per bucket, merged into one ring or not."""
    X = workloads.rank_buffers(P, n, "normal", 0.01, seed=90 + P + n)
    per = to_device(X, "f32")
    one = to_device(X, "f32")
    sent_per = torch.zeros(P, dtype=torch.int64, device=DEV)
    sent_one = torch.zeros(P, dtype=torch.int64, device=DEV)
    for k in range(0, n, E):
        ddp.allreduce_stepwise([x[k:k + E] for x in per], "mean", C, sent=sent_per)
    ddp.allreduce_stepwise(one, "mean", C, sent=sent_one, bucket_elems=E)
    torch.cuda.synchronize()
    got = to_host(one)
    assert_same_bits(got, to_host(per), "one call per bucket")
    assert torch.equal(sent_per, sent_one)
    for k in range(0, n, E):
        want, _ = oracle.ring_allreduce(X[:, k:k + E], "mean", C)
        assert_same_bits(got[:, k:k + E], want, f"bucket at {k}")

