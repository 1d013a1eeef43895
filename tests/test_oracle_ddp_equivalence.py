"""The pages' data-parallel equivalence, checked through the ring oracle.

"Distributed Training", "Data parallelism and all-reduce": for a loss
averaged over a batch split into W equal shards, the average of the shard
gradients is the full-batch gradient, so ranks that all-reduce with Mean and
then step locally stay identical.  "How to Apply It" checks this with one
process playing four ranks and prints the relative differences (float64 at
round-off level, float32 around 1e-7) and an exact factor 4 when the
accumulated loss is not divided by the number of micro-batches.

Here the all-reduce is the oracle's ring (not a plain mean), on a tiny MLP
with fixed random weights and synthetic data; only the orders of magnitude
of the pages' numbers transfer, their exact values belong to their conv net.
"""

import json
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle

W = 4
B = 32


def make_mlp(dtype):
    torch.manual_seed(0)
    net = torch.nn.Sequential(
        torch.nn.Linear(16, 32), torch.nn.Tanh(),
        torch.nn.Linear(32, 32), torch.nn.Tanh(),
        torch.nn.Linear(32, 3))
    return net.to(dtype)


def data(dtype):
    g = torch.Generator().manual_seed(1)
    X = torch.randn(B, 16, generator=g, dtype=torch.float64).to(dtype)
    y = torch.randint(0, 3, (B,), generator=g)
    return X, y


def loss_gradient(net, X, y):
    """Gradient of the mean cross-entropy over (X, y) with respect to every
    parameter, concatenated in parameter order (torch.autograd.grad, so no
    .grad state is kept between calls)."""
    params = list(net.parameters())
    loss = F.cross_entropy(net(X), y)
    return torch.cat([g.reshape(-1) for g in torch.autograd.grad(loss, params)]).detach()


def shard_gradients(net, X, y):
    """(W, n) gradients of the W equal shards.  Rank r takes samples r,
    r + W, r + 2W, ... -- the split an unshuffled distributed sampler gives
    when W divides the batch."""
    return np.stack([loss_gradient(net, X[r::W], y[r::W]).numpy() for r in range(W)])


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _printed(golden_dir):
    with open(os.path.join(golden_dir, "pages_printed.json")) as f:
        return json.load(f)["dp_equivalence"]


def test_ring_mean_of_shards_is_full_batch_gradient_float64(golden_dir):
    printed = _printed(golden_dir)
    net = make_mlp(torch.float64)
    X, y = data(torch.float64)
    g_full = loss_gradient(net, X, y).numpy()
    G = shard_gradients(net, X, y)
    Y, _ = oracle.ring_allreduce(G, "mean", W, in_dtype="f64")
    for r in range(W):
        d = rel(Y[r], g_full)
        # round-off level, same order as the pages' 6.7e-16
        assert d < 100 * printed["rel_diff_float64"], d
        assert np.array_equal(Y[r], Y[0])


def test_ring_mean_of_shards_is_full_batch_gradient_float32(golden_dir):
    printed = _printed(golden_dir)
    net = make_mlp(torch.float32)
    X, y = data(torch.float32)
    g_full = loss_gradient(net, X, y).numpy()
    G = shard_gradients(net, X, y)
    Y, _ = oracle.ring_allreduce(G, "mean", W)
    d = rel(Y[0], g_full)
    assert d < 100 * printed["rel_diff_float32"], d
    assert d > 0.0    # float32 reductions in another order do not match exactly


def test_sum_without_division_is_exactly_W_times(golden_dir):
    printed = _printed(golden_dir)
    net = make_mlp(torch.float64)
    X, y = data(torch.float64)
    g_full = loss_gradient(net, X, y).numpy()
    G = shard_gradients(net, X, y)
    Y, _ = oracle.ring_allreduce(G, "sum", W, in_dtype="f64")
    ratio = np.linalg.norm(Y[0]) / np.linalg.norm(g_full)
    assert f"{ratio:.12f}" == printed["accumulation_without_division_norm_ratio"]


def test_replicas_stay_identical_after_local_momentum_step():
    """CS336 Lecture 8, "Data Parallelism (DDP)": after the all-reduce each
    rank steps its own optimizer and the weights stay in sync."""
    net = make_mlp(torch.float32)
    X, y = data(torch.float32)
    G = shard_gradients(net, X, y)
    w0 = torch.cat([p.detach().reshape(-1) for p in net.parameters()]).numpy()
    Y, _ = oracle.ring_allreduce(G, "mean", W)
    states = [oracle.sgd_momentum(Y[r], w0, np.zeros_like(w0), 1e-3, 0.9)
              for r in range(W)]
    for w, v in states[1:]:
        assert np.array_equal(w, states[0][0]) and np.array_equal(v, states[0][1])
