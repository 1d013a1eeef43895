"""Synchronized batch normalization through the all-reduce, as the pages
describe it ("Distributed Training", "Synchronized batch normalization" and
"How to Apply It", part 2): every rank contributes its per-channel sum and
sum of squares, the all-reduce adds them, and the pooled statistics equal
batch normalization over the whole batch (the pages print a max abs
difference of 3.3e-14 in float64)."""

import numpy as np
import torch
import torch.nn.functional as F

import oracle

W = 4


def shards_of_activations(dtype):
    g = torch.Generator().manual_seed(3)
    h = torch.randn(32, 8, 6, 6, generator=g, dtype=torch.float64).to(dtype)
    return h, [h[r::W] for r in range(W)]


def test_pooled_statistics_equal_whole_batch_bn_float64():
    h, parts = shards_of_activations(torch.float64)
    s1 = np.stack([p.sum((0, 2, 3)).numpy() for p in parts])
    s2 = np.stack([(p * p).sum((0, 2, 3)).numpy() for p in parts])
    S1, _ = oracle.ring_allreduce(s1, "sum", W, in_dtype="f64")
    S2, _ = oracle.ring_allreduce(s2, "sum", W, in_dtype="f64")
    n = sum(p.shape[0] * p.shape[2] * p.shape[3] for p in parts)
    for r in range(W):
        mean = S1[r] / n
        var = S2[r] / n - mean ** 2
        normed = (h - torch.from_numpy(mean)[None, :, None, None]) / torch.sqrt(
            torch.from_numpy(var)[None, :, None, None] + 1e-5)
        ref = F.batch_norm(h, None, None, None, None, True, 0.0, 1e-5)
        assert (normed - ref).abs().max().item() < 1e-12
