"""The hot path in its setting, on the GPU: P replicas of a small model
compute their shard gradients directly into bucket views of one arena
(DDP's "gradients as bucket views": no pack or unpack), every bucket is
all-reduced with Mean and the fused SGD-momentum step updates the fp32
master weights.  Checked bit for bit against the oracle on the same
gradients, and against full-batch SGD within float32 rounding; plus
synchronized batch-norm statistics through the multi-tensor path, and HIP
graph capture and replay of a bucket step."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from gpu_helpers import DEV, assert_same_bits

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")


def test_ddp_step_with_bucket_views_and_fused_sgd():
    W, B = 4, 64
    torch.manual_seed(0)
    net = torch.nn.Sequential(torch.nn.Linear(32, 256), torch.nn.Tanh(),
                              torch.nn.Linear(256, 256), torch.nn.Tanh(),
                              torch.nn.Linear(256, 10)).to(DEV)
    params = list(net.parameters())
    shapes = [tuple(p.shape) for p in params]
    g = torch.Generator(device=DEV).manual_seed(1)
    X = torch.randn(B, 32, device=DEV, generator=g)
    y = torch.randint(0, 10, (B,), device=DEV, generator=g)
    plan = ddp.GradBucketer(shapes, torch.float32, 64 << 10, device=DEV)   # several buckets
    assert plan.n_buckets > 3
    arena = plan.alloc_arena(W)
    arena.zero_()
    for r in range(W):                      # rank r's backward writes into its arena row
        views = plan.tensor_views(arena[r])
        for p, v in zip(params, views):
            p.grad = v
        F.cross_entropy(net(X[r::W]), y[r::W]).backward()
        for p, v in zip(params, views):
            assert p.grad.data_ptr() == v.data_ptr()     # accumulated in place
    master = torch.zeros(plan.n_buckets * plan.bucket_elems, device=DEV)
    for p, v in zip(params, plan.tensor_views(master)):
        v.copy_(p.detach())
    mom = torch.zeros_like(master)
    grads_host = arena.cpu().numpy()
    master_host, mom_host = master.cpu().numpy(), mom.cpu().numpy()
    E = plan.bucket_elems
    for k in range(plan.n_buckets):
        lo, n = k * E, plan.bucket_len(k)
        ddp.allreduce_sgd([plan.bucket_view(arena[r], k) for r in range(W)], master[lo:lo + n],
                          mom[lo:lo + n], 0.1, 0.9, "mean", W)
    torch.cuda.synchronize()
    got_w = master.cpu().numpy()
    for k in range(plan.n_buckets):
        lo, n = k * E, plan.bucket_len(k)
        gk, _ = oracle.ring_allreduce(grads_host[:, lo:lo + n], "mean", W)
        ow, ov = oracle.sgd_momentum(gk[0], master_host[lo:lo + n], mom_host[lo:lo + n], 0.1, 0.9)
        assert_same_bits(got_w[lo:lo + n], ow, f"bucket {k}")
    # against one device's full-batch SGD step
    net.zero_grad(set_to_none=True)
    F.cross_entropy(net(X), y).backward()
    for p, v, v0 in zip(params, plan.tensor_views(master), plan.tensor_views(torch.from_numpy(master_host).to(DEV))):
        want = v0 - 0.1 * p.grad
        assert torch.allclose(v, want, rtol=0, atol=1e-6), float((v - want).abs().max())


def test_no_sync_accumulation_then_one_bucketed_all_reduce():
    """Gradient accumulation without synchronization ("Distributed
    Training", DDP's no_sync): every rank runs backward on two micro-batches
    into the same bucket views, with no all-reduce in between, and the
    accumulated gradients then go through one bucketed all-reduce with
    Mean.  Bit for bit the oracle's ring over the accumulated gradients of
    every bucket, and within float32 rounding of the full-batch gradient of
    the mean micro-batch loss."""
    W, B, M = 4, 64, 2
    torch.manual_seed(5)
    net = torch.nn.Sequential(torch.nn.Linear(32, 128), torch.nn.Tanh(), torch.nn.Linear(128, 10)).to(DEV)
    params = list(net.parameters())
    g = torch.Generator(device=DEV).manual_seed(6)
    X = torch.randn(M, B, 32, device=DEV, generator=g)
    y = torch.randint(0, 10, (M, B), device=DEV, generator=g)
    plan = ddp.GradBucketer([tuple(p.shape) for p in params], torch.float32, 8 << 10, device=DEV)
    assert plan.n_buckets > 2
    arena = plan.alloc_arena(W)
    arena.zero_()
    for r in range(W):
        views = plan.tensor_views(arena[r])
        for p, v in zip(params, views):
            p.grad = v
        for mb in range(M):                 # no all-reduce between micro-batches
            (F.cross_entropy(net(X[mb, r::W]), y[mb, r::W]) / M).backward()
    rows = [arena[r, :plan.total] for r in range(W)]
    before = np.stack([x.cpu().numpy() for x in rows])
    ddp.allreduce(rows, "mean", W, out=rows, bucket_elems=plan.bucket_elems)
    torch.cuda.synchronize()
    got = np.stack([x.cpu().numpy() for x in rows])
    E = plan.bucket_elems
    for k in range(plan.n_buckets):
        lo, n = k * E, plan.bucket_len(k)
        want, _ = oracle.ring_allreduce(before[:, lo:lo + n], "mean", W)
        assert_same_bits(got[:, lo:lo + n], want, f"bucket {k}")
    net.zero_grad(set_to_none=True)
    for mb in range(M):
        (F.cross_entropy(net(X[mb]), y[mb]) / M).backward()
    for p, v in zip(params, plan.tensor_views(rows[0])):
        assert torch.allclose(v, p.grad, rtol=0, atol=1e-6), float((v - p.grad).abs().max())


def test_synchronized_batchnorm_statistics():
    """Per-channel sums and sums of squares of W shards, all-reduced as two
    small tensors in one launch, give the whole batch's statistics."""
    W = 4
    g = torch.Generator(device=DEV).manual_seed(3)
    h = torch.randn(64, 32, 14, 14, device=DEV, generator=g)
    parts = [h[r::W] for r in range(W)]
    s1 = [p.sum((0, 2, 3)) for p in parts]
    s2 = [(p * p).sum((0, 2, 3)) for p in parts]
    m = ddp.MultiAllReduce([(32,), (32,)], W, torch.float32, device=DEV)
    out = m([[s1[r], s2[r]] for r in range(W)], "sum", W)
    torch.cuda.synchronize()
    for t, src in enumerate((s1, s2)):
        X = np.stack([x.cpu().numpy() for x in src])
        want, _ = oracle.ring_allreduce(X, "sum", W)
        for r in range(W):
            assert_same_bits(out[r][t].cpu().numpy(), want[r], f"stat {t} rank {r}")
    n = 64 * 14 * 14
    mean = out[0][0] / n
    var = out[0][1] / n - mean * mean
    ref_mean = h.mean((0, 2, 3))
    ref_var = h.var((0, 2, 3), unbiased=False)
    assert torch.allclose(mean, ref_mean, atol=1e-5)
    assert torch.allclose(var, ref_var, rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("bucketed", [False, True])
def test_graph_capture_and_replay_of_a_bucket_step(bucketed):
    """The launches of a bucket step (one call per bucket, or one bucketed
    call) captured in a HIP graph and replayed several times, with eager
    work and synchronizations between replays, give the eager result every
    time."""
    P = 8
    plan = ddp.GradBucketer(workloads.model_shapes("resnet50"), torch.float32, 25 << 20,
                            device=DEV)
    g = plan.alloc_arena(P)
    o = plan.alloc_arena(P)
    views = [([plan.bucket_view(g[r], k) for r in range(P)],
              [plan.bucket_view(o[r], k) for r in range(P)]) for k in range(plan.n_buckets)]
    rows = ([g[r, :plan.total] for r in range(P)], [o[r, :plan.total] for r in range(P)])

    def step():
        if bucketed:
            ddp.allreduce(rows[0], "mean", P, out=rows[1], bucket_elems=plan.bucket_elems)
            return
        for a, b in views:
            ddp.allreduce(a, "mean", P, out=b)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for rep in range(3):
        for r in range(P):
            workloads.torch_normal_(g[r], 0.01, seed=10 * rep + r)     # eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replayed = o.clone()
        step()                                                         # eager reference
        torch.cuda.synchronize()
        assert torch.equal(replayed.view(torch.int32), o.view(torch.int32)), rep
