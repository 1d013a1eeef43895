"""GPU parity of the multi-tensor (small-message) all-reduce: every tensor
bit for bit the oracle's ring on that tensor alone, including tiny tensors
whose chunks are shorter than a tile, tensors not 16-byte aligned, the
partial last tile, bf16; and the lecture's per-parameter DDP step on a tiny
MLP."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from gpu_helpers import DEV, assert_same_bits, oracle_ring

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")


def bits_of(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    return t.cpu().numpy().reshape(-1)


def make(P, shapes, dtype, seed, misalign=0):
    rng = np.random.default_rng(seed)
    host, dev = [], []
    for r in range(P):
        hs, ds = [], []
        for s in shapes:
            n = int(np.prod(s, dtype=np.int64))
            x = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 21, n))).astype(np.float32)
            if dtype == torch.bfloat16:
                x = workloads.to_bf16_bits(x)
                src = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
            else:
                src = torch.from_numpy(x).to(DEV)
            store = torch.empty(n + misalign, dtype=dtype, device=DEV)
            t = store[misalign:misalign + n].view(s)
            t.copy_(src.view(s))
            hs.append(x)
            ds.append(t)
        host.append(hs)
        dev.append(ds)
    return host, dev


@pytest.mark.parametrize("pair", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("P", [1, 3, 8, 16])
@pytest.mark.parametrize("misalign", [0, 1])
def test_multi_equals_oracle_per_tensor(pair, P, misalign):
    it, ot = pair
    tdt = torch.bfloat16 if it == "bf16" else torch.float32
    odt = torch.bfloat16 if ot == "bf16" else torch.float32
    shapes = [(1,), (7,), (64,), (3, 5), (1000,), (4096,), (4097,), (33, 129), (70001,), (0,)]
    host, dev = make(P, shapes, tdt, seed=P + misalign, misalign=misalign)
    m = ddp.MultiAllReduce(shapes, P, tdt, odt, device=DEV)
    for C in (P, 2 * P + 1):
        for op in ("sum", "mean"):
            out = m(dev, op, C)
            torch.cuda.synchronize()
            for t, s in enumerate(shapes):
                X = np.stack([host[r][t] for r in range(P)])
                if X.shape[1] == 0:
                    continue
                want = oracle_ring(X, op, C, in_dtype=it, out_dtype=ot)
                got = np.stack([bits_of(out[r][t]) for r in range(P)])
                assert_same_bits(got, want, f"{it}->{ot} P={P} t={t} C={C} {op}")


def test_multi_in_place_equals_single_calls():
    P = 8
    shapes = workloads.resnet50_shapes()
    _, dev = make(P, shapes, torch.float32, seed=5)
    single = [ddp.allreduce([dev[r][t].reshape(-1) for r in range(P)], "mean", P)
              for t in range(len(shapes))]
    m = ddp.MultiAllReduce(shapes, P, torch.float32, device=DEV)
    m(dev, "mean", P, out=dev)
    torch.cuda.synchronize()
    for t in range(len(shapes)):
        for r in range(P):
            assert torch.equal(dev[r][t].reshape(-1).view(torch.int32),
                               single[t][r].view(torch.int32)), (t, r)


def test_per_parameter_ddp_step_on_a_tiny_mlp():
    """CS336 Lecture 8, "Data Parallelism (DDP)": each rank computes the
    gradient of its shard, every param.grad is all-reduced with AVG, and the
    ranks hold the full-batch gradient."""
    W = 4
    torch.manual_seed(0)
    net = torch.nn.Sequential(torch.nn.Linear(16, 32), torch.nn.Tanh(), torch.nn.Linear(32, 3))
    g = torch.Generator().manual_seed(1)
    X = torch.randn(32, 16, generator=g)
    y = torch.randint(0, 3, (32,), generator=g)

    def grads(xb, yb):
        net.zero_grad()
        F.cross_entropy(net(xb), yb).backward()
        return [p.grad.detach().clone() for p in net.parameters()]

    full = grads(X, y)
    shard = [grads(X[r::W], y[r::W]) for r in range(W)]
    shapes = [tuple(p.shape) for p in net.parameters()]
    m = ddp.MultiAllReduce(shapes, W, torch.float32, device=DEV)
    dev = [[t.to(DEV) for t in shard[r]] for r in range(W)]
    out = m(dev, "mean", W)
    torch.cuda.synchronize()
    for t, s in enumerate(shapes):
        Xs = np.stack([shard[r][t].numpy().reshape(-1) for r in range(W)])
        want, _ = oracle.ring_allreduce(Xs, "mean", W)
        for r in range(W):
            assert_same_bits(out[r][t].cpu().numpy().reshape(-1), want[r], f"param {t}")
        d = np.linalg.norm(out[0][t].cpu().numpy() - full[t].numpy()) / np.linalg.norm(full[t].numpy())
        assert d < 1e-5
