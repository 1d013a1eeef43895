"""GPU parity of the ZeRO stage 1 step against the oracle's phase-by-phase
simulation (reduce-scatter, the owner's momentum step, all-gather of the
updated parameters), bit for bit, and its equality with the replicated
fused SGD step."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, assert_same_bits, to_device, to_host, torch_dtype

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")


def state(n, seed):
    w = workloads.rank_buffers(1, n, "normal", 0.02, seed=seed)[0]
    v = workloads.rank_buffers(1, n, "normal", 1e-3, seed=seed + 1)[0]
    return w, v


def grads(P, n, dtype, seed):
    X = workloads.rank_buffers(P, n, "wide", seed=seed)
    return workloads.to_bf16_bits(X) if dtype == "bf16" else X


def run(X, gt, pt, w, v, lr, mu, op, C, inplace=False):
    g = to_device(X, gt)
    wd = torch.from_numpy(w.copy()).to(DEV)
    vd = torch.from_numpy(v.copy()).to(DEV)
    params = g if inplace else [torch.empty(X.shape[1], dtype=torch_dtype(pt), device=DEV) for _ in g]
    ddp.zero1_sgd_step(g, wd, vd, lr, mu, params, op, C)
    torch.cuda.synchronize()
    return to_host(params), wd.cpu().numpy(), vd.cpu().numpy()


@pytest.mark.parametrize("gt,pt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
def test_zero1_equals_oracle(gt, pt, P):
    for n in (1, 9, 4101, 70001):
        for C in sorted({P, 3, 2 * P}):
            op = ("mean", "sum")[(n + C) % 2]
            X = grads(P, n, gt, seed=P * 1000 + n + C)
            w, v = state(n, seed=n + C)
            got_p, got_w, got_v = run(X, gt, pt, w, v, 1e-3, 0.9, op, C)
            want_p, want_w, want_v, _ = oracle.zero1_sgd_step(X, w, v, 1e-3, 0.9, op, C, gt, pt)
            what = f"{gt}->{pt} P={P} n={n} C={C} {op}"
            assert_same_bits(got_w[None], want_w[None], what + " w")
            assert_same_bits(got_v[None], want_v[None], what + " v")
            assert_same_bits(got_p, want_p, what + " params")


def test_zero1_in_place_over_the_gradients():
    P, n = 8, 100_003
    X = grads(P, n, "bf16", seed=5)
    w, v = state(n, seed=6)
    got_p, got_w, _ = run(X, "bf16", "bf16", w, v, 1e-3, 0.9, "mean", P, inplace=True)
    want_p, want_w, _, _ = oracle.zero1_sgd_step(X, w, v, 1e-3, 0.9, "mean", P, "bf16", "bf16")
    assert_same_bits(got_p, want_p, "in place")
    assert_same_bits(got_w[None], want_w[None], "in place w")


def test_zero1_equals_replicated_fused_sgd():
    """Stage 1 only partitions the state: the GPU's two calls give the same
    master weights and momentum, and the parameters are their rounding."""
    P, n = 8, 1_000_003
    X = grads(P, n, "bf16", seed=7)
    w, v = state(n, seed=8)
    p1, w1, v1 = run(X, "bf16", "bf16", w, v, 1e-3, 0.9, "mean", P)
    wd = torch.from_numpy(w.copy()).to(DEV)
    vd = torch.from_numpy(v.copy()).to(DEV)
    ddp.allreduce_sgd(to_device(X, "bf16"), wd, vd, 1e-3, 0.9, "mean", P)
    torch.cuda.synchronize()
    assert_same_bits(w1[None], wd.cpu().numpy()[None], "w")
    assert_same_bits(v1[None], vd.cpu().numpy()[None], "v")
    want = oracle.f32_to_bf16_bits(w1)
    for r in range(P):
        assert_same_bits(p1[r][None], want[None], f"rank {r}")


def test_zero1_full_vit_bucket():
    """A full 25 MiB bf16 bucket of the ViT-B/16 gradient set (13,107,200
    elements x 8 ranks), N(0, 1e-3) gradients, master weights N(0, 0.02),
    momentum N(0, 1e-3), lr 1e-3, mu 0.9, bf16 parameters."""
    P, n = 8, 13_107_200
    X = workloads.to_bf16_bits(workloads.rank_buffers(P, n, "normal", 1e-3, seed=9))
    w, v = state(n, seed=10)
    got_p, got_w, got_v = run(X, "bf16", "bf16", w, v, 1e-3, 0.9, "mean", P)
    want_p, want_w, want_v, _ = oracle.zero1_sgd_step(X, w, v, 1e-3, 0.9, "mean", P, "bf16", "bf16")
    assert_same_bits(got_w[None], want_w[None], "w")
    assert_same_bits(got_v[None], want_v[None], "v")
    assert_same_bits(got_p, want_p, "params")
    assert np.array_equal(got_p[0], got_p[P - 1])
