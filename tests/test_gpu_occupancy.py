"""The cap on resident workgroups per CU is a launch-shape choice, not part
of the method: every kernel family gives the oracle's bits whatever cap it
runs with (ddp_set_wg_per_cu), including no cap and the smallest one."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, assert_same_bits, oracle_ring, to_device, to_host, torch_dtype

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")

CAPS = [0, 2, 3, 7, 16, -1]


@pytest.fixture(autouse=True)
def builtin_caps_afterwards():
    yield
    for family in ddp.KERNEL_FAMILIES:
        ddp.ddp_set_wg_per_cu(family, -1)


def draw(P, n, dtype, seed):
    X = workloads.rank_buffers(P, n, dist="wide", seed=seed)
    return workloads.to_bf16_bits(X) if dtype == "bf16" else X


@pytest.mark.parametrize("pair", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
def test_ring_same_bits_at_every_cap(pair):
    it, ot = pair
    P, n, C = 8, 300_007, 8
    X = draw(P, n, it, seed=41)
    want = oracle_ring(X, "mean", C, in_dtype=it, out_dtype=ot)
    for cap in CAPS:
        ddp.ddp_set_wg_per_cu("ring", cap)
        out = ddp.allreduce(to_device(X, it), "mean", C, out_dtype=torch_dtype(ot))
        torch.cuda.synchronize()
        assert_same_bits(to_host(out), want, f"{it}->{ot} cap={cap}")


def test_bucketed_call_same_bits_at_every_cap():
    """The bucketed call (the full buckets as one ring and the partial one
    as a second segment, one launch) at every cap."""
    P, C, E = 8, 8, 32768
    n = 3 * E + 12347
    X = draw(P, n, "f32", seed=47)
    want = np.concatenate([oracle_ring(X[:, lo:lo + E], "mean", C) for lo in range(0, n, E)], axis=1)
    assert ddp.ddp_buckets_launch_count(P, C, ddp.F32, ddp.F32, False, n, E) == 1
    for cap in CAPS:
        ddp.ddp_set_wg_per_cu("ring", cap)
        out = ddp.allreduce(to_device(X, "f32"), "mean", C, bucket_elems=E)
        torch.cuda.synchronize()
        assert_same_bits(to_host(out), want, f"cap={cap}")


def test_fused_sgd_same_bits_at_every_cap():
    P, n, C = 8, 200_003, 8
    G = draw(P, n, "bf16", seed=42)
    w0 = workloads.rank_buffers(1, n, "normal", 0.02, seed=43)[0]
    v0 = workloads.rank_buffers(1, n, "normal", 1e-3, seed=44)[0]
    g, _ = oracle.ring_allreduce(G, "mean", C, in_dtype="bf16", out_dtype="f32")
    ow, ov = oracle.sgd_momentum(g[0], w0, v0, 1e-3, 0.9)
    want_out = oracle_ring(G, "mean", C, in_dtype="bf16", out_dtype="bf16")
    for cap in CAPS:
        ddp.ddp_set_wg_per_cu("ring_sgd", cap)
        for with_out in (False, True):
            w = torch.from_numpy(w0.copy()).to(DEV)
            v = torch.from_numpy(v0.copy()).to(DEV)
            grads = to_device(G, "bf16")
            out = [torch.empty_like(t) for t in grads] if with_out else None
            ddp.allreduce_sgd(grads, w, v, 1e-3, 0.9, "mean", C, out=out)
            torch.cuda.synchronize()
            assert_same_bits(w.cpu().numpy(), ow, f"w cap={cap} out={with_out}")
            assert_same_bits(v.cpu().numpy(), ov, f"v cap={cap} out={with_out}")
            if with_out:
                assert_same_bits(to_host(out), want_out, f"grads cap={cap}")


def test_tree_halves_and_stepwise_same_bits_at_every_cap():
    P, n, C = 8, 250_001, 8
    X = draw(P, n, "f32", seed=45)
    want_tree, _ = oracle.tree_allreduce(X, "mean", 2)
    want_ring = oracle_ring(X, "mean", C)
    for cap in CAPS:
        for family in ("tree", "reduce_scatter", "all_gather", "step"):
            ddp.ddp_set_wg_per_cu(family, cap)
        tree = ddp.allreduce_tree(to_device(X, "f32"), "mean", 2)
        halves = ddp.reduce_scatter(to_device(X, "f32"), "mean", C)
        ddp.all_gather(halves, C)
        steps = to_device(X, "f32")
        ddp.allreduce_stepwise(steps, "mean", C)
        torch.cuda.synchronize()
        assert_same_bits(to_host(tree), want_tree, f"tree cap={cap}")
        assert_same_bits(to_host(halves), want_ring, f"reduce-scatter + all-gather cap={cap}")
        assert_same_bits(to_host(steps), want_ring, f"stepwise cap={cap}")


def test_multi_tensor_and_bucket_copy_same_bits_at_every_cap():
    P, C = 4, 4
    shapes = [(1,), (7,), (3, 5), (1000,), (4097,), (33, 129), (70001,)]
    rng = np.random.default_rng(46)
    host = [[(rng.standard_normal(s) * np.exp2(rng.integers(-20, 21, s))).astype(np.float32)
             for s in shapes] for _ in range(P)]
    dev = [[torch.from_numpy(x).to(DEV) for x in hs] for hs in host]
    want = [oracle_ring(np.stack([host[r][t].reshape(-1) for r in range(P)]), "sum", C)
            for t in range(len(shapes))]
    bucket_bytes = 16 << 10
    packed = [oracle.pack(host[r], 4, bucket_bytes) for r in range(P)]
    m = ddp.MultiAllReduce(shapes, P, torch.float32, device=DEV)
    b = ddp.GradBucketer(shapes, torch.float32, bucket_bytes, device=DEV)
    table = b.pointer_table(dev)
    bufs = b.alloc_buckets(P)
    for cap in CAPS:
        ddp.ddp_set_wg_per_cu("multi", cap)
        ddp.ddp_set_wg_per_cu("bucket_copy", cap)
        out = m(dev, "sum", C)
        torch.cuda.synchronize()
        for t in range(len(shapes)):
            got = np.stack([out[r][t].cpu().numpy().reshape(-1) for r in range(P)])
            assert_same_bits(got, want[t], f"multi t={t} cap={cap}")
        back = [[torch.zeros_like(x) for x in ds] for ds in dev]
        back_table = b.pointer_table(back)
        for k in range(b.n_buckets):        # one bucket buffer per rank: pack, check, unpack
            b.pack(table, k, bufs)
            torch.cuda.synchronize()
            for r in range(P):
                assert np.array_equal(bufs[r][:b.bucket_len(k)].cpu().numpy(), packed[r][k]), (cap, k, r)
            b.unpack(back_table, k, bufs)
        torch.cuda.synchronize()
        for r in range(P):
            for t in range(len(shapes)):
                assert np.array_equal(back[r][t].cpu().numpy(), host[r][t]), (cap, r, t)
