"""GPU parity of the ring all-reduce and the fused SGD step against the CPU
oracle: bit for bit, through the C ABI, on seeded inputs sized to span many
tiles plus a ragged tail, and on the edge cases of the method."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, assert_same_bits, oracle_ring, to_device, to_host, torch_dtype

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")


def gpu_ring(X, op, C, in_dtype="f32", out_dtype=None, inplace=False):
    out_dtype = out_dtype or in_dtype
    ins = to_device(X, in_dtype)
    outs = ins if inplace else [torch.empty_like(t, dtype=torch_dtype(out_dtype)) for t in ins]
    ddp.allreduce(ins, op, C, out=outs)
    torch.cuda.synchronize()
    return to_host(outs)


def draw(P, n, dtype, seed, dist="wide"):
    X = workloads.rank_buffers(P, n, dist=dist, seed=seed)
    return workloads.to_bf16_bits(X) if dtype == "bf16" else X


def test_p4_65536_f32_sum():
    """P = 4 ranks, 65,536 fp32 gradients N(0,1) per rank, 4 chunks, Sum."""
    X = workloads.rank_buffers(4, 65536, "normal", 1.0, seed=0)
    Y = gpu_ring(X, "sum", 4)
    assert_same_bits(Y, oracle_ring(X, "sum", 4), "P=4, 65,536 fp32, Sum, 4 chunks")
    for r in range(1, 4):
        assert np.array_equal(Y[r].view(np.uint32), Y[0].view(np.uint32))


def test_hand_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "ring_hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        X = np.array(c["inputs"], np.float32)
        Y = gpu_ring(X, "sum", c["chunking"])
        assert (Y == np.array(c["sum"], np.float32)[None, :]).all(), c["name"]
        Ym = gpu_ring(X, "mean", c["chunking"])
        want = np.array([int(h, 16) for h in c["mean_f32_bits"]], np.uint32)
        assert (Ym.view(np.uint32) == want[None, :]).all(), c["name"]


SIZES = [1, 3, 5, 37, 1000, 4099, 70001]


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 7, 8, 9, 12, 16])
def test_sweep_f32(P):
    for n in SIZES:
        for C in sorted({1, P, 2 * P + 1, n}):
            for op in ("sum", "mean"):
                X = draw(P, n, "f32", seed=P * 7919 + n + C)
                got = gpu_ring(X, op, C)
                assert_same_bits(got, oracle_ring(X, op, C), f"P={P} n={n} C={C} {op}")


@pytest.mark.parametrize("pair", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("P", [2, 3, 4, 6, 8, 12, 16])
def test_sweep_mixed_types(pair, P):
    it, ot = pair
    for n in (1, 7, 9, 1000, 16391, 70001):
        for C in sorted({1, P, 3 * P + 1, n}):
            for op in ("sum", "mean"):
                X = draw(P, n, it, seed=P * 31 + n + C)
                got = gpu_ring(X, op, C, it, ot)
                want = oracle_ring(X, op, C, in_dtype=it, out_dtype=ot)
                assert_same_bits(got, want, f"{it}->{ot} P={P} n={n} C={C} {op}")


@pytest.mark.parametrize("P", list(range(1, 17)))
def test_bf16_to_f32_every_rank_count(P):
    """bf16 -> float32, the type pair whose kernels pause at each
    workgroup's start by rank count: bit-exact against the oracle for every
    P, across tiles, chunk boundaries and a ragged tail."""
    for n in (9, 70001):
        for C in sorted({1, P, 2 * P + 1}):
            X = draw(P, n, "bf16", seed=P * 131 + n + C)
            got = gpu_ring(X, "mean", C, "bf16", "f32")
            want = oracle_ring(X, "mean", C, in_dtype="bf16", out_dtype="f32")
            assert_same_bits(got, want, f"bf16->f32 P={P} n={n} C={C}")


def test_many_tiles_and_chunk_boundaries():
    """Sizes where chunk boundaries fall inside tiles and inside vectors."""
    for P, n, C in ((8, 1_000_003, 8), (8, 1_048_576 + 12, 16), (4, 524_287, 4),
                    (8, 2_000_001, 24), (3, 999_999, 3)):
        X = draw(P, n, "f32", seed=n)
        assert_same_bits(gpu_ring(X, "mean", C), oracle_ring(X, "mean", C), f"P={P} n={n}")


def test_in_place():
    for it in ("f32", "bf16"):
        X = draw(8, 100_003, it, seed=1)
        got = gpu_ring(X, "mean", 8, it, it, inplace=True)
        assert_same_bits(got, oracle_ring(X, "mean", 8, in_dtype=it), it)


def test_special_values():
    P, n = 4, 64
    X = workloads.rank_buffers(P, n, "normal", 1.0, seed=3)
    X[0, 0] = np.inf
    X[1, 1], X[2, 1] = np.inf, -np.inf
    X[0, 2] = np.nan
    X[:, 3] = -0.0
    X[:, 4] = np.float32(2.0 ** -140)              # subnormal
    X[:, 5] = np.float32(3.0e38)                   # overflows to inf when summed
    X[:, 6] = np.float32(1.0e-45)                  # smallest subnormal
    for op in ("sum", "mean"):
        for C in (1, 4, 64):
            got = gpu_ring(X, op, C)
            assert_same_bits(got, oracle_ring(X, op, C), f"{op} C={C}")
    assert np.isinf(gpu_ring(X, "sum", 4)[0, 5])
    assert gpu_ring(X, "sum", 4)[0, 4] == np.float32(2.0 ** -138)
    assert np.signbit(gpu_ring(X, "sum", 4)[0, 3])


def test_integer_valued_exact_sum():
    for P in (2, 8, 16):
        X = workloads.rank_buffers(P, 50_000, "int", 1024, seed=P)
        got = gpu_ring(X, "sum", P)
        assert np.array_equal(got[0].astype(np.int64), X.astype(np.int64).sum(0))


def test_mean_is_sum_over_P_on_gpu():
    for P in (3, 5, 6, 7, 8):
        X = draw(P, 30_001, "f32", seed=P)
        s = gpu_ring(X, "sum", P)
        m = gpu_ring(X, "mean", P)
        assert_same_bits(m, s / np.float32(P), f"P={P}")


def test_deterministic():
    X = draw(8, 300_007, "f32", seed=11)
    assert_same_bits(gpu_ring(X, "mean", 8), gpu_ring(X, "mean", 8), "two runs")


def test_bf16_within_relative_tolerance_of_exact():
    """bf16 inputs, fp32 accumulation: within 1e-2 relative of the exact
    mean of the bf16 values, measured as the pages measure (norm of the
    difference over the norm of the reference)."""
    P, n = 8, 200_000
    X = workloads.to_bf16_bits(workloads.rank_buffers(P, n, "normal", 1e-3, seed=5))
    exact = oracle.bf16_bits_to_f32(X).astype(np.float64).sum(0) / P
    for ot in ("bf16", "f32"):
        got = gpu_ring(X, "mean", P, "bf16", ot)[0]
        g = oracle.bf16_bits_to_f32(got) if ot == "bf16" else got
        rel = np.linalg.norm(g.astype(np.float64) - exact) / np.linalg.norm(exact)
        assert rel <= 1e-2, (ot, rel)


def test_more_than_one_launch():
    """Buffers over 2^29 elements are split into launches; the chunk order
    runs across the split."""
    P, n, C = 2, (1 << 29) + 77, 3
    ins = [torch.empty(n, dtype=torch.float32, device=DEV) for _ in range(P)]
    for r, t in enumerate(ins):
        workloads.torch_normal_(t, 1.0, seed=100 + r)
    outs = [torch.empty_like(t) for t in ins]
    ddp.allreduce(ins, "sum", C, out=outs)
    torch.cuda.synchronize()
    L = -(-n // C)
    idx = np.unique(np.concatenate([
        np.arange(0, 64), np.arange(L - 40, L + 40), np.arange(2 * L - 40, 2 * L + 40),
        np.arange((1 << 29) - 40, (1 << 29) + 40), np.arange(n - 64, n),
        np.random.default_rng(0).integers(0, n, 2000)]))
    it = torch.from_numpy(idx).to(DEV)
    V = np.stack([t[it].cpu().numpy() for t in ins])
    start = oracle.chunk_start_ranks_at(n, C, P, idx)
    want = oracle.ring_allreduce_sampled(V, start, "sum")
    got = np.stack([t[it].cpu().numpy() for t in outs])
    assert_same_bits(got, want, "split launch")
    del ins, outs
    torch.cuda.empty_cache()


def sampled_indices(n, C, extra=()):
    """Indices around every chunk boundary, the launch split at 2^29, both
    ends, and random ones."""
    L = -(-n // C)
    parts = [np.arange(0, 64), np.arange(n - 64, n), np.arange((1 << 29) - 40, (1 << 29) + 40),
             np.random.default_rng(1).integers(0, n, 2000)]
    parts += [np.arange(max(0, j * L - 40), min(n, j * L + 40)) for j in range(1, C)]
    parts += list(extra)
    return np.unique(np.concatenate(parts))


def test_more_than_one_launch_bf16_to_f32():
    """bf16 -> fp32 (outputs twice as wide as the inputs) carries the chunk
    order across the split at 2^29 elements."""
    P, n, C = 3, (1 << 29) + 77, 4
    ins = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    for r, t in enumerate(ins):
        workloads.torch_normal_(t, 1.0, seed=200 + r)
    outs = [torch.empty(n, dtype=torch.float32, device=DEV) for _ in range(P)]
    ddp.allreduce(ins, "mean", C, out=outs)
    torch.cuda.synchronize()
    idx = sampled_indices(n, C)
    it = torch.from_numpy(idx).to(DEV)
    V = np.stack([t[it].view(torch.int16).cpu().numpy().view(np.uint16) for t in ins])
    start = oracle.chunk_start_ranks_at(n, C, P, idx)
    want = oracle.ring_allreduce_sampled(V, start, "mean", in_dtype="bf16", out_dtype="f32")
    got = np.stack([t[it].cpu().numpy() for t in outs])
    assert_same_bits(got, want, "split launch, bf16 -> f32")
    del ins, outs
    torch.cuda.empty_cache()


def test_chunks_longer_than_2_30_elements():
    """Chunks longer than 2^30 elements: a launch of 2^29 elements then holds
    at most one chunk boundary, which the launch's chunk map must place
    exactly (here inside the fourth launch); in place, bf16, Mean."""
    P, n, C = 3, 3 * (1 << 30) + 4097, 2
    L = -(-n // C)
    assert L > (1 << 30)
    bufs = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    for r, t in enumerate(bufs):
        workloads.torch_normal_(t, 1.0, seed=400 + r)
    splits = [np.arange(max(0, k * (1 << 29) - 40), min(n, k * (1 << 29) + 40)) for k in range(1, 7)]
    idx = sampled_indices(n, C, extra=splits)
    it = torch.from_numpy(idx).to(DEV)
    V = np.stack([t[it].view(torch.int16).cpu().numpy().view(np.uint16) for t in bufs])
    ddp.allreduce(bufs, "mean", C, out=bufs)
    torch.cuda.synchronize()
    start = oracle.chunk_start_ranks_at(n, C, P, idx)
    assert set(start.tolist()) == {0, 1}
    want = oracle.ring_allreduce_sampled(V, start, "mean", in_dtype="bf16", out_dtype="bf16")
    got = np.stack([t[it].view(torch.int16).cpu().numpy().view(np.uint16) for t in bufs])
    assert_same_bits(got, want, "chunks over 2^30 elements")
    del bufs
    torch.cuda.empty_cache()


def test_more_than_one_launch_fused_sgd():
    """The optimizer state is offset with the gradients at every launch."""
    P, n, C = 3, (1 << 29) + 77, 3
    grads = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    for r, t in enumerate(grads):
        workloads.torch_normal_(t, 1e-3, seed=300 + r)
    w = torch.empty(n, dtype=torch.float32, device=DEV)
    v = torch.empty(n, dtype=torch.float32, device=DEV)
    workloads.torch_normal_(w, 0.02, seed=310)
    workloads.torch_normal_(v, 1e-3, seed=311)
    idx = sampled_indices(n, C)
    it = torch.from_numpy(idx).to(DEV)
    w0 = w[it].cpu().numpy()
    v0 = v[it].cpu().numpy()
    ddp.allreduce_sgd(grads, w, v, 1e-3, 0.9, "mean", C)
    torch.cuda.synchronize()
    V = np.stack([t[it].view(torch.int16).cpu().numpy().view(np.uint16) for t in grads])
    start = oracle.chunk_start_ranks_at(n, C, P, idx)
    g = oracle.ring_allreduce_sampled(V, start, "mean", in_dtype="bf16", out_dtype="f32")[0]
    w1, v1 = oracle.sgd_momentum(g, w0, v0, 1e-3, 0.9)
    assert_same_bits(w[it].cpu().numpy(), w1, "split launch, w")
    assert_same_bits(v[it].cpu().numpy(), v1, "split launch, v")
    del grads, w, v
    torch.cuda.empty_cache()


# ------------------------------------------------------------- fused SGD ----

@pytest.mark.parametrize("gt,ot", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("P", [1, 3, 8])
def test_fused_sgd(gt, ot, P):
    for n in (5, 10_007, 262_147):
        for C in (P, 2 * P + 1):
            X = draw(P, n, gt, seed=n + P, dist="normal")
            if gt == "f32":
                X = X * np.float32(1e-3)
            w0 = workloads.rank_buffers(1, n, "normal", 0.02, seed=1)[0]
            v0 = workloads.rank_buffers(1, n, "normal", 1e-3, seed=2)[0]
            grads = to_device(X, gt)
            w = torch.from_numpy(w0.copy()).to(DEV)
            v = torch.from_numpy(v0.copy()).to(DEV)
            outs = [torch.empty(n, dtype=torch_dtype(ot), device=DEV) for _ in range(P)]
            ddp.allreduce_sgd(grads, w, v, 1e-3, 0.9, "mean", C, out=outs)
            # second step with the same gradients and no gradient output
            w2 = w.clone()
            v2 = v.clone()
            ddp.allreduce_sgd(grads, w2, v2, 1e-3, 0.9, "mean", C)
            torch.cuda.synchronize()
            g = oracle_ring(X, "mean", C, in_dtype=gt, out_dtype="f32")[0]
            ow, ov = oracle.sgd_momentum(g, w0, v0, 1e-3, 0.9)
            ow2, ov2 = oracle.sgd_momentum(g, ow, ov, 1e-3, 0.9)
            tag = f"{gt}->{ot} P={P} n={n} C={C}"
            assert_same_bits(w.cpu().numpy(), ow, "w " + tag)
            assert_same_bits(v.cpu().numpy(), ov, "v " + tag)
            assert_same_bits(w2.cpu().numpy(), ow2, "w2 " + tag)
            assert_same_bits(v2.cpu().numpy(), ov2, "v2 " + tag)
            assert_same_bits(to_host(outs), oracle_ring(X, "mean", C, in_dtype=gt, out_dtype=ot),
                             "grads " + tag)


def test_fused_sgd_sum_and_zero_momentum():
    P, n = 4, 9_999
    X = draw(P, n, "f32", seed=3, dist="normal")
    w0 = workloads.rank_buffers(1, n, "normal", 1.0, seed=4)[0]
    v0 = workloads.rank_buffers(1, n, "normal", 1.0, seed=5)[0]
    w = torch.from_numpy(w0.copy()).to(DEV)
    v = torch.from_numpy(v0.copy()).to(DEV)
    ddp.allreduce_sgd(to_device(X, "f32"), w, v, 0.5, 0.0, "sum", P)
    torch.cuda.synchronize()
    g = oracle_ring(X, "sum", P)[0]
    ow, ov = oracle.sgd_momentum(g, w0, v0, 0.5, 0.0)
    assert_same_bits(w.cpu().numpy(), ow, "w")
    assert_same_bits(v.cpu().numpy(), ov, "v")
    assert np.array_equal(v.cpu().numpy(), g)


@pytest.mark.parametrize("layout", ["flat buffer, off lines", "alloc_state"])
@pytest.mark.parametrize("bucketed", [False, True])
def test_fused_sgd_state_layouts(layout, bucketed):
    """Master weights and momentum 16-byte aligned but inside 128-byte lines
    (w 16 bytes in, v 32 bytes in, both carved from one flat buffer, the
    gradients 16 bytes in), and the buffers GradBucketer.alloc_state lays
    out, as one call and as a bucketed call: bit for bit the oracle's ring
    Mean and momentum step, every bucket its own ring."""
    P, n, C = 8, 262_147, 8
    E = 65_536                          # bf16 elements per bucket of the bucketed call
    X = draw(P, n, "bf16", seed=41, dist="normal")
    w0 = workloads.rank_buffers(1, n, "normal", 0.02, seed=42)[0]
    v0 = workloads.rank_buffers(1, n, "normal", 1e-3, seed=43)[0]
    rows = [torch.empty(n + 64, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    grads = [r[8:8 + n] for r in rows]
    for g, h in zip(grads, to_device(X, "bf16")):
        g.copy_(h)
    if layout == "alloc_state":
        plan = ddp.GradBucketer([(n,)], torch.bfloat16, 2 * E, device=DEV)
        w, v = plan.alloc_state()
        assert w.data_ptr() % 128 == 0 and v.data_ptr() % 128 == 0
    else:
        flat = torch.empty(2 * n + 64, dtype=torch.float32, device=DEV)
        vo = -(-(4 + n) // 4) * 4
        w, v = flat[4:4 + n], flat[vo:vo + n]
        assert w.data_ptr() % 128 == 16 and v.data_ptr() % 128 == 32
    w.copy_(torch.from_numpy(w0))
    v.copy_(torch.from_numpy(v0))
    outs = [torch.empty(n, dtype=torch.float32, device=DEV) for _ in range(P)]
    ddp.allreduce_sgd(grads, w, v, 1e-3, 0.9, "mean", C, out=outs, bucket_elems=E if bucketed else None)
    w2, v2 = w.clone(), v.clone()
    ddp.allreduce_sgd(grads, w, v, 1e-3, 0.9, "mean", C, bucket_elems=E if bucketed else None)
    torch.cuda.synchronize()
    if bucketed:
        g = np.concatenate([oracle_ring(X[:, lo:lo + E], "mean", C, in_dtype="bf16", out_dtype="f32")[0]
                            for lo in range(0, n, E)])
    else:
        g = oracle_ring(X, "mean", C, in_dtype="bf16", out_dtype="f32")[0]
    ow, ov = oracle.sgd_momentum(g, w0, v0, 1e-3, 0.9)
    ow2, ov2 = oracle.sgd_momentum(g, ow, ov, 1e-3, 0.9)
    tag = f"{layout}, {'bucketed' if bucketed else 'one call'}"
    assert_same_bits(w2.cpu().numpy(), ow, "w, first step, " + tag)
    assert_same_bits(v2.cpu().numpy(), ov, "v, first step, " + tag)
    assert_same_bits(w.cpu().numpy(), ow2, "w, second step, " + tag)
    assert_same_bits(v.cpu().numpy(), ov2, "v, second step, " + tag)
    for r in range(P):
        assert_same_bits(outs[r].cpu().numpy(), g, f"gradient out rank {r}, " + tag)


def test_fused_steps_round_every_operation_once():
    """The two hand-worked cases where a fused multiply-add would differ
    (mu * v a tie that rounds to even and is then cancelled by g; lr * v
    rounded up and then cancelled by w), repeated over several tiles and a
    ragged tail, through every fused optimizer entry point: P = 2 ranks,
    Sum, rank 1 all zeros, so the reduced gradient is rank 0's exactly."""
    n = 3 * 4096 + 5
    case = np.arange(n) % 2
    g = np.where(case == 0, -11324620 * 2.0 ** -22, 3.0).astype(np.float32)
    w0 = np.where(case == 0, 0.5, 10066330 * 2.0 ** -25).astype(np.float32)
    v0 = np.where(case == 0, 3.0, 0.0).astype(np.float32)
    want_w = np.where(case == 0, 0.5, 0.0).astype(np.float32)
    want_v = np.where(case == 0, 0.0, 3.0).astype(np.float32)
    X = np.stack([g, np.zeros(n, np.float32)])
    ow, ov = oracle.sgd_momentum(g, w0, v0, 0.1, 0.9)
    assert np.array_equal(ow, want_w) and np.array_equal(ov, want_v)

    w = torch.from_numpy(w0.copy()).to(DEV)
    v = torch.from_numpy(v0.copy()).to(DEV)
    ddp.allreduce_sgd(to_device(X, "f32"), w, v, 0.1, 0.9, "sum", 2)
    torch.cuda.synchronize()
    assert_same_bits(w.cpu().numpy(), want_w, "allreduce_sgd w")
    assert_same_bits(v.cpu().numpy(), want_v, "allreduce_sgd v")

    w = torch.from_numpy(w0.copy()).to(DEV)
    v = torch.from_numpy(v0.copy()).to(DEV)
    params = [torch.empty(n, device=DEV) for _ in range(2)]
    ddp.zero1_sgd_step(to_device(X, "f32"), w, v, 0.1, 0.9, params, "sum", 2)
    torch.cuda.synchronize()
    assert_same_bits(w.cpu().numpy(), want_w, "zero1 w")
    assert_same_bits(v.cpu().numpy(), want_v, "zero1 v")
    assert_same_bits(to_host(params), np.stack([want_w, want_w]), "zero1 params")

    m = ddp.MultiAllReduce([(n,)], 2, torch.float32, device=DEV)
    grads = [[t] for t in to_device(X, "f32")]
    w = torch.from_numpy(w0.copy()).to(DEV)
    v = torch.from_numpy(v0.copy()).to(DEV)
    run = m.bind_sgd(grads, [w], [v])
    run(0.1, 0.9, "sum", 2)
    torch.cuda.synchronize()
    assert_same_bits(w.cpu().numpy(), want_w, "multi w")
    assert_same_bits(v.cpu().numpy(), want_v, "multi v")
