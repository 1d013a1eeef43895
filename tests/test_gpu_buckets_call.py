"""GPU parity of the bucketed calls (allreduce_ring_buckets,
allreduce_fused_sgd_buckets): every bucket of the flat rank buffers equals,
bit for bit, the oracle's ring over that bucket alone and the single-bucket
call on it -- on the path that joins consecutive full buckets into one ring
(C a multiple of P, E a multiple of C) and on the bucket-by-bucket path,
with and without a partial last bucket, in place, and for every pair of
element types."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, assert_same_bits, oracle_ring, to_device, to_host, torch_dtype

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")


def draw(P, n, dtype, seed):
    X = workloads.rank_buffers(P, n, dist="wide", seed=seed)
    return workloads.to_bf16_bits(X) if dtype == "bf16" else X


def per_bucket_oracle(X, op, C, E, it, ot):
    P, n = X.shape
    parts = [oracle_ring(X[:, lo:min(n, lo + E)], op, C, in_dtype=it, out_dtype=ot)
             for lo in range(0, n, E)]
    return np.concatenate(parts, axis=1)


# (P, C, E, n): joint full buckets and the tail in one launch (two
# segments: tails of whole tiles and chunks at least a tile long, with a
# ragged end), joint path with a short tail, joint without a tail, C not a
# multiple of P, E not a multiple of C, one bucket, a tail only, one full
# bucket and a tail, 16 ranks
CASES = [
    (4, 4, 16384, 3 * 16384 + 5001),
    (8, 8, 32768, 2 * 32768 + 12347),
    (3, 6, 12288, 4 * 12288 + 9001),
    (8, 8, 16384, 3 * 16384 + 1001),
    (4, 4, 10000, 4 * 10000),
    (3, 6, 6000, 5 * 6000 + 13),
    (8, 17, 8192, 3 * 8192 + 5),
    (5, 5, 4104, 4 * 4104 + 3),
    (2, 2, 8192, 8192),
    (4, 8, 65536, 4097),
    (4, 4, 8192, 8192 + 3001),
    (8, 17, 65536, 65536 + 9000),
    (16, 16, 16384, 2 * 16384 + 7777),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("pair", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_buckets_equal_oracle_and_single_calls(case, pair):
    P, C, E, n = case
    it, ot = pair
    X = draw(P, n, it, seed=P * 1000 + C + n % 97)
    want = per_bucket_oracle(X, "mean", C, E, it, ot)
    out = ddp.allreduce(to_device(X, it), "mean", C, out_dtype=torch_dtype(ot), bucket_elems=E)
    torch.cuda.synchronize()
    assert_same_bits(to_host(out), want, f"{it}->{ot} P={P} C={C} E={E} n={n}")
    ins = to_device(X, it)
    single = [torch.empty(n, dtype=torch_dtype(ot), device=DEV) for _ in range(P)]
    for lo in range(0, n, E):
        hi = min(n, lo + E)
        ddp.allreduce([t[lo:hi] for t in ins], "mean", C, out=[t[lo:hi] for t in single])
    torch.cuda.synchronize()
    assert_same_bits(to_host(single), to_host(out), "single-bucket calls")


@pytest.mark.parametrize("case", CASES[:6])
def test_buckets_in_place_and_sum(case):
    P, C, E, n = case
    X = draw(P, n, "f32", seed=7 + n)
    ts = to_device(X, "f32")
    ddp.allreduce(ts, "sum", C, out=ts, bucket_elems=E)
    torch.cuda.synchronize()
    assert_same_bits(to_host(ts), per_bucket_oracle(X, "sum", C, E, "f32", "f32"), f"case {case}")


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("gt", ["bf16", "f32"])
def test_fused_sgd_buckets_equal_oracle(case, gt):
    P, C, E, n = case
    X = draw(P, n, gt, seed=P + C + n)
    w0 = workloads.rank_buffers(1, n, "normal", 0.02, seed=8)[0]
    v0 = workloads.rank_buffers(1, n, "normal", 1e-3, seed=9)[0]
    g = per_bucket_oracle(X, "mean", C, E, gt, "f32")[0]
    ow, ov = oracle.sgd_momentum(g, w0, v0, 1e-3, 0.9)
    for with_out in (False, True):
        w = torch.from_numpy(w0.copy()).to(DEV)
        v = torch.from_numpy(v0.copy()).to(DEV)
        grads = to_device(X, gt)
        out = [torch.empty_like(t) for t in grads] if with_out else None
        ddp.allreduce_sgd(grads, w, v, 1e-3, 0.9, "mean", C, out=out, bucket_elems=E)
        torch.cuda.synchronize()
        tag = f"{gt} P={P} C={C} E={E} n={n} out={with_out}"
        assert_same_bits(w.cpu().numpy(), ow, "w " + tag)
        assert_same_bits(v.cpu().numpy(), ov, "v " + tag)
        if with_out:
            assert_same_bits(to_host(out), per_bucket_oracle(X, "mean", C, E, gt, gt), "grads " + tag)


def test_buckets_across_launch_splits():
    """Joint full buckets longer than one launch (2^29 elements): P = 2,
    bf16, 5 buckets of 2^27 + 2^20 elements and a tail; the chunk numbering
    carries across the split.  Checked on sampled elements against the
    oracle's per-element ring of each bucket."""
    P, C = 2, 4
    E = (1 << 27) + (1 << 20)
    n = 5 * E + 12345
    ins = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    for r in range(P):
        for lo in range(0, n, 1 << 26):
            workloads.torch_normal_(ins[r][lo:min(n, lo + (1 << 26))], 1.0, seed=50 + 10 * r + lo // (1 << 26))
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([rng.integers(0, n, 20000)] +
                                   [np.arange(max(0, k * E - 8), min(n, k * E + 8)) for k in range(1, 6)] +
                                   [np.arange(k * E + j * (E // C) - 4, k * E + j * (E // C) + 4)
                                    for k in range(5) for j in range(1, C)])).astype(np.int64)
    it = torch.from_numpy(idx).to(DEV)
    V = np.stack([t[it].view(torch.int16).cpu().numpy().view(np.uint16) for t in ins])
    ddp.allreduce(ins, "mean", C, out=ins, bucket_elems=E)
    torch.cuda.synchronize()
    got = np.stack([t[it].view(torch.int16).cpu().numpy().view(np.uint16) for t in ins])
    start = np.empty(idx.size, dtype=np.int64)
    for k in range(-(-n // E)):
        sel = (idx >= k * E) & (idx < (k + 1) * E)
        start[sel] = oracle.chunk_start_ranks_at(min(E, n - k * E), C, P, idx[sel] - k * E)
    want = oracle.ring_allreduce_sampled(V, start, "mean", in_dtype="bf16", out_dtype="bf16")
    assert_same_bits(got, want, "sampled")


@pytest.mark.parametrize("case", CASES[:5])
@pytest.mark.parametrize("gt,pt", [("bf16", "bf16"), ("f32", "f32")])
def test_zero1_buckets_equal_oracle(case, gt, pt):
    """zero1_sgd_step_buckets: every bucket's ZeRO stage 1 step as the
    oracle's phase-by-phase simulation of that bucket alone."""
    P, C, E, n = case
    X = draw(P, n, gt, seed=3 * P + C + n)
    w0 = workloads.rank_buffers(1, n, "normal", 0.02, seed=10)[0]
    v0 = workloads.rank_buffers(1, n, "normal", 1e-3, seed=11)[0]
    g = to_device(X, gt)
    w = torch.from_numpy(w0.copy()).to(DEV)
    v = torch.from_numpy(v0.copy()).to(DEV)
    params = [torch.empty(n, dtype=torch_dtype(pt), device=DEV) for _ in range(P)]
    ddp.zero1_sgd_step(g, w, v, 1e-3, 0.9, params, "mean", C, bucket_elems=E)
    torch.cuda.synchronize()
    got_p, got_w, got_v = to_host(params), w.cpu().numpy(), v.cpu().numpy()
    for lo in range(0, n, E):
        hi = min(n, lo + E)
        want_p, want_w, want_v, _ = oracle.zero1_sgd_step(X[:, lo:hi], w0[lo:hi], v0[lo:hi], 1e-3, 0.9, "mean",
                                                          C, gt, pt)
        what = f"{gt}->{pt} P={P} C={C} E={E} n={n} bucket at {lo}"
        assert_same_bits(got_w[None, lo:hi], want_w[None], what + " w")
        assert_same_bits(got_v[None, lo:hi], want_v[None], what + " v")
        assert_same_bits(got_p[:, lo:hi], want_p, what + " params")


def test_tree_over_the_flat_buffer_equals_per_bucket_calls():
    """The tree's order of additions is the same for every element, so one
    tree all-reduce over the flat buffer gives every bucket's own tree
    all-reduce, bit for bit (no bucketed variant is needed)."""
    P, E, n = 8, 16384, 3 * 16384 + 5001
    X = draw(P, n, "f32", seed=12)
    flat = ddp.allreduce_tree(to_device(X, "f32"), "mean", 2)
    ins = to_device(X, "f32")
    per = [torch.empty(n, device=DEV) for _ in range(P)]
    for lo in range(0, n, E):
        hi = min(n, lo + E)
        ddp.allreduce_tree([t[lo:hi] for t in ins], "mean", 2, out=[t[lo:hi] for t in per])
    torch.cuda.synchronize()
    assert_same_bits(to_host(flat), to_host(per), "flat tree vs per-bucket trees")
    want, _ = oracle.tree_allreduce(X, "mean", 2)
    assert_same_bits(to_host(flat), want, "flat tree vs oracle")
