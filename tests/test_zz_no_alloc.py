"""GPU check of the allocation-free multi-tensor all-reduce
(allreduce_multi_ring_noalloc, for callers that cannot allocate device
memory): through the C ABI its outputs equal, bit for bit, those of the
multi-tensor call that takes device tables (allreduce_multi_ring_emulated)
on the same tensors, on two calls in a row, the second with fewer and
smaller tensors (the scratch area keeps the first call's tables, and the
second must not read them), and both equal the oracle's ring per tensor."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import DEV, assert_same_bits, oracle_ring

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")
from gradient_all_reduce_allreduce_amd import _native as N  # noqa: E402


def bits_of(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    return t.cpu().numpy().reshape(-1)


def make(P, numels, dtype, seed, offset=0):
    """P ranks' tensors as views at `offset` elements into their own buffers."""
    rng = np.random.default_rng(seed)
    host, dev = [], []
    for r in range(P):
        hs, ds = [], []
        for n in numels:
            x = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 21, n))).astype(np.float32)
            if dtype == torch.bfloat16:
                x = workloads.to_bf16_bits(x)
                src = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
            else:
                src = torch.from_numpy(x).to(DEV)
            store = torch.empty(n + offset, dtype=dtype, device=DEV)
            t = store[offset:offset + n]
            t.copy_(src)
            hs.append(x)
            ds.append(t)
        host.append(hs)
        dev.append(ds)
    return host, dev


def with_device_tables(op, P, C, numels, ins, in_code, outs, out_code):
    """The existing entry point, its plan and tables built and uploaded by
    the caller (rank 0's input lines, as the allocation-free call plans)."""
    T = len(numels)
    tiles, total, tile = ddp.ddp_multi_plan(numels, P, in_code, out_code,
                                            align_to=[ins[0][t].data_ptr() for t in range(T)])
    tiles_dev = torch.from_numpy(tiles.view(np.uint8).copy()).to(DEV)
    bmap_dev = torch.from_numpy(ddp.ddp_multi_block_map(tiles, total).copy()).to(DEV)
    pin = torch.tensor([x.data_ptr() for row in ins for x in row], dtype=torch.int64).to(DEV)
    pout = torch.tensor([x.data_ptr() for row in outs for x in row], dtype=torch.int64).to(DEV)
    st = N.lib().allreduce_multi_ring_emulated(
        op, P, C, T, tiles_dev.data_ptr(), total, tile, bmap_dev.data_ptr(), pin.data_ptr(),
        in_code, pout.data_ptr(), out_code, ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert st == N.DDP_OK, N.last_error()
    torch.cuda.synchronize()
    return (tiles_dev, bmap_dev, pin, pout)


def no_alloc(op, P, C, numels, ins, in_code, outs, out_code):
    """The allocation-free entry point, called through the C ABI."""
    T = len(numels)
    arr = (ctypes.c_int64 * T)(*numels)
    st = N.lib().allreduce_multi_ring_noalloc(
        op, P, C, T, arr, N.pointer_array([x.data_ptr() for row in ins for x in row]), in_code,
        N.pointer_array([x.data_ptr() for row in outs for x in row]), out_code,
        ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert st == N.DDP_OK, N.last_error()


CASES = [
    # (P, C, in, out, op, first numels, second numels, view offset)
    (8, 8, "f32", "f32", N.DDP_MEAN,
     [1, 7, 64, 1000, 4097, 70001, 0, 262144 + 33], [5, 4097, 129], 0),
    (4, 9, "bf16", "f32", N.DDP_SUM,
     [3, 4096, 33 * 129, 100003, 17], [100, 2], 1),
    (3, 3, "bf16", "bf16", N.DDP_MEAN,
     [70001, 1, 2, 65536], [65535], 8),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_no_alloc_equals_device_table_call_twice(case):
    P, C, it, ot, op, first, second, offset = CASES[case]
    tin = torch.bfloat16 if it == "bf16" else torch.float32
    tout = torch.bfloat16 if ot == "bf16" else torch.float32
    cin = N.DDP_BF16 if it == "bf16" else N.DDP_F32
    cout = N.DDP_BF16 if ot == "bf16" else N.DDP_F32
    opname = "mean" if op == N.DDP_MEAN else "sum"
    for call, numels in enumerate((first, second)):
        print(f"no-alloc case {case} call {call}: P={P} C={C} {it}->{ot} T={len(numels)}", flush=True)
        host, ins = make(P, numels, tin, seed=100 * case + call, offset=offset)
        want = [[torch.full((n,), 7.0, dtype=tout, device=DEV) for n in numels] for _ in range(P)]
        got = [[torch.full((n,), -3.0, dtype=tout, device=DEV) for n in numels] for _ in range(P)]
        keep = with_device_tables(op, P, C, numels, ins, cin, want, cout)
        no_alloc(op, P, C, numels, ins, cin, got, cout)
        torch.cuda.synchronize()
        del keep
        for t, n in enumerate(numels):
            g = np.stack([bits_of(got[r][t]) for r in range(P)])
            w = np.stack([bits_of(want[r][t]) for r in range(P)])
            assert_same_bits(g, w, f"case {case} call {call} tensor {t}")
            if n == 0:
                continue
            X = np.stack([host[r][t] for r in range(P)])
            assert_same_bits(g, oracle_ring(X, opname, C, in_dtype=it, out_dtype=ot),
                             f"oracle case {case} call {call} tensor {t}")


def test_no_alloc_repeated_tables():
    """The same tensors again right after (the call finds its tables already
    in the scratch area and skips the copy), then other tensors, then the
    first ones again: every call equals the oracle."""
    P, C = 8, 8
    sets = [[4097, 9, 70001, 1], [33, 129 * 7]]
    data = [make(P, n, torch.float32, seed=40 + k) for k, n in enumerate(sets)]
    # One output list per set, reused, so that a repeat has the same tables.
    out_sets = [[[torch.empty((n,), device=DEV) for n in numels] for _ in range(P)] for numels in sets]
    for k in (0, 0, 1, 0, 1, 1):
        numels = sets[k]
        host, ins = data[k]
        outs = out_sets[k]
        print(f"no-alloc repeated: set {k}", flush=True)
        for row in outs:
            for x in row:
                x.fill_(-3.0)
        no_alloc(N.DDP_MEAN, P, C, numels, ins, N.DDP_F32, outs, N.DDP_F32)
        torch.cuda.synchronize()
        for t in range(len(numels)):
            X = np.stack([host[r][t] for r in range(P)])
            g = np.stack([bits_of(outs[r][t]) for r in range(P)])
            assert_same_bits(g, oracle_ring(X, "mean", C), f"set {k} tensor {t}")


def _want(host, numels, P, C):
    return [oracle_ring(np.stack([host[r][t] for r in range(P)]), "mean", C) for t in range(len(numels))]


def _check(outs, want, what):
    for t, w in enumerate(want):
        g = np.stack([bits_of(outs[r][t]) for r in range(len(outs))])
        assert_same_bits(g, w, f"{what} tensor {t}")


def test_no_alloc_alternating_outputs():
    """The same inputs into two output sets in turn, with enough tensors for
    several fill launches: only the output pointer table changes between
    calls, and only the launches' runs that changed are written again.
    Every call equals the oracle."""
    P, C = 8, 8
    rng = np.random.default_rng(7)
    numels = [int(x) for x in rng.integers(1, 3000, 300)]   # tables of 300 tensors: 43,520 bytes, 6 fill runs
    host, ins = make(P, numels, torch.float32, seed=71)
    want = _want(host, numels, P, C)
    outs = [[[torch.empty((n,), device=DEV) for n in numels] for _ in range(P)] for _ in range(2)]
    for k in (0, 1, 0, 1, 1, 0):
        print(f"no-alloc alternating outputs: set {k}", flush=True)
        for row in outs[k]:
            for x in row:
                x.fill_(-3.0)
        no_alloc(N.DDP_MEAN, P, C, numels, ins, N.DDP_F32, outs[k], N.DDP_F32)
        torch.cuda.synchronize()
        _check(outs[k], want, f"output set {k}")


def test_no_alloc_graph_replays():
    """Captured in a HIP graph, the call's table writes are captured with its
    launch, so every replay rewrites the scratch area first: replays between
    eager calls on other tensors (which rewrite the area, and which must not
    skip their writes once a replay may have run) each give the oracle's
    result, and so does every eager call."""
    P, C = 8, 8
    na, nb = [4097, 9, 70001, 1], [33, 129 * 7, 5]
    host_a, ins_a = make(P, na, torch.float32, seed=61)
    host_b, ins_b = make(P, nb, torch.float32, seed=62)
    out_a = [[torch.empty((n,), device=DEV) for n in na] for _ in range(P)]
    out_b = [[torch.empty((n,), device=DEV) for n in nb] for _ in range(P)]
    want_a, want_b = _want(host_a, na, P, C), _want(host_b, nb, P, C)
    print("no-alloc graph: eager call before capture", flush=True)
    no_alloc(N.DDP_MEAN, P, C, na, ins_a, N.DDP_F32, out_a, N.DDP_F32)
    torch.cuda.synchronize()
    _check(out_a, want_a, "eager a")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        no_alloc(N.DDP_MEAN, P, C, na, ins_a, N.DDP_F32, out_a, N.DDP_F32)
    torch.cuda.synchronize()
    for rep in range(4):
        print(f"no-alloc graph: replay {rep}", flush=True)
        for row in out_a + out_b:
            for x in row:
                x.fill_(-3.0)
        no_alloc(N.DDP_MEAN, P, C, nb, ins_b, N.DDP_F32, out_b, N.DDP_F32)
        torch.cuda.synchronize()
        _check(out_b, want_b, f"eager b before replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        _check(out_a, want_a, f"replay {rep}")
        for row in out_b:
            for x in row:
                x.fill_(-3.0)
        no_alloc(N.DDP_MEAN, P, C, nb, ins_b, N.DDP_F32, out_b, N.DDP_F32)
        torch.cuda.synchronize()
        _check(out_b, want_b, f"eager b after replay {rep}")


def test_no_alloc_in_place():
    """Output = input (in place) on the allocation-free call."""
    P, C, numels = 4, 4, [4097, 9, 70001]
    host, ins = make(P, numels, torch.float32, seed=5)
    print("no-alloc in place: P=4 C=4 f32", flush=True)
    no_alloc(N.DDP_SUM, P, C, numels, ins, N.DDP_F32, ins, N.DDP_F32)
    torch.cuda.synchronize()
    for t in range(len(numels)):
        X = np.stack([host[r][t] for r in range(P)])
        g = np.stack([bits_of(ins[r][t]) for r in range(P)])
        assert_same_bits(g, oracle_ring(X, "sum", C), f"in place tensor {t}")
