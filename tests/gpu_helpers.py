"""Shared helpers of the GPU parity tests: moving seeded inputs to the
device, calling the library through the binding, reading results back, and
the oracle calls the results are compared with."""

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")


def to_device(X, dtype):
    """(P, n) numpy array -> list of P contiguous device tensors.  For bf16
    the numpy array holds raw bit patterns (uint16)."""
    out = []
    for r in range(X.shape[0]):
        if dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(X[r]).view(np.int16)).to(DEV)
            out.append(t.view(torch.bfloat16))
        else:
            out.append(torch.from_numpy(np.ascontiguousarray(X[r], dtype=np.float32)).to(DEV))
    return out


def to_host(ts):
    """List of device tensors -> (P, n) numpy (float32, or uint16 bits)."""
    rows = []
    for t in ts:
        if t.dtype == torch.bfloat16:
            rows.append(t.view(torch.int16).cpu().numpy().view(np.uint16))
        else:
            rows.append(t.cpu().numpy())
    return np.stack(rows) if rows else np.zeros((0, 0), np.float32)


def torch_dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def oracle_ring(X, op, C, in_dtype="f32", out_dtype=None):
    """The oracle's ring; for many chunks the per-element form of the same
    stepwise simulation (identical results, see the oracle's own tests)."""
    P, n = X.shape
    if C <= 64:
        Y, _ = oracle.ring_allreduce(X, op, C, in_dtype=in_dtype, out_dtype=out_dtype)
        return Y
    start = oracle.chunk_start_ranks(n, C, P)
    return oracle.ring_allreduce_sampled(X, start, op, in_dtype=in_dtype, out_dtype=out_dtype)


def assert_same_bits(got, want, what=""):
    """Bitwise equality; two NaNs of any payload count as equal."""
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.uint16:
        gb, wb = got, want
        g_nan = (gb & 0x7FFF) > 0x7F80
        w_nan = (wb & 0x7FFF) > 0x7F80
    else:
        gb, wb = got.view(np.uint32), want.view(np.uint32)
        g_nan, w_nan = np.isnan(got), np.isnan(want)
    assert np.array_equal(g_nan, w_nan), what
    bad = np.flatnonzero((gb != wb) & ~g_nan)
    assert bad.size == 0, f"{what}: {bad.size} elements differ, first at {bad[:5]}"
