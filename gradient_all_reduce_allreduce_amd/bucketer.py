"""Gradient bucketer: ragged per-parameter gradients <-> fixed-size buckets.

DDP packs gradients into buckets (25 MB by default), filled in the reverse
order of the parameters, and every rank reduces the buckets in the same
order ("Distributed Training", "Data parallelism and all-reduce").  The plan
comes from the library's ``ddp_bucket_plan``; pack and unpack run as HIP
kernels for all P ranks per launch.  The library checks each bucket's
segments and the tensors' addresses on the host before launching; this
class only holds the plan and the tensor address tables it passes.
"""

import math

import numpy as np

from . import api


class GradBucketer:
    def __init__(self, shapes, dtype, bucket_bytes=25 << 20, device="cuda"):
        import torch
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.numels = [int(math.prod(s)) for s in self.shapes]
        self.dtype = dtype
        self.code = api.torch_dtype_code(dtype)
        self.elem_bytes = torch.empty(0, dtype=dtype).element_size()
        self.bucket_bytes = int(bucket_bytes)
        self.bucket_elems = self.bucket_bytes // self.elem_bytes
        segs, nb, total, fp = api.ddp_bucket_plan(self.numels, self.code, self.bucket_bytes)
        self.segments = segs
        self.n_buckets = nb
        self.total = total
        self.fingerprint = fp
        self.bucket_lengths = [min(self.bucket_elems, total - b * self.bucket_elems)
                               for b in range(nb)]
        first = np.searchsorted(segs["bucket"], np.arange(nb + 1), side="left")
        self._seg_first = [int(x) for x in first]
        self._numels = np.ascontiguousarray(self.numels, dtype=np.int64)
        self.device = torch.device(device)

    def bucket_len(self, b):
        return self.bucket_lengths[b]

    def segment_range(self, b):
        """(first segment index, count) of bucket b in the segment table."""
        return self._seg_first[b], self._seg_first[b + 1] - self._seg_first[b]

    def check_rank_tensors(self, rank_tensors):
        """Every rank must hold tensors of exactly the planned shapes (the
        emulated "same order on every rank" rule)."""
        for r, ts in enumerate(rank_tensors):
            if len(ts) != len(self.shapes):
                raise ValueError(f"rank {r}: {len(ts)} tensors, plan has {len(self.shapes)}")
            for t, (x, s) in enumerate(zip(ts, self.shapes)):
                if tuple(x.shape) != s or x.dtype != self.dtype or not x.is_contiguous() \
                        or x.device != self.device:
                    raise ValueError(f"rank {r} tensor {t} does not match the plan")

    def pointer_table(self, rank_tensors):
        """Host table [P * T] of the tensors' device addresses, rank-major,
        checked against the plan once.  The table keeps the tensors alive;
        pack and unpack always copy to and from these same tensors."""
        self.check_rank_tensors(rank_tensors)
        return TensorTable(rank_tensors, self.device)

    # Extra distance between consecutive rank rows of an arena, in bytes.
    ROW_STAGGER = 4096

    def alloc_arena(self, P, dtype=None):
        """A [P, n_buckets * E] view holding every rank's gradients in bucket
        order (DDP's "gradients as bucket views" layout: no pack or unpack
        copies).  Each rank's row is padded to whole buckets, rounded up to
        a multiple of 4 KiB, plus 4 KiB, so with buckets of a whole number of
        KiB rank r's copy of bucket k starts at r * (n_buckets * bucket_bytes
        + 4096) + k * bucket_bytes.  Every row starts 4 KiB-aligned, so the
        all-reduce's 1 KiB wave accesses never split a 128-byte line, and
        the 4 KiB stagger keeps the P copies the all-reduce reads at the
        same offset from lining up in memory (measured about 1% faster than
        rows exactly a whole number of buckets apart, and about 19% faster
        than rows that are not 128-byte aligned).  Each row is contiguous;
        the [P, n_buckets * E] view as a whole is not (row stride n_buckets *
        E + 4096 bytes' worth of elements).  ``dtype``: the element type
        (default the plan's), e.g. float32 outputs of bf16 gradients."""
        import torch
        dtype = dtype or self.dtype
        cols = max(1, self.n_buckets) * self.bucket_elems
        es = torch.empty(0, dtype=dtype).element_size()
        line = self.ROW_STAGGER // es
        stride = -(-cols // line) * line + line
        return torch.empty(P, stride, dtype=dtype, device=self.device)[:, :cols]

    def alloc_state(self, count=2):
        """``count`` float32 buffers of ``total`` elements in bucket order,
        e.g. the master weights and momentum of the fused optimizer step
        (bucket b's state is ``x[b * bucket_elems:][:bucket_len(b)]``).  They
        share one allocation laid out like ``alloc_arena`` rows, so each
        starts 4 KiB-aligned.  The fused step's tiles start at the
        gradients' 128-byte lines; a state buffer that starts inside a line
        leaves two partly written lines at every wave store.  Carving both
        from one flat buffer of 2 * total floats does that whenever total is
        not a multiple of 32: with the ViT-B/16 set (P = 8, bf16 gradients,
        no gradient output) momentum 32 bytes into a line ran 7.6% slower
        one call per bucket and 11% slower as one bucketed call, 64 bytes
        into a line 3.5% and 7.4%."""
        import torch
        rows = self.alloc_arena(count, torch.float32)
        return [rows[i, :self.total] for i in range(count)]

    def bucket_view(self, arena_row, b):
        """Bucket b of one rank's arena row (its live elements only)."""
        lo = b * self.bucket_elems
        return arena_row[lo:lo + self.bucket_len(b)]

    def tensor_views(self, arena_row):
        """The rank's per-parameter gradient tensors as views of its arena
        row (parameter order, planned shapes)."""
        views = [None] * len(self.shapes)
        offs = {}
        flat = 0
        for t in reversed(range(len(self.shapes))):
            offs[t] = flat
            flat += self.numels[t]
        for t, s in enumerate(self.shapes):
            views[t] = arena_row[offs[t]:offs[t] + self.numels[t]].view(s)
        return views

    def alloc_buckets(self, P):
        """P bucket buffers of full bucket capacity."""
        import torch
        return [torch.empty(self.bucket_elems, dtype=self.dtype, device=self.device)
                for _ in range(P)]

    def _check_copy(self, table, b, rank_buckets):
        """The table must be this plan's, for as many ranks as buckets given;
        every bucket buffer a contiguous tensor of at least bucket_len(b)
        elements.  (The library checks the segments and addresses.)"""
        if not 0 <= b < self.n_buckets:
            raise ValueError(f"bucket {b} outside 0..{self.n_buckets - 1}")
        P = len(rank_buckets)
        if not isinstance(table, TensorTable) or table.P != P or table.T != len(self.shapes) \
                or table.device != self.device:
            raise ValueError("pointer table must come from pointer_table() for these P ranks")
        for r, x in enumerate(rank_buckets):
            if x.dtype != self.dtype or x.device != self.device or not x.is_contiguous() \
                    or x.numel() < self.bucket_len(b):
                raise ValueError(f"rank {r}: bucket buffer must be a contiguous {self.dtype} tensor "
                                 f"of at least {self.bucket_len(b)} elements on {self.device}")

    def _copy(self, fn, table, b, rank_buckets):
        self._check_copy(table, b, rank_buckets)
        first, count = self.segment_range(b)
        fn(len(rank_buckets), self.code, self.segments[first:first + count], count, self._numels,
           len(self.shapes), table.ptrs, [x.data_ptr() for x in rank_buckets], self.bucket_len(b),
           api.current_stream(self.device))

    def pack(self, table, b, rank_buckets):
        """Gather bucket b of every rank (tensors of ``pointer_table``) into
        ``rank_buckets`` on the current stream."""
        self._copy(api.ddp_bucket_pack, table, b, rank_buckets)

    def unpack(self, table, b, rank_buckets):
        """Scatter bucket b of every rank back into its tensors."""
        self._copy(api.ddp_bucket_unpack, table, b, rank_buckets)


class TensorTable:
    """The device addresses of P ranks' T tensors as one host array
    (rank-major), with the tensors it points to kept alive."""

    def __init__(self, rank_tensors, device):
        import ctypes
        self.P = len(rank_tensors)
        self.T = len(rank_tensors[0]) if rank_tensors else 0
        self.device = device
        self.tensors = [list(ts) for ts in rank_tensors]
        self.ptrs = (ctypes.c_void_p * (self.P * self.T))(*[x.data_ptr() for ts in rank_tensors for x in ts])
