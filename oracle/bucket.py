"""Gradient bucketing: reverse parameter order, fixed-size flat buckets.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages: DDP packs gradients into buckets (25 MB by default in the
PyTorch version they describe), fills them in the reverse order of the
model's parameters, and every rank must reduce the buckets in the same order
("Distributed Training", "Data parallelism and all-reduce"); FSDP flattens a
unit's parameters into one tensor ("Sharded data parallelism"); collectives
that move larger tensors per call use bandwidth better ("Communication
costs").

Readings: a bucket holds exactly bucket_bytes // element_size elements
except the last; tensors are laid end to end in reverse order and the flat
range is cut at bucket boundaries, so a tensor may straddle two or more
buckets; zero-size tensors contribute nothing.

Parity status: pinned by the tests (pack then unpack is the identity, every
element lands in exactly one slot, the bucket lengths add up to the total,
the ResNet-50 and ViT-B/16 totals including the pages' ViT-B/16 closed form).
"""

import numpy as np


def bucket_plan(numels, elem_bytes, bucket_bytes):
    """Plan the buckets for tensors of the given sizes (in parameter order).

    Returns (segments, bucket_lengths).  Each segment is a tuple
    (tensor, bucket, src_off, dst_off, length) in elements: elements
    [src_off, src_off + length) of tensor ``tensor`` (flattened in C order)
    occupy [dst_off, dst_off + length) of bucket ``bucket``.  Segments are
    listed in bucket order and, within a bucket, by increasing dst_off.
    """
    E = bucket_bytes // elem_bytes
    if E < 1:
        raise ValueError("bucket smaller than one element")
    segments = []
    flat = 0
    for t in reversed(range(len(numels))):
        remaining = int(numels[t])
        src = 0
        while remaining > 0:
            b, off = divmod(flat, E)
            take = min(remaining, E - off)
            segments.append((t, b, src, off, take))
            src += take
            flat += take
            remaining -= take
    total = flat
    n_buckets = -(-total // E)
    lengths = [min(E, total - b * E) for b in range(n_buckets)]
    return segments, lengths


def pack(tensors, elem_bytes, bucket_bytes):
    """Flatten the tensors (one rank's gradients, in parameter order) in
    reverse order, lay them end to end and cut the result into buckets."""
    E = bucket_bytes // elem_bytes
    flat = [np.asarray(t).reshape(-1) for t in reversed(list(tensors))]
    if not flat:
        return []
    whole = np.concatenate(flat)
    return [whole[i:i + E].copy() for i in range(0, whole.size, E)]


def unpack(buckets, shapes):
    """Inverse of ``pack``: rebuild tensors of the given shapes (parameter
    order) from the buckets."""
    if buckets:
        whole = np.concatenate([np.asarray(b).reshape(-1) for b in buckets])
    else:
        whole = np.zeros(0)
    out = [None] * len(shapes)
    pos = 0
    for t in reversed(range(len(shapes))):
        size = int(np.prod(shapes[t], dtype=np.int64))
        out[t] = whole[pos:pos + size].reshape(shapes[t]).copy()
        pos += size
    if pos != whole.size:
        raise ValueError("buckets do not match the tensor shapes")
    return out
