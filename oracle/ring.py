"""Chunked ring all-reduce, simulated step by step on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests,
``smoke()`` and the CPU-baseline leg of the benchmark, never by the product.

What the pages fix
------------------
* An all-reduce takes one equal-size tensor from every rank and gives every
  rank the elementwise reduction ("Distributed Training", section "Data
  parallelism and all-reduce"; CS336 Lecture 8, "Collective Operations").
* The reduction is Sum or Mean; with Mean every replica receives the average
  gradient (Burn distributed guide, reduction configuration section).
* The ring strategy: peers form a ring and pass slices of the tensor around
  it (Burn collective blog, "Methods", Ring); a ring all-reduce is a
  reduce-scatter followed by an all-gather, each moving (W-1)/W of the model
  per device ("Distributed Training", "Sharded data parallelism" on FSDP's
  communication volume, and the printed traffic of "How to Apply It").
* Float32 sums taken in a different order differ in the last digits
  ("Distributed Training", Pitfalls, "Reproducibility"), so the order of
  additions is part of the result and is fixed here.

Readings where the pages are silent (each listed in the design notes)
---------------------------------------------------------------------
* Ring direction: rank r sends to rank (r + 1) mod P.
* Chunks: chunk length L = ceil(n / C); chunk j covers
  [min(jL, n), min((j+1)L, n)) and starts its reduce-scatter at rank
  j mod P.  With C = P this is the textbook ring; C = kP pipelines k rounds.
* Partial sums travel in the accumulation type (fp32 for fp32 and bf16
  inputs, fp64 for fp64 inputs); bf16 inputs are widened exactly first.
* Mean divides once, by P, at the chunk's owner after the full sum, with a
  correctly rounded IEEE division in the accumulation type.
* Output conversion to bf16 rounds to nearest even (``oracle.bf16``).

Parity status: the association order itself is a reading (no page shows
the step schedule); it is pinned by the tests against an independently
derived closed-form fold, hand-worked examples, exact integer sums, the
recursive-summation error bound and the pages' printed traffic figures.
"""

import numpy as np

from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits

SUM = "sum"
MEAN = "mean"


def chunk_length(n, chunking):
    """Length L = ceil(n / C) of every chunk but possibly the trailing ones."""
    if chunking < 1:
        raise ValueError("chunking must be >= 1")
    return -(-n // chunking) if n > 0 else 0


def chunk_start_ranks(n, chunking, P):
    """Start rank of the reduce-scatter for every element (int64 array).

    Element i lies in chunk floor(i / L); that chunk starts at rank
    (chunk mod P).  Reading of the Ring strategy in the Burn collective blog,
    "Methods".
    """
    return chunk_start_ranks_at(n, chunking, P, np.arange(n, dtype=np.int64))


def chunk_start_ranks_at(n, chunking, P, idx):
    """Start ranks of the elements with the given indices of an n-element
    buffer (the same rule as ``chunk_start_ranks``, without materialising
    all n of them)."""
    L = chunk_length(n, chunking)
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size == 0:
        return np.zeros(0, dtype=np.int64)
    return (idx // L) % P


def _widen(X, in_dtype):
    """Rank inputs -> (P, n) array in the accumulation type."""
    if in_dtype == "f32":
        return np.array(X, dtype=np.float32, copy=True)
    if in_dtype == "f64":
        return np.array(X, dtype=np.float64, copy=True)
    if in_dtype == "bf16":
        return bf16_bits_to_f32(np.asarray(X, dtype=np.uint16)).copy()
    raise ValueError(f"unknown input dtype {in_dtype!r}")


def _narrow(A, out_dtype):
    if out_dtype in ("f32", "f64"):
        return A.astype(np.float32 if out_dtype == "f32" else np.float64)
    if out_dtype == "bf16":
        return f32_to_bf16_bits(A.astype(np.float32))
    raise ValueError(f"unknown output dtype {out_dtype!r}")


def _chunks(n, P, C):
    L = chunk_length(n, C)
    chunks = [(min(j * L, n), min((j + 1) * L, n)) for j in range(C)]
    start = [j % P for j in range(C)]
    owner = [(s + P - 1) % P for s in start]
    return chunks, start, owner


def _reduce_scatter_steps(A, chunks, start, sent):
    """The P-1 reduce-scatter steps, in place on A (P, n).  Every send of a
    step reads the buffers as they stood at the start of the step (S), so
    the sends are simultaneous."""
    P = A.shape[0]
    for t in range(P - 1):
        S = A.copy()
        for r in range(P):
            dst = (r + 1) % P
            for j, (lo, hi) in enumerate(chunks):
                if start[j] == (r - t) % P:
                    A[dst, lo:hi] = S[r, lo:hi] + A[dst, lo:hi]
                    sent[r] += hi - lo


def _all_gather_steps(A, chunks, owner, sent):
    """The P-1 all-gather steps: the owner's finished chunk is forwarded
    around the ring."""
    P = A.shape[0]
    for t in range(P - 1):
        S = A.copy()
        for r in range(P):
            dst = (r + 1) % P
            for j, (lo, hi) in enumerate(chunks):
                if owner[j] == (r - t) % P:
                    A[dst, lo:hi] = S[r, lo:hi]
                    sent[r] += hi - lo


def _check(A, op):
    if A.ndim != 2:
        raise ValueError("X must have shape (P, n)")
    if A.shape[0] < 1:
        raise ValueError("P must be >= 1")
    if op not in (SUM, MEAN):
        raise ValueError(f"unknown op {op!r}")


def ring_allreduce(X, op=SUM, chunking=None, in_dtype="f32", out_dtype=None):
    """All-reduce P rank buffers by simulating the ring one step at a time.

    X: array-like of shape (P, n) -- rank r's buffer is X[r].  For
    ``in_dtype="bf16"`` the entries are raw bfloat16 bit patterns (uint16).
    op: ``"sum"`` or ``"mean"``.  chunking: C >= 1 (default P).
    Returns (Y, sent): Y of shape (P, n) in ``out_dtype`` (default: the input
    dtype) holding every rank's result, and ``sent[r]`` = number of elements
    rank r put on the wire over the whole all-reduce.
    """
    A = _widen(X, in_dtype)
    _check(A, op)
    P, n = A.shape
    C = P if chunking is None else int(chunking)
    chunks, start, owner = _chunks(n, P, C)
    sent = np.zeros(P, dtype=np.int64)

    _reduce_scatter_steps(A, chunks, start, sent)

    # Mean: the owner of each chunk now holds the full sum; divide once.
    if op == MEAN:
        div = A.dtype.type(P)
        for j, (lo, hi) in enumerate(chunks):
            A[owner[j], lo:hi] = A[owner[j], lo:hi] / div

    _all_gather_steps(A, chunks, owner, sent)
    return _narrow(A, out_dtype or in_dtype), sent


def chunk_owners(n, chunking, P):
    """Owner rank of every element: the rank where the chunk's reduce-scatter
    ends, (start + P - 1) mod P."""
    return (chunk_start_ranks(n, chunking, P) + P - 1) % P


def ring_reduce_scatter(X, op=SUM, chunking=None, in_dtype="f32", out_dtype=None):
    """The first half of the ring on its own: P-1 reduce-scatter steps, then
    Mean at each chunk's owner.  ("Distributed Training", "Sharded data
    parallelism": FSDP reduce-scatters the gradients so that each rank ends
    holding its shard; CS336 Lecture 8, "Collective Operations": each rank
    receives a unique chunk of the reduced tensor.)

    Returns (Y, owner, sent): Y (P, n) in ``out_dtype`` is every rank's
    buffer after the steps -- only Y[owner[i], i] is the finished reduction
    of element i, the other entries are partial sums of the ring --, owner
    (n,) the owning rank of each element, sent[r] the elements rank r sent.
    """
    A = _widen(X, in_dtype)
    _check(A, op)
    P, n = A.shape
    C = P if chunking is None else int(chunking)
    chunks, start, owner = _chunks(n, P, C)
    sent = np.zeros(P, dtype=np.int64)
    _reduce_scatter_steps(A, chunks, start, sent)
    if op == MEAN:
        div = A.dtype.type(P)
        for j, (lo, hi) in enumerate(chunks):
            A[owner[j], lo:hi] = A[owner[j], lo:hi] / div
    return _narrow(A, out_dtype or in_dtype), chunk_owners(n, C, P), sent


def ring_all_gather(B, chunking=None):
    """The second half of the ring on its own: P-1 steps forwarding each
    chunk from its owner, so every rank ends with the owner's values.
    (CS336 Lecture 8, "Collective Operations": all-gather gives every rank
    the complete tensor.)  B: (P, n) array of any dtype; only
    B[owner[i], i] matters.  Returns (Y, sent)."""
    A = np.array(B, copy=True)
    if A.ndim != 2 or A.shape[0] < 1:
        raise ValueError("B must have shape (P, n)")
    P, n = A.shape
    C = P if chunking is None else int(chunking)
    chunks, _, owner = _chunks(n, P, C)
    sent = np.zeros(P, dtype=np.int64)
    _all_gather_steps(A, chunks, owner, sent)
    return A, sent


def ring_allreduce_sampled(V, start, op=SUM, in_dtype="f32", out_dtype=None):
    """The same ring, for elements taken out of a larger buffer.

    V: shape (P, m) -- the P rank values of m sampled elements.
    start: shape (m,) -- each element's reduce-scatter start rank (from
    ``chunk_start_ranks`` of the full buffer, evaluated at the sampled
    indices).  Elements do not interact in an all-reduce, so simulating the
    ring on the sample gives exactly the values the full-buffer ring gives at
    those indices.  Returns Y of shape (P, m).
    """
    A = _widen(V, in_dtype)
    P, m = A.shape
    start = np.asarray(start, dtype=np.int64)
    if start.shape != (m,):
        raise ValueError("start must have one entry per sampled element")
    cols = np.arange(m)
    for t in range(P - 1):
        S = A.copy()
        src = (start + t) % P
        dst = (src + 1) % P
        A[dst, cols] = S[src, cols] + A[dst, cols]
    owner = (start + P - 1) % P
    if op == MEAN:
        A[owner, cols] = A[owner, cols] / A.dtype.type(P)
    for t in range(P - 1):
        S = A.copy()
        src = (owner + t) % P
        dst = (src + 1) % P
        A[dst, cols] = S[src, cols]
    return _narrow(A, out_dtype or in_dtype)
