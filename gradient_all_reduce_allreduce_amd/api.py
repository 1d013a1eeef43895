"""Python binding of the C ABI: the same entry points, argument marshalling
only.  Every step of the all-reduce runs in the HIP library; PyTorch is used
here for device memory, pointers and the current stream.

Raw entry points (same names and argument order as the C header, pointers as
Python ints, stream as an int handle or None):
    ddp_bucket_plan, ddp_bucket_pack, ddp_bucket_unpack,
    allreduce_ring_emulated, allreduce_fused_sgd, allreduce_ring_buckets,
    allreduce_fused_sgd_buckets, zero1_sgd_step_emulated, zero1_sgd_step_buckets,
    ddp_buckets_launch_count,
    reducescatter_ring_emulated, reducescatter_ring_buckets,
    allgather_ring_emulated, allgather_ring_buckets, allreduce_ring_stepwise,
    allreduce_ring_stepwise_buckets, allreduce_tree_emulated, allreduce_hierarchical_buckets,
    allreduce_hierarchical_emulated, ddp_multi_plan, ddp_multi_block_map, allreduce_multi_ring_emulated,
    allreduce_multi_fused_sgd, allreduce_multi_ring_noalloc, ddp_set_wg_per_cu
Tensor-level helpers:
    allreduce(tensors, op, chunking, out)            -> list of outputs
    allreduce_sgd(grads, w, v, lr, mu, op, chunking, out)
    zero1_sgd_step(grads, w, v, lr, mu, params, op, chunking)
    reduce_scatter, all_gather, allreduce_stepwise, allreduce_tree,
    allreduce_hierarchical, MultiAllReduce
"""

import ctypes

import numpy as np

from . import _native as N

SUM = N.DDP_SUM
MEAN = N.DDP_MEAN
F32 = N.DDP_F32
BF16 = N.DDP_BF16
MAX_RANKS = N.DDP_MAX_RANKS


class DdpError(RuntimeError):
    """A non-OK status from the library; ``status`` holds the code."""

    def __init__(self, status, message):
        super().__init__(f"{N.STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _check(status):
    if status != N.DDP_OK:
        raise DdpError(status, N.last_error())


def _op(op):
    if op in (SUM, MEAN):
        return op
    return {"sum": SUM, "mean": MEAN}[op]


# ----------------------------------------------------------- raw entry ----

SEGMENT_DTYPE = np.dtype([("tensor", "<i4"), ("bucket", "<i4"), ("src_off", "<i8"),
                          ("dst_off", "<i8"), ("len", "<i8")])
assert SEGMENT_DTYPE.itemsize == ctypes.sizeof(N.Segment)


def ddp_bucket_plan(numels, dtype, bucket_bytes):
    """Plan buckets (host only).  Returns (segments, n_buckets, total_elems,
    fingerprint); segments is a numpy structured array in the C layout."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    T = int(numels.size)
    c_numels = numels.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    n_segs = ctypes.c_int64(0)
    n_buckets = ctypes.c_int32(0)
    total = ctypes.c_int64(0)
    fp = ctypes.c_uint64(0)
    lib = N.lib()
    _check(lib.ddp_bucket_plan(c_numels, T, dtype, bucket_bytes, None, 0, ctypes.byref(n_segs),
                               ctypes.byref(n_buckets), ctypes.byref(total), ctypes.byref(fp)))
    segs = np.zeros(n_segs.value, dtype=SEGMENT_DTYPE)
    _check(lib.ddp_bucket_plan(c_numels, T, dtype, bucket_bytes,
                               segs.ctypes.data_as(ctypes.POINTER(N.Segment)), segs.size,
                               ctypes.byref(n_segs), ctypes.byref(n_buckets),
                               ctypes.byref(total), ctypes.byref(fp)))
    return segs, n_buckets.value, total.value, fp.value


def _host_addr(x, dtype=None):
    """Address of a host array: a numpy array (converted to ``dtype`` if
    given), a ctypes object or an int address; None stays NULL."""
    if x is None or isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        if dtype is not None and x.dtype != dtype:
            raise TypeError(f"expected a {dtype} array, got {x.dtype}")
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("host arrays must be contiguous")
        return x.ctypes.data
    return ctypes.addressof(x)


def _ptr_array(ptrs):
    if isinstance(ptrs, ctypes.Array):
        return ptrs
    return N.pointer_array(ptrs)


def ddp_bucket_pack(P, dtype, segs, n_segs, numels, n_tensors, tensor_ptrs, rank_bucket, bucket_len,
                    stream=None):
    """segs: the bucket's segments (a SEGMENT_DTYPE numpy array or a host
    address); numels: int64 numpy array (or address); tensor_ptrs: P *
    n_tensors device addresses, rank-major (a list or a ctypes array)."""
    _check(N.lib().ddp_bucket_pack(P, dtype, _host_addr(segs, SEGMENT_DTYPE), n_segs,
                                   _host_addr(numels, np.int64), n_tensors, _ptr_array(tensor_ptrs),
                                   N.pointer_array(rank_bucket), bucket_len, stream))


def ddp_bucket_unpack(P, dtype, segs, n_segs, numels, n_tensors, tensor_ptrs, rank_bucket, bucket_len,
                      stream=None):
    _check(N.lib().ddp_bucket_unpack(P, dtype, _host_addr(segs, SEGMENT_DTYPE), n_segs,
                                     _host_addr(numels, np.int64), n_tensors, _ptr_array(tensor_ptrs),
                                     N.pointer_array(rank_bucket), bucket_len, stream))


def allreduce_ring_emulated(op, P, chunking, rank_in, in_dtype, rank_out, out_dtype, n,
                            stream=None):
    _check(N.lib().allreduce_ring_emulated(_op(op), P, chunking, N.pointer_array(rank_in),
                                           in_dtype, N.pointer_array(rank_out), out_dtype, n,
                                           stream))


def allreduce_fused_sgd(op, P, chunking, rank_grad, grad_dtype, n, master_w, momentum, lr, mu,
                        rank_grad_out, out_dtype, stream=None):
    out = N.pointer_array(rank_grad_out) if rank_grad_out is not None else None
    _check(N.lib().allreduce_fused_sgd(_op(op), P, chunking, N.pointer_array(rank_grad),
                                       grad_dtype, n, master_w, momentum, lr, mu, out,
                                       out_dtype, stream))


def allreduce_ring_buckets(op, P, chunking, rank_in, in_dtype, rank_out, out_dtype, n, bucket_elems,
                           stream=None):
    _check(N.lib().allreduce_ring_buckets(_op(op), P, chunking, N.pointer_array(rank_in), in_dtype,
                                          N.pointer_array(rank_out), out_dtype, n, bucket_elems, stream))


def allreduce_fused_sgd_buckets(op, P, chunking, rank_grad, grad_dtype, n, bucket_elems, master_w,
                                momentum, lr, mu, rank_grad_out, out_dtype, stream=None):
    out = N.pointer_array(rank_grad_out) if rank_grad_out is not None else None
    _check(N.lib().allreduce_fused_sgd_buckets(_op(op), P, chunking, N.pointer_array(rank_grad),
                                               grad_dtype, n, bucket_elems, master_w, momentum, lr, mu,
                                               out, out_dtype, stream))


def zero1_sgd_step_emulated(op, P, chunking, rank_grad, grad_dtype, n, master_w, momentum, lr, mu,
                            rank_param_out, param_dtype, stream=None):
    _check(N.lib().zero1_sgd_step_emulated(_op(op), P, chunking, N.pointer_array(rank_grad), grad_dtype,
                                           n, master_w, momentum, lr, mu,
                                           N.pointer_array(rank_param_out), param_dtype, stream))


def ddp_buckets_launch_count(P, chunking, in_dtype, out_dtype, sgd, n, bucket_elems):
    """Kernel launches one bucketed call makes for these arguments (host only)."""
    out = ctypes.c_int64(0)
    _check(N.lib().ddp_buckets_launch_count(P, chunking, in_dtype, out_dtype, 1 if sgd else 0, n,
                                            bucket_elems, ctypes.byref(out)))
    return out.value


def zero1_sgd_step_buckets(op, P, chunking, rank_grad, grad_dtype, n, bucket_elems, master_w, momentum,
                           lr, mu, rank_param_out, param_dtype, stream=None):
    _check(N.lib().zero1_sgd_step_buckets(_op(op), P, chunking, N.pointer_array(rank_grad), grad_dtype,
                                          n, bucket_elems, master_w, momentum, lr, mu,
                                          N.pointer_array(rank_param_out), param_dtype, stream))


def reducescatter_ring_emulated(op, P, chunking, rank_in, in_dtype, rank_out, out_dtype, n,
                                stream=None):
    _check(N.lib().reducescatter_ring_emulated(_op(op), P, chunking, N.pointer_array(rank_in),
                                               in_dtype, N.pointer_array(rank_out), out_dtype, n,
                                               stream))


def reducescatter_ring_buckets(op, P, chunking, rank_in, in_dtype, rank_out, out_dtype, n, bucket_elems,
                               stream=None):
    _check(N.lib().reducescatter_ring_buckets(_op(op), P, chunking, N.pointer_array(rank_in), in_dtype,
                                              N.pointer_array(rank_out), out_dtype, n, bucket_elems, stream))


def allgather_ring_buckets(P, chunking, rank_buf, dtype, n, bucket_elems, stream=None):
    _check(N.lib().allgather_ring_buckets(P, chunking, N.pointer_array(rank_buf), dtype, n, bucket_elems,
                                          stream))


def allreduce_ring_stepwise_buckets(op, P, chunking, rank_buf, dtype, n, bucket_elems, sent_dev=None,
                                    stream=None):
    _check(N.lib().allreduce_ring_stepwise_buckets(_op(op), P, chunking, N.pointer_array(rank_buf), dtype, n,
                                                   bucket_elems, sent_dev, stream))


def allgather_ring_emulated(P, chunking, rank_buf, dtype, n, stream=None):
    _check(N.lib().allgather_ring_emulated(P, chunking, N.pointer_array(rank_buf), dtype, n,
                                           stream))


def allreduce_ring_stepwise(op, P, chunking, rank_buf, dtype, n, sent_dev=None, stream=None):
    _check(N.lib().allreduce_ring_stepwise(_op(op), P, chunking, N.pointer_array(rank_buf),
                                           dtype, n, sent_dev, stream))


def allreduce_tree_emulated(op, P, branching, rank_in, in_dtype, rank_out, out_dtype, n,
                            stream=None):
    _check(N.lib().allreduce_tree_emulated(_op(op), P, branching, N.pointer_array(rank_in),
                                           in_dtype, N.pointer_array(rank_out), out_dtype, n,
                                           stream))


STRATEGY_RING = 0
STRATEGY_TREE = 1
STRATEGY_CENTRALIZED = 2
_STRATEGIES = {"ring": STRATEGY_RING, "tree": STRATEGY_TREE, "centralized": STRATEGY_CENTRALIZED}


def _strategy(st):
    return st if isinstance(st, int) else _STRATEGIES[st]


def allreduce_hierarchical_emulated(op, nodes, local_ranks, local_strategy, local_param,
                                    global_strategy, global_param, rank_in, in_dtype, rank_out,
                                    out_dtype, n, stream=None):
    _check(N.lib().allreduce_hierarchical_emulated(
        _op(op), nodes, local_ranks, _strategy(local_strategy), local_param or 0,
        _strategy(global_strategy), global_param or 0, N.pointer_array(rank_in), in_dtype,
        N.pointer_array(rank_out), out_dtype, n, stream))


def allreduce_hierarchical_buckets(op, nodes, local_ranks, local_strategy, local_param,
                                   global_strategy, global_param, rank_in, in_dtype, rank_out,
                                   out_dtype, n, bucket_elems, stream=None):
    _check(N.lib().allreduce_hierarchical_buckets(
        _op(op), nodes, local_ranks, _strategy(local_strategy), local_param or 0,
        _strategy(global_strategy), global_param or 0, N.pointer_array(rank_in), in_dtype,
        N.pointer_array(rank_out), out_dtype, n, bucket_elems, stream))


TILES_DTYPE = np.dtype([("numel", "<i8"), ("first_tile", "<i4"), ("lead", "<i4")])


def ddp_multi_plan(numels, P, in_dtype, out_dtype, align_to=None):
    """Tile plan of a multi-tensor all-reduce (host only).  Returns (tiles,
    total_tiles, tile_elems); tiles is a numpy structured array in the C
    layout.  ``align_to``: one address per tensor (e.g. rank 0's inputs) to
    put the tiles on 128-byte lines of, or None."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    tiles = np.zeros(numels.size, dtype=TILES_DTYPE)
    total = ctypes.c_int64(0)
    tile = ctypes.c_int64(0)
    _check(N.lib().ddp_multi_plan(numels.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                  numels.size, P, in_dtype, out_dtype,
                                  None if align_to is None else N.pointer_array(align_to),
                                  tiles.ctypes.data_as(ctypes.POINTER(N.TensorTiles)),
                                  ctypes.byref(total), ctypes.byref(tile)))
    return tiles, total.value, tile.value


def ddp_multi_block_map(tiles, total_tiles):
    """Block map of a multi-tensor plan (host only): entry k is the tensor
    holding tile 64 k.  Returns an int32 numpy array."""
    tiles = np.ascontiguousarray(tiles, dtype=TILES_DTYPE)
    n_blocks = ctypes.c_int64(0)
    c_tiles = tiles.ctypes.data_as(ctypes.POINTER(N.TensorTiles))
    lib = N.lib()
    _check(lib.ddp_multi_block_map(c_tiles, tiles.size, total_tiles, None, 0, ctypes.byref(n_blocks)))
    out = np.zeros(n_blocks.value, dtype=np.int32)
    _check(lib.ddp_multi_block_map(c_tiles, tiles.size, total_tiles,
                                   out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), out.size,
                                   ctypes.byref(n_blocks)))
    return out


def allreduce_multi_ring_emulated(op, P, chunking, n_tensors, tiles_dev, total_tiles, tile_elems,
                                  block_first_dev, in_ptrs_dev, in_dtype, out_ptrs_dev, out_dtype,
                                  stream=None):
    _check(N.lib().allreduce_multi_ring_emulated(_op(op), P, chunking, n_tensors, tiles_dev,
                                                 total_tiles, tile_elems, block_first_dev, in_ptrs_dev,
                                                 in_dtype, out_ptrs_dev, out_dtype, stream))


def allreduce_multi_fused_sgd(op, P, chunking, n_tensors, tiles_dev, total_tiles, tile_elems,
                              block_first_dev, in_ptrs_dev, grad_dtype, w_ptrs_dev, v_ptrs_dev, lr, mu,
                              out_ptrs_dev, out_dtype, stream=None):
    _check(N.lib().allreduce_multi_fused_sgd(_op(op), P, chunking, n_tensors, tiles_dev, total_tiles,
                                             tile_elems, block_first_dev, in_ptrs_dev, grad_dtype,
                                             w_ptrs_dev, v_ptrs_dev, lr, mu, out_ptrs_dev, out_dtype,
                                             stream))


def allreduce_multi_ring_noalloc(op, P, chunking, numels, in_ptrs, in_dtype, out_ptrs, out_dtype,
                                 stream=None):
    """The multi-tensor all-reduce from host arrays, with its tables in the
    library's per-GPU scratch area (no device allocation).  ``numels``: T
    element counts; ``in_ptrs``/``out_ptrs``: P * T device addresses,
    rank-major."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    T = numels.size
    if len(in_ptrs) != P * T or len(out_ptrs) != P * T:
        raise ValueError(f"need {P * T} input and output pointers")
    _check(N.lib().allreduce_multi_ring_noalloc(
        _op(op), P, chunking, T, numels.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        N.pointer_array(in_ptrs), in_dtype, N.pointer_array(out_ptrs), out_dtype, stream))


def ddp_set_wg_per_cu(family, wg_per_cu):
    """Tuning knob: cap the resident workgroups per CU of one kernel family
    (a name of ``KERNEL_FAMILIES`` or its ddp_kernel_family value) for later
    launches; 0 = no cap, -1 = the built-in choice.  Results do not change."""
    if isinstance(family, str):
        if family not in N.KERNEL_FAMILIES:
            raise ValueError(f"unknown kernel family {family!r}; one of {sorted(N.KERNEL_FAMILIES)}")
        family = N.KERNEL_FAMILIES[family]
    _check(N.lib().ddp_set_wg_per_cu(family, wg_per_cu))


KERNEL_FAMILIES = dict(N.KERNEL_FAMILIES)


# --------------------------------------------------------- torch level ----

def torch_dtype_code(dtype):
    import torch
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported element type {dtype}")


def current_stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _stream_for(tables):
    """Handle of the stream current on the tables' device.  The tables were
    allocated on the stream current at bind time; a launch on another stream
    is recorded on them, so that torch's allocator does not hand their memory
    out again before that launch has read it."""
    import torch
    s = torch.cuda.current_stream(tables[0].device)
    for t in tables:
        if t.device.type == "cuda":
            t.record_stream(s)
    return s.cuda_stream


def _same_device(a, b, what):
    if a[0].device != b[0].device:
        raise ValueError(f"{what}: outputs must live on the inputs' device")


def _rank_tensors(tensors, what):
    tensors = list(tensors)
    if not 1 <= len(tensors) <= MAX_RANKS:
        raise ValueError(f"{what}: need 1..{MAX_RANKS} rank tensors, got {len(tensors)}")
    t0 = tensors[0]
    for t in tensors:
        if not t.is_cuda:
            raise ValueError(f"{what}: tensors must live on the GPU")
        if t.device != t0.device or t.dtype != t0.dtype or t.numel() != t0.numel():
            raise ValueError(f"{what}: every rank needs the same device, dtype and size")
        if not t.is_contiguous():
            raise ValueError(f"{what}: tensors must be contiguous")
    return tensors


def allreduce(tensors, op="sum", chunking=None, out=None, out_dtype=None, bucket_elems=None):
    """All-reduce a list of P equal-size GPU tensors (one per rank) in the
    chunked ring order.  ``out``: list of P output tensors ("in place" when
    they are the inputs); default: new tensors of ``out_dtype`` (default the
    input dtype).  ``bucket_elems``: the tensors are flat gradient buffers
    of consecutive buckets of that many elements, each bucket all-reduced as
    its own ring (one call for all of them); None: one bucket.  Enqueued on
    the current stream; returns the outputs."""
    import torch
    tensors = _rank_tensors(tensors, "allreduce")
    P = len(tensors)
    if out is None:
        dt = out_dtype or tensors[0].dtype
        out = [torch.empty(tensors[0].shape, dtype=dt, device=tensors[0].device) for _ in range(P)]
    out = _rank_tensors(out, "allreduce out")
    if len(out) != P or out[0].numel() != tensors[0].numel():
        raise ValueError("allreduce: out must match the inputs")
    _same_device(tensors, out, "allreduce")
    if bucket_elems is not None:
        allreduce_ring_buckets(op, P, chunking or P, [t.data_ptr() for t in tensors],
                               torch_dtype_code(tensors[0].dtype), [t.data_ptr() for t in out],
                               torch_dtype_code(out[0].dtype), tensors[0].numel(), bucket_elems,
                               current_stream(tensors[0].device))
        return out
    allreduce_ring_emulated(op, P, chunking or P, [t.data_ptr() for t in tensors],
                            torch_dtype_code(tensors[0].dtype), [t.data_ptr() for t in out],
                            torch_dtype_code(out[0].dtype), tensors[0].numel(),
                            current_stream(tensors[0].device))
    return out


def allreduce_tree(tensors, op="sum", branching=2, out=None, out_dtype=None):
    """All-reduce along the b-ary tree (branching >= P-1: the centralized
    strategy).  Arguments as for ``allreduce``."""
    import torch
    tensors = _rank_tensors(tensors, "allreduce_tree")
    P = len(tensors)
    if out is None:
        dt = out_dtype or tensors[0].dtype
        out = [torch.empty(tensors[0].shape, dtype=dt, device=tensors[0].device) for _ in range(P)]
    out = _rank_tensors(out, "allreduce_tree out")
    if len(out) != P or out[0].numel() != tensors[0].numel():
        raise ValueError("allreduce_tree: out must match the inputs")
    _same_device(tensors, out, "allreduce_tree")
    allreduce_tree_emulated(op, P, branching, [t.data_ptr() for t in tensors],
                            torch_dtype_code(tensors[0].dtype), [t.data_ptr() for t in out],
                            torch_dtype_code(out[0].dtype), tensors[0].numel(),
                            current_stream(tensors[0].device))
    return out


def allreduce_hierarchical(tensors, nodes, op="sum", local=("ring", None), global_=("ring", None),
                           out=None, out_dtype=None, bucket_elems=None):
    """Two-level all-reduce: ``nodes`` nodes of len(tensors) / nodes ranks
    (node-major), each level with its own strategy, given as (name,
    parameter) with name "ring" (parameter: chunk count, None = the level's
    member count), "tree" (branching) or "centralized".  Other arguments as
    for ``allreduce`` (``bucket_elems``: every bucket its own two-level
    all-reduce)."""
    import torch
    tensors = _rank_tensors(tensors, "allreduce_hierarchical")
    P = len(tensors)
    if nodes < 1 or P % nodes:
        raise ValueError("allreduce_hierarchical: nodes must divide the rank count")
    if out is None:
        dt = out_dtype or tensors[0].dtype
        out = [torch.empty(tensors[0].shape, dtype=dt, device=tensors[0].device) for _ in range(P)]
    out = _rank_tensors(out, "allreduce_hierarchical out")
    if len(out) != P or out[0].numel() != tensors[0].numel():
        raise ValueError("allreduce_hierarchical: out must match the inputs")
    _same_device(tensors, out, "allreduce_hierarchical")
    args = (op, nodes, P // nodes, local[0], local[1], global_[0], global_[1], [t.data_ptr() for t in tensors],
            torch_dtype_code(tensors[0].dtype), [t.data_ptr() for t in out], torch_dtype_code(out[0].dtype),
            tensors[0].numel())
    if bucket_elems is not None:
        allreduce_hierarchical_buckets(*args, bucket_elems, current_stream(tensors[0].device))
    else:
        allreduce_hierarchical_emulated(*args, current_stream(tensors[0].device))
    return out


def reduce_scatter(tensors, op="sum", chunking=None, out=None, out_dtype=None, bucket_elems=None):
    """Reduce-scatter: out[owner(i)][i] receives element i's reduction
    (owner = the rank where the chunk's ring ends); every other element of
    ``out`` is left as it was.  ``bucket_elems``: every bucket of that many
    elements its own ring, as for ``allreduce``.  Returns ``out``."""
    import torch
    tensors = _rank_tensors(tensors, "reduce_scatter")
    P = len(tensors)
    if out is None:
        dt = out_dtype or tensors[0].dtype
        out = [torch.empty(tensors[0].shape, dtype=dt, device=tensors[0].device) for _ in range(P)]
    out = _rank_tensors(out, "reduce_scatter out")
    if len(out) != P or out[0].numel() != tensors[0].numel():
        raise ValueError("reduce_scatter: out must match the inputs")
    _same_device(tensors, out, "reduce_scatter")
    args = (op, P, chunking or P, [t.data_ptr() for t in tensors], torch_dtype_code(tensors[0].dtype),
            [t.data_ptr() for t in out], torch_dtype_code(out[0].dtype), tensors[0].numel())
    if bucket_elems is not None:
        reducescatter_ring_buckets(*args, bucket_elems, current_stream(tensors[0].device))
    else:
        reducescatter_ring_emulated(*args, current_stream(tensors[0].device))
    return out


def all_gather(tensors, chunking=None, bucket_elems=None):
    """All-gather in place: every rank receives each element from the rank
    that owns it.  ``bucket_elems``: every bucket of that many elements its
    own ring, as for ``allreduce``.  Returns the tensors."""
    tensors = _rank_tensors(tensors, "all_gather")
    args = (len(tensors), chunking or len(tensors), [t.data_ptr() for t in tensors],
            torch_dtype_code(tensors[0].dtype), tensors[0].numel())
    if bucket_elems is not None:
        allgather_ring_buckets(*args, bucket_elems, current_stream(tensors[0].device))
    else:
        allgather_ring_emulated(*args, current_stream(tensors[0].device))
    return tensors


def allreduce_stepwise(tensors, op="sum", chunking=None, sent=None, bucket_elems=None):
    """All-reduce fp32 rank tensors in place, one ring step per launch.
    ``sent``: optional int64 GPU tensor of P counters, increased by the
    elements each rank sends.  ``bucket_elems``: every bucket of that many
    elements its own ring, as for ``allreduce``.  Returns the tensors."""
    import torch
    tensors = _rank_tensors(tensors, "allreduce_stepwise")
    if sent is not None and (sent.dtype != torch.int64 or sent.numel() != len(tensors)
                             or sent.device != tensors[0].device or not sent.is_contiguous()):
        raise ValueError("allreduce_stepwise: sent must be a contiguous int64 tensor of P on the "
                         "tensors' device")
    args = (op, len(tensors), chunking or len(tensors), [t.data_ptr() for t in tensors],
            torch_dtype_code(tensors[0].dtype), tensors[0].numel())
    sent_ptr = sent.data_ptr() if sent is not None else None
    if bucket_elems is not None:
        allreduce_ring_stepwise_buckets(*args, bucket_elems, sent_ptr, current_stream(tensors[0].device))
    else:
        allreduce_ring_stepwise(*args, sent_ptr, current_stream(tensors[0].device))
    return tensors


class MultiAllReduce:
    """All-reduce many tensors per rank in one launch (the per-parameter
    small-message path).  Plans once for a list of shapes; ``__call__`` takes
    P lists of T tensors (rank-major) and optional P output lists."""

    def __init__(self, shapes, P, dtype, out_dtype=None, device="cuda", block_map=True):
        import torch
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.P = P
        self.dtype = dtype
        self.out_dtype = out_dtype or dtype
        self.device = torch.device(device)
        numels = [int(np.prod(s, dtype=np.int64)) for s in self.shapes]
        # The plan (and every table bound to it) lists the tensors smallest
        # first: the few-tile tensors, whose tiles do the least work per
        # prologue, then run while the launch fills the chip rather than in
        # its tail (measured 1.6-2% faster on the 161 ResNet-50 tensors,
        # level on the ViT-B/16 and ragged sets).  Each tensor's result does
        # not depend on the order.  plan_order[i] is the caller's index of
        # the i-th planned tensor.
        self.plan_order = sorted(range(len(numels)), key=lambda t: numels[t])
        self._planned_numels = [numels[t] for t in self.plan_order]
        # The block map lets each workgroup find its tensor with one table
        # read and a short search instead of a search over the whole plan
        # (block_map=False: the whole-plan search; same results).
        self._use_block_map = block_map
        self.tiles, self.total_tiles, self.tile_elems = ddp_multi_plan(
            self._planned_numels, P, torch_dtype_code(dtype), torch_dtype_code(self.out_dtype))
        self.tiles_dev, self.block_map, self.block_map_dev = self._upload(self.tiles, self.total_tiles)

    def _upload(self, tiles, total):
        import torch
        tiles_dev = torch.from_numpy(tiles.view(np.uint8).copy()).to(self.device)
        bmap = ddp_multi_block_map(tiles, total) if self._use_block_map else None
        bmap_dev = torch.from_numpy(bmap.copy()).to(self.device) if bmap is not None else None
        return tiles_dev, bmap, bmap_dev

    def _plan_for(self, rank_lists):
        """(tiles_dev, total_tiles, block_map_dev) for these tensors: the
        shared plan, or, when some tensor starts off a 128-byte line (a view
        into a larger buffer), a plan whose tiles follow rank 0's lines."""
        addrs = [rank_lists[0][t].data_ptr() for t in self.plan_order]
        tiles, total, _ = ddp_multi_plan(self._planned_numels, self.P, torch_dtype_code(self.dtype),
                                         torch_dtype_code(self.out_dtype), align_to=addrs)
        if not np.any(tiles["lead"]):
            return self.tiles_dev, self.total_tiles, self.block_map_dev
        tiles_dev, _, bmap_dev = self._upload(tiles, total)
        return tiles_dev, total, bmap_dev

    def _table(self, lists, dtype):
        import torch
        if len(lists) != self.P:
            raise ValueError(f"need {self.P} rank lists")
        ptrs = []
        for ts in lists:
            if len(ts) != len(self.shapes):
                raise ValueError("every rank needs one tensor per planned shape")
            for x, s in zip(ts, self.shapes):
                if tuple(x.shape) != s or x.dtype != dtype or not x.is_contiguous() \
                        or x.device != self.device:
                    raise ValueError("tensor does not match the plan")
            ptrs.extend(ts[t].data_ptr() for t in self.plan_order)
        return torch.tensor(ptrs, dtype=torch.int64).to(self.device)

    def bind(self, rank_lists, out=None):
        """Validate the tensors once and upload their pointer tables; returns
        a launcher ``run(op="sum", chunking=None)`` that enqueues the whole
        multi-tensor all-reduce with one call on the stream current at that
        call.  The launcher keeps the bound tensors (and ``out``, default:
        new tensors) alive; it always reduces those same tensors."""
        import torch
        if out is None:
            out = [[torch.empty(s, dtype=self.out_dtype, device=self.device) for s in self.shapes]
                   for _ in range(self.P)]
        tin = self._table(rank_lists, self.dtype)
        tout = self._table(out, self.out_dtype)
        tiles_dev, total, bmap_dev = self._plan_for(rank_lists)
        args = (self.P, len(self.shapes), tiles_dev.data_ptr(), total, self.tile_elems,
                bmap_dev.data_ptr() if bmap_dev is not None else None, tin.data_ptr(),
                torch_dtype_code(self.dtype), tout.data_ptr(), torch_dtype_code(self.out_dtype))
        tables = tuple(t for t in (tiles_dev, bmap_dev, tin, tout) if t is not None)

        def run(op="sum", chunking=None):
            P, T, tiles, total, tile, bmap, pin, dtin, pout, dtout = args
            allreduce_multi_ring_emulated(op, P, chunking or P, T, tiles, total, tile, bmap, pin, dtin,
                                          pout, dtout, _stream_for(tables))
            return out

        # The launcher holds raw device addresses: it must own every table
        # they point into, the tile plan included, so that it stays valid
        # after this object is dropped (``MultiAllReduce(...).bind(...)``),
        # and every tensor whose address a table holds, so that a tensor
        # the caller drops (e.g. a gradient replaced by zero_grad(set_to_none=
        # True)) is never freed and reused while the launcher can still
        # write it.  The launcher reduces exactly the tensors it was bound
        # to; new gradient tensors need a new bind().
        run.tables = tables
        run.tensors = (rank_lists, out)
        run.out = out
        return run

    def _state_table(self, ts):
        import torch
        if len(ts) != len(self.shapes):
            raise ValueError("one optimizer-state tensor per planned shape")
        for x, s in zip(ts, self.shapes):
            if tuple(x.shape) != s or x.dtype != torch.float32 or not x.is_contiguous() \
                    or x.device != self.device:
                raise ValueError("optimizer state must be contiguous float32 tensors of the planned shapes")
        return torch.tensor([ts[t].data_ptr() for t in self.plan_order], dtype=torch.int64).to(self.device)

    def bind_sgd(self, rank_grads, w, v, out=None):
        """Like bind(), for the all-reduce fused with one SGD-momentum step
        per tensor: ``w`` and ``v`` are lists of T float32 tensors (each
        parameter's master weights and momentum, updated in place); ``out``:
        optional P lists receiving the reduced gradients.  Returns
        ``run(lr, mu, op="mean", chunking=None)``."""
        tin = self._table(rank_grads, self.dtype)
        tout = self._table(out, self.out_dtype) if out is not None else None
        tw = self._state_table(w)
        tv = self._state_table(v)
        T = len(self.shapes)
        tiles_dev, total, bmap_dev = self._plan_for(rank_grads)

        tables = tuple(t for t in (tiles_dev, bmap_dev, tin, tout, tw, tv) if t is not None)

        def run(lr, mu, op="mean", chunking=None):
            allreduce_multi_fused_sgd(op, self.P, chunking or self.P, T, tiles_dev.data_ptr(), total,
                                      self.tile_elems, bmap_dev.data_ptr() if bmap_dev is not None else None,
                                      tin.data_ptr(),
                                      torch_dtype_code(self.dtype), tw.data_ptr(), tv.data_ptr(), lr, mu,
                                      tout.data_ptr() if tout is not None else None,
                                      torch_dtype_code(self.out_dtype), _stream_for(tables))
            return out

        run.tables = tables                    # owned by the launcher, as in bind()
        run.tensors = (rank_grads, w, v, out)  # every tensor the tables point to
        return run

    def __call__(self, rank_lists, op="sum", chunking=None, out=None):
        """bind() and launch once."""
        run = self.bind(rank_lists, out)
        self._last = run              # the tables must outlive the launch
        return run(op, chunking)


def zero1_sgd_step(grads, w, v, lr, mu, params, op="mean", chunking=None, bucket_elems=None):
    """ZeRO stage 1 step: reduce-scatter the rank gradients, the momentum
    step on the float32 master weights ``w`` and momentum ``v`` (updated in
    place; element i is its chunk owner's shard), and all-gather of the
    updated weights into every rank's ``params`` tensor (float32 or
    bfloat16; may be the gradient tensors themselves).  ``bucket_elems``: as
    for ``allreduce``.  Returns ``params``."""
    import torch
    grads = _rank_tensors(grads, "zero1_sgd_step")
    params = _rank_tensors(params, "zero1_sgd_step params")
    for t in (w, v):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != grads[0].numel() \
                or t.device != grads[0].device:
            raise ValueError("zero1_sgd_step: w and v must be contiguous float32 tensors of the "
                             "gradient's size on its device")
    if len(params) != len(grads) or params[0].numel() != grads[0].numel():
        raise ValueError("zero1_sgd_step: one parameter tensor per rank, of the gradient's size")
    _same_device(grads, params, "zero1_sgd_step")
    if bucket_elems is not None:
        zero1_sgd_step_buckets(op, len(grads), chunking or len(grads), [g.data_ptr() for g in grads],
                               torch_dtype_code(grads[0].dtype), grads[0].numel(), bucket_elems,
                               w.data_ptr(), v.data_ptr(), lr, mu, [p.data_ptr() for p in params],
                               torch_dtype_code(params[0].dtype), current_stream(grads[0].device))
        return params
    zero1_sgd_step_emulated(op, len(grads), chunking or len(grads), [g.data_ptr() for g in grads],
                            torch_dtype_code(grads[0].dtype), grads[0].numel(), w.data_ptr(),
                            v.data_ptr(), lr, mu, [p.data_ptr() for p in params],
                            torch_dtype_code(params[0].dtype), current_stream(grads[0].device))
    return params


def allreduce_sgd(grads, w, v, lr, mu, op="mean", chunking=None, out=None, bucket_elems=None):
    """All-reduce the rank gradients, then one SGD-momentum step on the
    float32 master weights ``w`` and momentum ``v`` (updated in place).
    ``out``: optional list of P tensors receiving the reduced gradient.
    ``bucket_elems``: as for ``allreduce`` (w and v in the same layout)."""
    import torch
    grads = _rank_tensors(grads, "allreduce_sgd")
    for t in (w, v):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != grads[0].numel() \
                or t.device != grads[0].device:
            raise ValueError("allreduce_sgd: w and v must be contiguous float32 tensors of the "
                             "gradient's size on its device")
    out_ptrs, out_code = None, F32
    if out is not None:
        out = _rank_tensors(out, "allreduce_sgd out")
        if len(out) != len(grads) or out[0].numel() != grads[0].numel():
            raise ValueError("allreduce_sgd: out must match the gradients")
        _same_device(grads, out, "allreduce_sgd")
        out_ptrs = [t.data_ptr() for t in out]
        out_code = torch_dtype_code(out[0].dtype)
    if bucket_elems is not None:
        allreduce_fused_sgd_buckets(op, len(grads), chunking or len(grads), [g.data_ptr() for g in grads],
                                    torch_dtype_code(grads[0].dtype), grads[0].numel(), bucket_elems,
                                    w.data_ptr(), v.data_ptr(), lr, mu, out_ptrs, out_code,
                                    current_stream(grads[0].device))
        return out
    allreduce_fused_sgd(op, len(grads), chunking or len(grads), [g.data_ptr() for g in grads],
                        torch_dtype_code(grads[0].dtype), grads[0].numel(), w.data_ptr(),
                        v.data_ptr(), lr, mu, out_ptrs, out_code, current_stream(grads[0].device))
    return out
