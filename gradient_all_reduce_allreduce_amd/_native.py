"""ctypes view of the C ABI in include/ddp_allreduce.h.

Loads ``libddp_allreduce.so`` from this package directory.  There is no
fallback: if the library is missing or fails to load, every entry point
raises, because a CPU substitute would silently change what is being
measured and checked.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libddp_allreduce.so")

DDP_OK = 0
DDP_E_ARG = -1
DDP_E_UNSUPPORTED = -2
DDP_E_ALIGN = -3
DDP_E_OVERLAP = -4
DDP_E_PLAN = -5
DDP_E_HIP = -6
STATUS_NAMES = {
    DDP_OK: "DDP_OK", DDP_E_ARG: "DDP_E_ARG", DDP_E_UNSUPPORTED: "DDP_E_UNSUPPORTED",
    DDP_E_ALIGN: "DDP_E_ALIGN", DDP_E_OVERLAP: "DDP_E_OVERLAP", DDP_E_PLAN: "DDP_E_PLAN",
    DDP_E_HIP: "DDP_E_HIP",
}

DDP_SUM = 0
DDP_MEAN = 1
DDP_F32 = 0
DDP_BF16 = 1
DDP_MAX_RANKS = 16

# ddp_kernel_family
KERNEL_FAMILIES = {"ring": 0, "ring_sgd": 1, "tree": 2, "reduce_scatter": 3, "all_gather": 4,
                   "multi": 5, "bucket_copy": 6, "step": 7}


class Segment(ctypes.Structure):
    """ddp_segment: elements [src_off, src_off+len) of tensor `tensor`
    occupy [dst_off, dst_off+len) of bucket `bucket`."""
    _fields_ = [("tensor", ctypes.c_int32), ("bucket", ctypes.c_int32),
                ("src_off", ctypes.c_int64), ("dst_off", ctypes.c_int64),
                ("len", ctypes.c_int64)]


class TensorTiles(ctypes.Structure):
    """ddp_tensor_tiles: a tensor's element count, first tile and lead (the
    length of a short first tile, 0 for none)."""
    _fields_ = [("numel", ctypes.c_int64), ("first_tile", ctypes.c_int32), ("lead", ctypes.c_int32)]


_c_void_pp = ctypes.POINTER(ctypes.c_void_p)
_SIGNATURES = {
    "ddp_bucket_plan": (ctypes.c_int, [
        ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, ctypes.c_int, ctypes.c_int64,
        ctypes.POINTER(Segment), ctypes.c_int64, ctypes.POINTER(ctypes.c_int64),
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
        ctypes.POINTER(ctypes.c_uint64)]),
    "ddp_bucket_pack": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_int32, _c_void_pp, _c_void_pp, ctypes.c_int64, ctypes.c_void_p]),
    "ddp_bucket_unpack": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_int32, _c_void_pp, _c_void_pp, ctypes.c_int64, ctypes.c_void_p]),
    "allreduce_ring_emulated": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, _c_void_pp,
        ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]),
    "allreduce_fused_sgd": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, _c_void_pp,
        ctypes.c_int, ctypes.c_void_p]),
    "allreduce_ring_buckets": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, _c_void_pp,
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "allreduce_fused_sgd_buckets": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, _c_void_pp,
        ctypes.c_int, ctypes.c_void_p]),
    "ddp_buckets_launch_count": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int, ctypes.c_int, ctypes.c_int32, ctypes.c_int64,
        ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "zero1_sgd_step_buckets": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, _c_void_pp,
        ctypes.c_int, ctypes.c_void_p]),
    "zero1_sgd_step_emulated": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, _c_void_pp,
        ctypes.c_int, ctypes.c_void_p]),
    "reducescatter_ring_emulated": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, _c_void_pp,
        ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]),
    "allgather_ring_emulated": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]),
    "allreduce_ring_stepwise": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p]),
    "reducescatter_ring_buckets": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, _c_void_pp,
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "allgather_ring_buckets": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p]),
    "allreduce_ring_stepwise_buckets": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "allreduce_tree_emulated": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _c_void_pp, ctypes.c_int, _c_void_pp,
        ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]),
    "allreduce_hierarchical_emulated": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int, ctypes.c_int32, ctypes.c_int,
        ctypes.c_int32, _c_void_pp, ctypes.c_int, _c_void_pp, ctypes.c_int, ctypes.c_int64,
        ctypes.c_void_p]),
    "allreduce_hierarchical_buckets": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int, ctypes.c_int32, ctypes.c_int,
        ctypes.c_int32, _c_void_pp, ctypes.c_int, _c_void_pp, ctypes.c_int, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p]),
    "ddp_multi_plan": (ctypes.c_int, [
        ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, ctypes.c_int32, ctypes.c_int, ctypes.c_int,
        _c_void_pp, ctypes.POINTER(TensorTiles), ctypes.POINTER(ctypes.c_int64),
        ctypes.POINTER(ctypes.c_int64)]),
    "ddp_multi_block_map": (ctypes.c_int, [
        ctypes.POINTER(TensorTiles), ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32),
        ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "allreduce_multi_ring_emulated": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "allreduce_multi_fused_sgd": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_void_p]),
    "allreduce_multi_ring_noalloc": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.POINTER(ctypes.c_int64), _c_void_pp, ctypes.c_int, _c_void_pp, ctypes.c_int,
        ctypes.c_void_p]),
    "ddp_set_wg_per_cu": (ctypes.c_int, [ctypes.c_int, ctypes.c_int32]),
    "ddp_last_error": (ctypes.c_char_p, []),
}

_lib = None


class NativeLibraryMissing(RuntimeError):
    pass


def lib():
    """The loaded C library (loaded once).  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NativeLibraryMissing(
                f"{LIB_PATH} is not built; run "
                "`python -m gradient_all_reduce_allreduce_amd.build` first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (restype, argtypes) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = restype
            fn.argtypes = argtypes
        _lib = handle
    return _lib


def last_error():
    msg = lib().ddp_last_error()
    return msg.decode() if msg else ""


def pointer_array(ptrs):
    """Host array of device pointers (void*[]) from Python ints."""
    arr = (ctypes.c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr
