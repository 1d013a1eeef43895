"""Benchmark: the data-parallel gradient all-reduce on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--bucketed] [--no-secondary]
    python bench.py --suite                 every entry point at its workload's shape
    python bench.py --kernel-run NAME       one workload of the suite, untimed (for counters)
    python bench.py --occupancy-sweep       the measurements behind the built-in occupancy caps
    python bench.py --calibrate-copy        a plain copy of known size (scales memory counters)

Headline workload: P = 8 emulated ranks, each holding the gradients of a
2,017,529,856-parameter dense transformer (d = 2048, 24 blocks, MLP width
14,336, vocabulary 50,000, untied embedding and head; 292 tensors) in bf16,
drawn from N(0, 1e-4), laid out as views of 100 MiB buckets filled in
reverse parameter order (38 full buckets of 52,428,800 elements and a tail
of 25,235,456).  One step all-reduces every bucket with Mean in the chunked
ring order (8 chunks), fp32 accumulation, every rank receiving its own
float32 copy of the result: one allreduce_ring_emulated call (one launch)
per bucket, as data-parallel training issues one all-reduce per bucket.

Metric: effective HBM GB/s = algorithmic bytes / time, where the
algorithmic bytes of one all-reduce of n elements over P ranks are
P*n*(s_in + s_out) (every rank's input read once, every rank's output
written once): 48 bytes per element here, 96.8 GB per step.  Inputs are
resident in HBM before the timed region; a step streams far more than the
256 MB last-level cache.

Prints one JSON line: the step throughput, each launch's duration spread,
the dominant kernel's roofline (its launches timed with HIP events on the
stream they run on: the timed steps hold nothing but its launches, so a
profiler's average over the run is that launch's duration), the ResNet-50
set with 25 MiB buckets as a second workload (one call per bucket, and one
bucketed call), and the CPU oracle timed on a bounded sample of the
headline workload.  --bucketed adds the headline buckets in one bucketed
call (launches of another length, so a profiler's average over that run no
longer describes the per-bucket launch).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published peak
METRIC = "all-reduce effective HBM GB/s per bucket (P ranks) and % of MI355X HBM peak"
HEADLINE = "p8-transformer2b-bf16-mean-f32out-100MiB"
HEADLINE_KERNEL = "ring_reduce_kernel<8, true, false, false>"
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "ring_reduce_p8_bf16_f32_transformer2b_traffic.md")
KERNEL_SOURCES = ["ring_reduce_impl.h", "ring_reduce.hip", "ring_reduce_bf16_f32.hip", "launch.h"]


def kernel_source_hash():
    """SHA-256 of the dominant kernel's sources with comments and blank
    lines removed: an edit of the comments leaves the measured kernel, and
    so its recorded counters, valid."""
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gradient_all_reduce_allreduce_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()


def profile_fields(path):
    """The machine-read "- key: value" lines of a profile summary."""
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip()
    return fields


def measured_traffic(alg_bytes_per_step, launches_per_step):
    """HBM bytes per launch of the dominant kernel (the step's launches on
    average) from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source and on steps of the current shape; otherwise
    None."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = profile_fields(TRAFFIC_PROFILE)
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    if fields.get("algorithmic_bytes_per_step") != str(alg_bytes_per_step):
        return None
    if fields.get("launches_per_step") != str(launches_per_step):
        return None
    try:
        return round(float(fields["hbm_bytes_per_step"]) / launches_per_step, 1)
    except (KeyError, ValueError):
        return None


def cpu_baseline(samples, P, C, min_seconds=10.0, max_runs=6):
    """The oracle (NumPy, one thread) on whole buckets of the headline
    workload, the sampled buckets in turn, until at least min_seconds have
    passed (at most max_runs bucket all-reduces).  samples: list of
    (label, (P, n) uint16 bf16 bit patterns)."""
    import oracle
    done_bytes = 0
    runs = []
    t0 = time.perf_counter()
    while len(runs) < max_runs and time.perf_counter() - t0 < min_seconds:
        label, X = samples[len(runs) % len(samples)]
        oracle.ring_allreduce(X, "mean", C, in_dtype="bf16", out_dtype="f32")
        done_bytes += X.shape[0] * X.shape[1] * (2 + 4)
        runs.append(label)
    dt = time.perf_counter() - t0
    return {
        "value": round(done_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(runs)} whole-bucket all-reduces ({', '.join(runs)}) of the same gradient set "
                  f"(P={P}, bf16 -> f32, Mean, C={C}), stepwise ring simulation in NumPy on one "
                  f"thread, {dt:.1f} s; the host has {os.cpu_count()} cores",
    }


# --------------------------------------------------------------------------
# Workload setups shared by the headline, the suite and the kernel runs.
# --------------------------------------------------------------------------

def arena_sets(plan, P, n_sets, std, seed0, out_dtype=None):
    """Buffer sets of bucket views into per-rank arenas: per set, the
    (inputs, outputs) of every bucket, and the P input and output rows that
    hold the buckets end to end."""
    import workloads
    sets, rows = [], []
    for s_ in range(n_sets):
        g = plan.alloc_arena(P)
        for r in range(P):
            workloads.torch_normal_(g[r], std, seed=seed0 + 77 * s_ + r)
        o = plan.alloc_arena(P, out_dtype)
        E = plan.bucket_elems
        sets.append([([plan.bucket_view(g[r], k) for r in range(P)],
                      [o[r, k * E:k * E + plan.bucket_len(k)] for r in range(P)])
                     for k in range(plan.n_buckets)])
        rows.append(([g[r, :plan.total] for r in range(P)], [o[r, :plan.total] for r in range(P)]))
    return sets, rows


class Work:
    """One timed workload: fn(i) runs step i on the current stream."""

    def __init__(self, label, fn, nbytes, kernel, launches=None, steps=None, note=None,
                 host_timing=False, bytes_with_copies=None):
        self.label = label
        self.fn = fn
        self.nbytes = int(nbytes)
        self.kernel = kernel
        self.launches = launches
        self.steps = steps            # fixed step count (else the run's --steps)
        self.note = note
        self.host_timing = host_timing
        self.bytes_with_copies = bytes_with_copies


WORKS = {}      # name -> (group, setup(ctx) -> Work)


def work(name, group):
    def deco(f):
        WORKS[name] = (group, f)
        return f
    return deco


def _dev():
    import torch
    return torch.device("cuda:0")


def _resnet(ctx):
    if "resnet" not in ctx:
        import torch

        import gradient_all_reduce_allreduce_amd as ddp
        import workloads
        plan = ddp.GradBucketer(workloads.model_shapes("resnet50"), torch.float32, 25 << 20, device=_dev())
        sets, rows = arena_sets(plan, 8, 2, 0.01, 0)
        ctx["resnet"] = (plan, sets, rows)
    return ctx["resnet"]


def _resnet_tensors(ctx):
    if "resnet_tensors" not in ctx:
        import torch

        import gradient_all_reduce_allreduce_amd as ddp
        import workloads
        dev = _dev()
        shapes = workloads.model_shapes("resnet50")
        plan = ddp.GradBucketer(shapes, torch.float32, 25 << 20, device=dev)
        tensors = [[workloads.torch_normal_(torch.empty(s_, device=dev), 0.01, seed=300 + 1000 * r + t)
                    for t, s_ in enumerate(shapes)] for r in range(8)]
        ctx["resnet_tensors"] = (plan, shapes, tensors)
    return ctx["resnet_tensors"]


def _vit(ctx):
    if "vit" not in ctx:
        import torch

        import gradient_all_reduce_allreduce_amd as ddp
        import workloads
        dev = _dev()
        plan = ddp.GradBucketer(workloads.model_shapes("vit_b16"), torch.bfloat16, 25 << 20, device=dev)
        sets, rows = arena_sets(plan, 8, 2, 1e-3, 100)
        w = workloads.torch_normal_(torch.empty(plan.total, device=dev), 0.02, seed=7)
        v = torch.zeros(plan.total, device=dev)
        ctx["vit"] = (plan, sets, rows, w, v)
    return ctx["vit"]


def _ragged(ctx):
    if "ragged" not in ctx:
        import torch

        import gradient_all_reduce_allreduce_amd as ddp
        import workloads
        dev = _dev()
        sizes = workloads.ragged_sizes()
        plan = ddp.GradBucketer([(n,) for n in sizes], torch.float32, 25 << 20, device=dev)
        tensors = [[workloads.torch_uniform_(torch.empty(n, device=dev), -1.0, 1.0, seed=5000 * r + t)
                    for t, n in enumerate(sizes)] for r in range(4)]
        ctx["ragged"] = (plan, sizes, tensors)
    return ctx["ragged"]


def _tf2b(ctx):
    """The headline gradient set: one arena of bf16 inputs and one of float32
    outputs (97 GB together; one buffer set already defeats the 256 MB
    last-level cache)."""
    if "tf2b" not in ctx:
        import torch

        import gradient_all_reduce_allreduce_amd as ddp
        import workloads
        cfg = workloads.CONFIGS[HEADLINE]
        dev = _dev()
        plan = ddp.GradBucketer(workloads.model_shapes(cfg["model"]), torch.bfloat16, cfg["bucket_bytes"],
                                device=dev)
        g = plan.alloc_arena(cfg["P"])
        for r in range(cfg["P"]):
            workloads.torch_normal_(g[r], cfg["dist"][1], seed=500 + r)
        o = plan.alloc_arena(cfg["P"], torch.float32)
        ctx["tf2b"] = (plan, g, o)
    return ctx["tf2b"]


def _bucket_args(plan, g, o, P):
    """Per bucket: (input pointers, output pointers, elements) for the raw
    entry point, prepared once."""
    E = plan.bucket_elems
    out = []
    for k in range(plan.n_buckets):
        n = plan.bucket_len(k)
        out.append(([g[r, k * E:].data_ptr() for r in range(P)], [o[r, k * E:].data_ptr() for r in range(P)], n))
    return out


# Kernel names as a profiler prints them (without namespaces and arguments).
RING = "ring_reduce_kernel<8, false, false, false>"
RING_SGD_BF16 = "ring_reduce_kernel<8, true, true, true>"
RING_SGD_BF16_NO_OUT = "ring_reduce_kernel<8, true, false, true>"   # no gradient output
TREE = "tree_reduce_kernel<8, false, false>"


@work("ring-p4-65536", "small")
def _w_small(ctx):
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    dev = _dev()
    x = [torch.empty(65536, device=dev).normal_() for _ in range(4)]
    o = [torch.empty_like(t) for t in x]
    ctx["small"] = (x, o)
    return Work("p4 f32 sum n=65,536 (2 MB per call, cache resident: launch-bound)",
                lambda i: ddp.allreduce(x, "sum", 4, out=o), 4 * 65536 * 8,
                "ring_reduce_kernel<4, false, false, false>", 1, host_timing=True,
                note="time per call on the stream; host_us_per_call is the Python call alone")


@work("ring-p4-65536-cabi", "small")
def _w_small_c(ctx):
    import torch

    from gradient_all_reduce_allreduce_amd import _native
    if "small" not in ctx:
        _w_small(ctx)
    x, o = ctx["small"]
    lib = _native.lib()
    pin = _native.pointer_array([t.data_ptr() for t in x])
    pout = _native.pointer_array([t.data_ptr() for t in o])
    sh = torch.cuda.current_stream(_dev()).cuda_stream

    def c_call(i):
        if lib.allreduce_ring_emulated(_native.DDP_SUM, 4, 4, pin, _native.DDP_F32, pout,
                                       _native.DDP_F32, 65536, sh) != 0:
            raise RuntimeError(_native.last_error())
    return Work("p4 f32 sum n=65,536, C ABI call with prepared arguments", c_call, 4 * 65536 * 8,
                "ring_reduce_kernel<4, false, false, false>", 1, host_timing=True,
                note="time per call on the stream; host_us_per_call is the ctypes call alone")


@work("ring-resnet50", "resnet")
def _w_ring_resnet(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sets, _ = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, bucket views, one call per bucket",
                lambda i: [ddp.allreduce(a, "mean", 8, out=o) for a, o in sets[i % 2]],
                8 * plan.total * 8, RING, plan.n_buckets)


@work("ring-resnet50-bucketed", "resnet")
def _w_ring_resnet_b(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, _, rows = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, bucket views, all buckets in one bucketed call",
                lambda i: ddp.allreduce(rows[i % 2][0], "mean", 8, out=rows[i % 2][1],
                                        bucket_elems=plan.bucket_elems),
                8 * plan.total * 8, RING,
                ddp.ddp_buckets_launch_count(8, 8, ddp.F32, ddp.F32, False, plan.total, plan.bucket_elems),
                note="every bucket its own ring, the same bits")


@work("tree-resnet50", "resnet")
def _w_tree(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sets, _ = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, tree b=2 on bucket views, one call per bucket",
                lambda i: [ddp.allreduce_tree(a, "mean", 2, out=o) for a, o in sets[i % 2]],
                8 * plan.total * 8, TREE, plan.n_buckets)


@work("tree-resnet50-flat", "resnet")
def _w_tree_flat(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, _, rows = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, tree b=2 over the flat buffer (every bucket's tree, one launch)",
                lambda i: ddp.allreduce_tree(rows[i % 2][0], "mean", 2, out=rows[i % 2][1]),
                8 * plan.total * 8, TREE, 1,
                note="the tree's order is the same for every element: the same bits as one tree per bucket")


@work("hier-resnet50-2x4-ring-ring", "resnet")
def _w_hier1(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sets, _ = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, two-level 2 nodes x 4: ring in the nodes, ring over them",
                lambda i: [ddp.allreduce_hierarchical(a, 2, "mean", ("ring", None), ("ring", None), out=o)
                           for a, o in sets[i % 2]],
                8 * plan.total * 8, TREE, plan.n_buckets)


@work("hier-resnet50-2x4-ring-ring-bucketed", "resnet")
def _w_hier1_b(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, _, rows = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, two-level 2 nodes x 4: ring in the nodes, ring over them, all buckets in "
                "one bucketed call",
                lambda i: ddp.allreduce_hierarchical(rows[i % 2][0], 2, "mean", ("ring", None), ("ring", None),
                                                     out=rows[i % 2][1], bucket_elems=plan.bucket_elems),
                8 * plan.total * 8, TREE, 2,
                note="every bucket its own two-level ring, the same bits; the full buckets go out as one")


@work("hier-resnet50-4x2-tree-ring", "resnet")
def _w_hier2(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sets, _ = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, two-level 4 nodes x 2: tree in the nodes, ring over them",
                lambda i: [ddp.allreduce_hierarchical(a, 4, "mean", ("tree", 2), ("ring", None), out=o)
                           for a, o in sets[i % 2]],
                8 * plan.total * 8, TREE, plan.n_buckets)


@work("rs-resnet50", "resnet")
def _w_rs(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sets, _ = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, reduce-scatter alone (owner-only writes), one call per bucket",
                lambda i: [ddp.reduce_scatter(a, "mean", 8, out=o) for a, o in sets[i % 2]],
                8 * plan.total * 4 + plan.total * 4, "ring_rs_kernel<8, false, false>",
                plan.n_buckets, note="reads P*n, writes n (each element to its owner)")


@work("ag-resnet50", "resnet")
def _w_ag(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sets, _ = _resnet(ctx)
    return Work("resnet50 p8 f32, all-gather alone (owner to every other rank), one call per bucket",
                lambda i: [ddp.all_gather(o, 8) for _, o in sets[i % 2]],
                plan.total * 4 + 7 * plan.total * 4, "ring_ag_kernel<8, 4>", plan.n_buckets,
                note="reads n, writes (P-1)*n")


@work("rs-resnet50-bucketed", "resnet")
def _w_rs_b(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, _, rows = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, reduce-scatter alone, all buckets in one bucketed call",
                lambda i: ddp.reduce_scatter(rows[i % 2][0], "mean", 8, out=rows[i % 2][1],
                                             bucket_elems=plan.bucket_elems),
                8 * plan.total * 4 + plan.total * 4, "ring_rs_kernel<8, false, false>", 2,
                note="every bucket its own ring, the same bits; the full buckets go out as one ring of "
                     "buckets x 8 chunks")


@work("ag-resnet50-bucketed", "resnet")
def _w_ag_b(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, _, rows = _resnet(ctx)
    return Work("resnet50 p8 f32, all-gather alone, all buckets in one bucketed call",
                lambda i: ddp.all_gather(rows[i % 2][1], 8, bucket_elems=plan.bucket_elems),
                plan.total * 4 + 7 * plan.total * 4, "ring_ag_kernel<8, 4>", 2,
                note="every bucket its own ring, the same bits; the full buckets go out as one ring of "
                     "buckets x 8 chunks")


@work("stepwise-resnet50", "resnet")
def _w_step(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sets, _ = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, stepwise ring (2(P-1) launches per bucket, in place)",
                lambda i: [ddp.allreduce_stepwise(o, "mean", 8) for _, o in sets[i % 2]],
                8 * plan.total * 8, "ring_step_kernel<8>", 14 * plan.n_buckets, steps=20,
                note="moves 35n floats per bucket against 16n")


@work("stepwise-resnet50-bucketed", "resnet")
def _w_step_b(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, _, rows = _resnet(ctx)
    return Work("resnet50 p8 f32 mean, stepwise ring, all buckets in one bucketed call (in place)",
                lambda i: ddp.allreduce_stepwise(rows[i % 2][1], "mean", 8, bucket_elems=plan.bucket_elems),
                8 * plan.total * 8, "ring_step_kernel<8>", 28, steps=20,
                note="every bucket its own ring, the same bits and per-rank sends; the full buckets go out as "
                     "one ring of buckets x 8 chunks: 2(P-1) launches for them and 2(P-1) for the tail")


@work("multi-resnet50", "resnet_tensors")
def _w_multi(ctx):
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    plan, shapes, tensors = _resnet_tensors(ctx)
    outs = [[torch.empty(s_, device=_dev()) for s_ in shapes] for _ in range(8)]
    run = ddp.MultiAllReduce(shapes, 8, torch.float32, device=_dev()).bind(tensors, outs)
    return Work("resnet50 p8 f32 mean, 161 separate tensors, one multi-tensor launch",
                lambda i: run("mean"), 8 * plan.total * 8, "multi_ring_kernel<8, false, false, false>", 1)


def _noalloc_runner(ctx, shapes, tensors, n_out):
    """fn(i) calling allreduce_multi_ring_noalloc on the tensors (smallest
    first, as MultiAllReduce orders them), into output set i % n_out."""
    import ctypes

    import numpy as np
    import torch

    from gradient_all_reduce_allreduce_amd import _native as N
    numels = [int(np.prod(s_, dtype=np.int64)) for s_ in shapes]
    order = sorted(range(len(numels)), key=lambda t: numels[t])
    c_numels = (ctypes.c_int64 * len(order))(*[numels[t] for t in order])
    c_in = N.pointer_array([tensors[r][t].data_ptr() for r in range(8) for t in order])
    outs = [[[torch.empty(s_, device=_dev()) for s_ in shapes] for _ in range(8)] for _ in range(n_out)]
    c_outs = [N.pointer_array([o[r][t].data_ptr() for r in range(8) for t in order]) for o in outs]
    ctx.setdefault("noalloc_outs", []).append(outs)

    def run(i):
        stream = ctypes.c_void_p(torch.cuda.current_stream(_dev()).cuda_stream)
        st = N.lib().allreduce_multi_ring_noalloc(N.DDP_MEAN, 8, 8, len(order), c_numels, c_in, N.DDP_F32,
                                                  c_outs[i % n_out], N.DDP_F32, stream)
        if st != N.DDP_OK:
            raise RuntimeError(N.last_error())
    return run


@work("multi-noalloc-resnet50-alternating", "resnet_tensors")
def _w_multi_noalloc_alt(ctx):
    """As multi-noalloc-resnet50, alternating between two output sets, so
    that every call writes its tables (4 fill launches of 30,016 bytes)."""
    plan, shapes, tensors = _resnet_tensors(ctx)
    run = _noalloc_runner(ctx, shapes, tensors, 2)
    return Work("resnet50 p8 f32 mean, 161 separate tensors, allocation-free multi-tensor call, tables "
                "written on every call (two output sets alternating)", run, 8 * plan.total * 8,
                "multi_ring_kernel<8, false, false, false>", 1, host_timing=True,
                note="against multi-noalloc-resnet50: the cost of writing the tables on every call")


@work("multi-noalloc-resnet50", "resnet_tensors")
def _w_multi_noalloc(ctx):
    """The same 161 tensors through the allocation-free entry point, the
    same outputs every call: the tables are written on the first call only,
    later calls plan on the host and launch."""
    plan, shapes, tensors = _resnet_tensors(ctx)
    run = _noalloc_runner(ctx, shapes, tensors, 1)
    return Work("resnet50 p8 f32 mean, 161 separate tensors, allocation-free multi-tensor call (host plan, "
                "tables in the scratch area, one launch)", run, 8 * plan.total * 8,
                "multi_ring_kernel<8, false, false, false>", 1, host_timing=True,
                note="against multi-resnet50: the same tensors every call, so the tables are copied on the "
                     "first call only and later calls plan on the host and launch")


@work("multi-resnet50-views", "resnet")
def _w_multi_views(ctx):
    """The multi-tensor launch over the same 161 tensors laid out as views of
    the per-rank arena rows the bucketed call reads (gradients as bucket
    views): the kernel on the bucketed call's memory layout."""
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    import workloads
    plan, _, rows = _resnet(ctx)
    shapes = workloads.model_shapes("resnet50")
    runs = []
    for ins, outs in rows:
        tin = [plan.tensor_views(x) for x in ins]
        tout = [plan.tensor_views(x) for x in outs]
        runs.append(ddp.MultiAllReduce(shapes, 8, torch.float32, device=_dev()).bind(tin, tout))
    return Work("resnet50 p8 f32 mean, 161 tensors as views of the bucketed call's arena rows, one "
                "multi-tensor launch", lambda i: runs[i % 2]("mean"), 8 * plan.total * 8,
                "multi_ring_kernel<8, false, false, false>", 1,
                note="the same memory layout as the bucketed call: separates the kernel from the layout")


@work("multi-sgd-resnet50", "resnet_tensors")
def _w_multi_sgd(ctx):
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    plan, shapes, tensors = _resnet_tensors(ctx)
    mw = [torch.empty(s_, device=_dev()).normal_(0, 0.02) for s_ in shapes]
    mv = [torch.zeros(s_, device=_dev()) for s_ in shapes]
    run = ddp.MultiAllReduce(shapes, 8, torch.float32, device=_dev()).bind_sgd(tensors, mw, mv)
    return Work("resnet50 p8 f32 mean, 161 separate tensors, one launch with fused sgd-momentum per tensor",
                lambda i: run(1e-3, 0.9, "mean"), 8 * plan.total * 4 + 16 * plan.total,
                "multi_ring_kernel<8, false, false, true>", 1)


def _packed(ctx, key):
    plan, _, tensors = _resnet_tensors(ctx) if key == "resnet" else _ragged(ctx)
    if key + "_table" not in ctx:
        ctx[key + "_table"] = plan.pointer_table(tensors)
    return plan, tensors, ctx[key + "_table"]


@work("packed-step-resnet50", "resnet_tensors")
def _w_packed(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, _, table = _packed(ctx, "resnet")
    bufs = plan.alloc_buckets(8)

    def packed_step(i):
        for k in range(plan.n_buckets):
            n = plan.bucket_len(k)
            plan.pack(table, k, bufs)
            ddp.allreduce([x[:n] for x in bufs], "mean", 8, out=[x[:n] for x in bufs])
            plan.unpack(table, k, bufs)
    nbytes = 8 * plan.total * 8
    return Work("resnet50 p8 f32 mean, pack -> all-reduce -> unpack", packed_step, nbytes, None,
                bytes_with_copies=3 * nbytes,
                note="gbps counts the all-reduce bytes; with_copies_gbps adds pack and unpack traffic")


@work("pack-resnet50", "resnet_tensors")
def _w_pack(ctx):
    plan, _, table = _packed(ctx, "resnet")
    bufs = plan.alloc_buckets(8)
    return Work("resnet50 p8 f32, pack alone (161 tensors -> 4 buckets, all ranks, one bucket buffer set)",
                lambda i: [plan.pack(table, k, bufs) for k in range(plan.n_buckets)],
                8 * plan.total * 8, "bucket_copy_kernel<true>",
                note="the bucket buffers (200 MiB) are reused for every bucket, as a DDP step does, "
                     "so the last-level cache holds part of them")


@work("unpack-resnet50", "resnet_tensors")
def _w_unpack(ctx):
    plan, _, table = _packed(ctx, "resnet")
    bufs = plan.alloc_buckets(8)
    return Work("resnet50 p8 f32, unpack alone (4 buckets -> 161 tensors, all ranks, one bucket buffer set)",
                lambda i: [plan.unpack(table, k, bufs) for k in range(plan.n_buckets)],
                8 * plan.total * 8, "bucket_copy_kernel<false>")


@work("pack-resnet50-fresh", "resnet_tensors")
def _w_pack_fresh(ctx):
    plan, _, table = _packed(ctx, "resnet")
    per_bucket = [plan.alloc_buckets(8) for _ in range(plan.n_buckets)]
    return Work("resnet50 p8 f32, pack alone, a bucket buffer set per bucket",
                lambda i: [plan.pack(table, k, per_bucket[k]) for k in range(plan.n_buckets)],
                8 * plan.total * 8, "bucket_copy_kernel<true>")


@work("unpack-resnet50-fresh", "resnet_tensors")
def _w_unpack_fresh(ctx):
    plan, _, table = _packed(ctx, "resnet")
    per_bucket = [plan.alloc_buckets(8) for _ in range(plan.n_buckets)]
    return Work("resnet50 p8 f32, unpack alone, a bucket buffer set per bucket",
                lambda i: [plan.unpack(table, k, per_bucket[k]) for k in range(plan.n_buckets)],
                8 * plan.total * 8, "bucket_copy_kernel<false>")


def _sgd_work(ctx, with_out, bucketed):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sets, rows, w, v = _vit(ctx)
    E = plan.bucket_elems

    def sgd_step(i):
        for k, (a, o) in enumerate(sets[i % 2]):
            lo, n = k * E, plan.bucket_len(k)
            ddp.allreduce_sgd(a, w[lo:lo + n], v[lo:lo + n], 1e-3, 0.9, "mean", 8,
                              out=o if with_out else None)

    def sgd_bucketed(i):
        ddp.allreduce_sgd(rows[i % 2][0], w, v, 1e-3, 0.9, "mean", 8,
                          out=rows[i % 2][1] if with_out else None, bucket_elems=E)
    label = ("vitb16 p8 bf16 mean + fused sgd-momentum (w, v fp32), " +
             ("gradients also written (bf16)" if with_out else "no gradient output") +
             (", all buckets in one bucketed call" if bucketed else ", one call per bucket"))
    launches = (ddp.ddp_buckets_launch_count(8, 8, ddp.BF16, ddp.BF16, True, plan.total, E)
                if bucketed else plan.n_buckets)
    return Work(label, sgd_bucketed if bucketed else sgd_step,
                8 * plan.total * (4 if with_out else 2) + 16 * plan.total,
                RING_SGD_BF16 if with_out else RING_SGD_BF16_NO_OUT, launches,
                note="every bucket its own ring, the same bits" if bucketed else None)


@work("sgd-vitb16", "vit")
def _w_sgd(ctx):
    return _sgd_work(ctx, False, False)


@work("sgd-vitb16-out", "vit")
def _w_sgd_out(ctx):
    return _sgd_work(ctx, True, False)


@work("sgd-vitb16-bucketed", "vit")
def _w_sgd_b(ctx):
    return _sgd_work(ctx, False, True)


@work("sgd-vitb16-out-bucketed", "vit")
def _w_sgd_out_b(ctx):
    return _sgd_work(ctx, True, True)


@work("zero1-vitb16", "vit")
def _w_zero1(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sets, _, w, v = _vit(ctx)
    E = plan.bucket_elems

    def zero1_step(i):
        for k, (a, o) in enumerate(sets[i % 2]):
            lo, n = k * E, plan.bucket_len(k)
            ddp.zero1_sgd_step(a, w[lo:lo + n], v[lo:lo + n], 1e-3, 0.9, o, "mean", 8)
    return Work("vitb16 p8 bf16 mean, ZeRO stage 1 step (owner sgd-momentum, bf16 parameters to every rank)",
                zero1_step, 8 * plan.total * 4 + 16 * plan.total,
                RING_SGD_BF16, plan.n_buckets)


@work("zero1-vitb16-bucketed", "vit")
def _w_zero1_b(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, _, rows, w, v = _vit(ctx)
    return Work("vitb16 p8 bf16 mean, ZeRO stage 1 step, all buckets in one bucketed call",
                lambda i: ddp.zero1_sgd_step(rows[i % 2][0], w, v, 1e-3, 0.9, rows[i % 2][1], "mean", 8,
                                             bucket_elems=plan.bucket_elems),
                8 * plan.total * 4 + 16 * plan.total, RING_SGD_BF16,
                ddp.ddp_buckets_launch_count(8, 8, ddp.BF16, ddp.BF16, True, plan.total, plan.bucket_elems),
                note="every bucket its own ring, the same bits")


@work("packed-step-ragged2000", "ragged")
def _w_ragged_step(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, sizes, table = _packed(ctx, "ragged")
    bufs = plan.alloc_buckets(4)

    def ragged_step(i):
        for k in range(plan.n_buckets):
            n = plan.bucket_len(k)
            plan.pack(table, k, bufs)
            ddp.allreduce([x[:n] for x in bufs], "sum", 4, out=[x[:n] for x in bufs])
            plan.unpack(table, k, bufs)
    nbytes = 4 * plan.total * 8
    return Work(f"ragged 2000 tensors p4 f32 sum, pack -> all-reduce -> unpack ({plan.n_buckets} buckets)",
                ragged_step, nbytes, None, steps=10, bytes_with_copies=3 * nbytes,
                note="gbps counts the all-reduce bytes; with_copies_gbps adds pack and unpack traffic")


@work("pack-ragged2000", "ragged")
def _w_ragged_pack(ctx):
    plan, _, table = _packed(ctx, "ragged")
    bufs = plan.alloc_buckets(4)
    return Work(f"ragged 2000 tensors p4 f32, pack alone ({plan.n_buckets} buckets, all ranks)",
                lambda i: [plan.pack(table, k, bufs) for k in range(plan.n_buckets)],
                4 * plan.total * 8, "bucket_copy_kernel<true>", steps=10)


@work("unpack-ragged2000", "ragged")
def _w_ragged_unpack(ctx):
    plan, _, table = _packed(ctx, "ragged")
    bufs = plan.alloc_buckets(4)
    return Work(f"ragged 2000 tensors p4 f32, unpack alone ({plan.n_buckets} buckets, all ranks)",
                lambda i: [plan.unpack(table, k, bufs) for k in range(plan.n_buckets)],
                4 * plan.total * 8, "bucket_copy_kernel<false>", steps=10)


@work("bucketed-step-ragged2000", "ragged")
def _w_ragged_bucketed(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, _, table = _packed(ctx, "ragged")
    arena = plan.alloc_arena(4)
    E = plan.bucket_elems
    slots = [[arena[r, k * E:k * E + plan.bucket_len(k)] for r in range(4)] for k in range(plan.n_buckets)]
    flat = [arena[r, :plan.total] for r in range(4)]

    def ragged_bucketed(i):
        for k in range(plan.n_buckets):
            plan.pack(table, k, slots[k])
        ddp.allreduce(flat, "sum", 4, out=flat, bucket_elems=E)
        for k in range(plan.n_buckets):
            plan.unpack(table, k, slots[k])
    nbytes = 4 * plan.total * 8
    return Work("ragged 2000 tensors p4 f32 sum, pack every bucket -> one bucketed all-reduce -> unpack",
                ragged_bucketed, nbytes, None, steps=10, bytes_with_copies=3 * nbytes,
                note="gbps counts the all-reduce bytes; with_copies_gbps adds pack and unpack traffic")


@work("multi-ragged2000", "ragged")
def _w_ragged_multi(ctx):
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    plan, sizes, tensors = _ragged(ctx)
    run = ddp.MultiAllReduce([(n,) for n in sizes], 4, torch.float32, device=_dev()).bind(tensors, tensors)
    return Work("ragged 2000 tensors p4 f32 sum, one multi-tensor launch, in place",
                lambda i: run("sum"), 4 * plan.total * 8, "multi_ring_kernel<4, false, false, false>", 1, steps=10)


def _split_rows(ctx):
    """Two buffer sets of P = 8 contiguous rank rows (inputs and outputs) of
    25,559,040 floats (99,840 tiles of the multi-tensor kernel), rows 4 KiB
    apart: the same memory handed to the multi-tensor kernel as one tensor
    per rank or as 160 equal ones."""
    if "split" not in ctx:
        import torch

        import workloads
        n = 99840 * 256
        stride = n + 1024
        sets = []
        for s_ in range(2):
            g = torch.empty(8 * stride, device=_dev())
            workloads.torch_normal_(g, 0.01, seed=700 + s_)
            o = torch.empty(8 * stride, device=_dev())
            sets.append(([g[r * stride:r * stride + n] for r in range(8)],
                         [o[r * stride:r * stride + n] for r in range(8)]))
        ctx["split"] = (n, sets)
    return ctx["split"]


def _split_work(ctx, T):
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    n, sets = _split_rows(ctx)
    each = n // T
    m = ddp.MultiAllReduce([(each,)] * T, 8, torch.float32, device=_dev())
    runs = [m.bind([[x[t * each:(t + 1) * each] for t in range(T)] for x in ins],
                   [[y[t * each:(t + 1) * each] for t in range(T)] for y in outs]) for ins, outs in sets]
    return runs, 8 * n * 8


@work("multi-split1", "split")
def _w_split1(ctx):
    runs, nbytes = _split_work(ctx, 1)
    return Work("p8 f32 mean, contiguous rank rows of 25,559,040 floats as one tensor per rank, one "
                "multi-tensor launch", lambda i: runs[i % 2]("mean"), nbytes,
                "multi_ring_kernel<8, false, false, false>", 1,
                note="with multi-split160: the multi-tensor kernel's cost per tensor on the same memory")


@work("multi-split160", "split")
def _w_split160(ctx):
    runs, nbytes = _split_work(ctx, 160)
    return Work("p8 f32 mean, the same rows as 160 equal tensors per rank (624 tiles each), one "
                "multi-tensor launch", lambda i: runs[i % 2]("mean"), nbytes,
                "multi_ring_kernel<8, false, false, false>", 1,
                note="no partial tile and no tile across a chunk boundary: only the tensor count differs")


@work("ring-transformer2b", "tf2b")
def _w_tf2b(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, g, o = _tf2b(ctx)
    args = _bucket_args(plan, g, o, 8)
    return Work(f"transformer-2b p8 bf16 -> f32 mean ({plan.n_buckets} x 100 MiB buckets), one call per bucket",
                lambda i: [ddp.allreduce_ring_emulated("mean", 8, 8, a, ddp.BF16, b, ddp.F32, n) for a, b, n in args],
                8 * plan.total * 6, HEADLINE_KERNEL, plan.n_buckets, steps=5)


@work("ring-transformer2b-bucketed", "tf2b")
def _w_tf2b_b(ctx):
    import gradient_all_reduce_allreduce_amd as ddp
    plan, g, o = _tf2b(ctx)
    ins = [g[r, :plan.total] for r in range(8)]
    outs = [o[r, :plan.total] for r in range(8)]
    return Work(f"transformer-2b p8 bf16 -> f32 mean ({plan.n_buckets} x 100 MiB buckets), one bucketed call",
                lambda i: ddp.allreduce(ins, "mean", 8, out=outs, bucket_elems=plan.bucket_elems),
                8 * plan.total * 6, HEADLINE_KERNEL,
                ddp.ddp_buckets_launch_count(8, 8, ddp.BF16, ddp.F32, False, plan.total, plan.bucket_elems),
                steps=5, note="every bucket its own ring, the same bits")


def _time(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def run_suite(steps, warmup, names=None):
    """Every registered workload (or the named ones) timed at its shape; one
    JSON line each.  Rates are algorithmic bytes (what the method must read
    and write) over time, with the inputs resident in HBM."""
    import torch
    torch.cuda.set_device(_dev())
    ctx = {}
    group = None
    for name, (grp, setup) in WORKS.items():
        if names and name not in names:
            continue
        if grp != group:
            ctx.clear()
            torch.cuda.empty_cache()
            group = grp
        w = setup(ctx)
        k = w.steps or steps
        ms = _time(w.fn, k, min(warmup, max(1, k // 4)) if w.steps else warmup)
        line = {"suite": name, "label": w.label, "kernel": w.kernel, "ms": round(ms, 4),
                "algorithmic_bytes": w.nbytes, "gbps": round(w.nbytes / (ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(w.nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if w.launches:
            line["launches_per_step"] = w.launches
            line["avg_launch_us"] = round(ms * 1e3 / w.launches, 2)
        if w.bytes_with_copies:
            line["with_copies_gbps"] = round(w.bytes_with_copies / (ms * 1e-3) / 1e9, 1)
        if w.host_timing:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(k):
                w.fn(i)
            line["host_us_per_call"] = round((time.perf_counter() - t0) / k * 1e6, 2)
            torch.cuda.synchronize()
        if w.note:
            line["note"] = w.note
        print(json.dumps(line), flush=True)
        del w
    ctx.clear()
    torch.cuda.empty_cache()
    return 0


def run_kernel(name, steps, warmup):
    """One registered workload, untimed: W + K steps and nothing else of
    this package, so that a profiler's per-kernel counters over the run
    divided by W + K are one step's.  Prints what a step must move."""
    import torch
    if name not in WORKS:
        print(f"unknown workload {name!r}; known: {', '.join(WORKS)}", file=sys.stderr)
        return 2
    torch.cuda.set_device(_dev())
    ctx = {}
    w = WORKS[name][1](ctx)
    torch.cuda.synchronize()
    for i in range(warmup + steps):
        w.fn(i)
    torch.cuda.synchronize()
    print(json.dumps({"kernel_run": name, "label": w.label, "kernel": w.kernel, "steps": warmup + steps,
                      "algorithmic_bytes_per_step": w.nbytes, "launches_per_step": w.launches}), flush=True)
    return 0


def run_occupancy_sweep(caps=(2, 3, 4, 5, 6, 8, 10, 12, 16)):
    """Time the fused all-reduce and the fused optimizer step at every cap on
    resident workgroups per CU (ddp_set_wg_per_cu), for each rank count and
    element-type pair, on four 25 MiB buckets per rank (two buffer sets);
    one JSON line per case with the rate at every cap and the built-in
    choice's rate.  The tables of launch.h hold the fastest cap per case."""
    import torch

    import gradient_all_reduce_allreduce_amd as ddp

    dev = _dev()

    def timed(fn, steps=20):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def sweep(name, family, fn, nbytes):
        rates = {}
        for k in caps:
            ddp.ddp_set_wg_per_cu(family, k)
            rates[k] = round(nbytes / timed(fn) / 1e6, 1)
        ddp.ddp_set_wg_per_cu(family, -1)
        builtin = round(nbytes / timed(fn) / 1e6, 1)
        best = max(rates, key=rates.get)
        print(json.dumps({"occupancy": name, "family": family, "best_cap": best, "builtin_gbps": builtin,
                          "gbps_by_cap": rates}), flush=True)

    bucket = 25 << 20
    nb = 4
    names = {torch.float32: "f32", torch.bfloat16: "bf16"}
    for P in (2, 3, 4, 5, 6, 8, 12, 16):
        for it, ot in ((torch.float32, torch.float32), (torch.float32, torch.bfloat16),
                       (torch.bfloat16, torch.float32), (torch.bfloat16, torch.bfloat16)):
            n = bucket // (2 if it == torch.bfloat16 else 4)
            g = torch.empty(2, P, nb * n, dtype=it, device=dev).normal_(0, 0.01)
            o = torch.empty(2, P, nb * n, dtype=ot, device=dev)
            views = [[([g[s_, r, k * n:(k + 1) * n] for r in range(P)],
                       [o[s_, r, k * n:(k + 1) * n] for r in range(P)]) for k in range(nb)] for s_ in range(2)]
            sweep(f"ring P={P} {names[it]}->{names[ot]}", "ring",
                  lambda: [[ddp.allreduce(a, "mean", P, out=b) for a, b in st] for st in views],
                  2 * nb * n * P * (g.element_size() + o.element_size()))
            del g, o, views
        for it in (torch.bfloat16, torch.float32):
            n = bucket // (2 if it == torch.bfloat16 else 4)
            g = torch.empty(P, nb * n, dtype=it, device=dev).normal_(0, 0.01)
            o = torch.empty(P, nb * n, dtype=it, device=dev)
            w = torch.zeros(nb * n, device=dev)
            v = torch.zeros(nb * n, device=dev)
            for with_out in (False, True):
                sweep(f"sgd P={P} {names[it]} grads, {'with' if with_out else 'no'} gradient output", "ring_sgd",
                      lambda: [ddp.allreduce_sgd([g[r, k * n:(k + 1) * n] for r in range(P)], w[k * n:(k + 1) * n],
                                                 v[k * n:(k + 1) * n], 1e-3, 0.9, "mean", P,
                                                 out=[o[r, k * n:(k + 1) * n] for r in range(P)] if with_out else None)
                               for k in range(nb)],
                      nb * n * (P * g.element_size() * (2 if with_out else 1) + 16))
            del g, o, w, v
        torch.cuda.empty_cache()
    return 0


# --------------------------------------------------------------------------
# The headline line.
# --------------------------------------------------------------------------

def timed_region(fn, steps, stream):
    """K steps bracketed by events on the stream the kernels run on, with a
    device synchronisation on both sides; ms per step."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def secondary_resnet50(steps, warmup):
    """The ResNet-50 gradient set (P = 8, fp32, Mean, C = 8, 25 MiB buckets:
    3 full + a tail) as a second workload: one call per bucket, and one
    bucketed call (each bucket its own ring, the same bits; one launch)."""
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    ctx = {}
    out = {"workload": "resnet50-gradient-set all-reduce: P=8 ranks x 161 fp32 tensors (25,557,032 "
                       "params) N(0,0.01), 25 MiB buckets (3 full + tail of 5,896,232), grads as bucket "
                       "views of per-rank arenas, Mean, 8 ring chunks, two buffer sets alternating",
           "kernel": RING}
    for key, name in (("one_call_per_bucket", "ring-resnet50"), ("bucketed_call", "ring-resnet50-bucketed")):
        w = WORKS[name][1](ctx)
        stream = torch.cuda.current_stream()
        for i in range(warmup):
            w.fn(i)
        ms = timed_region(w.fn, steps, stream)
        gbs = w.nbytes / (ms * 1e-3) / 1e9
        out[key] = {"value": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                    "ms_per_step": round(ms, 4), "launches_per_step": w.launches,
                    "avg_launch_us": round(ms * 1e3 / w.launches, 2), "steps": steps}
    out["bytes_per_step"] = w.nbytes
    del w
    ctx.clear()
    torch.cuda.empty_cache()
    return out


def headline(args):
    import numpy as np
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    import workloads
    from gradient_all_reduce_allreduce_amd import _native

    cfg = workloads.CONFIGS[HEADLINE]
    P, C = cfg["P"], cfg["chunking"]
    dev = _dev()
    torch.cuda.set_device(dev)
    ctx = {}
    plan, g, o = _tf2b(ctx)
    lens = [plan.bucket_len(k) for k in range(plan.n_buckets)]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    lib = _native.lib()
    # Arguments of every bucket's call prepared once, as a training loop
    # that issues one all-reduce per bucket would hold them.
    calls = [(_native.pointer_array(a), _native.pointer_array(b), n) for a, b, n in _bucket_args(plan, g, o, P)]

    def launch(a, b, n):
        if lib.allreduce_ring_emulated(_native.DDP_MEAN, P, C, a, _native.DDP_BF16, b, _native.DDP_F32,
                                       n, sh) != 0:
            raise RuntimeError(_native.last_error())

    def step(i):
        """One step: every bucket with one single-bucket call (one launch)."""
        for a, b, n in calls:
            launch(a, b, n)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region 1: K steps bracketed by events.
    ms_step = timed_region(step, args.steps, stream)
    bytes_step = sum(P * n * (2 + 4) for n in lens)
    value = bytes_step / (ms_step * 1e-3) / 1e9

    # The step is nothing but launches of the dominant kernel, back to back
    # on one stream, so region 1 also gives that kernel's average launch
    # duration: step time / launches per step.
    launches = len(lens)
    avg_ms = ms_step / launches
    avg_bytes = bytes_step / launches
    achieved = avg_bytes / (avg_ms * 1e-3) / 1e9

    # Region 2: the same K steps with an event pair around every launch
    # (the pairs add about 2 us per launch): each launch's duration.
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        for (a, b, n), (e0, e1) in zip(calls, ev[i]):
            e0.record(stream)
            launch(a, b, n)
            e1.record(stream)
    torch.cuda.synchronize()
    durs = np.array([[e0.elapsed_time(e1) for e0, e1 in row] for row in ev])   # ms, [K, launches]
    full = np.array([n == plan.bucket_elems for n in lens])
    full_d = np.sort(durs[:, full].ravel())
    tail_d = np.sort(durs[:, ~full].ravel()) if (~full).any() else None
    per_step = np.sort(durs.sum(axis=1))

    def spread(d, n):
        med = float(np.median(d))
        return {"elements": int(n), "launches": int(d.size), "median_us": round(med * 1e3, 2),
                "min_us": round(float(d[0]) * 1e3, 2), "max_us": round(float(d[-1]) * 1e3, 2),
                "median_gbs": round(P * n * 6 / (med * 1e-3) / 1e9, 1)}

    bucketed = {"value": None,
                "note": "not timed by default: one bucketed call puts consecutive full buckets in launches of up "
                        "to 2^29 elements, another length of the same kernel, which would change a profiler's "
                        "average over this run; `bench.py --bucketed` adds it (the same bits as one call per "
                        "bucket)"}
    if args.bucketed:
        ins = [g[r, :plan.total] for r in range(P)]
        outs = [o[r, :plan.total] for r in range(P)]
        bucket_step = (lambda i: ddp.allreduce(ins, "mean", C, out=outs, bucket_elems=plan.bucket_elems))
        for i in range(args.warmup):
            bucket_step(i)
        ms_b = timed_region(bucket_step, args.steps, stream)
        nl = ddp.ddp_buckets_launch_count(P, C, ddp.BF16, ddp.F32, False, plan.total, plan.bucket_elems)
        bucketed = {"value": round(bytes_step / (ms_b * 1e-3) / 1e9, 1),
                    "frac_of_peak": round(bytes_step / (ms_b * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "ms_per_step": round(ms_b, 4), "launches_per_step": nl,
                    "note": "every bucket in one allreduce_ring_buckets call: each bucket its own ring "
                            "(the same bits as one call per bucket), consecutive full buckets in launches "
                            "of up to 2^29 elements"}

    samples = []
    if not args.no_cpu_baseline:
        mid = plan.n_buckets // 2
        E = plan.bucket_elems
        for label, k in (("first", 0), ("middle", mid), ("tail", plan.n_buckets - 1)):
            X = g[:, k * E:k * E + lens[k]].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            samples.append((f"{label} bucket {k}, {lens[k]:,} elements", X))
    del calls, g, o, plan
    ctx.clear()
    torch.cuda.empty_cache()

    secondary = None if args.no_secondary else secondary_resnet50(max(args.steps, 100), args.warmup)

    traffic = measured_traffic(bytes_step, launches)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "transformer-2b gradient-set all-reduce: P=8 ranks x 292 bf16 tensors "
                        "(2,017,529,856 params: d=2048, 24 blocks, MLP 14,336, vocab 50,000, untied) "
                        "N(0,1e-4), 100 MiB buckets (38 full + tail of 25,235,456), grads as bucket views "
                        "of a per-rank arena, Mean with fp32 accumulation and fp32 output, 8 ring chunks; "
                        "one allreduce_ring_emulated call (one launch) per bucket",
            "P": P, "chunking": C, "op": "mean", "in_dtype": "bf16", "out_dtype": "f32",
            "bucket_bytes": cfg["bucket_bytes"], "buckets": launches, "elements_per_rank": sum(lens),
            "bytes_per_step": bytes_step,
        },
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": HEADLINE_KERNEL,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_ms * 1e3, 2),
            "launches_per_step": launches,
            "algorithmic_bytes_per_launch": round(avg_bytes, 1),
            "timing": "events around the timed steps, which hold only this kernel's launches (one per "
                      "bucket); achieved and traffic are per launch, averaged over the step's launches",
        },
        "per_launch": {
            "full_bucket": spread(full_d, max(lens)),
            "tail_bucket": spread(tail_d, min(lens)) if tail_d is not None else None,
            "per_step_median_ms": round(float(np.median(per_step)), 4),
            "per_step_min_ms": round(float(per_step[0]), 4),
            "note": "a second pass of K steps with an event pair around every launch (about 2 us each)",
        },
        "bucketed_call": bucketed,
        "resnet50_25MiB": secondary,
        "cpu_baseline": None,
    }
    if samples:
        out["cpu_baseline"] = cpu_baseline(samples, P, C)
    print(json.dumps(out), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; --suite 200, --kernel-run 3)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 5; --suite 20, --kernel-run 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the ResNet-50 set with 25 MiB buckets")
    ap.add_argument("--bucketed", action="store_true",
                    help="also time the headline buckets in one bucketed call (launches of another "
                         "length: a profiler's average over the run then mixes both)")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the headline line, time every workload of the suite (one JSON "
                         "line each)")
    ap.add_argument("--only", nargs="*", default=None,
                    help="with --suite: only these workloads")
    ap.add_argument("--kernel-run", default=None, metavar="NAME",
                    help="run one workload of the suite W + K times, untimed (for a profiler's "
                         "counters); --list-workloads names them")
    ap.add_argument("--list-workloads", action="store_true")
    ap.add_argument("--occupancy-sweep", action="store_true",
                    help="time the fused all-reduce and optimizer step at every cap on resident "
                         "workgroups per CU (the measurements behind the built-in caps)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 10 times (a kernel of known "
                         "traffic, to scale the memory counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the P ranks are emulated as P buffers in one "
              f"GPU's HBM; --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2
    if args.list_workloads:
        for name, (grp, _) in WORKS.items():
            print(name, grp)
        return 0

    import torch

    if args.calibrate_copy:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": a.numel() * 4,
                          "bytes_written": b.numel() * 4, "launches": 10}))
        return 0
    if args.suite:
        return run_suite(200 if args.steps is None else args.steps,
                         20 if args.warmup is None else args.warmup, args.only)
    if args.kernel_run:
        return run_kernel(args.kernel_run, 3 if args.steps is None else args.steps,
                          1 if args.warmup is None else args.warmup)
    args.steps = 20 if args.steps is None else args.steps
    args.warmup = 5 if args.warmup is None else args.warmup
    if args.occupancy_sweep:
        return run_occupancy_sweep()
    return headline(args)


if __name__ == "__main__":
    sys.exit(main())
