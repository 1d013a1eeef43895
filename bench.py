"""Benchmark: the data-parallel gradient all-reduce on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--per-bucket]

Workload (the configuration the headline metric is quoted on): P = 8
emulated ranks, each holding a ResNet-50-shaped gradient set of 161 fp32
tensors (25,557,032 parameters) drawn from N(0, 0.01), laid out as views of
25 MiB buckets filled in reverse parameter order (3 full buckets and a
partial tail).  One step all-reduces every bucket with Mean in the chunked
ring order (8 chunks), every rank receiving its own copy of the result, in
one bucketed call (each bucket its own ring; one launch holds the 3 full
buckets as one ring and the tail bucket as a second segment).  The same
buckets with one call each are timed beside it with --per-bucket.

Metric: effective HBM GB/s = algorithmic bytes / time, where the algorithmic
bytes of one all-reduce of n elements over P ranks are P*n*(s_in + s_out)
(every rank's input read once, every rank's output written once).  Inputs
are resident in HBM before the timed region; the step streams 1.6 GB, far
more than the 256 MB last-level cache, and two buffer sets alternate.

Prints one JSON line with the step throughput, the dominant kernel's
roofline (its launches timed with HIP events on the stream they run on: the
timed steps consist of nothing but its launches, so a profiler's average
over the run is that launch's duration) and the CPU oracle timed on a
bounded sample of the same workload.  --per-bucket adds the same buckets
with one call each (with each bucket's median and minimum launch time from
an event pair around every launch).
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
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "ring_reduce_p8_f32_resnet50_traffic.md")
KERNEL_SOURCES = ["ring_reduce_impl.h", "ring_reduce.hip", "ring_reduce_f32_f32.hip", "launch.h"]


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


def measured_traffic(alg_bytes_per_launch):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source
    and on launches of the current shape; otherwise None."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    with open(TRAFFIC_PROFILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip().lstrip("- ").strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    if fields.get("algorithmic_bytes_per_launch") != str(alg_bytes_per_launch):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(grads_host, bucket_lens, P, C, min_seconds=10.0, max_passes=20):
    """The oracle (NumPy, single thread) on whole buckets of the same
    gradient set, bucket after bucket and pass after pass, until at least
    min_seconds have passed (bounded by max_passes over the set)."""
    import oracle
    done_bytes = 0
    t0 = time.perf_counter()
    buckets = 0
    for _ in range(max_passes):
        for X in grads_host:
            oracle.ring_allreduce(X, "mean", C)
            buckets += 1
            done_bytes += X.shape[0] * X.shape[1] * 8
            if time.perf_counter() - t0 > min_seconds:
                break
        if time.perf_counter() - t0 > min_seconds:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(done_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{buckets} bucket all-reduces over the {len(bucket_lens)} buckets of the "
                  f"same gradient set (P={P}, fp32, Mean, C={C}), stepwise ring simulation in NumPy, "
                  f"{dt:.1f} s; host has {os.cpu_count()} cores",
    }


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


def run_suite(steps, warmup):
    """Every entry point at the shape of its workload; one JSON line each.
    Rates are algorithmic bytes (what the method must read and write) over
    time, with the inputs resident in HBM."""
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    import workloads

    dev = torch.device("cuda:0")

    def report(name, ms, nbytes, **extra):
        line = {"suite": name, "ms": round(ms, 4), "algorithmic_bytes": int(nbytes),
                "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        line.update(extra)
        print(json.dumps(line), flush=True)

    def arena_sets(plan, P, n_sets=2, std=0.01, out_dtype=None):
        """Buffer sets of bucket views into per-rank arenas: per set, the
        (inputs, outputs) of every bucket, and the P input and output rows
        that hold the buckets end to end."""
        sets, rows = [], []
        for s_ in range(n_sets):
            g = plan.alloc_arena(P)
            for r in range(P):
                workloads.torch_normal_(g[r], std, seed=77 * s_ + r)
            o = plan.alloc_arena(P, out_dtype)
            E = plan.bucket_elems
            sets.append([([plan.bucket_view(g[r], k) for r in range(P)],
                          [o[r, k * E:k * E + plan.bucket_len(k)] for r in range(P)])
                         for k in range(plan.n_buckets)])
            rows.append(([g[r, :plan.total] for r in range(P)], [o[r, :plan.total] for r in range(P)]))
        return sets, rows

    # 4 ranks x 65,536 fp32, Sum, 4 chunks, out of place.  2 MB
    # per call sits in the last-level cache, so the call is bound by launch
    # and host overhead: a parity case, not a bandwidth one.
    x1 = [torch.empty(65536, device=dev).normal_() for _ in range(4)]
    o1 = [torch.empty_like(t) for t in x1]
    ms1 = _time(lambda i: ddp.allreduce(x1, "sum", 4, out=o1), steps, warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ddp.allreduce(x1, "sum", 4, out=o1)
    host_us = (time.perf_counter() - t0) / steps * 1e6
    torch.cuda.synchronize()
    report("p4 f32 sum n=65,536 (2 MB per call, cache resident: launch-bound)", ms1, 4 * 65536 * 8,
           host_us_per_call=round(host_us, 2),
           note="time per call on the stream; host_us_per_call is the Python call alone")
    # The same call through the C ABI with its arguments prepared once (what
    # a C caller or a bound launcher pays per call).
    from gradient_all_reduce_allreduce_amd import _native
    lib = _native.lib()
    pin = _native.pointer_array([t.data_ptr() for t in x1])
    pout = _native.pointer_array([t.data_ptr() for t in o1])
    sh = torch.cuda.current_stream(dev).cuda_stream

    def c_call(i):
        if lib.allreduce_ring_emulated(_native.DDP_SUM, 4, 4, pin, _native.DDP_F32, pout,
                                       _native.DDP_F32, 65536, sh) != 0:
            raise RuntimeError(_native.last_error())
    ms1c = _time(c_call, steps, warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        c_call(i)
    host_c_us = (time.perf_counter() - t0) / steps * 1e6
    torch.cuda.synchronize()
    report("p4 f32 sum n=65,536, C ABI call with prepared arguments", ms1c, 4 * 65536 * 8,
           host_us_per_call=round(host_c_us, 2),
           note="time per call on the stream; host_us_per_call is the ctypes call alone")
    del x1, o1

    # ResNet-50 gradient set, P=8: bucket views (the headline step), the multi-tensor launch
    # over the 161 separate per-parameter tensors, and pack/unpack
    P = 8
    shapes = workloads.model_shapes("resnet50")
    plan = ddp.GradBucketer(shapes, torch.float32, 25 << 20, device=dev)
    nbytes = P * plan.total * 8
    sets, rows = arena_sets(plan, P)
    report("resnet50 p8 f32 mean, bucket views",
           _time(lambda i: [ddp.allreduce(a, "mean", P, out=o) for a, o in sets[i % 2]], steps, warmup),
           nbytes)
    report("resnet50 p8 f32 mean, bucket views, all buckets in one bucketed call",
           _time(lambda i: ddp.allreduce(rows[i % 2][0], "mean", P, out=rows[i % 2][1],
                                         bucket_elems=plan.bucket_elems), steps, warmup),
           nbytes, note="every bucket its own ring, the same bits; 1 launch per step")
    report("resnet50 p8 f32 mean, tree b=2 on bucket views",
           _time(lambda i: [ddp.allreduce_tree(a, "mean", 2, out=o) for a, o in sets[i % 2]], steps, warmup),
           nbytes)
    report("resnet50 p8 f32 mean, tree b=2 over the flat buffer (every bucket's tree, one launch)",
           _time(lambda i: ddp.allreduce_tree(rows[i % 2][0], "mean", 2, out=rows[i % 2][1]), steps, warmup),
           nbytes, note="the tree's order is the same for every element: the same bits as one tree per bucket")
    report("resnet50 p8 f32 mean, two-level 2 nodes x 4: ring in the nodes, ring over them",
           _time(lambda i: [ddp.allreduce_hierarchical(a, 2, "mean", ("ring", None), ("ring", None), out=o)
                            for a, o in sets[i % 2]], steps, warmup),
           nbytes)
    report("resnet50 p8 f32 mean, two-level 4 nodes x 2: tree in the nodes, ring over them",
           _time(lambda i: [ddp.allreduce_hierarchical(a, 4, "mean", ("tree", 2), ("ring", None), out=o)
                            for a, o in sets[i % 2]], steps, warmup),
           nbytes)
    report("resnet50 p8 f32 mean, reduce-scatter alone (owner-only writes), one call per bucket",
           _time(lambda i: [ddp.reduce_scatter(a, "mean", P, out=o) for a, o in sets[i % 2]], steps, warmup),
           P * plan.total * 4 + plan.total * 4, note="reads P*n, writes n (each element to its owner)")
    report("resnet50 p8 f32, all-gather alone (owner to every other rank), one call per bucket",
           _time(lambda i: [ddp.all_gather(o, P) for _, o in sets[i % 2]], steps, warmup),
           plan.total * 4 + (P - 1) * plan.total * 4, note="reads n, writes (P-1)*n")
    report("resnet50 p8 f32 mean, stepwise ring (2(P-1) launches per bucket, in place)",
           _time(lambda i: [ddp.allreduce_stepwise(o, "mean", P) for _, o in sets[i % 2]],
                 max(2, steps // 10), 2), nbytes, note="moves 35n floats per bucket against 16n")
    del sets, rows
    tensors = [[torch.empty(s_, device=dev).normal_(0, 0.01) for s_ in shapes] for _ in range(P)]
    outs = [[torch.empty(s_, device=dev) for s_ in shapes] for _ in range(P)]
    run = ddp.MultiAllReduce(shapes, P, torch.float32, device=dev).bind(tensors, outs)
    report("resnet50 p8 f32 mean, 161 separate tensors, one multi-tensor launch",
           _time(lambda i: run("mean"), steps, warmup), nbytes)
    mw = [torch.empty(s_, device=dev).normal_(0, 0.02) for s_ in shapes]
    mv = [torch.zeros(s_, device=dev) for s_ in shapes]
    run_sgd = ddp.MultiAllReduce(shapes, P, torch.float32, device=dev).bind_sgd(tensors, mw, mv)
    report("resnet50 p8 f32 mean, 161 separate tensors, one launch with fused sgd-momentum per tensor",
           _time(lambda i: run_sgd(1e-3, 0.9, "mean"), steps, warmup), P * plan.total * 4 + 16 * plan.total)
    del mw, mv, run_sgd
    table = plan.pointer_table(tensors)
    bufs = plan.alloc_buckets(P)

    def packed_step(i):
        for k in range(plan.n_buckets):
            n = plan.bucket_len(k)
            plan.pack(table, k, bufs)
            ddp.allreduce([x[:n] for x in bufs], "mean", P, out=[x[:n] for x in bufs])
            plan.unpack(table, k, bufs)
    ms = _time(packed_step, steps, warmup)
    report("resnet50 p8 f32 mean, pack -> all-reduce -> unpack", ms, nbytes,
           with_copies_gbps=round(3 * nbytes / (ms * 1e-3) / 1e9, 1),
           note="gbps counts the all-reduce bytes; with_copies_gbps adds pack and unpack traffic")
    copy_bytes = P * plan.total * 4 * 2     # every rank's gradients read once and written once
    report("resnet50 p8 f32, pack alone (161 tensors -> 4 buckets, all ranks)",
           _time(lambda i: [plan.pack(table, k, bufs) for k in range(plan.n_buckets)], steps, warmup),
           copy_bytes)
    report("resnet50 p8 f32, unpack alone (4 buckets -> 161 tensors, all ranks)",
           _time(lambda i: [plan.unpack(table, k, bufs) for k in range(plan.n_buckets)], steps, warmup),
           copy_bytes)
    # The lines above reuse one set of P bucket buffers (200 MiB) for every
    # bucket, as a DDP step does, so the last-level cache can hold part of
    # them; with a buffer set per bucket (800 MiB) every byte goes to HBM.
    per_bucket = [plan.alloc_buckets(P) for _ in range(plan.n_buckets)]
    report("resnet50 p8 f32, pack alone, a bucket buffer set per bucket",
           _time(lambda i: [plan.pack(table, k, per_bucket[k]) for k in range(plan.n_buckets)], steps, warmup),
           copy_bytes)
    report("resnet50 p8 f32, unpack alone, a bucket buffer set per bucket",
           _time(lambda i: [plan.unpack(table, k, per_bucket[k]) for k in range(plan.n_buckets)], steps, warmup),
           copy_bytes)
    del tensors, outs, run, table, bufs, per_bucket
    torch.cuda.empty_cache()

    # ViT-B/16 bf16 gradients, P=8, Mean, fused SGD-momentum
    plan = ddp.GradBucketer(workloads.model_shapes("vit_b16"), torch.bfloat16, 25 << 20, device=dev)
    sets, rows = arena_sets(plan, P, std=1e-3)
    w = torch.empty(plan.total, device=dev).normal_(0, 0.02)
    v = torch.zeros(plan.total, device=dev)
    E = plan.bucket_elems

    def sgd_step(i, with_out):
        for k, (a, o) in enumerate(sets[i % 2]):
            lo, n = k * E, plan.bucket_len(k)
            ddp.allreduce_sgd(a, w[lo:lo + n], v[lo:lo + n], 1e-3, 0.9, "mean", P,
                              out=o if with_out else None)
    report("vitb16 p8 bf16 mean + fused sgd-momentum (w, v fp32), no gradient output",
           _time(lambda i: sgd_step(i, False), steps, warmup), P * plan.total * 2 + 16 * plan.total)
    report("vitb16 p8 bf16 mean + fused sgd-momentum, gradients also written (bf16)",
           _time(lambda i: sgd_step(i, True), steps, warmup), P * plan.total * 4 + 16 * plan.total)
    for with_out in (False, True):
        report("vitb16 p8 bf16 mean + fused sgd-momentum, " +
               ("gradients also written (bf16), " if with_out else "no gradient output, ") +
               "all buckets in one bucketed call",
               _time(lambda i: ddp.allreduce_sgd(rows[i % 2][0], w, v, 1e-3, 0.9, "mean", P,
                                                 out=rows[i % 2][1] if with_out else None,
                                                 bucket_elems=E), steps, warmup),
               P * plan.total * (4 if with_out else 2) + 16 * plan.total,
               note="every bucket its own ring, the same bits; 1 launch per step")

    def zero1_step(i):
        for k, (a, o) in enumerate(sets[i % 2]):
            lo, n = k * E, plan.bucket_len(k)
            ddp.zero1_sgd_step(a, w[lo:lo + n], v[lo:lo + n], 1e-3, 0.9, o, "mean", P)
    report("vitb16 p8 bf16 mean, ZeRO stage 1 step (owner sgd-momentum, bf16 parameters to every rank)",
           _time(zero1_step, steps, warmup), P * plan.total * 4 + 16 * plan.total)
    report("vitb16 p8 bf16 mean, ZeRO stage 1 step, all buckets in one bucketed call",
           _time(lambda i: ddp.zero1_sgd_step(rows[i % 2][0], w, v, 1e-3, 0.9, rows[i % 2][1], "mean", P,
                                              bucket_elems=E), steps, warmup),
           P * plan.total * 4 + 16 * plan.total, note="every bucket its own ring, the same bits; 1 launch per step")
    del sets, rows, w, v
    torch.cuda.empty_cache()

    # 2,000 ragged fp32 tensors, P=4, Sum, 25 MiB buckets
    P4 = 4
    sizes = workloads.ragged_sizes()
    shapes4 = [(n,) for n in sizes]
    plan = ddp.GradBucketer(shapes4, torch.float32, 25 << 20, device=dev)
    tensors = [[torch.empty(n, device=dev).uniform_(-1, 1) for n in sizes] for _ in range(P4)]
    table = plan.pointer_table(tensors)
    bufs = plan.alloc_buckets(P4)
    nbytes4 = P4 * plan.total * 8

    def ragged_step(i):
        for k in range(plan.n_buckets):
            n = plan.bucket_len(k)
            plan.pack(table, k, bufs)
            ddp.allreduce([x[:n] for x in bufs], "sum", P4, out=[x[:n] for x in bufs])
            plan.unpack(table, k, bufs)
    ms = _time(ragged_step, max(2, steps // 20), 1)
    report(f"ragged {len(sizes)} tensors p4 f32 sum, pack -> all-reduce -> unpack "
           f"({plan.n_buckets} buckets)", ms, nbytes4,
           with_copies_gbps=round(3 * nbytes4 / (ms * 1e-3) / 1e9, 1),
           note="gbps counts the all-reduce bytes; with_copies_gbps adds pack and unpack traffic")
    report(f"ragged {len(sizes)} tensors p4 f32, pack alone ({plan.n_buckets} buckets, all ranks)",
           _time(lambda i: [plan.pack(table, k, bufs) for k in range(plan.n_buckets)], max(2, steps // 20), 1),
           P4 * plan.total * 8)
    report(f"ragged {len(sizes)} tensors p4 f32, unpack alone ({plan.n_buckets} buckets, all ranks)",
           _time(lambda i: [plan.unpack(table, k, bufs) for k in range(plan.n_buckets)], max(2, steps // 20), 1),
           P4 * plan.total * 8)
    arena = plan.alloc_arena(P4)
    E4 = plan.bucket_elems
    slots = [[arena[r, k * E4:k * E4 + plan.bucket_len(k)] for r in range(P4)] for k in range(plan.n_buckets)]
    flat = [arena[r, :plan.total] for r in range(P4)]

    def ragged_bucketed(i):
        for k in range(plan.n_buckets):
            plan.pack(table, k, slots[k])
        ddp.allreduce(flat, "sum", P4, out=flat, bucket_elems=E4)
        for k in range(plan.n_buckets):
            plan.unpack(table, k, slots[k])
    ms = _time(ragged_bucketed, max(2, steps // 20), 1)
    report(f"ragged {len(sizes)} tensors p4 f32 sum, pack every bucket -> one bucketed "
           f"all-reduce -> unpack", ms, nbytes4,
           with_copies_gbps=round(3 * nbytes4 / (ms * 1e-3) / 1e9, 1),
           note="gbps counts the all-reduce bytes; with_copies_gbps adds pack and unpack traffic")
    del arena, slots, flat
    run = ddp.MultiAllReduce(shapes4, P4, torch.float32, device=dev).bind(tensors, tensors)
    report(f"ragged {len(sizes)} tensors p4 f32 sum, one multi-tensor launch, in place",
           _time(lambda i: run("sum"), max(2, steps // 20), 1), nbytes4)
    del tensors, table, bufs, run
    torch.cuda.empty_cache()

    # 2B-parameter transformer, P=8, bf16 in, fp32 out, 100 MiB buckets
    plan = ddp.GradBucketer(workloads.model_shapes("transformer_2b"), torch.bfloat16, 100 << 20,
                            device=dev)
    g = plan.alloc_arena(P)
    for r in range(P):
        workloads.torch_normal_(g[r], 1e-4, seed=500 + r)
    o = plan.alloc_arena(P, torch.float32)
    E = plan.bucket_elems
    views = [([plan.bucket_view(g[r], k) for r in range(P)],
              [o[r, k * E:k * E + plan.bucket_len(k)] for r in range(P)]) for k in range(plan.n_buckets)]
    report(f"transformer-2b p8 bf16 -> f32 mean ({plan.n_buckets} x 100 MiB buckets)",
           _time(lambda i: [ddp.allreduce(a, "mean", P, out=b) for a, b in views], 3, 1),
           P * plan.total * 6)
    report(f"transformer-2b p8 bf16 -> f32 mean ({plan.n_buckets} x 100 MiB buckets), one bucketed call",
           _time(lambda i: ddp.allreduce([g[r, :plan.total] for r in range(P)], "mean", P,
                                         out=[o[r, :plan.total] for r in range(P)],
                                         bucket_elems=E), 3, 1),
           P * plan.total * 6, note="every bucket its own ring, the same bits")
    del g, o, views
    torch.cuda.empty_cache()
    return 0


def run_occupancy_sweep(caps=(2, 3, 4, 5, 6, 8, 10, 12, 16)):
    """Time the fused all-reduce and the fused optimizer step at every cap on
    resident workgroups per CU (ddp_set_wg_per_cu), for each rank count and
    element-type pair, on four 25 MiB buckets per rank (two buffer sets);
    one JSON line per case with the rate at every cap and the built-in
    choice's rate.  The tables of launch.h hold the fastest cap per case."""
    import torch

    import gradient_all_reduce_allreduce_amd as ddp

    dev = torch.device("cuda:0")

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


def one_call_per_bucket(timed, bucket_calls, lens, P, bytes_step, steps):
    """Timed region 2: the step's buckets with one single-bucket call (one
    launch) each; region 3: the same with an event pair around every launch
    (on the stream it runs on; the pairs add about 2 us each) for each
    bucket's median and minimum."""
    import numpy as np
    import torch
    ms_calls = timed(bucket_calls)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in lens] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        bucket_calls(i, ev[i])
    torch.cuda.synchronize()
    durs = [[ev[i][k][0].elapsed_time(ev[i][k][1]) for k in range(len(lens))] for i in range(steps)]
    per_bucket = []
    for k, n in enumerate(lens):
        col = sorted(row[k] for row in durs)
        med = float(np.median(col))
        per_bucket.append({"elements": n, "median_us": round(med * 1e3, 2),
                           "min_us": round(col[0] * 1e3, 2),
                           "median_gbs": round(P * n * 8 / (med * 1e-3) / 1e9, 1)})
    per_set = sorted(map(sum, durs))
    gbs = bytes_step / (ms_calls * 1e-3) / 1e9
    return {
        "ms_per_step": round(ms_calls, 4),
        "value": round(gbs, 1),
        "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "avg_launch_us": round(ms_calls / len(lens) * 1e3, 2),
        "per_bucket": per_bucket,
        "per_set_median_ms": round(float(np.median(per_set)), 4),
        "per_set_min_ms": round(per_set[0], 4),
        "note": "the same buckets, one allreduce_ring_emulated call (one launch) each; per_bucket "
                "from an event pair around every launch, which adds about 2 us",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the headline line, time every entry point at the shape "
                         "of its workload (one JSON line each)")
    ap.add_argument("--occupancy-sweep", action="store_true",
                    help="time the fused all-reduce and optimizer step at every cap on resident "
                         "workgroups per CU (the measurements behind the built-in caps)")
    ap.add_argument("--per-bucket", action="store_true",
                    help="also time the same buckets with one single-bucket call each (adds the "
                         "one_call_per_bucket object; its launches have another shape, so a "
                         "profiler's average over the run no longer describes the step's launch)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 10 times (a kernel of known "
                         "traffic, to scale the memory counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the P ranks are emulated as P buffers in one "
              f"GPU's HBM; --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gradient_all_reduce_allreduce_amd as ddp
    import workloads

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
        return run_suite(args.steps, args.warmup)
    if args.occupancy_sweep:
        return run_occupancy_sweep()

    cfg = workloads.CONFIGS["p8-resnet50-f32-mean-25MiB"]
    P, C = cfg["P"], cfg["chunking"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shapes = workloads.model_shapes("resnet50")
    plan = ddp.GradBucketer(shapes, torch.float32, cfg["bucket_bytes"], device=dev)
    E = plan.bucket_elems
    lens = [plan.bucket_len(k) for k in range(plan.n_buckets)]

    # Two buffer sets of inputs and outputs, each an arena of P rows padded
    # to whole buckets (grads as bucket views: bucket k of rank r is
    # row r, elements [k*E, k*E + len_k)).
    sets = []
    for s in range(2):
        g = plan.alloc_arena(P)
        for r in range(P):
            workloads.torch_normal_(g[r], cfg["dist"][1], seed=1000 * s + r)
        sets.append((g, plan.alloc_arena(P)))
    views = []
    for g, o in sets:
        views.append([([plan.bucket_view(g[r], k) for r in range(P)],
                       [plan.bucket_view(o[r], k) for r in range(P)], n)
                      for k, n in enumerate(lens)])
    rows = [([g[r, :plan.total] for r in range(P)], [o[r, :plan.total] for r in range(P)])
            for g, o in sets]

    stream = torch.cuda.current_stream(dev)

    def step(i):
        """The step: every bucket in one bucketed call, each bucket its own
        ring (bit for bit the one-call-per-bucket result)."""
        ins, outs = rows[i % 2]
        ddp.allreduce(ins, "mean", C, out=outs, bucket_elems=E)

    def bucket_calls(i, events=None):
        """The same buckets, one single-bucket call each."""
        for k, (ins, outs, n) in enumerate(views[i % 2]):
            if events is not None:
                events[k][0].record(stream)
            ddp.allreduce(ins, "mean", C, out=outs)
            if events is not None:
                events[k][1].record(stream)

    for i in range(args.warmup):
        step(i)
        if args.per_bucket:
            bucket_calls(i)
    torch.cuda.synchronize()

    def timed(fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(args.steps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    # Timed region 1: the step throughput, K steps bracketed by events.
    ms_step = timed(step)
    bytes_step = sum(P * n * (4 + 4) for n in lens)
    value = bytes_step / (ms_step * 1e-3) / 1e9

    # The step is nothing but launches of the dominant kernel, back to back
    # on one stream, so region 1 also gives that kernel's average launch
    # duration: step time / launches per step.
    launches_per_step = ddp.ddp_buckets_launch_count(P, C, ddp.F32, ddp.F32, False, plan.total, E)
    avg_ms = ms_step / launches_per_step
    avg_bytes = bytes_step / launches_per_step
    achieved = avg_bytes / (avg_ms * 1e-3) / 1e9

    # Per-step spread: the same K steps again with an event pair around
    # each (the pairs add about 2 us per step); the same launches only.
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(pairs):
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)

    traffic = measured_traffic(int(avg_bytes))
    one_call = None
    if args.per_bucket:
        one_call = one_call_per_bucket(timed, bucket_calls, lens, P, bytes_step, args.steps)

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
            "workload": "resnet50-gradient-set all-reduce: P=8 ranks x 161 fp32 tensors "
                        "(25,557,032 params) N(0,0.01), 25 MiB buckets (3 full + tail of "
                        "5,896,232), grads as bucket views of a per-rank arena padded to "
                        "whole buckets + 4 KiB, Mean, 8 ring chunks; one bucketed call per step "
                        "(every bucket its own ring; one launch: the 3 full buckets as one "
                        "ring, the tail bucket as a second segment with its own chunks)",
            "P": P, "chunking": C, "op": "mean", "bucket_bytes": cfg["bucket_bytes"],
            "buckets": len(lens), "elements_per_rank": plan.total,
            "bytes_per_step": bytes_step,
        },
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "ring_reduce_kernel<P=8, f32 -> f32>",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_ms * 1e3, 2),
            "launches_per_step": launches_per_step,
            "algorithmic_bytes_per_launch": int(avg_bytes),
            "timing": "events around the timed steps, which hold only this kernel's launches",
        },
        "per_step": {
            "median_ms": round(float(np.median(step_ms)), 4),
            "min_ms": round(step_ms[0], 4),
            "max_ms": round(step_ms[-1], 4),
            "note": "an event pair around every step (about 2 us each), a second pass of K steps",
        },
        "one_call_per_bucket": one_call,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        g = sets[0][0]
        host = [np.ascontiguousarray(g[:, k * E:k * E + n].cpu().numpy()) for k, n in enumerate(lens)]
        del sets, views, rows
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(host, lens, P, C)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
