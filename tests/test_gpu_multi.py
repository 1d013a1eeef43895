"""GPU parity of the multi-tensor (small-message) all-reduce: every tensor
bit for bit the oracle's ring on that tensor alone, including tiny tensors
whose chunks are shorter than a tile, tensors not 16-byte aligned, the
partial last tile, bf16; and the lecture's per-parameter DDP step on a tiny
MLP."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from gpu_helpers import DEV, assert_same_bits, oracle_ring

pytestmark = pytest.mark.gpu
ddp = pytest.importorskip("gradient_all_reduce_allreduce_amd")


def bits_of(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    return t.cpu().numpy().reshape(-1)


def make(P, shapes, dtype, seed, misalign=0):
    rng = np.random.default_rng(seed)
    host, dev = [], []
    for r in range(P):
        hs, ds = [], []
        for s in shapes:
            n = int(np.prod(s, dtype=np.int64))
            x = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 21, n))).astype(np.float32)
            if dtype == torch.bfloat16:
                x = workloads.to_bf16_bits(x)
                src = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
            else:
                src = torch.from_numpy(x).to(DEV)
            store = torch.empty(n + misalign, dtype=dtype, device=DEV)
            t = store[misalign:misalign + n].view(s)
            t.copy_(src.view(s))
            hs.append(x)
            ds.append(t)
        host.append(hs)
        dev.append(ds)
    return host, dev


@pytest.mark.parametrize("pair", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("P", [1, 3, 8, 16])
@pytest.mark.parametrize("misalign", [0, 1])
def test_multi_equals_oracle_per_tensor(pair, P, misalign):
    it, ot = pair
    tdt = torch.bfloat16 if it == "bf16" else torch.float32
    odt = torch.bfloat16 if ot == "bf16" else torch.float32
    shapes = [(1,), (7,), (64,), (3, 5), (1000,), (4096,), (4097,), (33, 129), (70001,), (0,)]
    host, dev = make(P, shapes, tdt, seed=P + misalign, misalign=misalign)
    m = ddp.MultiAllReduce(shapes, P, tdt, odt, device=DEV)
    for C in (P, 2 * P + 1):
        for op in ("sum", "mean"):
            out = m(dev, op, C)
            torch.cuda.synchronize()
            for t, s in enumerate(shapes):
                X = np.stack([host[r][t] for r in range(P)])
                if X.shape[1] == 0:
                    continue
                want = oracle_ring(X, op, C, in_dtype=it, out_dtype=ot)
                got = np.stack([bits_of(out[r][t]) for r in range(P)])
                assert_same_bits(got, want, f"{it}->{ot} P={P} t={t} C={C} {op}")


def test_launcher_run_on_another_stream():
    """A launcher bound on one stream and run on another, then dropped while
    the launch may still be in flight: its tables are recorded on the stream
    that reads them, so new allocations cannot take their memory early."""
    P, C = 4, 4
    shapes = [(7,), (4097,), (70001,)]
    host, dev = make(P, shapes, torch.float32, seed=17)
    run = ddp.MultiAllReduce(shapes, P, torch.float32, device=DEV).bind(dev)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        out = run("sum", C)
    del run
    junk = [torch.full((1 << 16,), 7.0, device=DEV) for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    for t in range(len(shapes)):
        want = oracle_ring(np.stack([host[r][t] for r in range(P)]), "sum", C)
        got = np.stack([bits_of(out[r][t]) for r in range(P)])
        assert_same_bits(got, want, f"t={t}")
    del junk


def test_multi_in_place_equals_single_calls():
    P = 8
    shapes = workloads.resnet50_shapes()
    _, dev = make(P, shapes, torch.float32, seed=5)
    single = [ddp.allreduce([dev[r][t].reshape(-1) for r in range(P)], "mean", P)
              for t in range(len(shapes))]
    m = ddp.MultiAllReduce(shapes, P, torch.float32, device=DEV)
    m(dev, "mean", P, out=dev)
    torch.cuda.synchronize()
    for t in range(len(shapes)):
        for r in range(P):
            assert torch.equal(dev[r][t].reshape(-1).view(torch.int32),
                               single[t][r].view(torch.int32)), (t, r)


def test_per_parameter_ddp_step_on_a_tiny_mlp():
    """CS336 Lecture 8, "Data Parallelism (DDP)": each rank computes the
    gradient of its shard, every param.grad is all-reduced with AVG, and the
    ranks hold the full-batch gradient."""
    W = 4
    torch.manual_seed(0)
    net = torch.nn.Sequential(torch.nn.Linear(16, 32), torch.nn.Tanh(), torch.nn.Linear(32, 3))
    g = torch.Generator().manual_seed(1)
    X = torch.randn(32, 16, generator=g)
    y = torch.randint(0, 3, (32,), generator=g)

    def grads(xb, yb):
        net.zero_grad()
        F.cross_entropy(net(xb), yb).backward()
        return [p.grad.detach().clone() for p in net.parameters()]

    full = grads(X, y)
    shard = [grads(X[r::W], y[r::W]) for r in range(W)]
    shapes = [tuple(p.shape) for p in net.parameters()]
    m = ddp.MultiAllReduce(shapes, W, torch.float32, device=DEV)
    dev = [[t.to(DEV) for t in shard[r]] for r in range(W)]
    out = m(dev, "mean", W)
    torch.cuda.synchronize()
    for t, s in enumerate(shapes):
        Xs = np.stack([shard[r][t].numpy().reshape(-1) for r in range(W)])
        want, _ = oracle.ring_allreduce(Xs, "mean", W)
        for r in range(W):
            assert_same_bits(out[r][t].cpu().numpy().reshape(-1), want[r], f"param {t}")
        d = np.linalg.norm(out[0][t].cpu().numpy() - full[t].numpy()) / np.linalg.norm(full[t].numpy())
        assert d < 1e-5


# ------------------------------------------------- fused optimizer step ----

def sgd_state(shapes, seed, misalign=0):
    """Per tensor float32 master weights and momentum (host copies and
    device tensors, optionally misaligned views)."""
    rng = np.random.default_rng(seed)
    host, dev = [], []
    for s in shapes:
        n = int(np.prod(s, dtype=np.int64))
        pair_h, pair_d = [], []
        for scale in (0.02, 1e-3):
            x = (rng.standard_normal(n) * scale).astype(np.float32)
            store = torch.empty(n + misalign, dtype=torch.float32, device=DEV)
            t = store[misalign:misalign + n].view(s)
            t.copy_(torch.from_numpy(x).view(s))
            pair_h.append(x)
            pair_d.append(t)
        host.append(pair_h)
        dev.append(pair_d)
    return host, dev


@pytest.mark.parametrize("pair", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("P", [1, 3, 8])
@pytest.mark.parametrize("misalign", [0, 1])
@pytest.mark.parametrize("with_out", [False, True])
def test_multi_fused_sgd_equals_oracle_per_tensor(pair, P, misalign, with_out):
    """Every tensor: the oracle's ring on that tensor alone, then its
    momentum step, bit for bit; the reduced gradients when asked for."""
    it, ot = pair
    tdt = torch.bfloat16 if it == "bf16" else torch.float32
    odt = torch.bfloat16 if ot == "bf16" else torch.float32
    shapes = [(1,), (7,), (64,), (3, 5), (1000,), (4096,), (4097,), (33, 129), (70001,), (0,)]
    host, dev = make(P, shapes, tdt, seed=10 * P + misalign, misalign=misalign)
    sh, sd = sgd_state(shapes, seed=P, misalign=misalign)
    m = ddp.MultiAllReduce(shapes, P, tdt, odt, device=DEV)
    out = [[torch.empty(s, dtype=odt, device=DEV) for s in shapes] for _ in range(P)] if with_out else None
    run = m.bind_sgd(dev, [p[0] for p in sd], [p[1] for p in sd], out=out)
    C = 2 * P + 1
    run(1e-3, 0.9, "mean", C)
    torch.cuda.synchronize()
    for t, s in enumerate(shapes):
        X = np.stack([host[r][t] for r in range(P)])
        if X.shape[1] == 0:
            continue
        g = oracle_ring(X, "mean", C, in_dtype=it, out_dtype="f32")[0]
        w1, v1 = oracle.sgd_momentum(g, sh[t][0], sh[t][1], 1e-3, 0.9)
        what = f"{it}->{ot} P={P} t={t} misalign={misalign}"
        assert_same_bits(sd[t][0].cpu().numpy().reshape(1, -1), w1[None], what + " w")
        assert_same_bits(sd[t][1].cpu().numpy().reshape(1, -1), v1[None], what + " v")
        if with_out:
            want = oracle_ring(X, "mean", C, in_dtype=it, out_dtype=ot)
            got = np.stack([bits_of(out[r][t]) for r in range(P)])
            assert_same_bits(got, want, what + " grads")


def test_multi_fused_sgd_equals_bucketed_fused_sgd():
    """The per-parameter fused step on 161 ResNet-50 tensors updates the
    weights exactly as the single-tensor fused step does per tensor."""
    P = 8
    shapes = workloads.resnet50_shapes()
    _, dev = make(P, shapes, torch.float32, seed=6)
    _, sd = sgd_state(shapes, seed=7)
    ref = [(p[0].clone(), p[1].clone()) for p in sd]
    m = ddp.MultiAllReduce(shapes, P, torch.float32, device=DEV)
    m.bind_sgd(dev, [p[0] for p in sd], [p[1] for p in sd])(1e-3, 0.9, "mean", P)
    for t in range(len(shapes)):
        ddp.allreduce_sgd([dev[r][t].reshape(-1) for r in range(P)], ref[t][0].reshape(-1),
                          ref[t][1].reshape(-1), 1e-3, 0.9, "mean", P)
    torch.cuda.synchronize()
    for t in range(len(shapes)):
        assert torch.equal(sd[t][0].view(torch.int32), ref[t][0].view(torch.int32)), t
        assert torch.equal(sd[t][1].view(torch.int32), ref[t][1].view(torch.int32)), t


def test_per_parameter_ddp_training_steps_on_a_tiny_mlp():
    """The lecture's DDP loop, every step on the GPU in one launch: each rank
    computes its shard's gradients, all of them are all-reduced with AVG and
    each replica's SGD-momentum step follows.  Over three steps the weights
    track single-device training on the full batch (float32 round-off) and
    match the oracle's ring + step bit for bit."""
    W = 4
    torch.manual_seed(0)
    net = torch.nn.Sequential(torch.nn.Linear(16, 32), torch.nn.Tanh(), torch.nn.Linear(32, 3))
    ref = torch.nn.Sequential(torch.nn.Linear(16, 32), torch.nn.Tanh(), torch.nn.Linear(32, 3))
    ref.load_state_dict(net.state_dict())
    opt = torch.optim.SGD(ref.parameters(), lr=0.1, momentum=0.9)
    g = torch.Generator().manual_seed(1)
    shapes = [tuple(p.shape) for p in net.parameters()]
    w_dev = [p.detach().to(DEV).contiguous() for p in net.parameters()]
    v_dev = [torch.zeros_like(p) for p in w_dev]
    w_host = [p.detach().numpy().reshape(-1).copy() for p in net.parameters()]
    v_host = [np.zeros_like(x) for x in w_host]
    m = ddp.MultiAllReduce(shapes, W, torch.float32, device=DEV)
    for step in range(3):
        X = torch.randn(32, 16, generator=g)
        y = torch.randint(0, 3, (32,), generator=g)
        shard = []
        for r in range(W):
            with torch.no_grad():
                for p, wd in zip(net.parameters(), w_dev):
                    p.copy_(wd.cpu())
            net.zero_grad()
            F.cross_entropy(net(X[r::W]), y[r::W]).backward()
            shard.append([p.grad.detach().clone() for p in net.parameters()])
        dev = [[t.to(DEV) for t in shard[r]] for r in range(W)]
        m.bind_sgd(dev, w_dev, v_dev)(0.1, 0.9, "mean", W)
        torch.cuda.synchronize()
        for t in range(len(shapes)):
            Xs = np.stack([shard[r][t].numpy().reshape(-1) for r in range(W)])
            gm, _ = oracle.ring_allreduce(Xs, "mean", W)
            w_host[t], v_host[t] = oracle.sgd_momentum(gm[0], w_host[t], v_host[t], 0.1, 0.9)
            assert_same_bits(w_dev[t].cpu().numpy().reshape(1, -1), w_host[t][None], f"step {step} w{t}")
        opt.zero_grad()
        F.cross_entropy(ref(X), y).backward()
        opt.step()
    for p, wd in zip(ref.parameters(), w_dev):
        d = (np.linalg.norm(wd.cpu().numpy() - p.detach().numpy()) /
             np.linalg.norm(p.detach().numpy()))
        assert d < 1e-5, d


def _many_block_shapes(seed, T=600):
    """Tensors of sizes around the tile and chunk edges (and empty ones), so
    that the plan's tiles span many 64-tile blocks whose first tile lies
    inside a tensor, at a tensor's start, or on an empty tensor."""
    rng = np.random.default_rng(seed)
    sizes = rng.choice([0, 1, 7, 255, 256, 257, 2047, 2048, 2049, 16384, 70001], size=T)
    return [(int(n),) for n in sizes]


@pytest.mark.parametrize("pair,P", [(("f32", "f32"), 8), (("bf16", "f32"), 8), (("f32", "f32"), 5),
                                    (("bf16", "bf16"), 7), (("f32", "bf16"), 2)])
def test_block_map_search_equals_whole_plan_search_and_oracle(pair, P):
    """With the block map each workgroup starts its search in its block's
    tensor (and, up to P = 8, reads ahead the tables of the tensor 768 tiles
    on); the results are bit for bit those of the whole-plan search, and
    every tensor is the oracle's ring on that tensor alone."""
    it, ot = pair
    tdt = torch.bfloat16 if it == "bf16" else torch.float32
    odt = torch.bfloat16 if ot == "bf16" else torch.float32
    C = P
    shapes = _many_block_shapes(21)
    host, dev = make(P, shapes, tdt, seed=22)
    fast = ddp.MultiAllReduce(shapes, P, tdt, odt, device=DEV)
    plain = ddp.MultiAllReduce(shapes, P, tdt, odt, device=DEV, block_map=False)
    assert fast.total_tiles > 768 + 64 * 20 and fast.block_map.size == -(-fast.total_tiles // 64)
    a = fast(dev, "mean", C)
    b = plain(dev, "mean", C)
    torch.cuda.synchronize()
    for t, s in enumerate(shapes):
        for r in range(P):
            assert np.array_equal(bits_of(a[r][t]), bits_of(b[r][t])), (t, r)
        X = np.stack([host[r][t] for r in range(P)])
        if X.shape[1] == 0:
            continue
        want = oracle_ring(X, "mean", C, in_dtype=it, out_dtype=ot)
        got = np.stack([bits_of(a[r][t]) for r in range(P)])
        assert_same_bits(got, want, f"{it}->{ot} t={t} n={s[0]}")


def test_block_map_fused_sgd_equals_whole_plan_search():
    P = 8
    shapes = _many_block_shapes(23, T=400)
    _, dev = make(P, shapes, torch.float32, seed=24)
    _, sd1 = sgd_state(shapes, seed=25)
    _, sd2 = sgd_state(shapes, seed=25)
    ddp.MultiAllReduce(shapes, P, torch.float32, device=DEV).bind_sgd(
        dev, [p[0] for p in sd1], [p[1] for p in sd1])(1e-3, 0.9, "mean", P)
    ddp.MultiAllReduce(shapes, P, torch.float32, device=DEV, block_map=False).bind_sgd(
        dev, [p[0] for p in sd2], [p[1] for p in sd2])(1e-3, 0.9, "mean", P)
    torch.cuda.synchronize()
    for t in range(len(shapes)):
        assert torch.equal(sd1[t][0].view(torch.int32), sd2[t][0].view(torch.int32)), t
        assert torch.equal(sd1[t][1].view(torch.int32), sd2[t][1].view(torch.int32)), t


def test_multi_fused_sgd_on_vit_bf16_equals_single_tensor_fused_sgd():
    """The per-parameter fused step on the 152 ViT-B/16 bf16 gradient tensors
    (P = 8, Mean, bf16 gradients written back too) gives, tensor by tensor,
    the bits of the single-tensor fused step: weights, momentum and the
    reduced bf16 gradients."""
    P = 8
    shapes = workloads.vit_b16_shapes()
    g = torch.Generator(device=DEV).manual_seed(31)
    dev = [[torch.empty(s, device=DEV).normal_(0, 1e-3, generator=g).to(torch.bfloat16) for s in shapes]
           for _ in range(P)]
    sd = [(torch.empty(s, device=DEV).normal_(0, 0.02, generator=g),
           torch.empty(s, device=DEV).normal_(0, 1e-3, generator=g)) for s in shapes]
    ref = [(p[0].clone(), p[1].clone()) for p in sd]
    out = [[torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes] for _ in range(P)]
    m = ddp.MultiAllReduce(shapes, P, torch.bfloat16, device=DEV)
    m.bind_sgd(dev, [p[0] for p in sd], [p[1] for p in sd], out=out)(1e-3, 0.9, "mean", P)
    ref_out = []
    for t in range(len(shapes)):
        o = [torch.empty(shapes[t], dtype=torch.bfloat16, device=DEV).reshape(-1) for _ in range(P)]
        ddp.allreduce_sgd([dev[r][t].reshape(-1) for r in range(P)], ref[t][0].reshape(-1),
                          ref[t][1].reshape(-1), 1e-3, 0.9, "mean", P, out=o)
        ref_out.append(o)
    torch.cuda.synchronize()
    for t in range(len(shapes)):
        assert torch.equal(sd[t][0].view(torch.int32), ref[t][0].view(torch.int32)), t
        assert torch.equal(sd[t][1].view(torch.int32), ref[t][1].view(torch.int32)), t
        for r in range(P):
            assert torch.equal(out[r][t].reshape(-1).view(torch.int16), ref_out[t][r].view(torch.int16)), (t, r)


@pytest.mark.parametrize("pair,sgd", [(("f32", "f32"), False), (("bf16", "f32"), False), (("f32", "f32"), True),
                                      (("bf16", "bf16"), False)])
def test_tensors_as_views_off_lines_equal_oracle(pair, sgd):
    """Tensors that are views of one buffer per rank, at 16-byte but mostly
    not 128-byte boundaries (rows of equal stride, as gradients as bucket
    views lie): the plan gives them short first tiles so that whole tiles
    sit on lines.  Every tensor is still the oracle's ring on that tensor
    alone (with its momentum step when fused), bit for bit."""
    it, ot = pair
    tdt = torch.bfloat16 if it == "bf16" else torch.float32
    odt = torch.bfloat16 if ot == "bf16" else torch.float32
    P = 8
    rng = np.random.default_rng(41)
    numels = [int(n) * 8 for n in rng.choice([1, 3, 40, 129, 1000, 8191], size=120)]
    offs, o = [], 8
    for n in numels:
        offs.append(o)
        o += n
    stride = -(-o // 64) * 64 + 1024
    shapes = [(n,) for n in numels]
    host = []
    base_in = torch.empty(P * stride, dtype=tdt, device=DEV)
    base_out = torch.empty(P * stride, dtype=odt, device=DEV)
    views_in, views_out = [], []
    for r in range(P):
        x = (rng.standard_normal(o) * np.exp2(rng.integers(-10, 11, o))).astype(np.float32)
        if tdt == torch.bfloat16:
            x = workloads.to_bf16_bits(x)
            base_in[r * stride:r * stride + o].copy_(torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16))
        else:
            base_in[r * stride:r * stride + o].copy_(torch.from_numpy(x).to(DEV))
        host.append(x)
        views_in.append([base_in[r * stride + a:r * stride + a + n] for a, n in zip(offs, numels)])
        views_out.append([base_out[r * stride + a:r * stride + a + n] for a, n in zip(offs, numels)])
    m = ddp.MultiAllReduce(shapes, P, tdt, odt, device=DEV)
    addrs = [views_in[0][t].data_ptr() for t in m.plan_order]
    tiles, total, _ = ddp.ddp_multi_plan([numels[t] for t in m.plan_order], P, ddp.api.torch_dtype_code(tdt),
                                         ddp.api.torch_dtype_code(odt), align_to=addrs)
    assert (tiles["lead"] > 0).sum() > 60 and total > m.total_tiles
    C = P
    if not sgd:
        m.bind(views_in, views_out)("mean", C)
    else:
        sh, sd = sgd_state(shapes, seed=42)
        m.bind_sgd(views_in, [p[0] for p in sd], [p[1] for p in sd], out=views_out)(1e-3, 0.9, "mean", C)
    torch.cuda.synchronize()
    for t, (a, n) in enumerate(zip(offs, numels)):
        X = np.stack([host[r][a:a + n] for r in range(P)])
        want = oracle_ring(X, "mean", C, in_dtype=it, out_dtype=ot)
        got = np.stack([bits_of(views_out[r][t]) for r in range(P)])
        assert_same_bits(got, want, f"{it}->{ot} t={t} n={n} off={a}")
        if sgd:
            g = oracle_ring(X, "mean", C, in_dtype=it, out_dtype="f32")[0]
            w1, v1 = oracle.sgd_momentum(g, sh[t][0], sh[t][1], 1e-3, 0.9)
            assert_same_bits(sd[t][0].cpu().numpy().reshape(1, -1), w1[None], f"t={t} w")
            assert_same_bits(sd[t][1].cpu().numpy().reshape(1, -1), v1[None], f"t={t} v")
