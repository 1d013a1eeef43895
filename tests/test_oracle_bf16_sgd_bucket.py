"""Pins for the oracle's bf16 conversion, SGD-momentum step and bucketing."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

# ---------------------------------------------------------------- bf16 ----

HAND_CASES = [
    (0x3F800000, 0x3F80),   # 1.0 exact
    (0x3F808000, 0x3F80),   # tie, lower neighbour even
    (0x3F818000, 0x3F82),   # tie, lower neighbour odd -> up
    (0x3F808001, 0x3F81),   # just above the tie
    (0x3F807FFF, 0x3F80),   # just below the tie
    (0xBF818000, 0xBF82),   # negative tie rounds away from zero to even
    (0x7F7F7FFF, 0x7F7F),   # below the largest finite bf16's upper half-ulp
    (0x7F7F8000, 0x7F80),   # tie at the top: overflow to +inf
    (0x7F7FFFFF, 0x7F80),   # float32 max -> +inf
    (0xFF7FFFFF, 0xFF80),   # -float32 max -> -inf
    (0x80000000, 0x8000),   # -0
    (0x00000000, 0x0000),   # +0
    (0x00000001, 0x0000),   # smallest subnormal rounds to 0
    (0x00008000, 0x0000),   # subnormal tie, lower even
    (0x00018000, 0x0002),   # subnormal tie, lower odd
    (0x00010000, 0x0001),   # smallest bf16 subnormal, exact
    (0x7F800000, 0x7F80),   # +inf
    (0xFF800000, 0xFF80),   # -inf
    (0x7FC00000, 0x7FC0),   # quiet NaN
    (0x7F800001, 0x7FC0),   # signalling NaN with payload only in the low half
    (0xFF800001, 0xFFC0),   # negative signalling NaN
    (0x7F812345, 0x7FC1),   # NaN payload kept in the upper half, quiet bit set
]


def test_bf16_hand_cases():
    src = np.array([c[0] for c in HAND_CASES], np.uint32).view(np.float32)
    want = np.array([c[1] for c in HAND_CASES], np.uint16)
    got = oracle.f32_to_bf16_bits(src)
    for (s, w), g in zip(HAND_CASES, got):
        assert int(g) == w, (hex(s), hex(int(g)), hex(w))


def test_bf16_widening_is_a_shift():
    b = np.arange(0, 1 << 16, 7, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(b)
    assert np.array_equal(f.view(np.uint32), b.astype(np.uint32) << 16)


def test_bf16_matches_exact_nearest_on_random_patterns():
    """Exact rational check: the result is a nearest bf16 and, on a tie,
    the one with the even significand."""
    rng = np.random.default_rng(0)
    u = rng.integers(0, 0x7F800000, size=3000, dtype=np.uint32)
    u |= (rng.integers(0, 2, size=3000, dtype=np.uint32) << 31)
    x = u.view(np.float32)
    got = oracle.f32_to_bf16_bits(x)
    for xi, gi in zip(x, got):
        q = Fraction(float(xi))
        y = Fraction(float(oracle.bf16_bits_to_f32(np.array([gi]))[0]))
        for d in (-1, 1):
            nb_bits = np.array([int(gi) + d], np.int64)
            if nb_bits[0] < 0 or (nb_bits[0] & 0x7FFF) >= 0x7F80:
                continue
            nb = Fraction(float(oracle.bf16_bits_to_f32(nb_bits.astype(np.uint16))[0]))
            if (int(gi) & 0x8000) != (int(nb_bits[0]) & 0x8000):
                continue
            assert abs(y - q) <= abs(nb - q)
            if abs(y - q) == abs(nb - q):
                assert int(gi) & 1 == 0


def test_bf16_matches_torch_conversion():
    """torch's float32 -> bfloat16 conversion rounds to nearest even; on
    finite inputs the two agree bit for bit."""
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    mine = oracle.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, theirs)


# ----------------------------------------------------------------- SGD ----

def test_sgd_from_zero_momentum():
    g = workloads.rank_buffers(1, 1000, "normal", 1e-3, seed=1)[0]
    w = workloads.rank_buffers(1, 1000, "normal", 0.02, seed=2)[0]
    v = np.zeros(1000, np.float32)
    w1, v1 = oracle.sgd_momentum(g, w, v, 1e-3, 0.9)
    assert np.array_equal(v1, g)
    assert np.array_equal(w1, w - np.float32(1e-3) * g)


def test_sgd_mu_zero_is_plain_sgd():
    g = workloads.rank_buffers(1, 100, "normal", 1.0, seed=3)[0]
    w = workloads.rank_buffers(1, 100, "normal", 1.0, seed=4)[0]
    v = workloads.rank_buffers(1, 100, "normal", 1.0, seed=5)[0]
    w1, v1 = oracle.sgd_momentum(g, w, v, 0.5, 0.0)
    assert np.array_equal(v1, g)
    assert np.array_equal(w1, w - np.float32(0.5) * g)


def test_sgd_exact_closed_form():
    """lr = 2^-10, mu = 2^-1, integer gradients: every operation is exact, so
    k steps equal v_k = sum_j mu^(k-j) g_j and w_k = w_0 - lr sum_i v_i."""
    rng = np.random.default_rng(6)
    steps = 6
    G = rng.integers(-64, 65, size=(steps, 50)).astype(np.float32)
    w = rng.integers(-16, 17, size=50).astype(np.float32)
    v = np.zeros(50, np.float32)
    lr, mu = Fraction(1, 1024), Fraction(1, 2)
    wk, vk = w.copy(), v.copy()
    for k in range(steps):
        wk, vk = oracle.sgd_momentum(G[k], wk, vk, float(lr), float(mu))
    for i in range(50):
        vs = Fraction(0)
        ws = Fraction(float(w[i]))
        for k in range(steps):
            vs = mu * vs + Fraction(float(G[k, i]))
            ws = ws - lr * vs
        assert Fraction(float(vk[i])) == vs
        assert Fraction(float(wk[i])) == ws


def test_sgd_rounds_every_operation_once():
    """No multiply-add contraction (each product is rounded before the add):
    two hand-worked cases where a fused multiply-add would give another
    value.

    Momentum: mu = float32(0.9) = 15099494 * 2^-24 and v = 3.  The exact
    product 45298482 * 2^-24 = 11324620.5 * 2^-22 (a float32 in [2, 4) is a
    multiple of 2^-22) lies halfway between two floats; ties-to-even gives
    11324620 * 2^-22.  With g = -11324620 * 2^-22 the new momentum is 0
    exactly (fused: 2^-23), and the weight is unchanged.

    Weights: lr = float32(0.1) = 13421773 * 2^-27, v_new = 3 (from v = 0,
    g = 3).  The exact product 40265319 * 2^-27 = 10066329.75 * 2^-25 (a
    float32 in [1/4, 1/2) is a multiple of 2^-25) rounds to 10066330 * 2^-25.
    With w = 10066330 * 2^-25 the new weight is 0 exactly (fused: 2^-27)."""
    mu32, lr32 = np.float32(0.9), np.float32(0.1)
    assert int(mu32.view(np.uint32)) == 0x3F000000 | (15099494 - (1 << 23))
    assert int(lr32.view(np.uint32)) == (123 << 23) | (13421773 - (1 << 23))
    g = np.array([-11324620 * 2.0 ** -22, 3.0], np.float32)
    w = np.array([0.5, 10066330 * 2.0 ** -25], np.float32)
    v = np.array([3.0, 0.0], np.float32)
    w1, v1 = oracle.sgd_momentum(g, w, v, 0.1, 0.9)
    assert v1[0] == 0.0 and w1[0] == 0.5
    assert v1[1] == 3.0 and w1[1] == 0.0


def test_sgd_constant_gradient_geometric_series():
    g = np.full(10, 0.25, np.float32)
    w = np.zeros(10, np.float32)
    v = np.zeros(10, np.float32)
    mu, k = 0.9, 40
    for _ in range(k):
        w, v = oracle.sgd_momentum(g, w, v, 1e-3, mu)
    want = 0.25 * (1 - mu ** k) / (1 - mu)
    assert np.allclose(v, want, rtol=k * 2 ** -23 * 4)


def test_sgd_matches_torch_optim_sgd_float64():
    """torch.optim.SGD(momentum=mu) in float64 follows the same formula; the
    float32 oracle stays within float32 rounding of it."""
    rng = np.random.default_rng(7)
    n, steps = 500, 5
    w0 = rng.standard_normal(n).astype(np.float32) * 0.02
    G = (rng.standard_normal((steps, n)) * 1e-3).astype(np.float32)
    p = torch.nn.Parameter(torch.from_numpy(w0.astype(np.float64)))
    opt = torch.optim.SGD([p], lr=1e-3, momentum=0.9)
    w, v = w0.copy(), np.zeros(n, np.float32)
    for k in range(steps):
        p.grad = torch.from_numpy(G[k].astype(np.float64))
        opt.step()
        w, v = oracle.sgd_momentum(G[k], w, v, 1e-3, 0.9)
    ref = p.detach().numpy()
    assert np.max(np.abs(w - ref)) <= 4 * steps * 2 ** -24 * np.max(np.abs(ref))
    buf = opt.state[p]["momentum_buffer"].numpy()
    assert np.allclose(v, buf, rtol=1e-5, atol=1e-9)


# ------------------------------------------------------------- buckets ----

def test_pack_unpack_identity():
    shapes = [(3, 5), (7,), (0,), (4, 4, 2), (1,), (33,)]
    rng = np.random.default_rng(0)
    tensors = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    for bucket_bytes in (16, 32, 64, 400, 1 << 20):
        buckets = oracle.pack(tensors, 4, bucket_bytes)
        back = oracle.unpack(buckets, shapes)
        for a, b in zip(tensors, back):
            assert a.shape == b.shape and np.array_equal(a, b)


def test_plan_agrees_with_pack():
    shapes = [(3, 5), (7,), (0,), (4, 4, 2), (1,), (33,)]
    numels = [int(np.prod(s)) for s in shapes]
    rng = np.random.default_rng(1)
    tensors = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    for bucket_bytes in (16, 48, 64, 400):
        segs, lengths = oracle.bucket_plan(numels, 4, bucket_bytes)
        buckets = oracle.pack(tensors, 4, bucket_bytes)
        assert [b.size for b in buckets] == lengths
        covered = [np.zeros(L, np.int64) for L in lengths]
        for (t, b, src, dst, ln) in segs:
            assert ln > 0
            flat = tensors[t].reshape(-1)
            assert np.array_equal(buckets[b][dst:dst + ln], flat[src:src + ln])
            covered[b][dst:dst + ln] += 1
        assert all(np.all(c == 1) for c in covered)
        keys = [(b, dst) for (_, b, _, dst, _) in segs]
        assert keys == sorted(keys)
        E = bucket_bytes // 4
        assert all(L == E for L in lengths[:-1]) and 0 < lengths[-1] <= E


def test_bucket_counts_resnet50_vit_transformer(golden_dir):
    cases = [
        (workloads.resnet50_shapes(), 4, 25 << 20, 161, 25_557_032, 3, 5_896_232),
        (workloads.vit_b16_shapes(), 2, 25 << 20, 152, 86_567_656, 6, 7_924_456),
        (workloads.transformer_2b_shapes(), 2, 100 << 20, 292, 2_017_529_856,
         38, 25_235_456),
    ]
    for shapes, eb, bb, count, total, full, tail in cases:
        numels = [workloads.numel(s) for s in shapes]
        assert len(shapes) == count and sum(numels) == total
        segs, lengths = oracle.bucket_plan(numels, eb, bb)
        assert lengths[:-1] == [bb // eb] * full and lengths[-1] == tail
        assert sum(s[4] for s in segs) == total
        # reverse order: the first segment is the last tensor
        assert segs[0][0] == count - 1 and segs[-1][0] == 0


def test_vit_count_matches_pages_closed_form(golden_dir):
    """The pages count ViT-B/16 two ways (a meta-device model and a closed
    form) and print 86,567,656 for both."""
    with open(os.path.join(golden_dir, "pages_printed.json")) as f:
        printed = json.load(f)["vit_b16_parameters"]["count"]
    D, L, MLP, Pt, C, T = 768, 12, 3072, 16, 1000, 197
    block = 2 * 2 * D + (3 * D * D + 3 * D) + (D * D + D) + (D * MLP + MLP) + (MLP * D + D)
    closed = (3 * Pt * Pt * D + D) + D + T * D + L * block + 2 * D + (D * C + C)
    assert closed == printed
    assert sum(workloads.numel(s) for s in workloads.vit_b16_shapes()) == printed


def test_vit_shapes_match_torch_module_order():
    """The ViT-B/16 of the pages, built on the meta device: same shapes in
    the same registration order as the synthetic gradient set."""
    nn = torch.nn
    D, L, MLP, Pt, C, T = 768, 12, 3072, 16, 1000, 197

    class ViT(nn.Module):
        def __init__(self):
            super().__init__()
            self.patch = nn.Conv2d(3, D, Pt, stride=Pt)
            self.cls = nn.Parameter(torch.zeros(1, 1, D))
            self.pos = nn.Parameter(torch.zeros(1, T, D))
            self.blocks = nn.ModuleList(
                nn.TransformerEncoderLayer(D, 12, MLP, norm_first=True, batch_first=True)
                for _ in range(L))
            self.norm, self.head = nn.LayerNorm(D), nn.Linear(D, C)

    with torch.device("meta"):
        vit = ViT()
    assert [tuple(p.shape) for p in vit.parameters()] == workloads.vit_b16_shapes()
