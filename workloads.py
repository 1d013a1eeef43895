"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds shapes and random draws only -- none of the all-reduce's
arithmetic -- so that the oracle and the HIP path can be fed identical inputs
without sharing any code of the method.

Gradient sets stand in for the models the pages train (ResNet-50, ViT-B/16,
a large transformer); only the parameter *shapes* are taken from the
architectures, values are i.i.d. draws.  No dataset or trained weight is
used.
"""

import math

import numpy as np

MiB = 1 << 20


# --------------------------------------------------------------------------
# Parameter shapes, in the order a PyTorch module registers its parameters.
# --------------------------------------------------------------------------

def resnet50_shapes():
    """ResNet-50: 7x7 stem, bottleneck stages [3, 4, 6, 3] of widths
    64/128/256/512 with 4x expansion, 1x1 projection in each stage's first
    block, convolutions without bias, batch norm weight + bias, fc 2048->1000
    with bias.  161 tensors, 25,557,032 parameters."""
    shapes = [(64, 3, 7, 7), (64,), (64,)]
    inp = 64
    for width, blocks in zip((64, 128, 256, 512), (3, 4, 6, 3)):
        for b in range(blocks):
            out = 4 * width
            shapes += [(width, inp, 1, 1), (width,), (width,),
                       (width, width, 3, 3), (width,), (width,),
                       (out, width, 1, 1), (out,), (out,)]
            if b == 0:
                shapes += [(out, inp, 1, 1), (out,), (out,)]
            inp = out
    shapes += [(1000, 2048), (1000,)]
    return shapes


def vit_b16_shapes(D=768, layers=12, mlp=3072, patch=16, classes=1000,
                   tokens=197):
    """ViT-B/16 as built in "Distributed Training", "How to Apply It", part 3:
    class token and position embedding (a module's own parameters come
    first), patch conv with bias, 12 pre-norm
    encoder layers (fused qkv projection with bias, output projection, two
    MLP linears, two layer norms), final layer norm, linear head.
    152 tensors, 86,567,656 parameters."""
    shapes = [(1, 1, D), (1, tokens, D), (D, 3, patch, patch), (D,)]
    for _ in range(layers):
        shapes += [(3 * D, D), (3 * D,), (D, D), (D,),
                   (mlp, D), (mlp,), (D, mlp), (D,),
                   (D,), (D,), (D,), (D,)]
    shapes += [(D,), (D,), (classes, D), (classes,)]
    return shapes


def transformer_2b_shapes(d=2048, layers=24, ffn=14336, vocab=50000):
    """Dense decoder: untied token embedding and output head (vocab x d),
    24 pre-norm blocks (fused qkv with bias, output projection with bias, MLP
    d -> ffn -> d with biases, two layer norms), final layer norm.
    292 tensors, 2,017,529,856 parameters with ffn = 7d."""
    shapes = [(vocab, d)]
    for _ in range(layers):
        shapes += [(d,), (d,), (3 * d, d), (3 * d,), (d, d), (d,),
                   (d,), (d,), (ffn, d), (ffn,), (d, ffn), (d,)]
    shapes += [(d,), (d,), (vocab, d)]
    return shapes


def ragged_sizes(count=2000, lo=1e3, hi=4e6, seed=0):
    """Tensor sizes log-uniform in [lo, hi]: round(exp(U(ln lo, ln hi)))."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(lo), math.log(hi), size=count)
    return [int(v) for v in np.rint(np.exp(u)).astype(np.int64)]


def numel(shape):
    return int(np.prod(shape, dtype=np.int64))


# --------------------------------------------------------------------------
# Value draws.
# --------------------------------------------------------------------------

def rank_buffers(P, n, dist="normal", scale=1.0, seed=0, dtype=np.float32):
    """(P, n) array, rank-major, from numpy's default_rng(seed).

    dist "normal": N(0, scale) with scale the standard deviation;
    dist "uniform": U[-scale, scale]; dist "int": integers in
    [-scale, scale] stored as floats."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((P, n)) * scale
    elif dist == "uniform":
        x = rng.uniform(-scale, scale, size=(P, n))
    elif dist == "int":
        x = rng.integers(-int(scale), int(scale) + 1, size=(P, n))
    elif dist == "wide":
        # normal mantissas over a wide exponent range: makes the order of
        # additions visible in the low bits
        x = rng.standard_normal((P, n)) * np.exp2(
            rng.integers(-20, 21, size=(P, n)))
    else:
        raise ValueError(dist)
    return x.astype(dtype)


def to_bf16_bits(x):
    """float32 array -> bfloat16 bit patterns via torch's own conversion
    (round to nearest even), used only to draw bf16 inputs."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_normal_(t, std, seed):
    """Fill a torch tensor (any device, float dtype) with N(0, std) from a
    generator seeded with ``seed`` on that tensor's device."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    if t.dtype in (torch.float32, torch.float64):
        t.normal_(0.0, std, generator=g)
    else:
        tmp = torch.empty(t.shape, dtype=torch.float32, device=t.device)
        tmp.normal_(0.0, std, generator=g)
        t.copy_(tmp)
    return t


def torch_uniform_(t, lo, hi, seed):
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    t.uniform_(lo, hi, generator=g)
    return t


# --------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------

CONFIGS = {
    "p4-65536-f32-sum": dict(name="p4-65536-f32-sum", P=4, shapes=[(65536,)], dtype="f32",
                 out_dtype="f32", op="sum", chunking=4, bucket_bytes=None,
                 dist=("normal", 1.0), sgd=None),
    "p8-resnet50-f32-mean-25MiB": dict(name="p8-resnet50-f32-mean-25MiB", P=8, shapes=None,
                 model="resnet50", dtype="f32", out_dtype="f32", op="mean",
                 chunking=8, bucket_bytes=25 * MiB, dist=("normal", 0.01),
                 sgd=None),
    "p8-vitb16-bf16-mean-sgd-25MiB": dict(name="p8-vitb16-bf16-mean-sgd-25MiB", P=8, shapes=None,
                 model="vit_b16", dtype="bf16", out_dtype="bf16", op="mean",
                 chunking=8, bucket_bytes=25 * MiB, dist=("normal", 1e-3),
                 sgd=dict(lr=1e-3, mu=0.9, w_std=0.02, v_std=1e-3)),
    "p4-ragged2000-f32-sum-25MiB": dict(name="p4-ragged2000-f32-sum-25MiB", P=4, shapes=None,
                 model="ragged", dtype="f32", out_dtype="f32", op="sum",
                 chunking=4, bucket_bytes=25 * MiB, dist=("uniform", 1.0),
                 sgd=None),
    "p8-transformer2b-bf16-mean-f32out-100MiB": dict(name="p8-transformer2b-bf16-mean-f32out-100MiB", P=8,
                 shapes=None, model="transformer_2b", dtype="bf16",
                 out_dtype="f32", op="mean", chunking=8,
                 bucket_bytes=100 * MiB, dist=("normal", 1e-4), sgd=None),
}


def model_shapes(model):
    if model == "resnet50":
        return resnet50_shapes()
    if model == "vit_b16":
        return vit_b16_shapes()
    if model == "transformer_2b":
        return transformer_2b_shapes()
    if model == "ragged":
        return [(s,) for s in ragged_sizes()]
    raise ValueError(model)
