// ring_reduce_impl.h -- device code of the emulated ring all-reduce for
// CDNA4 (gfx950).  Included by the ring_reduce_*.hip translation units, each
// of which instantiates one (input type, output type) pair so that the
// kernels compile in parallel.
//
// P rank buffers of n elements sit in HBM.  For every element the kernel
// performs the additions a ring all-reduce over P devices performs -- the
// reduce-scatter carries the partial sum of a chunk from its start rank s
// through s+1, ..., s+P-1 (Burn collective blog, "Methods", Ring;
// "Distributed Training", "Sharded data parallelism": a ring all-reduce is
// a reduce-scatter followed by an all-gather) -- then applies Mean (Burn
// distributed guide, ReduceOperation), optionally one SGD-momentum step on
// float32 master weights (CS336 Lecture 8, "Data Parallelism (DDP)";
// "Distributed Training", "Mixed-Precision Training"), and writes the
// result to every rank (the all-gather).
//
// The work is bound by HBM bandwidth: per element it reads P inputs, writes
// P outputs and does P-1 float32 additions.  The design follows from that:
//   * each workgroup of 256 lanes owns one contiguous, balanced share of the
//     buffer and the grid equals the device's resident capacity, so every
//     workgroup streams concurrently and all finish together;
//   * each lane loads U 16-byte vectors from each of the P ranks per tile
//     (P*U loads in flight) with non-temporal hints, folds them in registers
//     and stores 16-byte vectors non-temporally: the data is touched once,
//     so nothing is staged in LDS and no cache lines are kept;
//   * addresses are a per-rank base in SGPRs plus one 32-bit lane offset
//     shared by all ranks (the host splits buffers over 2^29 elements into
//     several launches), which keeps VGPRs for data;
//   * the reduce-scatter start rank is uniform over a tile except where a
//     chunk boundary falls inside it; chunks are at least a tile long on
//     this path, so such a tile holds two start ranks and is folded in both
//     orders, selecting per element.  Chunks shorter than a tile go to a
//     one-element-per-lane kernel;
//   * bf16 inputs are widened exactly (a shift) inside the fold, float32
//     accumulation throughout, no FMA contraction, subnormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ddp {
namespace rr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;

struct RingArgs {
    const void* in[kMaxRanks];   // already offset to this launch's first element
    void* out[kMaxRanks];
    float* w;
    float* v;
    float lr;
    float mu;
    int64_t base;        // global index of this launch's first element
    int64_t L;           // chunk length ceil(n_total / C)
    uint32_t n;          // elements in this launch (< 2^29)
    uint32_t n_vec;      // elements covered by whole 16-byte input vectors
    uint32_t per_block;  // elements per workgroup, a multiple of 256 * V
    int32_t mean;
    int32_t write_out;
};

__device__ __forceinline__ u32x4 load16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store8(void* p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

// Element e of a 16-byte vector as float32.  A bf16 value is the upper half
// of a float32, so widening is exact; element 2k sits in the low half of
// word k.
template <bool BF16>
__device__ __forceinline__ float elem(const u32x4& x, int e) {
    if constexpr (BF16) {
        const uint32_t w = x[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
        return __uint_as_float(x[e]);
    }
}

// float32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet bit
// forced) so that rounding cannot turn it into infinity.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Mean: one division by P, correctly rounded.  For P a power of two the
// product with 2^-k is the exact quotient rounded once, i.e. the same value.
// Otherwise the quotient is taken in double and rounded to float: rounding a
// quotient of two floats first to 53 and then to 24 bits gives the correctly
// rounded result because 53 >= 2 * 24 + 2 (Figueroa, "When is double
// rounding innocuous?", SIGNUM Newsletter 30(3), 1995).
template <int P>
__device__ __forceinline__ float mean_of(float s) {
    if constexpr ((P & (P - 1)) == 0) {
        return s * (1.0f / static_cast<float>(P));
    } else {
        return static_cast<float>(static_cast<double>(s) / static_cast<double>(P));
    }
}

__device__ __forceinline__ void momentum_step(float g, float& w, float& v, float lr, float mu) {
#pragma clang fp contract(off)
    float vn = mu * v;
    vn = vn + g;
    const float step = lr * vn;
    w = w - step;
    v = vn;
}

// ---- the fold: ((x_S + x_{S+1}) + ...) + x_{S+P-1}, rank indices mod P ---

template <int P, int S, bool BF16, int U, int V>
__device__ __forceinline__ void fold_from(const u32x4 (&x)[P][U], float (&acc)[U][V]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float s = elem<BF16>(x[S][u], e);
#pragma unroll
            for (int k = 1; k < P; ++k) s = s + elem<BF16>(x[(S + k) % P][u], e);
            acc[u][e] = s;
        }
    }
}

// s is uniform across the workgroup: a chain of scalar branches.
template <int P, int S, bool BF16, int U, int V>
__device__ __forceinline__ void fold_uniform(int s, const u32x4 (&x)[P][U], float (&acc)[U][V]) {
    if constexpr (S + 1 < P) {
        if (s == S) {
            fold_from<P, S, BF16, U, V>(x, acc);
        } else {
            fold_uniform<P, S + 1, BF16, U, V>(s, x, acc);
        }
    } else {
        fold_from<P, S, BF16, U, V>(x, acc);
    }
}

template <int P, int S>
__device__ __forceinline__ float fold_scalar_from(const float (&xs)[P]) {
#pragma clang fp contract(off)
    float s = xs[S];
#pragma unroll
    for (int k = 1; k < P; ++k) s = s + xs[(S + k) % P];
    return s;
}

// s may differ between lanes.
template <int P, int S>
__device__ __forceinline__ float fold_scalar(int s, const float (&xs)[P]) {
    if constexpr (S + 1 < P) {
        if (s == S) return fold_scalar_from<P, S>(xs);
        return fold_scalar<P, S + 1>(s, xs);
    } else {
        return fold_scalar_from<P, S>(xs);
    }
}

// ---- one element per lane: tails and chunks shorter than a tile ----------

template <int P, bool INB, bool OUTB, bool SGD>
__device__ __forceinline__ void process_element(const RingArgs a, uint32_t i) {
#pragma clang fp contract(off)
    float xs[P];
#pragma unroll
    for (int r = 0; r < P; ++r) {
        if constexpr (INB) {
            const uint16_t h = static_cast<const uint16_t*>(a.in[r])[i];
            xs[r] = __uint_as_float(static_cast<uint32_t>(h) << 16);
        } else {
            xs[r] = static_cast<const float*>(a.in[r])[i];
        }
    }
    const int s = static_cast<int>(((a.base + i) / a.L) % P);
    float g = fold_scalar<P, 0>(s, xs);
    if (a.mean) g = mean_of<P>(g);
    if constexpr (SGD) {
        float w = a.w[i];
        float v = a.v[i];
        momentum_step(g, w, v, a.lr, a.mu);
        a.w[i] = w;
        a.v[i] = v;
        if (!a.write_out) return;
    }
#pragma unroll
    for (int r = 0; r < P; ++r) {
        if constexpr (OUTB) {
            static_cast<uint16_t*>(a.out[r])[i] = static_cast<uint16_t>(bf16_bits(g));
        } else {
            static_cast<float*>(a.out[r])[i] = g;
        }
    }
}

// ---- the vector path ------------------------------------------------------

// One tile: U rows of 256 16-byte vectors per rank.  FULL: every vector of
// the tile lies below blk_end (no per-vector predicate).
template <int P, bool INB, bool OUTB, bool SGD, int U, bool FULL>
__device__ __forceinline__ void process_tile(const RingArgs a, uint32_t t0, uint32_t blk_end) {
#pragma clang fp contract(off)
    constexpr int V = INB ? 8 : 4;        // elements per 16-byte input vector
    constexpr uint32_t IES = INB ? 2 : 4; // input element bytes
    constexpr uint32_t OES = OUTB ? 2 : 4;
    constexpr uint32_t TILE = static_cast<uint32_t>(kBlock) * U * V;
    const uint32_t tid = threadIdx.x;

    u32x4 x[P][U];
    float ws[U][V];
    float vs[U][V];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
        ok[u] = FULL || (i0 < blk_end);
        if (ok[u]) {
#pragma unroll
            for (int r = 0; r < P; ++r) x[r][u] = load16(static_cast<const char*>(a.in[r]) + i0 * IES);
            if constexpr (SGD) {
#pragma unroll
                for (int q = 0; q < V / 4; ++q) {
                    const u32x4 wq = load16(reinterpret_cast<const char*>(a.w) + (i0 + 4 * q) * 4u);
                    const u32x4 vq = load16(reinterpret_cast<const char*>(a.v) + (i0 + 4 * q) * 4u);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ws[u][4 * q + e] = __uint_as_float(wq[e]);
                        vs[u][4 * q + e] = __uint_as_float(vq[e]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < P; ++r) x[r][u] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // Chunks are at least TILE long here, so the tile holds one start rank,
    // or two with the boundary at element `split` of the launch.
    float acc[U][V];
    const uint32_t last = FULL ? t0 + TILE - 1 : ((t0 + TILE < blk_end ? t0 + TILE : blk_end) - 1);
    const int64_t j0 = (a.base + t0) / a.L;
    const int64_t j1 = (a.base + last) / a.L;
    fold_uniform<P, 0, INB, U, V>(static_cast<int>(j0 % P), x, acc);
    if (j1 != j0) {
        float acc2[U][V];
        fold_uniform<P, 0, INB, U, V>(static_cast<int>(j1 % P), x, acc2);
        const uint32_t split = static_cast<uint32_t>(j1 * a.L - a.base);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i0 = t0 + (u * kBlock + tid) * V;
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (i0 + e >= split) acc[u][e] = acc2[u][e];
        }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
        float g[V];
#pragma unroll
        for (int e = 0; e < V; ++e) g[e] = a.mean ? mean_of<P>(acc[u][e]) : acc[u][e];
        if constexpr (SGD) {
#pragma unroll
            for (int e = 0; e < V; ++e) momentum_step(g[e], ws[u][e], vs[u][e], a.lr, a.mu);
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                u32x4 wq, vq;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wq[e] = __float_as_uint(ws[u][4 * q + e]);
                    vq[e] = __float_as_uint(vs[u][4 * q + e]);
                }
                store16(reinterpret_cast<char*>(a.w) + (i0 + 4 * q) * 4u, wq);
                store16(reinterpret_cast<char*>(a.v) + (i0 + 4 * q) * 4u, vq);
            }
            if (!a.write_out) continue;
        }
        if constexpr (OUTB) {
            if constexpr (V == 8) {
                u32x4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = bf16_bits(g[2 * k]) | (bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
                for (int r = 0; r < P; ++r) store16(static_cast<char*>(a.out[r]) + i0 * OES, o);
            } else {
                u32x2 o;
#pragma unroll
                for (int k = 0; k < 2; ++k) o[k] = bf16_bits(g[2 * k]) | (bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
                for (int r = 0; r < P; ++r) store8(static_cast<char*>(a.out[r]) + i0 * OES, o);
            }
        } else {
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(g[4 * q + e]);
#pragma unroll
                for (int r = 0; r < P; ++r) store16(static_cast<char*>(a.out[r]) + (i0 + 4 * q) * OES, o);
            }
        }
    }
}

template <int P, bool INB, bool OUTB, bool SGD>
__global__ __launch_bounds__(kBlock) void ring_reduce_kernel(RingArgs a) {
    constexpr int U = ring_vectors_per_lane(P);
    constexpr int V = INB ? 8 : 4;
    constexpr uint32_t TILE = static_cast<uint32_t>(kBlock) * U * V;
    const uint32_t begin = blockIdx.x * a.per_block;
    const uint32_t end = begin + a.per_block < a.n_vec ? begin + a.per_block : a.n_vec;
    uint32_t t0 = begin;
    for (; t0 + TILE <= end; t0 += TILE) process_tile<P, INB, OUTB, SGD, U, true>(a, t0, end);
    if (t0 < end) process_tile<P, INB, OUTB, SGD, U, false>(a, t0, end);
    if (blockIdx.x == gridDim.x - 1) {
        const uint32_t i = a.n_vec + threadIdx.x;
        if (i < a.n) process_element<P, INB, OUTB, SGD>(a, i);
    }
}

// Chunks shorter than a tile (C large against n): one element per lane.
template <int P, bool INB, bool OUTB, bool SGD>
__global__ __launch_bounds__(kBlock) void ring_reduce_scalar_kernel(RingArgs a) {
    for (uint32_t i = blockIdx.x * kBlock + threadIdx.x; i < a.n; i += gridDim.x * kBlock)
        process_element<P, INB, OUTB, SGD>(a, i);
}

template <bool INB, bool OUTB, bool SGD, bool SCALAR>
const void* ring_kernel_for(int P) {
    switch (P) {
#define DDP_CASE(p)                                                                              \
    case p:                                                                                      \
        return SCALAR ? reinterpret_cast<const void*>(&ring_reduce_scalar_kernel<p, INB, OUTB, SGD>) \
                      : reinterpret_cast<const void*>(&ring_reduce_kernel<p, INB, OUTB, SGD>);
        DDP_CASE(1) DDP_CASE(2) DDP_CASE(3) DDP_CASE(4)
        DDP_CASE(5) DDP_CASE(6) DDP_CASE(7) DDP_CASE(8)
        DDP_CASE(9) DDP_CASE(10) DDP_CASE(11) DDP_CASE(12)
        DDP_CASE(13) DDP_CASE(14) DDP_CASE(15) DDP_CASE(16)
#undef DDP_CASE
        default:
            return nullptr;
    }
}

}  // namespace rr
}  // namespace ddp

// Defines ddp::ring_kernel_<name>(P, sgd, scalar) for one type pair.
#define DDP_RING_TYPE_PAIR(name, INB, OUTB)                                              \
    namespace ddp {                                                                      \
    const void* ring_kernel_##name(int P, int sgd, int scalar) {                         \
        if (sgd) return scalar ? rr::ring_kernel_for<INB, OUTB, true, true>(P)           \
                               : rr::ring_kernel_for<INB, OUTB, true, false>(P);         \
        return scalar ? rr::ring_kernel_for<INB, OUTB, false, true>(P)                   \
                      : rr::ring_kernel_for<INB, OUTB, false, false>(P);                 \
    }                                                                                    \
    }
