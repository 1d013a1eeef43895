// multi_tensor.hip -- many independent all-reduces in one launch, for
// gfx950: the small-message path.
//
// Without buckets, data-parallel training all-reduces every parameter's
// gradient on its own (CS336 Lecture 8, "Data Parallelism (DDP)": one
// all-reduce per param.grad); collectives on small tensors are inefficient,
// which is why DDP packs buckets ("Distributed Training", "Data parallelism
// and all-reduce", "Communication costs").  Here T tensors of P ranks are
// all-reduced by one launch: tensor t is its own ring all-reduce, with its
// own chunk length ceil(numel_t / C), exactly as if it were passed alone to
// allreduce_ring_emulated.  The host plan gives every tensor a run of tiles;
// a workgroup finds its tensor by a binary search over the plan (uniform,
// scalar loads) and then works like the single-tensor kernel: rotated rank
// pointers, one fixed fold, P output stores.  Optionally every tensor then
// takes one SGD-momentum step on its float32 master weights and momentum,
// as each replica's optimizer.step() does after the per-parameter
// all-reduces (same lecture section), with or without writing the reduced
// gradients.  Tiles of small tensors, tiles
// across a chunk boundary and tensors (or optimizer state) not 16-byte
// aligned take a per-element path whose rank pointers are read per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "ring_reduce_impl.h"

namespace ddp {
namespace {

using rr::kBlock;
using rr::u32x2;
using rr::u32x4;

struct MultiArgs {
    const ddp_tensor_tiles* tiles;   // [T], device
    const void* const* in;           // [P * T] device, rank-major
    void* const* out;                // [P * T] device, rank-major; null: no output
    float* const* w;                 // SGD: [T] device, master weights
    float* const* v;                 // SGD: [T] device, momentum
    float lr;
    float mu;
    int32_t T;
    int32_t chunking;
    int32_t mean;
};

typedef const __attribute__((address_space(4))) MultiArgs* KMulti;

__device__ __forceinline__ KMulti multi_args() {
    return (KMulti)(__builtin_amdgcn_kernarg_segment_ptr());
}

template <int P, bool INB, bool OUTB, bool SGD>
__device__ __forceinline__ void multi_element(KMulti a, int t, uint32_t i, uint32_t L) {
#pragma clang fp contract(off)
    const int T = a->T;
    const int s = static_cast<int>((i / L) % P);
    float g;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const void* p = a->in[static_cast<int64_t>(rr::rank_at(s, k, P)) * T + t];
        float xk;
        if constexpr (INB) {
            xk = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
        } else {
            xk = static_cast<const float*>(p)[i];
        }
        g = k == 0 ? xk : g + xk;
    }
    if (a->mean) g = rr::mean_of<P>(g);
    if constexpr (SGD) {
        float* wp = a->w[t];
        float* vp = a->v[t];
        float w = wp[i];
        float v = vp[i];
        rr::momentum_step(g, w, v, a->lr, a->mu);
        wp[i] = w;
        vp[i] = v;
        if (a->out == nullptr) return;
    }
#pragma unroll
    for (int r = 0; r < P; ++r) {
        void* o = a->out[static_cast<int64_t>(r) * T + t];
        if constexpr (OUTB) {
            static_cast<uint16_t*>(o)[i] = static_cast<uint16_t>(rr::bf16_bits(g));
        } else {
            static_cast<float*>(o)[i] = g;
        }
    }
}

template <int P, bool INB, bool OUTB, bool SGD>
__global__ __launch_bounds__(kBlock) void multi_ring_kernel(MultiArgs) {
#pragma clang fp contract(off)
    constexpr int U = ring_vectors_per_lane(P, false);
    constexpr int V = ring_lane_elems(INB, OUTB, false);
    constexpr uint32_t IES = INB ? 2 : 4;
    constexpr uint32_t OES = OUTB ? 2 : 4;
    constexpr int WIN = V * IES / 4;
    constexpr uint32_t TILE = static_cast<uint32_t>(kBlock) * U * V;
    const KMulti a = multi_args();
    const int T = a->T;
    const int64_t b = blockIdx.x;

    // The tensor whose tile run holds this workgroup: largest t with
    // first_tile <= b.
    int lo = 0;
    int hi = T - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a->tiles[mid].first_tile <= b) lo = mid; else hi = mid - 1;
    }
    const int t = lo;
    const int64_t numel = a->tiles[t].numel;
    const uint32_t t0 = static_cast<uint32_t>((b - a->tiles[t].first_tile) * TILE);
    if (static_cast<int64_t>(t0) >= numel) return;
    const uint32_t n = static_cast<uint32_t>(numel);
    // Tensors hold at most 2^29 elements (ddp_multi_plan), so the chunk
    // arithmetic fits 32 bits (a 64-bit division is a long sequence).
    const uint32_t L = static_cast<uint32_t>((numel + a->chunking - 1) / a->chunking);
    const uint32_t end = t0 + TILE < n ? t0 + TILE : n;
    const uint32_t j0 = t0 / L;
    const uint32_t j1 = (end - 1) / L;
    const uint32_t tid = threadIdx.x;

    const bool write_out = !SGD || a->out != nullptr;
    bool vector_path = j0 == j1 && end - t0 == TILE;
    uintptr_t align = 0;
#pragma unroll
    for (int r = 0; r < P; ++r) {
        align |= reinterpret_cast<uintptr_t>(a->in[static_cast<int64_t>(r) * T + t]);
        if (write_out) align |= reinterpret_cast<uintptr_t>(a->out[static_cast<int64_t>(r) * T + t]);
    }
    if constexpr (SGD) align |= reinterpret_cast<uintptr_t>(a->w[t]) | reinterpret_cast<uintptr_t>(a->v[t]);
    vector_path = vector_path && (align & 15u) == 0;

    if (!vector_path) {
        for (uint32_t i = t0 + tid; i < end; i += kBlock) multi_element<P, INB, OUTB, SGD>(a, t, i, L);
        return;
    }

    const int s0 = static_cast<int>(j0 % P);
    u32x4 x[P][U];
    constexpr int WV = SGD ? V / 4 : 1;   // 16-byte state vectors per lane vector
    u32x4 wq[U][WV];
    u32x4 vq[U][WV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const char* p = static_cast<const char*>(a->in[static_cast<int64_t>(rr::rank_at(s0, k, P)) * T + t]);
            x[k][u] = rr::load_lane<WIN>(p + i0 * IES);
        }
        if constexpr (SGD) {
#pragma unroll
            for (int q = 0; q < WV; ++q) {
                wq[u][q] = rr::load16(reinterpret_cast<const char*>(a->w[t]) + (i0 + 4 * q) * 4u);
                vq[u][q] = rr::load16(reinterpret_cast<const char*>(a->v[t]) + (i0 + 4 * q) * 4u);
            }
        }
    }
    float acc[U][V];
    rr::fold<P, 0, INB, U, V>(x, acc);
    const bool mean = a->mean != 0;
    const int rot = rr::store_rotation(P);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
        float g[V];
#pragma unroll
        for (int e = 0; e < V; ++e) g[e] = mean ? rr::mean_of<P>(acc[u][e]) : acc[u][e];
        if constexpr (SGD) {
#pragma unroll
            for (int q = 0; q < WV; ++q) {
                u32x4 wn, vn;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float w = __uint_as_float(wq[u][q][e]);
                    float v = __uint_as_float(vq[u][q][e]);
                    rr::momentum_step(g[4 * q + e], w, v, a->lr, a->mu);
                    wn[e] = __float_as_uint(w);
                    vn[e] = __float_as_uint(v);
                }
                rr::store16(a->w[t], n * 4u, (i0 + 4 * q) * 4u, wn);
                rr::store16(a->v[t], n * 4u, (i0 + 4 * q) * 4u, vn);
            }
            if (!write_out) continue;
        }
        if constexpr (OUTB && V == 8) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = rr::bf16_bits(g[2 * k]) | (rr::bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
            for (int q = 0; q < P; ++q)
                rr::store16(a->out[static_cast<int64_t>(rr::rank_at(rot, q, P)) * T + t], n * OES, i0 * OES, o);
        } else if constexpr (OUTB) {
            u32x2 o;
#pragma unroll
            for (int k = 0; k < 2; ++k) o[k] = rr::bf16_bits(g[2 * k]) | (rr::bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
            for (int q = 0; q < P; ++q)
                rr::store8(a->out[static_cast<int64_t>(rr::rank_at(rot, q, P)) * T + t], n * OES, i0 * OES, o);
        } else {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(g[e]);
#pragma unroll
            for (int q = 0; q < P; ++q)
                rr::store16(a->out[static_cast<int64_t>(rr::rank_at(rot, q, P)) * T + t], n * OES, i0 * OES, o);
        }
    }
}

template <bool INB, bool OUTB, bool SGD>
const void* multi_kernel_for(int P) {
    switch (P) {
#define DDP_CASE(p) \
    case p: return reinterpret_cast<const void*>(&multi_ring_kernel<p, INB, OUTB, SGD>);
        DDP_CASE(1) DDP_CASE(2) DDP_CASE(3) DDP_CASE(4)
        DDP_CASE(5) DDP_CASE(6) DDP_CASE(7) DDP_CASE(8)
        DDP_CASE(9) DDP_CASE(10) DDP_CASE(11) DDP_CASE(12)
        DDP_CASE(13) DDP_CASE(14) DDP_CASE(15) DDP_CASE(16)
#undef DDP_CASE
        default:
            return nullptr;
    }
}

}  // namespace

int64_t multi_tile_elems(int P, bool in_bf16, bool out_bf16) {
    return static_cast<int64_t>(kBlock) * ring_vectors_per_lane(P, false) * ring_lane_elems(in_bf16, out_bf16, false);
}

int launch_multi_ring(const MultiLaunch& l, const char** msg) {
    if (l.total_tiles <= 0) return 0;
    const void* fn;
    if (l.sgd) {
        fn = l.in_bf16 ? (l.out_bf16 ? multi_kernel_for<true, true, true>(l.P) : multi_kernel_for<true, false, true>(l.P))
                       : (l.out_bf16 ? multi_kernel_for<false, true, true>(l.P)
                                     : multi_kernel_for<false, false, true>(l.P));
    } else {
        fn = l.in_bf16 ? (l.out_bf16 ? multi_kernel_for<true, true, false>(l.P)
                                     : multi_kernel_for<true, false, false>(l.P))
                       : (l.out_bf16 ? multi_kernel_for<false, true, false>(l.P)
                                     : multi_kernel_for<false, false, false>(l.P));
    }
    if (fn == nullptr) {
        *msg = "no multi-tensor kernel for this rank count";
        return static_cast<int>(hipErrorInvalidValue);
    }
    MultiArgs a{};
    a.tiles = l.tiles;
    a.in = l.in;
    a.out = l.out;
    a.w = l.w;
    a.v = l.v;
    a.lr = l.lr;
    a.mu = l.mu;
    a.T = l.T;
    a.chunking = l.chunking;
    a.mean = l.op == DDP_MEAN;
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(l.total_tiles)), dim3(kBlock), args,
                                         lds_reserve(wg_per_cu_for(DDP_KF_MULTI, multi_wg_per_cu(l.P, l.sgd != 0))),
                                         static_cast<hipStream_t>(l.stream));
    if (e != hipSuccess) {
        *msg = "hipLaunchKernel(multi_ring)";
        return static_cast<int>(e);
    }
    return 0;
}

}  // namespace ddp
