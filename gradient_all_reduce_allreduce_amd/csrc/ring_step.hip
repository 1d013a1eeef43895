// ring_step.hip -- the ring all-reduce one step at a time, for gfx950.
//
// The literal algorithm: peers form a ring and pass slices of the tensor
// around it (Burn collective blog, "Methods", Ring); a ring all-reduce is a
// reduce-scatter followed by an all-gather ("Distributed Training",
// "Sharded data parallelism").  Each launch is one step of the ring over
// all P rank buffers (fp32, in place):
//   reduce-scatter step t: the chunk that started at rank s moves from
//     src = s+t to dst = s+t+1, which adds it to its own copy
//     (buf[dst] = buf[src] + buf[dst]); at the last step dst is the chunk's
//     owner, which applies Mean;
//   all-gather step t: the finished chunk moves from src = owner+t to
//     dst = src+1 (buf[dst] = buf[src]).
// Within one step every chunk is read at src and written at dst, and no
// chunk's src is another chunk's dst in the same step, so updating in place
// equals the simultaneous sends of the ring.  The per-element result is the
// same fold, bit for bit, as the fused single-pass kernel.  Optionally every
// launch adds to sent[r] the number of elements rank r sent, so the traffic
// of a ring (2(P-1)/P of the buffer per rank) can be read back.
//
// Each step reads 2n (reduce-scatter) or n (all-gather) floats and writes n;
// HBM-bound like the fused kernel, but it moves (3(P-1) + 2(P-1)) n floats in
// total against the fused kernel's 2Pn: this mode is the building block a
// multi-GPU ring would run per link, not the fast path on one GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch_step.h"
#include "ring_reduce_impl.h"

namespace ddp {
namespace {

using rr::kBlock;
using rr::u32x4;

struct StepArgs {
    float* buf[kMaxRanks];      // already offset to this launch's first element
    unsigned long long* sent;   // [P] element counters, or null
    int64_t base;               // global index of this launch's first element
    int64_t L;                  // chunk length ceil(n_total / C)
    uint32_t n;
    uint32_t n_vec;             // multiple of 4
    int32_t t;                  // step within the phase
    int32_t phase;              // 0 reduce-scatter, 1 all-gather
    int32_t mean_last;          // apply Mean at this (last reduce-scatter) step
};

typedef const __attribute__((address_space(4))) StepArgs* KStep;

__device__ __forceinline__ KStep step_args() {
    return (KStep)(__builtin_amdgcn_kernarg_segment_ptr());
}

constexpr int kStepU = 2;
constexpr uint32_t kStepTile = kBlock * kStepU * 4;

// Source and destination rank of this step for a chunk with start rank s.
template <int P>
__device__ __forceinline__ void step_ranks(KStep a, int s, int* src, int* dst) {
    const int from = a->phase == 0 ? s + a->t : s + P - 1 + a->t;
    *src = from % P;
    *dst = (from + 1) % P;
}

template <int P>
__device__ __forceinline__ void step_element(KStep a, uint32_t i) {
#pragma clang fp contract(off)
    const int s = static_cast<int>(((a->base + i) / a->L) % P);
    int src, dst;
    step_ranks<P>(a, s, &src, &dst);
    float v = a->buf[src][i];
    if (a->phase == 0) {
        v = v + a->buf[dst][i];
        if (a->mean_last) v = rr::mean_of<P>(v);
    }
    a->buf[dst][i] = v;
    if (a->sent) atomicAdd(a->sent + src, 1ull);
}

template <int P>
__global__ __launch_bounds__(kBlock) void ring_step_kernel(StepArgs) {
#pragma clang fp contract(off)
    const KStep a = step_args();
    const uint32_t tid = threadIdx.x;
    const uint32_t t0 = blockIdx.x * kStepTile;
    const uint32_t n_vec = a->n_vec;
    if (t0 < n_vec) {
        const uint32_t end = t0 + kStepTile < n_vec ? t0 + kStepTile : n_vec;
        const int64_t j0 = (a->base + t0) / a->L;
        const int64_t j1 = (a->base + end - 1) / a->L;
        if (j0 != j1) {
            // a chunk boundary inside the tile: element by element
            for (int u = 0; u < kStepU; ++u) {
                const uint32_t i0 = t0 + (u * kBlock + tid) * 4;
                if (i0 < end) {
                    for (int e = 0; e < 4; ++e) step_element<P>(a, i0 + e);
                }
            }
        } else {
            int src, dst;
            step_ranks<P>(a, static_cast<int>(j0 % P), &src, &dst);
            const char* ps = reinterpret_cast<const char*>(a->buf[src]);
            char* pd = reinterpret_cast<char*>(a->buf[dst]);
            u32x4 x[kStepU];
            u32x4 y[kStepU];
#pragma unroll
            for (int u = 0; u < kStepU; ++u) {
                const uint32_t i0 = t0 + (u * kBlock + tid) * 4;
                if (i0 < end) {
                    x[u] = rr::load16(ps + i0 * 4u);
                    if (a->phase == 0) y[u] = rr::load16(pd + i0 * 4u);
                }
            }
#pragma unroll
            for (int u = 0; u < kStepU; ++u) {
                const uint32_t i0 = t0 + (u * kBlock + tid) * 4;
                if (i0 >= end) continue;
                u32x4 o = x[u];
                if (a->phase == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float v = __uint_as_float(x[u][e]) + __uint_as_float(y[u][e]);
                        if (a->mean_last) v = rr::mean_of<P>(v);
                        o[e] = __float_as_uint(v);
                    }
                }
                rr::store16(pd, a->n * 4u, i0 * 4u, o);
            }
            if (a->sent && tid == 0) atomicAdd(a->sent + src, static_cast<unsigned long long>(end - t0));
        }
    }
    if (blockIdx.x == gridDim.x - 1) {
        const uint32_t i = n_vec + tid;
        if (i < a->n) step_element<P>(a, i);
    }
}

// Chunks shorter than a tile: one element per lane.
template <int P>
__global__ __launch_bounds__(kBlock) void ring_step_scalar_kernel(StepArgs) {
    const KStep a = step_args();
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < a->n) step_element<P>(a, i);
}

const void* step_kernel(int P, bool scalar) {
    switch (P) {
#define DDP_CASE(p)                                                                   \
    case p:                                                                           \
        return scalar ? reinterpret_cast<const void*>(&ring_step_scalar_kernel<p>) \
                      : reinterpret_cast<const void*>(&ring_step_kernel<p>);
        DDP_CASE(2) DDP_CASE(3) DDP_CASE(4) DDP_CASE(5)
        DDP_CASE(6) DDP_CASE(7) DDP_CASE(8) DDP_CASE(9)
        DDP_CASE(10) DDP_CASE(11) DDP_CASE(12) DDP_CASE(13)
        DDP_CASE(14) DDP_CASE(15) DDP_CASE(16)
#undef DDP_CASE
        default:
            return nullptr;
    }
}

}  // namespace

int launch_ring_stepwise(const StepLaunch& l, const char** msg) {
    if (l.n <= 0 || l.P < 2) return 0;   // one rank: nothing moves, Mean divides by 1
    const int64_t L = (l.n + l.chunking - 1) / l.chunking;
    const bool scalar = L < static_cast<int64_t>(kStepTile);
    const void* fn = step_kernel(l.P, scalar);
    if (fn == nullptr) {
        *msg = "no step kernel for this rank count";
        return static_cast<int>(hipErrorInvalidValue);
    }
    for (int phase = 0; phase < 2; ++phase) {
        for (int t = 0; t < l.P - 1; ++t) {
            for (int64_t base = 0; base < l.n; base += kMaxLaunchElems) {
                const int64_t n = l.n - base < kMaxLaunchElems ? l.n - base : kMaxLaunchElems;
                StepArgs a{};
                for (int r = 0; r < l.P; ++r) a.buf[r] = l.buf[r] + base;
                a.sent = reinterpret_cast<unsigned long long*>(l.sent);
                a.base = base;
                a.L = L;
                a.n = static_cast<uint32_t>(n);
                a.n_vec = static_cast<uint32_t>(n - n % 4);
                a.t = t;
                a.phase = phase;
                a.mean_last = phase == 0 && t == l.P - 2 && l.op == DDP_MEAN;
                int64_t grid = scalar ? (n + kBlock - 1) / kBlock : (a.n_vec + kStepTile - 1) / kStepTile;
                if (grid < 1) grid = 1;
                void* args[] = {&a};
                const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(kBlock), args,
                                                     lds_reserve(wg_per_cu_for(DDP_KF_STEP, kStepWgPerCu)),
                                                     static_cast<hipStream_t>(l.stream));
                if (e != hipSuccess) {
                    *msg = "hipLaunchKernel(ring_step)";
                    return static_cast<int>(e);
                }
            }
        }
    }
    return 0;
}

}  // namespace ddp
