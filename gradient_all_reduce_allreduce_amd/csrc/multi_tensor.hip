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
// allreduce_ring_emulated.  The host plan gives every tensor a run of tiles
// (with a short first tile when the tensor starts off a 128-byte line, so
// that the others cover whole lines); a workgroup finds its tensor by a
// binary search over the plan (uniform, scalar loads), narrowed by a map of
// every 64th tile's tensor, and then works like the single-tensor kernel:
// rotated rank pointers, one fixed fold, P output stores.  While its data
// is in flight it also reads the plan entry and rank pointers of the tensor
// a few rounds of tiles ahead, so that later tiles on the same CU find them
// in the scalar cache.  Between the search and the
// tile's first data load there is one more round trip: the tensor's entry,
// then every rank pointer in fold and store order, read with independent
// scalar loads issued together, with the chunk arithmetic in 32 bits.
// (Reading the pointers one pair at a time for an alignment test and again
// for the loads, with a 64-bit division for the chunk length, made a tile
// take about twice as long before its first load: on one 25.5M-element
// tensor the kernel ran at 3.2 TB/s with 4 workgroups per CU against the
// ring kernel's 6.5.)  Optionally every tensor then
// takes one SGD-momentum step on its float32 master weights and momentum,
// as each replica's optimizer.step() does after the per-parameter
// all-reduces (same lecture section), with or without writing the reduced
// gradients.  Tiles of small tensors, short first tiles, tiles across a
// chunk boundary and tensors (or optimizer state) not 16-byte aligned take
// a per-element path whose rank pointers are read per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstring>
#include <mutex>

#include "launch_multi.h"
#include "ring_reduce_impl.h"

namespace ddp {
namespace {

using rr::kBlock;
using rr::u32x2;
using rr::u32x4;

struct MultiArgs {
    const ddp_tensor_tiles* tiles;   // [T], device
    const int32_t* block_first;      // [ceil(tiles / kMultiBlockTiles)], device, or null
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
// The plan, the block map and the pointer tables as the kernel reads them:
// through the constant address space.  The kernel never writes them, and a
// uniform read there is always a scalar load.  Through plain pointers the
// reads are scalar only while the compiler can prove that nothing before
// them writes memory; anything it cannot see through (an s_sleep, an empty
// asm volatile) turns them into vector loads that wait behind the tiles'
// data, which measured 20-25% slower.
typedef const __attribute__((address_space(4))) ddp_tensor_tiles* CTiles;
typedef const __attribute__((address_space(4))) int32_t* CInts;
typedef const void* const __attribute__((address_space(4)))* CPtrs;

// Non-temporal loads through global-address-space pointers.  The tensors'
// addresses come from device tables, so the compiler cannot tell that they
// point to global memory and would issue flat loads, which also count
// against the scalar-load counter: the next wait for a scalar load would
// then drain the tile's data loads as well.
typedef const __attribute__((address_space(1))) u32x4* GlobalVec4;
typedef const __attribute__((address_space(1))) u32x2* GlobalVec2;

template <int W>
__device__ __forceinline__ u32x4 load_global(const char* p) {
    if constexpr (W == 4) {
        return __builtin_nontemporal_load((GlobalVec4)(p));
    } else {
        const u32x2 h = __builtin_nontemporal_load((GlobalVec2)(p));
        return u32x4{h[0], h[1], 0u, 0u};
    }
}

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
    const CTiles tiles = (CTiles)(a->tiles);
    const CInts block_first = (CInts)(a->block_first);
    const CPtrs in_tab = (CPtrs)(a->in);
    const CPtrs out_tab = (CPtrs)(a->out);
    const CPtrs w_tab = (CPtrs)(a->w);
    const CPtrs v_tab = (CPtrs)(a->v);

    // The tensor whose tile run holds this workgroup: largest t with
    // first_tile <= b, by a binary search over the plan.  With the block
    // map the search starts between the tensors holding tiles 64 k and
    // 64 (k + 1), where 64 k <= b < 64 (k + 1) (usually one tensor: no
    // step at all); without it, over the whole plan (8 dependent scalar
    // loads for 161 tensors; a 16-way search that reads 16 entries per
    // level in one round trip measured 7-20% slower).
    int lo = 0;
    int hi = T - 1;
    if (block_first != nullptr) {
        const uint32_t k = static_cast<uint32_t>(b) / kMultiBlockTiles;
        const int f = block_first[k];
        const int g = (k + 1) * kMultiBlockTiles < gridDim.x ? block_first[k + 1] : T - 1;
        // Clamped, so that a map of another plan reads only entries of this one.
        lo = f < 0 ? 0 : (f > T - 1 ? T - 1 : f);
        hi = g < lo ? lo : (g > T - 1 ? T - 1 : g);
    }
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tiles[mid].first_tile <= b) lo = mid; else hi = mid - 1;
    }
    const int t = lo;
    ddp_tensor_tiles tt;
    tt.numel = tiles[t].numel;
    tt.first_tile = tiles[t].first_tile;
    tt.lead = tiles[t].lead;
    // Tile k of the tensor: with a lead, [0, lead) and then whole tiles
    // from `lead` on (each on a 128-byte line of the address the plan was
    // aligned to); without, whole tiles from element 0.
    const int64_t kt = b - tt.first_tile;
    const int64_t lead = tt.lead;
    const int64_t start = lead == 0 ? kt * TILE : (kt == 0 ? 0 : lead + (kt - 1) * TILE);
    if (kt < 0 || start >= tt.numel) return;
    // Tensors hold at most 2^29 elements (ddp_multi_plan) and the chunk
    // count is below 2^31, so the chunk arithmetic fits 32 bits: three
    // 32-bit divisions by uniform values instead of 64-bit ones.
    const uint32_t t0 = static_cast<uint32_t>(start);
    const uint32_t n = static_cast<uint32_t>(tt.numel);
    const uint32_t C = static_cast<uint32_t>(a->chunking);
    const uint32_t L = n / C + (n % C != 0u);
    const uint32_t stop = lead != 0 && kt == 0 ? static_cast<uint32_t>(lead) : t0 + TILE;
    const uint32_t end = stop < n ? stop : n;
    const uint32_t j0 = t0 / L;
    const uint32_t j1 = (end - 1) / L;
    const uint32_t tid = threadIdx.x;
    const int s0 = static_cast<int>(j0 % P);
    const int rot = rr::store_rotation(P);

    // Every pointer the tile needs, read once, in fold and store order
    // (rank (s0 + k) mod P, rank (rot + q) mod P): independent scalar loads
    // issued together, one round trip.  The alignment test below reads the
    // same registers.
    const bool write_out = !SGD || a->out != nullptr;
    const char* src[P];
    char* dst[P];
#pragma unroll
    for (int k = 0; k < P; ++k)
        src[k] = static_cast<const char*>(in_tab[static_cast<int64_t>(rr::rank_at(s0, k, P)) * T + t]);
    if (write_out) {
#pragma unroll
        for (int q = 0; q < P; ++q)
            dst[q] = static_cast<char*>(const_cast<void*>(out_tab[static_cast<int64_t>(rr::rank_at(rot, q, P)) * T + t]));
    }
    char* wp = nullptr;
    char* vp = nullptr;
    if constexpr (SGD) {
        wp = static_cast<char*>(const_cast<void*>(w_tab[t]));
        vp = static_cast<char*>(const_cast<void*>(v_tab[t]));
    }

    uintptr_t align = 0;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        align |= reinterpret_cast<uintptr_t>(src[k]);
        if (write_out) align |= reinterpret_cast<uintptr_t>(dst[k]);
    }
    if constexpr (SGD) align |= reinterpret_cast<uintptr_t>(wp) | reinterpret_cast<uintptr_t>(vp);
    // The tile's byte offsets in each stream (whole tiles past a lead start
    // off a multiple of the tile size).
    align |= (t0 * IES) | (t0 * OES) | (SGD ? t0 * 4u : 0u);
    const bool vector_path = j0 == j1 && end - t0 == TILE && (align & 15u) == 0;

    if (!vector_path) {
        for (uint32_t i = t0 + tid; i < end; i += kBlock) multi_element<P, INB, OUTB, SGD>(a, t, i, L);
        return;
    }

    u32x4 x[P][U];
    constexpr int WV = SGD ? V / 4 : 1;   // 16-byte state vectors per lane vector
    u32x4 wq[U][WV];
    u32x4 vq[U][WV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
#pragma unroll
        for (int k = 0; k < P; ++k) x[k][u] = load_global<WIN>(src[k] + i0 * IES);
        if constexpr (SGD) {
#pragma unroll
            for (int q = 0; q < WV; ++q) {
                wq[u][q] = load_global<4>(wp + (i0 + 4 * q) * 4u);
                vq[u][q] = load_global<4>(vp + (i0 + 4 * q) * 4u);
            }
        }
    }
    // Every compute unit works on tiles of every tensor, so each tensor's
    // plan entry and rank pointers are first-time misses in each CU's
    // scalar cache, on the path between a tile's start and its first load.
    // Reading those of the tensor a few rounds of tiles ahead now, while
    // this tile's data is in flight, turns most of them into hits for the
    // tiles that follow on this CU.  The values are only kept alive until
    // the end (nothing uses them).  Up to P = 8: at P = 16 the 33 extra
    // pointers crowd the scalar registers and the launch got 2-6% slower.
    uint64_t warm = 0;
    if (P <= 8 && block_first != nullptr) {
        const uint32_t ahead = static_cast<uint32_t>(b) + kMultiPrefetchTiles;
        if (ahead < gridDim.x) {
            const int f = block_first[ahead / kMultiBlockTiles];
            const int tw = f < 0 ? 0 : (f > T - 1 ? T - 1 : f);
            constexpr int NW = 2 * P + 1 + (SGD ? 2 : 0);
            uint64_t w[NW];
            w[0] = static_cast<uint64_t>(tiles[tw].numel);
#pragma unroll
            for (int r = 0; r < P; ++r) {
                w[1 + r] = reinterpret_cast<uint64_t>(in_tab[static_cast<int64_t>(r) * T + tw]);
                w[1 + P + r] = write_out ? reinterpret_cast<uint64_t>(out_tab[static_cast<int64_t>(r) * T + tw]) : 0;
            }
            if constexpr (SGD) {
                w[2 * P + 1] = reinterpret_cast<uint64_t>(w_tab[tw]);
                w[2 * P + 2] = reinterpret_cast<uint64_t>(v_tab[tw]);
            }
#pragma unroll
            for (int i = 0; i < NW; ++i) warm |= w[i];
        }
    }
    float acc[U][V];
    rr::fold<P, 0, INB, U, V>(x, acc);
    const bool mean = a->mean != 0;
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
                rr::store16(wp, n * 4u, (i0 + 4 * q) * 4u, wn);
                rr::store16(vp, n * 4u, (i0 + 4 * q) * 4u, vn);
            }
            if (!write_out) continue;
        }
        if constexpr (OUTB && V == 8) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = rr::bf16_bits(g[2 * k]) | (rr::bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
            for (int q = 0; q < P; ++q) rr::store16(dst[q], n * OES, i0 * OES, o);
        } else if constexpr (OUTB) {
            u32x2 o;
#pragma unroll
            for (int k = 0; k < 2; ++k) o[k] = rr::bf16_bits(g[2 * k]) | (rr::bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
            for (int q = 0; q < P; ++q) rr::store8(dst[q], n * OES, i0 * OES, o);
        } else {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(g[e]);
#pragma unroll
            for (int q = 0; q < P; ++q) rr::store16(dst[q], n * OES, i0 * OES, o);
        }
    }
    asm volatile("" ::"s"(warm));
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

// The allocation-free multi-tensor call's tables (plan, block map, pointer
// tables) live here: one copy per GPU, loaded with the code object, held
// until the process ends.  Host code never names this array in a launch or
// copy: its name is a host-side stand-in, not a device address.  It uses the
// address hipGetSymbolAddress gives on each device instead.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

int noalloc_scratch(void* stream, void** ptr, int* device, const char** msg) {
    int dev = -1;
    hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                     : hipGetDevice(&dev);
    if (e != hipSuccess) {
        *msg = "hipStreamGetDevice/hipGetDevice (scratch)";
        return static_cast<int>(e);
    }
    if (dev < 0 || dev >= kMaxScratchDevices) {
        *msg = "device ordinal beyond the scratch table";
        return static_cast<int>(hipErrorInvalidDevice);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        // Look the address up once per device, with that device current.
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) {
            *msg = "hipGetDevice (scratch)";
            return static_cast<int>(e);
        }
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) {
            *msg = "hipSetDevice (scratch)";
            return static_cast<int>(e);
        }
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess || p == nullptr) {
            *msg = "hipGetSymbolAddress(scratch)";
            return static_cast<int>(e != hipSuccess ? e : hipErrorInvalidSymbol);
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *device = dev;
    return 0;
}

int stream_capturing(void* stream, bool* capturing, const char** msg) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &st);
    if (e != hipSuccess) {
        *msg = "hipStreamIsCapturing";
        return static_cast<int>(e);
    }
    *capturing = st != hipStreamCaptureStatusNone;
    return 0;
}

namespace {

// The tables reach the scratch area as kernel arguments: each fill launch
// carries up to kFillWords 8-byte words, one per lane over ceil(n / 64)
// one-wave workgroups (a single wave looping over them waited out a load
// per word: 7.4 us per launch), and writes them with vector stores.  A
// launch captured into a graph keeps its arguments, so every replay
// writes the same tables again.

struct FillArgs {
    uint64_t* dst;
    int32_t n;          // words, 1 .. kFillWords
    int32_t unused;
    uint64_t w[kFillWords];
};
static_assert(sizeof(FillArgs) <= 7800, "the fill's kernel arguments must stay under the 8,000 bytes measured to pass");

typedef const __attribute__((address_space(4))) FillArgs* KFill;

__global__ __launch_bounds__(kBlock) void table_fill_kernel(FillArgs) {
    const KFill a = (KFill)(__builtin_amdgcn_kernarg_segment_ptr());
    const int i = static_cast<int>(blockIdx.x) * kBlock + static_cast<int>(threadIdx.x);
    if (i < a->n) a->dst[i] = a->w[i];
}

}  // namespace

int fill_scratch(void* dst, const void* src, size_t bytes, void* stream, const char** msg) {
    if (bytes % sizeof(uint64_t) != 0) {
        *msg = "table bytes not a whole number of 8-byte words";
        return static_cast<int>(hipErrorInvalidValue);
    }
    const uint64_t* w = static_cast<const uint64_t*>(src);
    const size_t words = bytes / sizeof(uint64_t);
    FillArgs a;
    for (size_t k = 0; k < words; k += kFillWords) {
        const size_t n = words - k < static_cast<size_t>(kFillWords) ? words - k : static_cast<size_t>(kFillWords);
        a.dst = static_cast<uint64_t*>(dst) + k;
        a.n = static_cast<int32_t>(n);
        a.unused = 0;
        std::memcpy(a.w, w + k, n * sizeof(uint64_t));
        void* args[] = {&a};
        const unsigned grid = static_cast<unsigned>((n + kBlock - 1) / kBlock);
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&table_fill_kernel), dim3(grid),
                                             dim3(kBlock), args, 0, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) {
            *msg = "hipLaunchKernel(table_fill)";
            return static_cast<int>(e);
        }
    }
    return 0;
}

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
    a.block_first = l.block_first;
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
