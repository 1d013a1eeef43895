// hbm_patterns.hip -- what this GPU's HBM sustains for the access patterns
// of the all-reduce, measured with plain streaming kernels.
//
//   gradient_all_reduce_allreduce_amd/hbm_patterns
//
// The ring all-reduce of P buffers reads P streams and writes P streams; its
// roofline is HBM bandwidth for that read/write mix, not the read-only peak.
// Every kernel here moves one 16-byte vector per lane and stream, with
// one-wave (64-lane) workgroups, one tile each, as many workgroups as tiles,
// and LDS reserved so that at most `cap` workgroups share a CU (cap 0: the
// hardware's own occupancy).  Loads are non-temporal, stores device-scope
// buffer stores, as in the library.  Buffers hold random float bit patterns
// (the rates on all-zero buffers come out about 1% higher).  Each line is
// the mean over 40 launches timed with hipEvents, rotating over buffer sets
// larger in total than the 256 MB last-level cache, in GB/s of bytes moved
// (read + written):
//   read8       8 input streams, 25 MiB each
//   write8      8 output streams
//   copy        1 input stream -> 1 output stream, 200 MiB each
//   bcast 1 -> 7  the all-gather's pattern: 1 input stream, each tile
//               stored to 7 of the 8 output streams (25 MiB each), with
//               each store cache policy and load kind; and the
//               same with one output stream per workgroup, the 7 workgroups
//               that read one tile on one XCD (reads mostly from its L2)
//   LDS-staged  the all-reduce's pattern with the inputs brought into LDS
//               by direct global -> LDS loads, 1, 2 or 4 tiles per
//               workgroup (the next tile's loads in flight while one is
//               folded), float32 and bf16 -> float32; checked bit for bit
//               against the register kernels
//   red8 f32    the all-reduce's own pattern: 8 input streams summed into 8
//               identical output streams, 25 MiB each (the 16 buffers back to
//               back in one allocation)
//   red8 f32, 100 MiB streams   the same pattern, four times as much per
//               launch: the fixed cost of starting and draining a launch
//               weighs a quarter as much
//   red8 bf16->f32  8 bf16 input streams of 100 MiB, 8 float32 outputs
//   sgd step    the fused optimizer step: 8 bf16 gradient streams of 25 MiB
//               summed, float32 w and v read and written, and with output
//               the bf16 sum to 8 streams
//   red8 f32, separate allocations   the f32 pattern on 16 hipMallocs
//
//   gradient_all_reduce_allreduce_amd/hbm_patterns --launch-cost
//
// prints instead what a launch costs the GPU itself: empty one-wave kernels
// of 1 and of 25,600 workgroups (one 25 MiB float32 bucket's tiles), back to
// back on one stream behind about 1.5 ms of copying, so that the host has
// queued every measured launch before the GPU reaches them and the events
// around them time the GPU's side alone.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define CK(x)                                                                  \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                      \
        }                                                                      \
    } while (0)

constexpr int kW = 64;
constexpr unsigned kLdsPerCu = 160u * 1024u;
constexpr unsigned kLdsGranule = 1280u;

static unsigned lds_for(int cap) { return cap <= 0 ? 0u : kLdsPerCu / cap / kLdsGranule * kLdsGranule; }

struct Streams {
    const char* in[8];
    char* out[16];       // out[q] and out[q + 8] are the same stream (rotated store order)
    uint32_t out_bytes;  // size of each output stream
};

__device__ __forceinline__ void store16(char* base, uint32_t bytes, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000),
                                           off, 0, 16);
}

// Random float bit patterns of magnitude around 2^-7 (finite, both signs).
__global__ void fill_kernel(uint32_t* p, size_t n, uint32_t seed) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        uint32_t x = static_cast<uint32_t>(i) * 2654435761u ^ seed ^ static_cast<uint32_t>(i >> 32);
        x ^= x >> 16;
        x *= 0x7feb352du;
        x ^= x >> 15;
        x *= 0x846ca68bu;
        x ^= x >> 16;
        p[i] = (x & 0x807fffffu) | ((120u + ((x >> 23) & 3u)) << 23);
    }
}

// NR input streams, NW output streams; tile = one 16-byte vector per lane
// and stream.  With both, the outputs get the sum of the inputs (float32).
template <int NR, int NW>
__global__ __launch_bounds__(kW) void stream_kernel(Streams p, uint32_t* sink) {
    const uint32_t off = (blockIdx.x * kW + threadIdx.x) * 16u;
    u32x4 x[NR > 0 ? NR : 1];
#pragma unroll
    for (int r = 0; r < NR; ++r) x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.in[r] + off));
    u32x4 s = {off, off, off, off};
    if constexpr (NR > 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float acc = __uint_as_float(x[0][e]);
#pragma unroll
            for (int r = 1; r < NR; ++r) acc = acc + __uint_as_float(x[r][e]);
            s[e] = __float_as_uint(acc);
        }
    }
    if constexpr (NW == 0) {
        if ((s[0] ^ s[1] ^ s[2] ^ s[3]) == 0x9e3779b9u) sink[0] = 1u;   // keeps the loads
    } else {
        const int rot = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x % NW));
#pragma unroll
        for (int q = 0; q < NW; ++q) store16(p.out[rot + q], p.out_bytes, off, s);
    }
}

// The all-gather's pattern (one input stream, each tile stored to 7 of the
// 8 output streams) with the stores' cache policy as a parameter: 0 the
// default, 2 non-temporal, 16 device scope (sc1, the library's choice for
// the all-reduce), 18 both; and ordinary or non-temporal loads.
template <int POL, bool NT_LOAD>
__global__ __launch_bounds__(kW) void bcast_policy_kernel(Streams p, uint32_t* sink) {
    const uint32_t off = (blockIdx.x * kW + threadIdx.x) * 16u;
    const u32x4 y = NT_LOAD ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.in[0] + off))
                            : *reinterpret_cast<const u32x4*>(p.in[0] + off);
    const int rot = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x % 7));
#pragma unroll
    for (int q = 0; q < 7; ++q)
        __builtin_amdgcn_raw_buffer_store_b128(
            y, __builtin_amdgcn_make_buffer_rsrc(p.out[rot + q], 0, static_cast<int>(p.out_bytes), 0x00020000), off, 0,
            POL);
}

// The all-gather's pattern with one output stream per workgroup: the
// workgroups that copy one input tile to the 7 outputs sit on one XCD
// (workgroups are dispatched to the 8 XCDs round robin, so workgroup b runs
// on XCD b mod 8), so that the first read of a tile fills that XCD's L2 and
// the other six hit it.  Workgroup b: tile (b / 64) * 8 + b mod 8, output
// slot (b / 8) mod 8, slot 7 idle.  U vectors per lane.
template <int U>
__global__ __launch_bounds__(kW) void bcast_xcd_kernel(Streams p, uint32_t* sink) {
    const uint32_t b = blockIdx.x;
    const uint32_t slot = (b >> 3) & 7u;
    if (slot == 7u) return;
    const uint32_t tile = (b >> 6) * 8u + (b & 7u);
    u32x4 y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t off = ((tile * U + u) * kW + threadIdx.x) * 16u;
        y[u] = *reinterpret_cast<const u32x4*>(p.in[0] + off);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t off = ((tile * U + u) * kW + threadIdx.x) * 16u;
        store16(p.out[slot], p.out_bytes, off, y[u]);
    }
}

// stream_kernel with the stores' cache policy as a parameter (the values of
// bcast_policy_kernel).
template <int NR, int NW, int POL>
__global__ __launch_bounds__(kW) void stream_policy_kernel(Streams p, uint32_t* sink) {
    const uint32_t off = (blockIdx.x * kW + threadIdx.x) * 16u;
    u32x4 x[NR > 0 ? NR : 1];
#pragma unroll
    for (int r = 0; r < NR; ++r) x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.in[r] + off));
    u32x4 s = {off, off, off, off};
    if constexpr (NR > 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float acc = __uint_as_float(x[0][e]);
#pragma unroll
            for (int r = 1; r < NR; ++r) acc = acc + __uint_as_float(x[r][e]);
            s[e] = __float_as_uint(acc);
        }
    }
    const int rot = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x % NW));
#pragma unroll
    for (int q = 0; q < NW; ++q)
        __builtin_amdgcn_raw_buffer_store_b128(
            s, __builtin_amdgcn_make_buffer_rsrc(p.out[rot + q], 0, static_cast<int>(p.out_bytes), 0x00020000), off, 0,
            POL);
}

// stream_kernel with BS-lane workgroups: every wave still moves its own
// 64-lane tile, so only the number of workgroups to dispatch changes (a
// quarter of them with 256 lanes).
template <int NR, int NW, int BS>
__global__ __launch_bounds__(BS) void stream_bs_kernel(Streams p, uint32_t* sink) {
    const uint32_t off = (blockIdx.x * BS + threadIdx.x) * 16u;
    u32x4 x[NR > 0 ? NR : 1];
#pragma unroll
    for (int r = 0; r < NR; ++r) x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.in[r] + off));
    u32x4 s = {off, off, off, off};
    if constexpr (NR > 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float acc = __uint_as_float(x[0][e]);
#pragma unroll
            for (int r = 1; r < NR; ++r) acc = acc + __uint_as_float(x[r][e]);
            s[e] = __float_as_uint(acc);
        }
    }
    const int wave = static_cast<int>(blockIdx.x * (BS / 64) + threadIdx.x / 64);
    const int rot = __builtin_amdgcn_readfirstlane(wave % NW);
#pragma unroll
    for (int q = 0; q < NW; ++q) store16(p.out[rot + q], p.out_bytes, off, s);
}

// The bf16 -> float32 pattern with the stores' cache policy as a parameter.
template <int POL>
__global__ __launch_bounds__(kW) void red8_bf16_policy_kernel(Streams p, uint32_t* sink) {
    const uint32_t i = blockIdx.x * kW + threadIdx.x;   // 4-element group
    u32x2 x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p.in[r] + i * 8u));
    u32x4 s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint32_t w = x[r][e >> 1];
            const float v = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
            acc = r == 0 ? v : acc + v;
        }
        s[e] = __float_as_uint(acc);
    }
    const int rot = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x & 7));
#pragma unroll
    for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_raw_buffer_store_b128(
            s, __builtin_amdgcn_make_buffer_rsrc(p.out[rot + q], 0, static_cast<int>(p.out_bytes), 0x00020000),
            i * 16u, 0, POL);
}

// The bf16 -> float32 pattern: 8-byte bf16 loads (4 elements), 16-byte stores.
__global__ __launch_bounds__(kW) void red8_bf16_kernel(Streams p, uint32_t* sink) {
    const uint32_t i = blockIdx.x * kW + threadIdx.x;   // 4-element group
    u32x2 x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p.in[r] + i * 8u));
    u32x4 s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint32_t w = x[r][e >> 1];
            const float v = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
            acc = r == 0 ? v : acc + v;
        }
        s[e] = __float_as_uint(acc);
    }
    const int rot = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x & 7));
#pragma unroll
    for (int q = 0; q < 8; ++q) store16(p.out[rot + q], p.out_bytes, i * 16u, s);
}

// The fused optimizer step's pattern: 8 bf16 input streams (8-byte loads,
// 4 elements per lane) summed, one momentum step on float32 w and v (read
// and written, 16 bytes per lane each), and with WOUT the sum rounded to
// bf16 into 8 output streams (8-byte stores).  (The bf16 rounding here is
// a truncation: only the traffic matters.)
struct SgdStreams {
    const char* in[8];
    char* out[16];
    char* w;
    char* v;
    uint32_t out_bytes;
    uint32_t wv_bytes;
};

__device__ __forceinline__ void store8(char* base, uint32_t bytes, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000),
                                          off, 0, 16);
}

template <bool WOUT>
__global__ __launch_bounds__(kW) void sgd_kernel(SgdStreams p, uint32_t* sink) {
    const uint32_t i = blockIdx.x * kW + threadIdx.x;   // 4-element group
    u32x2 x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p.in[r] + i * 8u));
    const u32x4 wq = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.w + i * 16u));
    const u32x4 vq = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.v + i * 16u));
    u32x4 wn, vn;
    u32x2 o;
    float g[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint32_t w = x[r][e >> 1];
            const float val = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
            acc = r == 0 ? val : acc + val;
        }
        g[e] = acc * 0.125f;
        const float v1 = 0.9f * __uint_as_float(vq[e]) + g[e];
        vn[e] = __float_as_uint(v1);
        wn[e] = __float_as_uint(__uint_as_float(wq[e]) - 1e-3f * v1);
    }
    for (int k = 0; k < 2; ++k) o[k] = (__float_as_uint(g[2 * k]) >> 16) | (__float_as_uint(g[2 * k + 1]) & 0xffff0000u);
    store16(p.w, p.wv_bytes, i * 16u, wn);
    store16(p.v, p.wv_bytes, i * 16u, vn);
    if constexpr (WOUT) {
        const int rot = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x & 7));
#pragma unroll
        for (int q = 0; q < 8; ++q) store8(p.out[rot + q], p.out_bytes, i * 8u, o);
    } else {
        if ((o[0] ^ o[1]) == 0x9e3779b9u) sink[0] = 1u;
    }
}

// The all-reduce's pattern with the input tiles staged in LDS by direct
// global -> LDS loads (global_load_lds_dwordx4: lane i's 16 bytes land at
// the wave's LDS base + 16 i), then read back to registers, folded and
// stored as above.  T tiles per workgroup: the loads of tile t + 1 are
// issued (into the other LDS buffer) before tile t is folded and stored.
// The compiler does not order reads of LDS after these loads on its own,
// so every read waits explicitly for the vector memory counter to drain
// (loads and stores share that counter on this chip and may complete out
// of order with each other, so only vmcnt(0) is safe); the empty asm
// also keeps the LDS reads below the wait.
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* gbl_ptr;

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ES_IN 4: float32 inputs, a 64-lane tile of 4 elements per lane; ES_IN 2:
// bf16 inputs, a tile of 512 elements (the direct loads move 16 bytes per
// lane), read back transposed: lane i takes elements 4i..4i+3 and
// 256+4i..256+4i+3, so that each of its two 16-byte float32 stores per
// stream belongs to one contiguous 1 KB store of the wave.
template <int T, int ES_IN>
__global__ __launch_bounds__(kW) void red8_lds_kernel(Streams p, uint32_t* sink) {
    constexpr int VE = 16 / ES_IN;                  // elements per lane and tile
    __shared__ u32x4 buf[T > 1 ? 2 : 1][8][kW];
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    const uint32_t lane = threadIdx.x;
    const uint32_t tile0 = blockIdx.x * T;
#pragma unroll
    for (int r = 0; r < 8; ++r)
        __builtin_amdgcn_global_load_lds((gbl_ptr)(p.in[r] + (tile0 * kW + lane) * 16u), (lds_ptr)&buf[0][r][0], 16, 0, 0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        wait_vm_all();
        u32x4 x[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (ES_IN == 4) {
                x[r] = buf[t & 1][r][lane];
            } else {
                const u32x2v* row = reinterpret_cast<const u32x2v*>(&buf[t & 1][r][0]);
                const u32x2v lo2 = row[lane];        // elements 4 lane .. 4 lane + 3
                const u32x2v hi2 = row[kW + lane];   // elements 256 + 4 lane ..
                x[r] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
            }
        }
        if (t + 1 < T) {
            // the LDS reads above complete before the next loads overwrite
            // the other buffer's previous contents (read two tiles ago)
#pragma unroll
            for (int r = 0; r < 8; ++r)
                __builtin_amdgcn_global_load_lds((gbl_ptr)(p.in[r] + ((tile0 + t + 1) * kW + lane) * 16u),
                                                 (lds_ptr)&buf[(t + 1) & 1][r][0], 16, 0, 0);
        }
        float acc[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint32_t w = ES_IN == 4 ? x[r][e] : x[r][e >> 1];
                const float v = ES_IN == 4 ? __uint_as_float(w) : __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
                acc[e] = r == 0 ? v : acc[e] + v;
            }
        }
        // float32 output offset of lane's first element; the second half
        // of a bf16 tile is 256 elements (1 KB) further
        const uint32_t off = ((tile0 + t) * kW * VE + 4u * lane) * 4u;
        const int rot = __builtin_amdgcn_readfirstlane(static_cast<int>((tile0 + t) & 7));
#pragma unroll
        for (int h = 0; h < VE / 4; ++h) {
            u32x4 s;
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] = __float_as_uint(acc[4 * h + e]);
#pragma unroll
            for (int q = 0; q < 8; ++q) store16(p.out[rot + q], p.out_bytes, off + 1024u * h, s);
        }
    }
}

// Does nothing (the store is never taken: no stream is that long); the
// arguments are as large as the pattern kernels'.
__global__ __launch_bounds__(kW) void empty_kernel(Streams p, uint32_t* sink) {
    if (p.out_bytes == 0xffffffffu && threadIdx.x == 0) sink[0] = blockIdx.x;
}

// GPU-side microseconds per launch of `grid` empty workgroups at `cap`
// workgroups per CU (best of 3 batches of `iters`), behind `ahead` copy
// launches over `copy` sets of `copy_grid` workgroups.
static double launch_us(unsigned grid, int cap, const Streams& st, uint32_t* sink,
                        const std::vector<Streams>& copy, unsigned copy_grid, int ahead, int iters) {
    hipFuncAttributes at{};
    CK(hipFuncGetAttributes(&at, reinterpret_cast<const void*>(empty_kernel)));
    const unsigned want = lds_for(cap);
    const unsigned lds = want > at.sharedSizeBytes ? want - static_cast<unsigned>(at.sharedSizeBytes) : 0u;
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    double best = 1e30;
    for (int rep = 0; rep < 3; ++rep) {
        CK(hipDeviceSynchronize());
        for (int i = 0; i < ahead; ++i)
            hipLaunchKernelGGL((stream_kernel<1, 1>), dim3(copy_grid), dim3(kW), 0, 0, copy[i % copy.size()], sink);
        CK(hipEventRecord(a));
        for (int i = 0; i < iters; ++i) hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(kW), lds, 0, st, sink);
        CK(hipEventRecord(b));
        CK(hipGetLastError());
        CK(hipEventSynchronize(b));
        float ms = 0.f;
        CK(hipEventElapsedTime(&ms, a, b));
        if (ms * 1e3 / iters < best) best = ms * 1e3 / iters;
    }
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    return best;
}

template <typename K, typename S>
static double rate(K kernel, unsigned grid, int cap, const std::vector<S>& sets, uint32_t* sink,
                   double bytes_per_launch, int reps = 40, unsigned block = kW) {
    hipFuncAttributes at{};
    CK(hipFuncGetAttributes(&at, reinterpret_cast<const void*>(kernel)));
    const unsigned want = lds_for(cap);
    const unsigned lds = want > at.sharedSizeBytes ? want - static_cast<unsigned>(at.sharedSizeBytes) : 0u;
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    for (int i = 0; i < 3; ++i) hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), lds, 0, sets[i % sets.size()], sink);
    CK(hipGetLastError());
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(a));
    for (int i = 0; i < reps; ++i) hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), lds, 0, sets[i % sets.size()], sink);
    CK(hipEventRecord(b));
    CK(hipEventSynchronize(b));
    float ms = 0.f;
    CK(hipEventElapsedTime(&ms, a, b));
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    return bytes_per_launch / (ms / reps * 1e-3) / 1e9;
}

static void fill(char* p, size_t bytes, uint32_t seed) {
    hipLaunchKernelGGL(fill_kernel, dim3(4096), dim3(256), 0, 0, reinterpret_cast<uint32_t*>(p), bytes / 4, seed);
    CK(hipGetLastError());
}

// Streams of one set: inputs at `in`, outputs at `out`, each `stride` apart.
static Streams make_set(char* in, size_t in_stride, char* out, size_t out_stride, uint32_t out_bytes) {
    Streams s{};
    for (int r = 0; r < 8; ++r) s.in[r] = in + r * in_stride;
    for (int q = 0; q < 8; ++q) s.out[q] = s.out[q + 8] = out + q * out_stride;
    s.out_bytes = out_bytes;
    return s;
}

static int launch_cost(uint32_t* sink) {
    const size_t cb = size_t(200) << 20;
    char* arena = nullptr;
    CK(hipMalloc(&arena, cb * 4));
    fill(arena, cb * 4, 4u);
    std::vector<Streams> copy;
    for (int s = 0; s < 2; ++s) copy.push_back(make_set(arena + 2 * s * cb, cb, arena + (2 * s + 1) * cb, cb,
                                                        static_cast<uint32_t>(cb)));
    const unsigned g200 = static_cast<unsigned>(cb / 16 / kW);
    CK(hipDeviceSynchronize());
    const Streams st = copy[0];
    std::printf("GPU-side cost of one launch (empty one-wave workgroups, back to back on one stream)\n");
    std::printf("%-44s %8s %8s\n", "launch", "cap", "us");
    const struct { const char* name; unsigned grid; int cap; int iters; } rows[] = {
        {"1 workgroup", 1, 0, 200},
        {"1 workgroup, LDS for 5 per CU", 1, 5, 200},
        {"25,600 workgroups", 25600, 0, 150},
        {"25,600 workgroups, LDS for 5 per CU", 25600, 5, 150},
        {"102,400 workgroups, LDS for 5 per CU", 102400, 5, 60},
    };
    for (const auto& r : rows) {
        std::printf("%-44s %8d %8.2f\n", r.name, r.cap, launch_us(r.grid, r.cap, st, sink, copy, g200, 24, r.iters));
        std::fflush(stdout);
    }
    CK(hipFree(arena));
    return 0;
}

int main(int argc, char** argv) {
    const int caps[] = {0, 3, 4, 5, 6, 8, 12, 16};
    uint32_t* sink = nullptr;
    CK(hipMalloc(&sink, 64));
    if (argc > 1 && std::strcmp(argv[1], "--launch-cost") == 0) {
        const int rc = launch_cost(sink);
        CK(hipFree(sink));
        return rc;
    }

    // 25 MiB streams: 4 sets of 16 streams back to back (1.6 GiB); the
    // arena holds twice that for 2 sets of 100 MiB streams
    const size_t sb = size_t(25) << 20;
    const int nsets = 4;
    char* arena = nullptr;
    CK(hipMalloc(&arena, sb * 16 * nsets * 2));
    fill(arena, sb * 16 * nsets * 2, 1u);
    const size_t lb = 4 * sb;
    std::vector<Streams> red_long;
    for (int s = 0; s < 2; ++s)
        red_long.push_back(make_set(arena + s * 16 * lb, lb, arena + (s * 16 + 8) * lb, lb, static_cast<uint32_t>(lb)));
    const unsigned g100 = static_cast<unsigned>(lb / 16 / kW);
    std::vector<Streams> red;
    for (int s = 0; s < nsets; ++s)
        red.push_back(make_set(arena + s * 16 * sb, sb, arena + (s * 16 + 8) * sb, sb, static_cast<uint32_t>(sb)));
    const unsigned g25 = static_cast<unsigned>(sb / 16 / kW);

    // copy: 200 MiB streams, 4 pairs (1.6 GiB)
    const size_t cb = size_t(200) << 20;
    std::vector<Streams> copy;
    for (int s = 0; s < nsets; ++s)
        copy.push_back(make_set(arena + 2 * s * cb, cb, arena + (2 * s + 1) * cb, cb, static_cast<uint32_t>(cb)));
    const unsigned g200 = static_cast<unsigned>(cb / 16 / kW);

    // bf16 -> f32: 100 MiB bf16 inputs, 200 MiB float32 outputs, 2 sets (4.7 GiB)
    const size_t bin = size_t(100) << 20, bout = size_t(200) << 20;
    char* barena = nullptr;
    CK(hipMalloc(&barena, (bin + bout) * 8 * 2));
    fill(barena, (bin + bout) * 8 * 2, 2u);
    std::vector<Streams> bf;
    for (int s = 0; s < 2; ++s) {
        char* base = barena + s * (bin + bout) * 8;
        bf.push_back(make_set(base, bin, base + 8 * bin, bout, static_cast<uint32_t>(bout)));
    }
    const unsigned gbf = static_cast<unsigned>(bin / 8 / kW);

    // the fused optimizer step: bf16 gradients of 25 MiB per rank, w and v
    // float32 (50 MiB each), outputs bf16; 4 sets, carved from the bf16 arena
    const size_t gb = sb;                 // 25 MiB of bf16 per stream
    const size_t wvb = 2 * sb;            // 50 MiB of float32
    std::vector<SgdStreams> sgd;
    for (int s = 0; s < 4; ++s) {
        char* base = barena + s * (16 * gb + 2 * wvb);
        SgdStreams st{};
        for (int r = 0; r < 8; ++r) st.in[r] = base + r * gb;
        for (int q = 0; q < 8; ++q) st.out[q] = st.out[q + 8] = base + (8 + q) * gb;
        st.w = base + 16 * gb;
        st.v = base + 16 * gb + wvb;
        st.out_bytes = static_cast<uint32_t>(gb);
        st.wv_bytes = static_cast<uint32_t>(wvb);
        sgd.push_back(st);
    }
    const unsigned gsgd = static_cast<unsigned>(gb / 8 / kW);

    // separate allocations for the f32 pattern
    std::vector<char*> sep;
    for (int i = 0; i < 16 * nsets; ++i) {
        char* p = nullptr;
        CK(hipMalloc(&p, sb));
        fill(p, sb, 3u + i);
        sep.push_back(p);
    }
    std::vector<Streams> red_sep;
    for (int s = 0; s < nsets; ++s) {
        Streams st{};
        for (int r = 0; r < 8; ++r) st.in[r] = sep[s * 16 + r];
        for (int q = 0; q < 8; ++q) st.out[q] = st.out[q + 8] = sep[s * 16 + 8 + q];
        st.out_bytes = static_cast<uint32_t>(sb);
        red_sep.push_back(st);
    }
    CK(hipDeviceSynchronize());

    std::printf("%-36s", "pattern \\ workgroups per CU");
    for (int c : caps) std::printf(c ? "%8d" : "    none", c);
    std::printf("\n");
    auto row = [&](const char* name, auto kernel, unsigned grid, const auto& sets, double bytes) {
        std::printf("%-36s", name);
        for (int c : caps) std::printf("%8.0f", rate(kernel, grid, c, sets, sink, bytes));
        std::printf("   GB/s\n");
        std::fflush(stdout);
    };
    row("read8 (25 MiB streams)", stream_kernel<8, 0>, g25, red, 8.0 * sb);
    row("write8 (25 MiB streams)", stream_kernel<0, 8>, g25, red, 8.0 * sb);
    row("copy (200 MiB)", stream_kernel<1, 1>, g200, copy, 2.0 * cb);
    row("bcast 1 -> 7 (25 MiB streams)", stream_kernel<1, 7>, g25, red, 8.0 * sb);
    {
        // 128- and 256-lane workgroups: the caps are workgroups per CU, so
        // waves per CU = cap * 2 or cap * 4 (at least 2 workgroups per CU)
        auto row_bs = [&](const char* name, auto kernel, unsigned grid, const auto& sets, double bytes, unsigned bs) {
            std::printf("%-36s", name);
            for (int c : caps) {
                if (c != 0 && c < 2) { std::printf("%8s", "-"); continue; }
                std::printf("%8.0f", rate(kernel, grid, c, sets, sink, bytes, 40, bs));
            }
            std::printf("   GB/s\n");
            std::fflush(stdout);
        };
        row_bs("red8 f32 25 MiB, 128-lane wg", stream_bs_kernel<8, 8, 128>, g25 / 2, red, 16.0 * sb, 128);
        row_bs("red8 f32 25 MiB, 256-lane wg", stream_bs_kernel<8, 8, 256>, g25 / 4, red, 16.0 * sb, 256);
        row_bs("red8 f32 100 MiB, 128-lane wg", stream_bs_kernel<8, 8, 128>, g100 / 2, red_long, 16.0 * lb, 128);
        row_bs("red8 f32 100 MiB, 256-lane wg", stream_bs_kernel<8, 8, 256>, g100 / 4, red_long, 16.0 * lb, 256);
        row_bs("write8, 256-lane wg", stream_bs_kernel<0, 8, 256>, g25 / 4, red, 8.0 * sb, 256);
    }
    row("write8, stores nt", stream_policy_kernel<0, 8, 2>, g25, red, 8.0 * sb);
    row("write8, stores sc1 nt", stream_policy_kernel<0, 8, 18>, g25, red, 8.0 * sb);
    row("red8 f32 25 MiB, stores nt", stream_policy_kernel<8, 8, 2>, g25, red, 16.0 * sb);
    row("red8 f32 25 MiB, stores sc1 nt", stream_policy_kernel<8, 8, 18>, g25, red, 16.0 * sb);
    row("red8 f32 25 MiB, stores sc1", stream_policy_kernel<8, 8, 16>, g25, red, 16.0 * sb);
    row("red8 f32 100 MiB, stores nt", stream_policy_kernel<8, 8, 2>, g100, red_long, 16.0 * lb);
    row("red8 f32 100 MiB, stores sc1 nt", stream_policy_kernel<8, 8, 18>, g100, red_long, 16.0 * lb);
    row("red8 bf16->f32, stores nt", red8_bf16_policy_kernel<2>, gbf, bf, 8.0 * (bin + bout));
    row("red8 bf16->f32, stores sc1 nt", red8_bf16_policy_kernel<18>, gbf, bf, 8.0 * (bin + bout));
    row("red8 bf16->f32, stores sc1", red8_bf16_policy_kernel<16>, gbf, bf, 8.0 * (bin + bout));
    row("bcast 1 -> 7, stores default", bcast_policy_kernel<0, false>, g25, red, 8.0 * sb);
    row("bcast 1 -> 7, stores nt", bcast_policy_kernel<2, false>, g25, red, 8.0 * sb);
    row("bcast 1 -> 7, stores sc1", bcast_policy_kernel<16, false>, g25, red, 8.0 * sb);
    row("bcast 1 -> 7, stores sc1 nt", bcast_policy_kernel<18, false>, g25, red, 8.0 * sb);
    row("bcast 1 -> 7, nt loads, stores sc1", bcast_policy_kernel<16, true>, g25, red, 8.0 * sb);
    row("bcast 1 -> 7, nt loads, stores nt", bcast_policy_kernel<2, true>, g25, red, 8.0 * sb);
    row("bcast 1 -> 7, a stream per wg, XCD", bcast_xcd_kernel<1>, g25 * 8, red, 8.0 * sb);
    row("bcast 1 -> 7, the same, 2 vec/lane", bcast_xcd_kernel<2>, g25 * 4, red, 8.0 * sb);
    row("red8 f32 (25 MiB, one allocation)", stream_kernel<8, 8>, g25, red, 16.0 * sb);
    row("red8 f32 (25 MiB, separate allocs)", stream_kernel<8, 8>, g25, red_sep, 16.0 * sb);
    row("red8 f32 (100 MiB streams)", stream_kernel<8, 8>, g100, red_long, 16.0 * lb);
    row("red8 bf16->f32 (100 MiB inputs)", red8_bf16_kernel, gbf, bf, 8.0 * (bin + bout));
    row("sgd step, bf16 in, no output", sgd_kernel<false>, gsgd, sgd, 8.0 * gb + 4.0 * wvb);
    row("sgd step, bf16 in, bf16 out", sgd_kernel<true>, gsgd, sgd, 16.0 * gb + 4.0 * wvb);
    row("red8 f32 LDS-staged, 1 tile/wg", red8_lds_kernel<1, 4>, g25, red, 16.0 * sb);
    row("red8 f32 LDS-staged, 2 tiles/wg", red8_lds_kernel<2, 4>, g25 / 2, red, 16.0 * sb);
    row("red8 f32 LDS-staged, 4 tiles/wg", red8_lds_kernel<4, 4>, g25 / 4, red, 16.0 * sb);
    row("red8 f32 LDS-staged, 1 tile, 100 MiB", red8_lds_kernel<1, 4>, g100, red_long, 16.0 * lb);
    row("red8 bf16->f32 LDS-staged, 1 tile/wg", red8_lds_kernel<1, 2>, gbf / 2, bf, 8.0 * (bin + bout));
    row("red8 bf16->f32 LDS-staged, 2 tiles/wg", red8_lds_kernel<2, 2>, gbf / 4, bf, 8.0 * (bin + bout));

    // The staged kernels compute what the register kernels compute: the
    // same sums in the same order, compared bit for bit on one set.
    {
        std::vector<uint32_t> a(sb / 4), b(sb / 4);
        auto run_cmp = [&](const char* name, auto k1, unsigned g1, auto k2, unsigned g2, const Streams& st,
                           size_t bytes) {
            hipLaunchKernelGGL(k1, dim3(g1), dim3(kW), 0, 0, st, sink);
            CK(hipGetLastError());
            CK(hipMemcpy(a.data(), st.out[3], bytes, hipMemcpyDeviceToHost));
            CK(hipMemset(st.out[3], 0, bytes));
            hipLaunchKernelGGL(k2, dim3(g2), dim3(kW), 0, 0, st, sink);
            CK(hipGetLastError());
            CK(hipMemcpy(b.data(), st.out[3], bytes, hipMemcpyDeviceToHost));
            size_t bad = 0;
            for (size_t i = 0; i < bytes / 4; ++i) bad += a[i] != b[i];
            std::printf("check %-44s %zu of %zu words differ\n", name, bad, bytes / 4);
        };
        run_cmp("red8 f32: registers vs LDS-staged (1 tile)", stream_kernel<8, 8>, g25, red8_lds_kernel<1, 4>, g25,
                red[0], sb);
        run_cmp("red8 f32: registers vs LDS-staged (4 tiles)", stream_kernel<8, 8>, g25, red8_lds_kernel<4, 4>,
                g25 / 4, red[1], sb);
        run_cmp("red8 bf16->f32: registers vs LDS-staged (2 tiles)", red8_bf16_kernel, gbf, red8_lds_kernel<2, 2>,
                gbf / 4, bf[0], sb);
    }

    for (char* p : sep) CK(hipFree(p));
    CK(hipFree(barena));
    CK(hipFree(arena));
    CK(hipFree(sink));
    return 0;
}
