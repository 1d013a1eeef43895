// hbm_patterns.hip -- what this GPU's HBM sustains for the access patterns
// of the all-reduce, measured with plain streaming kernels.
//
//   gradient_all_reduce_allreduce_amd/hbm_patterns
//
// The ring all-reduce of P buffers reads P streams and writes P streams; its
// roofline is HBM bandwidth for that read/write mix, not the read-only peak.
// This program times, with hipEvents over 40 repetitions each:
//   read   -- 2 GiB read with 16-byte non-temporal loads (XOR-folded)
//   write  -- 2 GiB written with 16-byte stores, plain and non-temporal
//   copy   -- 2 GiB read + 2 GiB written, 16-byte non-temporal loads, and
//             non-temporal or ordinary stores
//   red8   -- the all-reduce's own pattern: 8 input streams summed into 8
//             identical output streams (25 MiB each, 4 rotating buffer sets
//             = 1.6 GiB, more than the last-level cache), with the 16
//             buffers (a) separately allocated, (b) packed back to back in
//             one allocation, (c) in one allocation with an extra 4 KiB
//             between neighbours; each with 2 vectors per lane and a common
//             store order, and with 1 vector per lane and the store order
//             rotated per wave (non-temporal or ordinary stores).
// Every kernel uses one tile of 256 lanes x U vectors per workgroup and as
// many workgroups as tiles.  Output: one line per measurement, GB/s of bytes
// moved (read + written).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CK(x)                                                                  \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                      \
        }                                                                      \
    } while (0)

constexpr int kBlock = 256;
constexpr int kU = 2;

__global__ __launch_bounds__(kBlock) void read_kernel(const u32x4* a, uint32_t nvec, uint32_t* sink) {
    const uint32_t t = blockIdx.x * (kBlock * kU);
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t i = t + u * kBlock + threadIdx.x;
        if (i < nvec) acc ^= __builtin_nontemporal_load(a + i);
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) sink[0] = 1u;   // keeps the loads
}

template <bool NT>
__global__ __launch_bounds__(kBlock) void write_kernel(u32x4* a, uint32_t nvec) {
    const uint32_t t = blockIdx.x * (kBlock * kU);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t i = t + u * kBlock + threadIdx.x;
        const u32x4 v = {i, i, i, i};
        if (i < nvec) {
            if (NT) __builtin_nontemporal_store(v, a + i); else a[i] = v;
        }
    }
}

template <bool NT>
__global__ __launch_bounds__(kBlock) void copy_kernel(const u32x4* a, u32x4* b, uint32_t nvec) {
    const uint32_t t = blockIdx.x * (kBlock * kU);
    u32x4 x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t i = t + u * kBlock + threadIdx.x;
        if (i < nvec) x[u] = __builtin_nontemporal_load(a + i);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t i = t + u * kBlock + threadIdx.x;
        if (i < nvec) {
            if (NT) __builtin_nontemporal_store(x[u], b + i); else b[i] = x[u];
        }
    }
}

struct Streams8 {
    const u32x4* in[8];
    u32x4* out[8];
};

// The same pattern with one 16-byte vector per lane and the order of the 8
// output stores rotated by the wave index (each wave starts at another
// output stream); NT selects non-temporal or ordinary stores.
template <bool NT>
__global__ __launch_bounds__(kBlock) void red8_rotated_kernel(Streams8 p, uint32_t nvec) {
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= nvec) return;
    u32x4 x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = __builtin_nontemporal_load(p.in[r] + i);
    u32x4 s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float acc = __uint_as_float(x[0][k]);
#pragma unroll
        for (int r = 1; r < 8; ++r) acc = acc + __uint_as_float(x[r][k]);
        s[k] = __float_as_uint(acc);
    }
    const int rot = __builtin_amdgcn_readfirstlane(static_cast<int>((blockIdx.x * (kBlock / 64) + threadIdx.x / 64) & 7));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int want = (q + rot) & 7;
        u32x4* o = p.out[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) o = want == j ? p.out[j] : o;
        if (NT) __builtin_nontemporal_store(s, o + i); else o[i] = s;
    }
}

__global__ __launch_bounds__(kBlock) void red8_kernel(Streams8 p, uint32_t nvec) {
    const uint32_t t = blockIdx.x * (kBlock * kU);
    u32x4 x[8][kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t i = t + u * kBlock + threadIdx.x;
#pragma unroll
        for (int r = 0; r < 8; ++r) x[r][u] = i < nvec ? __builtin_nontemporal_load(p.in[r] + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t i = t + u * kBlock + threadIdx.x;
        if (i >= nvec) continue;
        u32x4 s;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float acc = __uint_as_float(x[0][u][k]);
#pragma unroll
            for (int r = 1; r < 8; ++r) acc = acc + __uint_as_float(x[r][u][k]);
            s[k] = __float_as_uint(acc);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) __builtin_nontemporal_store(s, p.out[r] + i);
    }
}

template <typename F>
static float time_ms(F launch, int reps = 40) {
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    launch(0);
    launch(1);
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(a));
    for (int i = 0; i < reps; ++i) launch(i);
    CK(hipEventRecord(b));
    CK(hipEventSynchronize(b));
    float ms = 0.f;
    CK(hipEventElapsedTime(&ms, a, b));
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    return ms / reps;
}

static unsigned grid_for(uint32_t nvec) { return (nvec + kBlock * kU - 1) / (kBlock * kU); }

int main() {
    const size_t big = size_t(2) << 30;
    const uint32_t nvec = static_cast<uint32_t>(big / 16);
    char* A = nullptr;
    char* B = nullptr;
    uint32_t* sink = nullptr;
    CK(hipMalloc(&A, big));
    CK(hipMalloc(&B, big));
    CK(hipMalloc(&sink, 64));
    CK(hipMemset(A, 1, big));
    CK(hipMemset(B, 2, big));
    const unsigned g = grid_for(nvec);

    float ms = time_ms([&](int) { read_kernel<<<g, kBlock>>>(reinterpret_cast<const u32x4*>(A), nvec, sink); });
    std::printf("read  nt          : %7.0f GB/s\n", big / ms / 1e6);
    ms = time_ms([&](int) { write_kernel<false><<<g, kBlock>>>(reinterpret_cast<u32x4*>(A), nvec); });
    std::printf("write plain       : %7.0f GB/s\n", big / ms / 1e6);
    ms = time_ms([&](int) { write_kernel<true><<<g, kBlock>>>(reinterpret_cast<u32x4*>(A), nvec); });
    std::printf("write nt          : %7.0f GB/s\n", big / ms / 1e6);
    ms = time_ms([&](int) {
        copy_kernel<true><<<g, kBlock>>>(reinterpret_cast<const u32x4*>(A), reinterpret_cast<u32x4*>(B), nvec);
    });
    std::printf("copy  nt          : %7.0f GB/s\n", 2.0 * big / ms / 1e6);
    ms = time_ms([&](int) {
        copy_kernel<false><<<g, kBlock>>>(reinterpret_cast<const u32x4*>(A), reinterpret_cast<u32x4*>(B), nvec);
    });
    std::printf("copy  nt load, plain store: %7.0f GB/s\n", 2.0 * big / ms / 1e6);

    const size_t rb = size_t(25) << 20;               // 25 MiB per stream
    const uint32_t rv = static_cast<uint32_t>(rb / 16);
    const int sets = 4;
    std::vector<char*> separate;
    for (int s = 0; s < 16 * sets; ++s) {
        char* p = nullptr;
        CK(hipMalloc(&p, rb));
        CK(hipMemset(p, 0, rb));
        separate.push_back(p);
    }
    const size_t max_stride = rb + 4096;
    char* arena = nullptr;
    CK(hipMalloc(&arena, max_stride * 16 * sets));
    CK(hipMemset(arena, 0, max_stride * 16 * sets));
    const char* names[3] = {"separate allocations", "one allocation, stride 25 MiB",
                            "one allocation, stride 25 MiB + 4 KiB"};
    for (int layout = 0; layout < 3; ++layout) {
        const size_t stride = layout == 2 ? max_stride : rb;
        Streams8 ps[sets];
        for (int s = 0; s < sets; ++s) {
            for (int r = 0; r < 8; ++r) {
                char* in = layout == 0 ? separate[s * 16 + r] : arena + (s * 16 + r) * stride;
                char* out = layout == 0 ? separate[s * 16 + 8 + r] : arena + (s * 16 + 8 + r) * stride;
                ps[s].in[r] = reinterpret_cast<const u32x4*>(in);
                ps[s].out[r] = reinterpret_cast<u32x4*>(out);
            }
        }
        ms = time_ms([&](int i) { red8_kernel<<<grid_for(rv), kBlock>>>(ps[i % sets], rv); });
        std::printf("red8  %-38s: %7.0f GB/s (%.1f us per 25 MiB x 16 streams)\n", names[layout],
                    16.0 * rb / ms / 1e6, ms * 1e3);
        ms = time_ms([&](int i) { red8_rotated_kernel<true><<<(rv + kBlock - 1) / kBlock, kBlock>>>(ps[i % sets], rv); });
        std::printf("red8  %-38s: %7.0f GB/s (%.1f us) one vector per lane, rotated stores\n",
                    names[layout], 16.0 * rb / ms / 1e6, ms * 1e3);
        ms = time_ms([&](int i) { red8_rotated_kernel<false><<<(rv + kBlock - 1) / kBlock, kBlock>>>(ps[i % sets], rv); });
        std::printf("red8  %-38s: %7.0f GB/s (%.1f us) one vector per lane, rotated plain stores\n",
                    names[layout], 16.0 * rb / ms / 1e6, ms * 1e3);
    }
    for (char* p : separate) CK(hipFree(p));
    CK(hipFree(arena));
    CK(hipFree(A));
    CK(hipFree(B));
    CK(hipFree(sink));
    return 0;
}
