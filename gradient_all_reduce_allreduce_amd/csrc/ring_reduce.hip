// ring_reduce.hip -- host-side launch of the ring all-reduce kernels
// (device code in ring_reduce_impl.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <unordered_map>

#include "launch.h"
#include "ring_reduce_impl.h"

namespace ddp {
namespace {

// Buffers longer than this go out in several launches so that lane offsets
// stay 32-bit; a multiple of every vector width, so each launch's first
// element stays 16-byte aligned.
constexpr int64_t kMaxLaunchElems = int64_t(1) << 29;

const void* select_kernel(const RingLaunch& l, int scalar) {
    if (l.in_bf16) {
        return l.out_bf16 ? ring_kernel_bf16_bf16(l.P, l.sgd, scalar) : ring_kernel_bf16_f32(l.P, l.sgd, scalar);
    }
    return l.out_bf16 ? ring_kernel_f32_bf16(l.P, l.sgd, scalar) : ring_kernel_f32_f32(l.P, l.sgd, scalar);
}

struct DeviceInfo {
    int cus = 0;
    std::unordered_map<const void*, int> blocks_per_cu;
};

std::mutex g_mutex;
std::unordered_map<int, DeviceInfo> g_devices;

// Resident workgroups of `fn` on the current device (CUs x blocks per CU),
// or -(HIP error).
int resident_blocks(const void* fn, const char** msg) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *msg = "hipGetDevice";
        return -static_cast<int>(e);
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceInfo& info = g_devices[dev];
    if (info.cus == 0) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || cus <= 0) {
            *msg = "hipDeviceGetAttribute(MultiprocessorCount)";
            return -static_cast<int>(e == hipSuccess ? hipErrorInvalidValue : e);
        }
        info.cus = cus;
    }
    auto it = info.blocks_per_cu.find(fn);
    if (it == info.blocks_per_cu.end()) {
        int nb = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, rr::kBlock, 0);
        if (e != hipSuccess || nb <= 0) {
            *msg = "hipOccupancyMaxActiveBlocksPerMultiprocessor";
            return -static_cast<int>(e == hipSuccess ? hipErrorInvalidValue : e);
        }
        it = info.blocks_per_cu.emplace(fn, nb).first;
    }
    return info.cus * it->second;
}

}  // namespace

int launch_ring_reduce(const RingLaunch& l, const char** msg) {
    if (l.n <= 0) return 0;
    const int64_t V = l.in_bf16 ? 8 : 4;
    const int64_t tile = static_cast<int64_t>(rr::kBlock) * ring_vectors_per_lane(l.P) * V;
    const int64_t L = (l.n + l.chunking - 1) / l.chunking;
    const int scalar = L < tile ? 1 : 0;
    const void* fn = select_kernel(l, scalar);
    if (fn == nullptr) {
        *msg = "no kernel for this rank count";
        return static_cast<int>(hipErrorInvalidValue);
    }
    const int slots = resident_blocks(fn, msg);
    if (slots < 0) return -slots;
    const int ies = l.in_bf16 ? 2 : 4;
    const int oes = l.out_bf16 ? 2 : 4;

    for (int64_t base = 0; base < l.n; base += kMaxLaunchElems) {
        const int64_t n = l.n - base < kMaxLaunchElems ? l.n - base : kMaxLaunchElems;
        rr::RingArgs a{};
        for (int r = 0; r < l.P; ++r) {
            a.in[r] = static_cast<const char*>(l.in[r]) + base * ies;
            a.out[r] = l.out[r] ? static_cast<char*>(l.out[r]) + base * oes : nullptr;
        }
        a.w = l.w ? l.w + base : nullptr;
        a.v = l.v ? l.v + base : nullptr;
        a.lr = l.lr;
        a.mu = l.mu;
        a.base = base;
        a.L = L;
        a.n = static_cast<uint32_t>(n);
        a.n_vec = static_cast<uint32_t>(n - n % V);
        a.mean = l.op == DDP_MEAN;
        a.write_out = l.write_out;

        int64_t grid = 1;
        if (scalar) {
            a.per_block = 0;
            const int64_t need = (n + rr::kBlock - 1) / rr::kBlock;
            grid = need < slots ? need : slots;
        } else if (a.n_vec > 0) {
            // Balanced contiguous shares in whole rows of 256 vectors, one
            // share per resident workgroup.
            const int64_t row = rr::kBlock * V;
            const int64_t rows = (a.n_vec + row - 1) / row;
            const int64_t rows_per_block = (rows + slots - 1) / slots;
            a.per_block = static_cast<uint32_t>(rows_per_block * row);
            grid = (a.n_vec + a.per_block - 1) / a.per_block;
        } else {
            a.per_block = static_cast<uint32_t>(rr::kBlock * V);
        }
        if (grid < 1) grid = 1;
        void* args[] = {&a};
        const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(rr::kBlock), args, 0,
                                             static_cast<hipStream_t>(l.stream));
        if (e != hipSuccess) {
            *msg = "hipLaunchKernel(ring_reduce)";
            return static_cast<int>(e);
        }
    }
    return 0;
}

}  // namespace ddp
