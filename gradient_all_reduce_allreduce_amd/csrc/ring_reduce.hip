// ring_reduce.hip -- host-side launch of the ring kernels (device code in
// ring_reduce_impl.h): the fused all-reduce (optionally with SGD), and the
// reduce-scatter and all-gather halves on their own.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "ring_reduce_impl.h"

namespace ddp {
namespace {

const void* select_kernel(const RingLaunch& l, int scalar) {
    const int P = l.P;
    switch (l.mode) {
        case kReduceScatter:
            if (l.in_bf16) return l.out_bf16 ? ring_rs_kernel_bf16_bf16(P, scalar) : ring_rs_kernel_bf16_f32(P, scalar);
            return l.out_bf16 ? ring_rs_kernel_f32_bf16(P, scalar) : ring_rs_kernel_f32_f32(P, scalar);
        case kAllGather:
            return ring_ag_kernel(l.out_bf16 ? 2 : 4, P, scalar);
        case kTree:
            if (l.in_bf16) return l.out_bf16 ? tree_kernel_bf16_bf16(P, scalar) : tree_kernel_bf16_f32(P, scalar);
            return l.out_bf16 ? tree_kernel_f32_bf16(P, scalar) : tree_kernel_f32_f32(P, scalar);
        default:
            if (l.in_bf16) {
                return l.out_bf16 ? ring_kernel_bf16_bf16(P, l.sgd, scalar) : ring_kernel_bf16_f32(P, l.sgd, scalar);
            }
            return l.out_bf16 ? ring_kernel_f32_bf16(P, l.sgd, scalar) : ring_kernel_f32_f32(P, l.sgd, scalar);
    }
}

// Elements per lane vector and per tile of the vector kernel of this mode.
void tile_shape(const RingLaunch& l, int64_t* V, int64_t* tile) {
    if (l.mode == kAllGather) {
        *V = l.out_bf16 ? 8 : 4;
        *tile = static_cast<int64_t>(rr::kBlock) * *V;
        return;
    }
    const bool sgd = l.mode == kAllReduce && l.sgd;
    *V = ring_lane_elems(l.in_bf16 != 0, l.out_bf16 != 0, sgd);
    *tile = static_cast<int64_t>(rr::kBlock) * ring_vectors_per_lane(l.P, sgd) * *V;
}

// The 32-bit chunk map of a launch starting at global element `base` (see
// rr::ChunkMap): chunks of L elements, their start member taken modulo M.
// A launch holds at most 2^29 elements, so with d = L <= 2^30 every
// t + off stays below 2^31.  A longer chunk leaves at most one boundary in
// the launch, at local element tb; the divisor 2^30 with the origin shifted
// to put a multiple of it at tb gives the same chunk steps.
rr::ChunkMap chunk_map(int64_t base, int64_t L, int M) {
    constexpr int64_t kCap = int64_t(1) << 30;
    const int64_t first = base / L;
    const int64_t within = base - first * L;   // the launch's first element, inside its chunk
    rr::ChunkMap c;
    if (L <= kCap) {
        c.d = static_cast<uint32_t>(L);
        c.off = static_cast<uint32_t>(within);
    } else {
        const int64_t tb = L - within;            // first element of the next chunk
        c.d = static_cast<uint32_t>(kCap);
        c.off = tb <= kCap ? static_cast<uint32_t>(kCap - tb) : 0u;
    }
    c.m = 0xffffffffu / c.d;
    c.first = static_cast<uint32_t>(first % M);
    c.members = static_cast<uint32_t>(M);
    c.members_m = 0xffffffffu / c.members;
    return c;
}

// Resident workgroups per CU for the launches of this mode (launch.h).
int wg_per_cu(const RingLaunch& l) {
    const bool ib = l.in_bf16 != 0;
    const bool ob = l.out_bf16 != 0;
    switch (l.mode) {
        case kReduceScatter: return wg_per_cu_for(DDP_KF_REDUCE_SCATTER, kRsWgPerCu);
        case kAllGather: return wg_per_cu_for(DDP_KF_ALL_GATHER, kAgWgPerCu);
        case kTree: return wg_per_cu_for(DDP_KF_TREE, tree_wg_per_cu(l.P, ib, ob));
        default:
            if (l.sgd) return wg_per_cu_for(DDP_KF_RING_SGD, sgd_wg_per_cu(l.P, ib, l.write_out != 0));
            return wg_per_cu_for(DDP_KF_RING, ring_wg_per_cu(l.P, ib, ob));
    }
}

}  // namespace

int64_t ring_tile_elems(const RingLaunch& l) {
    int64_t V = 4, tile = 0;
    tile_shape(l, &V, &tile);
    return tile;
}

// Buffers longer than kMaxLaunchElems go out in several launches so that
// lane offsets stay 32-bit; it is a multiple of every lane-vector width, so
// each launch's first element stays 16-byte aligned.
int launch_ring_reduce(const RingLaunch& l, const char** msg) {
    if (l.n <= 0) return 0;
    if (l.mode == kAllGather && l.P == 1) return 0;   // one rank already holds everything
    int64_t V = 4, tile = 0;
    tile_shape(l, &V, &tile);
    const bool two = l.seg2 > 0 && l.seg2 < l.n;
    if (two && (l.mode != kAllReduce || l.n > kMaxLaunchElems || l.seg2 % tile != 0)) {
        *msg = "second segment not supported for this launch";
        return static_cast<int>(hipErrorInvalidValue);
    }
    // Chunk lengths: the ring's; for the tree strategies those of a ring
    // within the nodes (L) and over the nodes (Lg), or a length beyond any
    // index where a level's order is fixed.
    const int64_t kFixed = int64_t(1) << 62;
    const int groups = l.groups > 0 ? l.groups : 1;
    int64_t L, Lg = kFixed;
    if (l.mode == kTree) {
        L = l.local_chunking > 0 ? (l.n + l.local_chunking - 1) / l.local_chunking : kFixed;
        Lg = l.global_chunking > 0 ? (l.n + l.global_chunking - 1) / l.global_chunking : kFixed;
    } else if (two) {
        L = (l.seg2 + l.chunking - 1) / l.chunking;
        Lg = (l.n - l.seg2 + l.seg2_chunking - 1) / l.seg2_chunking;
    } else {
        L = (l.n + l.chunking - 1) / l.chunking;
    }
    // Chunks shorter than a tile would put several start ranks in one tile:
    // those calls use the one-element-per-lane kernels.
    const int scalar = (L < Lg ? L : Lg) < tile ? 1 : 0;
    const void* fn = select_kernel(l, scalar);
    if (fn == nullptr) {
        *msg = "no kernel for this rank count";
        return static_cast<int>(hipErrorInvalidValue);
    }
    const int ies = l.in_bf16 ? 2 : 4;
    const int oes = l.out_bf16 ? 2 : 4;

    for (int64_t base = 0; base < l.n; base += kMaxLaunchElems) {
        const int64_t n = l.n - base < kMaxLaunchElems ? l.n - base : kMaxLaunchElems;
        rr::RingArgs a{};
        for (int r = 0; r < l.P; ++r) {
            a.in[r] = l.in[r] ? static_cast<const char*>(l.in[r]) + base * ies : nullptr;
            a.out[r] = l.out[r] ? static_cast<char*>(l.out[r]) + base * oes : nullptr;
            a.in[r + l.P] = a.in[r];
            a.out[r + l.P] = a.out[r];
        }
        a.w = l.w ? l.w + base : nullptr;
        a.v = l.v ? l.v + base : nullptr;
        a.lr = l.lr;
        a.mu = l.mu;
        a.ring = chunk_map(base, L, l.mode == kTree ? l.P / groups : l.P);
        a.n = static_cast<uint32_t>(n);
        a.n_vec = static_cast<uint32_t>(n - n % V);
        a.mean = l.op == DDP_MEAN;
        a.write_out = l.write_out;
        a.parents = l.parents;
        a.global = two ? chunk_map(0, Lg, l.P) : chunk_map(base, Lg, groups);
        a.groups = groups;
        a.group_size = l.P / groups;
        a.seg2 = two ? static_cast<uint32_t>(l.seg2) : 0xffffffffu;

        int64_t grid;
        if (scalar) {
            grid = (n + rr::kBlock - 1) / rr::kBlock;
        } else {
            grid = (a.n_vec + tile - 1) / tile;   // one tile per workgroup
            if (grid < 1) grid = 1;               // the tail still needs a workgroup
        }
        rr::TreeArgs ta{};
        void* args[] = {&a};
        if (l.mode == kTree) {
            // Row s_g * Lr + s_l: rank k of the fold is node (s_g + k / Lr) mod G,
            // peer (s_l + k) mod Lr, as the kernels' level_ranks walks it.
            const int Lr = a.group_size;
            ta.ring = a;
            for (int sg = 0; sg < groups; ++sg)
                for (int sl = 0; sl < Lr; ++sl)
                    for (int k = 0; k < l.P; ++k)
                        ta.order_in[(sg * Lr + sl) * l.P + k] =
                            a.in[((sg + k / Lr) % groups) * Lr + (sl + k) % Lr];
            args[0] = &ta;
        }
        const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(rr::kBlock), args,
                                             lds_reserve(wg_per_cu(l)), static_cast<hipStream_t>(l.stream));
        if (e != hipSuccess) {
            *msg = "hipLaunchKernel(ring)";
            return static_cast<int>(e);
        }
    }
    return 0;
}

}  // namespace ddp
