// Internal interface between the C-ABI layer (api.cpp) and the HIP kernel
// translation units.  Not installed, not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/ddp_allreduce.h"

namespace ddp {

constexpr int kMaxRanks = DDP_MAX_RANKS;

// ---- launch shape -----------------------------------------------------------
//
// Every kernel here streams HBM with little arithmetic.  On MI355X the mix
// of reads and writes of the all-reduce (P input streams, P output streams)
// reaches its highest rate when few waves per CU keep requests in flight:
// 6.39 TB/s at 4 one-wave workgroups per CU against 5.7 TB/s with the CUs
// filled, in a plain 8-in/8-out streaming kernel.  A launch therefore
// reserves LDS it never touches, so that at most the chosen number of its
// workgroups fit on a CU at once; the dispatcher still hands tiles to
// whichever CU frees up.  The limit only pays where a tile's first load
// follows its start within a few dozen instructions: the multi-tensor and
// bucket-copy kernels, which search a table first, and the two halves of
// the ring measured slower with it, so they keep the hardware's occupancy.

constexpr unsigned kLdsBytesPerCu = 160u * 1024u;   // CDNA4 compute unit

// Dynamic LDS for a launch whose kernel already uses `static_bytes`, such
// that at most `wg_per_cu` workgroups are resident per CU (0: no limit).
constexpr unsigned lds_reserve(int wg_per_cu, unsigned static_bytes = 0) {
    if (wg_per_cu <= 0) return 0u;
    const unsigned per = (kLdsBytesPerCu / static_cast<unsigned>(wg_per_cu)) & ~1023u;
    return per > static_bytes ? per - static_bytes : 0u;
}

// Lanes per workgroup of the ring, tree and multi-tensor kernels: one wave,
// so that the resident waves of a CU start and finish tiles independently.
constexpr int kRingBlock = 64;
// Resident workgroups per CU for each kernel family (0: no limit).
constexpr int kRingWgPerCu = 4;     // fused all-reduce, tree strategies
constexpr int kSgdWgPerCu = 4;      // fused all-reduce + optimizer step
constexpr int kRsWgPerCu = 0;       // reduce-scatter half
constexpr int kAgWgPerCu = 0;       // all-gather half
constexpr int kMultiWgPerCu = 0;    // many tensors in one launch
constexpr int kStepWgPerCu = 0;     // one ring step per launch
constexpr int kCopyWgPerCu = 0;     // bucket pack / unpack

// What one launch sequence computes: the ring all-reduce (optionally with
// the fused optimizer step), one of its halves, or a fold along a tree
// (tree, centralized and two-level strategies).
enum RingMode { kAllReduce = 0, kReduceScatter = 1, kAllGather = 2, kTree = 3 };

// Everything launch_ring_reduce needs; validated by the caller (api.cpp).
struct RingLaunch {
    int mode;          // RingMode
    int P;
    int chunking;
    int op;            // DDP_SUM / DDP_MEAN
    int in_bf16;       // input element type is bf16
    int out_bf16;      // output element type is bf16
    int sgd;           // apply the momentum step to w, v
    int write_out;     // write to out[]: 1 the reduced gradient, 2 (with sgd) the updated weights
    const void* in[kMaxRanks];
    void* out[kMaxRanks];
    float* w;
    float* v;
    float lr;
    float mu;
    uint64_t parents;  // kTree: parent of fold register c in bits [4c, 4c+4)
    int groups;        // kTree: G nodes of P / G ranks, node-major (0 means 1)
    int local_chunking;   // kTree: chunk count of a ring within the nodes, 0 = fixed order
    int global_chunking;  // kTree: chunk count of a ring over the nodes, 0 = fixed order
    int64_t n;
    void* stream;
};

// Returns 0 on success, else a HIP error code; *msg names the failing call.
int launch_ring_reduce(const RingLaunch& l, const char** msg);

// Vectors of each rank a lane keeps in flight per tile: P * U loads.  One
// vector per lane (a tile of 256 or 512 elements per wave) measured fastest
// from P = 3 up; P <= 2 keeps more loads in flight with U = 4.  The fused
// optimizer step, whose outputs are the two 16-byte state vectors instead
// of P gradient copies, keeps two vectors per lane in flight.
constexpr int ring_vectors_per_lane(int P, bool sgd) {
    return P <= 2 ? 4 : (sgd ? 2 : 1);
}

// Elements per lane vector: 8 for bf16 -> bf16 (16-byte loads and stores),
// otherwise 4 so that float32 outputs and momentum state move as 16 bytes.
constexpr int ring_lane_elems(bool in_bf16, bool out_bf16, bool sgd) {
    return (in_bf16 && out_bf16 && !sgd) ? 8 : 4;
}

// Kernel entry points, one function per (input, output) element type pair;
// defined in ring_reduce_<in>_<out>.hip.  scalar: the one-element-per-lane
// variant for chunks shorter than a tile.
const void* ring_kernel_f32_f32(int P, int sgd, int scalar);
const void* ring_kernel_f32_bf16(int P, int sgd, int scalar);
const void* ring_kernel_bf16_f32(int P, int sgd, int scalar);
const void* ring_kernel_bf16_bf16(int P, int sgd, int scalar);
const void* ring_rs_kernel_f32_f32(int P, int scalar);
const void* ring_rs_kernel_f32_bf16(int P, int scalar);
const void* ring_rs_kernel_bf16_f32(int P, int scalar);
const void* ring_rs_kernel_bf16_bf16(int P, int scalar);
const void* tree_kernel_f32_f32(int P, int scalar);
const void* tree_kernel_f32_bf16(int P, int scalar);
const void* tree_kernel_bf16_f32(int P, int scalar);
const void* tree_kernel_bf16_bf16(int P, int scalar);
// All-gather kernels by element size (2 or 4 bytes); ring_allgather.hip.
const void* ring_ag_kernel(int elem_bytes, int P, int scalar);

// The ring one step per launch (ring_step.hip): fp32 rank buffers, in place.
struct StepLaunch {
    int P;
    int chunking;
    int op;
    float* buf[kMaxRanks];
    uint64_t* sent;    // device [P] counters of elements sent, or null
    int64_t n;
    void* stream;
};

int launch_ring_stepwise(const StepLaunch& l, const char** msg);

// Many tensors in one launch (multi_tensor.hip).
struct MultiLaunch {
    int P;
    int chunking;
    int op;
    int in_bf16;
    int out_bf16;
    int32_t T;
    const ddp_tensor_tiles* tiles;
    const void* const* in;
    void* const* out;           // may be null with sgd: no gradient output
    float* const* w;            // sgd: [T] device table of master weights
    float* const* v;            // sgd: [T] device table of momentum buffers
    float lr;
    float mu;
    int sgd;
    int64_t total_tiles;
    void* stream;
};

int64_t multi_tile_elems(int P, bool in_bf16, bool out_bf16);
int launch_multi_ring(const MultiLaunch& l, const char** msg);

struct CopyLaunch {
    int P;
    int elem_bytes;    // 2 or 4
    int pack;          // 1: tensors -> bucket, 0: bucket -> tensors
    const ddp_segment* segs;
    int64_t n_segs;
    const void* const* tensors;   // device array [P * n_tensors]
    int32_t n_tensors;
    void* bucket[kMaxRanks];
    int64_t bucket_len;
    void* stream;
};

int launch_bucket_copy(const CopyLaunch& l, const char** msg);

}  // namespace ddp
