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
// reaches its highest rate with few waves per CU keeping requests in
// flight: a plain 8-in/8-out streaming kernel moves 6.36-6.42 TB/s with 3
// or 4 one-wave workgroups per CU against 5.5 TB/s with the CUs filled.  A
// launch therefore reserves LDS it never touches, so that at most a chosen
// number of its workgroups fit on a CU at once; the dispatcher still hands
// tiles to whichever CU frees up.  The best number depends on how many
// bytes a wave moves per tile (the rank count and element types) and on
// how long a tile takes to reach its first load, so it was measured for
// each kernel family: the tables below hold the fastest of 2..16 on
// 25 MiB buckets.  ddp_set_wg_per_cu overrides a family's choice.

constexpr unsigned kLdsBytesPerCu = 160u * 1024u;   // CDNA4 compute unit
// LDS goes to workgroups in granules of 1,280 bytes on this chip (measured:
// a 53,760-byte request lets 3 workgroups share a CU, 54,272 bytes only 2),
// so a request that is a multiple of the granule fits exactly
// floor(160 KiB / request) workgroups per CU.
constexpr unsigned kLdsGranule = 1280u;

// Dynamic LDS for a launch whose kernel already uses `static_bytes` (its
// own __shared__ arrays, as the compiler laid them out), such that at most
// `wg_per_cu` workgroups are resident per CU (0: no limit).  Never fewer
// than 2 per CU: a workgroup asking for the whole 160 KiB is refused.
constexpr unsigned lds_reserve(int wg_per_cu, unsigned static_bytes = 0) {
    if (wg_per_cu <= 0) return 0u;
    const unsigned k = static_cast<unsigned>(wg_per_cu < 2 ? 2 : wg_per_cu);
    const unsigned per = kLdsBytesPerCu / k / kLdsGranule * kLdsGranule;
    return per > static_bytes ? per - static_bytes : 0u;
}

// Lanes per workgroup of the ring, tree and multi-tensor kernels: one wave,
// so that the resident waves of a CU start and finish tiles independently.
constexpr int kRingBlock = 64;

// The fused all-reduce: resident one-wave workgroups per CU by element
// types and rank count P = 1..16 (index 0 unused; P = 1, a copy, takes
// P = 2's value; P = 7, 9-11 and 13-15 interpolate the measured neighbours).
// Rows: f32 -> f32, f32 -> bf16, bf16 -> f32, bf16 -> bf16.
constexpr signed char kRingWg[4][17] = {
    //   P: 1   2   3   4   5  6  7  8  9 10 11 12 13 14 15 16
    {0, 4, 4, 12, 8, 8, 6, 5, 4, 4, 4, 3, 3, 3, 3, 3, 3},
    {0, 12, 12, 16, 10, 10, 8, 6, 5, 5, 4, 4, 4, 4, 4, 4, 4},
    {0, 6, 6, 16, 10, 10, 8, 6, 5, 5, 4, 4, 4, 3, 3, 3, 3},
    {0, 6, 6, 12, 10, 8, 6, 6, 5, 5, 4, 4, 4, 3, 3, 3, 3},
};
// The all-reduce fused with the optimizer step, by gradient type and
// whether the reduced gradients (or updated parameters) are written to the
// ranks: rows bf16 without, bf16 with, f32 without, f32 with.
constexpr signed char kSgdWg[4][17] = {
    //   P: 1   2   3   4   5  6  7  8  9 10 11 12 13 14 15 16
    {0, 6, 6, 12, 16, 10, 10, 8, 8, 8, 8, 6, 6, 6, 6, 6, 6},
    {0, 4, 4, 10, 8, 8, 6, 6, 6, 6, 5, 4, 4, 4, 4, 4, 4},
    {0, 8, 8, 12, 16, 10, 8, 10, 10, 8, 8, 6, 5, 5, 5, 5, 5},
    {0, 3, 3, 6, 5, 5, 4, 4, 3, 3, 3, 3, 3, 3, 3, 2, 2},
};
constexpr int ring_wg_per_cu(int P, bool in_bf16, bool out_bf16) {
    return kRingWg[(in_bf16 ? 2 : 0) + (out_bf16 ? 1 : 0)][P];
}
constexpr int sgd_wg_per_cu(int P, bool grad_bf16, bool writes_ranks) {
    return kSgdWg[(grad_bf16 ? 0 : 2) + (writes_ranks ? 1 : 0)][P];
}
// A pause at the start of every workgroup of the fused all-reduce, in
// units of 64 clocks (s_sleep): 0 except where measured faster.  It acts as
// a fraction of a workgroup below the cap: a new workgroup issues its loads
// a little after the one it replaces finished.  bf16 -> f32 at P = 8 and 5
// workgroups per CU, on 100 MiB buckets: 6,389 GB/s with no pause, 6,505-6,512
// with 3, 4 or 5, 6,451 with 8; at 6 per CU a pause of 12 came to 6,477.
// For bf16 -> f32 at other rank counts (100 MiB buckets, C = P, the caps
// above; pauses 0, 2, 4, 8, 12, 16, 24 tried) the best pause and its gain:
// P = 3: 12 (+1.0%), 4: 4 (+0.7%), 5: 16 (+1.6%), 6: 16 (+2.9%), 7: 8
// (+3.8%), 9: 12 (+3.1%), 10: 8 (+3.6%), 11: 8 (+3.4%), 12: 12 (+2.7%),
// 13: 8 (+4.5%), 14: 8 (+5.4%), 15: 12 (+3.7%), 16: 8 (+4.6%); P = 2: none
// helped.  The best length does not follow P smoothly (at P = 16 a pause of
// 4 was slower than none), so each is the measured one.  For the other type pairs the best pause
// gained under 0.3% at most rank counts (0.6-1.2% at P = 12 and 16 only),
// and with the optimizer step under 0.7% (one isolated 2%): they keep none.
constexpr signed char kRingStartSleepBf16F32[17] = {
    //   P: 1  2   3  4   5   6  7  8   9 10 11  12 13 14  15 16
    0, 0, 0, 12, 4, 16, 16, 8, 4, 12, 8, 8, 12, 8, 8, 12, 8,
};
constexpr int ring_start_sleep(int P, bool in_bf16, bool out_bf16, bool sgd) {
    return (in_bf16 && !out_bf16 && !sgd) ? kRingStartSleepBf16F32[P] : 0;
}

// The tree strategies measured best one workgroup above the ring (5 at
// P = 8, f32; 4 and 6 were slower, also with the order table).
constexpr int tree_wg_per_cu(int P, bool in_bf16, bool out_bf16) {
    return ring_wg_per_cu(P, in_bf16, out_bf16) + 1;
}
// The ring's halves, measured at P = 8, f32, ResNet-50 buckets.  (The
// multi-tensor, stepwise and bucket-copy kernels keep their caps in their
// own headers: launch_multi.h, launch_step.h, launch_copy.h.)
constexpr int kRsWgPerCu = 10;      // reduce-scatter half
constexpr int kAgWgPerCu = 12;      // all-gather half

// The cap ddp_set_wg_per_cu set for a family (ddp_kernel_family): -1 if
// none (use the built-in choice), else the cap (0: no cap).  api.cpp.
int wg_per_cu_override(int family);

// The cap a launch of `family` uses: the override if set, else `builtin`.
inline int wg_per_cu_for(int family, int builtin) {
    const int o = wg_per_cu_override(family);
    return o >= 0 ? o : builtin;
}

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
    // kAllReduce: elements [seg2, n) are a second ring of their own with
    // seg2_chunking chunks (0: none).  Only for a single launch (n <= 2^29)
    // with seg2 a multiple of ring_tile_elems and whole chunks before it.
    int64_t seg2;
    int seg2_chunking;
};

// Returns 0 on success, else a HIP error code; *msg names the failing call.
int launch_ring_reduce(const RingLaunch& l, const char** msg);

// Elements per workgroup tile of the vector ring kernel for this launch.
int64_t ring_tile_elems(const RingLaunch& l);

// Elements per launch; longer buffers go out in several launches.
constexpr int64_t kMaxLaunchElems = int64_t(1) << 29;

// Vectors of each rank a lane keeps in flight per tile: P * U loads.  One
// vector per lane (a tile of 256 or 512 elements per wave) measured fastest
// from P = 3 up, with the fused optimizer step too once its occupancy cap
// was tuned for it (3-5% over two vectors); P <= 2 keeps more loads in
// flight with U = 4.
constexpr int ring_vectors_per_lane(int P, bool /*sgd*/) {
    return P <= 2 ? 4 : 1;
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

}  // namespace ddp
