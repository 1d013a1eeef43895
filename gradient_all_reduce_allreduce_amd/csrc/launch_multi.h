// Launch interface of the multi-tensor kernel (multi_tensor.hip) between
// api.cpp and the kernel.  Internal, like launch.h.
#pragma once

#include "launch.h"

namespace ddp {

// Resident one-wave workgroups per CU.  The multi-tensor kernel searches
// its tile plan and reads its pointers from device tables before its first
// load, and wants a few more waves than the ring: 6 at P = 8 (161 ResNet-50
// tensors, 152 ViT-B/16 tensors in bf16), 8 with the optimizer step, 10 at
// P = 4 (2,000 ragged tensors), each measured best of 3..20.
constexpr int multi_wg_per_cu(int P, bool sgd) { return P >= 6 ? (sgd ? 8 : 6) : 10; }

// Tiles per entry of the block map (ddp_multi_block_map): entry k is the
// tensor holding tile k * kMultiBlockTiles.
constexpr int kMultiBlockTiles = 64;

// With the block map (and P <= 8), each tile's workgroup also reads the
// plan entry and rank pointers of the tensor holding the tile this many
// tiles ahead, while its own data is in flight: a later tile on the same
// CU then finds them in the scalar cache.  768 (half the resident
// workgroups of a launch at P = 8) measured best of 768, 1536 and 3072 on
// the 161 ResNet-50 tensors, the 2,000 ragged tensors and 160 equal ones.
constexpr int kMultiPrefetchTiles = 768;

// Many tensors in one launch (multi_tensor.hip).
struct MultiLaunch {
    int P;
    int chunking;
    int op;
    int in_bf16;
    int out_bf16;
    int32_t T;
    const ddp_tensor_tiles* tiles;
    const int32_t* block_first;   // device [ceil(total_tiles / kMultiBlockTiles)], or null
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

// Size of the per-GPU scratch area of allreduce_multi_ring_noalloc (its
// tables: plan, block map, input and output pointer tables).
constexpr int64_t kNoAllocScratchBytes = int64_t(1) << 20;
// 8-byte words of table one fill launch carries in its arguments.
constexpr int kFillWords = 944;
// Devices (ordinals 0 .. kMaxScratchDevices - 1) the call can run on.
constexpr int kMaxScratchDevices = 64;

int64_t multi_tile_elems(int P, bool in_bf16, bool out_bf16);
// The device address of the scratch area of the GPU of `stream` (the
// current GPU for the null stream), looked up once per device, and that
// device's ordinal.
int noalloc_scratch(void* stream, void** ptr, int* device, const char** msg);
// Whether `stream` is capturing a graph.
int stream_capturing(void* stream, bool* capturing, const char** msg);
// Writes `bytes` (a multiple of 8) of host data to device memory at `dst`
// in stream order, with kernels that carry the data in their arguments
// (so a captured call's graph rewrites it at every replay); the host data
// may be reused when this returns.
int fill_scratch(void* dst, const void* src, size_t bytes, void* stream, const char** msg);
int launch_multi_ring(const MultiLaunch& l, const char** msg);

}  // namespace ddp
