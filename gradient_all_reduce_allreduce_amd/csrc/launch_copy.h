// Launch interface of bucket pack and unpack (bucket_copy.hip) between
// api.cpp and the kernel.  Internal, like launch.h.
#pragma once

#include "launch.h"

namespace ddp {

// Resident 256-lane workgroups per CU (32 waves at a cap of 8): measured
// best at 8 with 2 vectors per lane, on the ResNet-50 set and on 2,000
// ragged tensors.
constexpr int kPackWgPerCu = 8;     // bucket pack
constexpr int kUnpackWgPerCu = 8;   // bucket unpack

// Bucket pack and unpack (bucket_copy.hip).  One launch covers a range of
// one bucket for all P ranks; its segment table travels in the kernel
// arguments (7.7 KB: kernel arguments of 8,000 bytes measured to arrive
// whole on this stack), so a launch holds at most
// copy_segments_per_launch(P) segments (110 at P = 8, enough for every
// bucket of the ResNet-50, ViT-B/16, transformer and 2,000-tensor sets) and
// a bucket with more goes out as several launches over consecutive ranges
// (api.cpp).
constexpr int kCopyMaxSegs = 128;     // segments per launch
constexpr int kCopyMaxPieces = 880;   // (segment, rank) tensor addresses per launch
constexpr int copy_segments_per_launch(int P) {
    return kCopyMaxPieces / P < kCopyMaxSegs ? kCopyMaxPieces / P : kCopyMaxSegs;
}
// Longest range of a bucket one launch covers, in elements (offsets inside
// a launch are 32-bit).
constexpr int64_t kCopyMaxLaunchElems = int64_t(1) << 30;

struct CopyLaunch {
    int P;
    int elem_bytes;    // 2 or 4
    int pack;          // 1: tensors -> bucket, 0: bucket -> tensors
    int32_t n_segs;    // segments of this launch, 1 .. copy_segments_per_launch(P)
    int32_t len;       // elements of the range, 1 .. kCopyMaxLaunchElems
    void* bucket[kMaxRanks];          // rank r's bucket at the range's first element (16-byte aligned)
    int32_t start[kCopyMaxSegs];      // segment k's first element in the range; start[0] = 0, increasing
    void* piece[kCopyMaxPieces];      // [k * P + r]: rank r's tensor address of segment k's first element
    void* stream;
};

// Elements per workgroup tile of the copy.
int64_t copy_tile_elems(int elem_bytes);
int launch_bucket_copy(const CopyLaunch& l, const char** msg);

}  // namespace ddp
