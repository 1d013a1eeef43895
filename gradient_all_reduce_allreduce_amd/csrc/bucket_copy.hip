// bucket_copy.hip -- gather a bucket out of ragged gradient tensors (pack)
// and scatter it back (unpack), all P ranks in one launch, for gfx950.
//
// DDP packs gradients into fixed-size buckets before the all-reduce and
// every rank fills them in the same order ("Distributed Training", "Data
// parallelism and all-reduce"; FSDP's flattened units, "Sharded data
// parallelism").  The segments of a bucket say which piece of which tensor
// occupies which range of the bucket.
//
// The host validates the bucket's segments (they tile the bucket in order
// and stay inside their tensors) and writes the part of the table a launch
// covers into the launch's kernel arguments: where each segment starts in
// the launch's range of the bucket, and each rank's address of the
// segment's first element in its tensor.  The kernel reads nothing else, so
// no device-side table can disagree with what the host checked.  A bucket
// with more segments than one launch's arguments hold goes out as several
// launches over consecutive ranges of the bucket (host side, api.cpp).
//
// A pure copy: bound by HBM bandwidth, 2 * bucket bytes per rank.  One
// workgroup per (tile of the range, rank), as many workgroups as tiles, so
// that the dispatcher keeps every CU busy.  One uniform binary search over
// the segment starts (scalar loads of the kernel arguments) finds the
// segment holding the tile's first element.  Most tiles lie inside that one
// segment (tensors are long against a tile): every vector then maps to the
// tensor at a uniform offset and the tile moves with no further lookup.
// Otherwise the workgroup stages the segments overlapping the tile in LDS,
// and each lane finds the segment of each of its vectors with a short
// binary search there.  A vector (16 bytes on the bucket side, always
// aligned) that lies inside one segment moves as one 16-byte access on the
// bucket side and, on the tensor side, as one 16-byte access when the
// tensor address is aligned, else as element-size accesses; a lane issues
// all of those loads before its first store, so kVecPerLane vectors per
// lane are in flight.  Vectors across a segment boundary move element by
// element afterwards.  Pack stores the bucket with device-scope buffer
// stores, unpack stores the tensors non-temporally; each measured fastest
// of the store policies tried (ordinary, non-temporal, device scope).
// Every element of the range is written exactly once (the segments tile
// it), so no synchronisation between workgroups is needed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch_copy.h"

namespace ddp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kVecPerLane = 2;   // 16-byte vectors per lane and tile

// The kernel arguments: one range [0, len) of a bucket, in elements
// relative to the range's first element.  Segment k covers [start[k],
// start[k + 1]) (the last one up to len); rank r's tensor address of its
// first element is piece[k * P + r], with P = gridDim.y.
struct CopyArgs {
    char* bucket[kMaxRanks];        // rank r's bucket at the range's first element
    char* piece[kCopyMaxPieces];
    int32_t start[kCopyMaxSegs];    // start[0] = 0, increasing
    int32_t n_segs;                 // 1 .. copy_segments_per_launch(P)
    int32_t len;                    // elements in the range, < 2^30
    int32_t tile_elems;             // elements per tile (multiple of 16 / es)
    int32_t es;                     // element bytes, 2 or 4
};
static_assert(sizeof(CopyArgs) <= 7800, "the copy's kernel arguments must stay under the 8,000 bytes measured to pass");

typedef const __attribute__((address_space(4))) CopyArgs* KCopy;

__device__ __forceinline__ KCopy copy_args() {
    return (KCopy)(__builtin_amdgcn_kernarg_segment_ptr());
}

__device__ __forceinline__ void copy_elem(char* dst, const char* src, int es) {
    if (es == 4) {
        *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
    } else {
        *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src);
    }
}

// One 16-byte vector's worth of elements (4 float32 or 8 bf16) at an
// address aligned only to the element size, and the inverse.
__device__ __forceinline__ u32x4 load_elems(const char* p, int es) {
    u32x4 v;
    if (es == 4) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = q[j];
    } else {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = static_cast<uint32_t>(q[2 * j]) | (static_cast<uint32_t>(q[2 * j + 1]) << 16);
    }
    return v;
}

__device__ __forceinline__ void store_elems_nt(char* p, u32x4 v, int es) {
    if (es == 4) {
        uint32_t* q = reinterpret_cast<uint32_t*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(static_cast<uint32_t>(v[j]), q + j);
    } else {
        uint16_t* q = reinterpret_cast<uint16_t*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            __builtin_nontemporal_store(static_cast<uint16_t>(v[j] & 0xffffu), q + 2 * j);
            __builtin_nontemporal_store(static_cast<uint16_t>(v[j] >> 16), q + 2 * j + 1);
        }
    }
}

// Bucket-side stores of pack: a buffer store with device scope (sc1), the
// policy of the all-reduce's result stores, over the tile (measured 2%
// faster than ordinary stores, and faster than non-temporal ones).
__device__ __forceinline__ void store16_tile(char* tile_base, int32_t tile_bytes, int32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(
        v, __builtin_amdgcn_make_buffer_rsrc(tile_base, 0, tile_bytes, 0x00020000),
        static_cast<uint32_t>(off), 0, 16);
}

// Largest index g in [0, count) with start[g] <= e (start ascending,
// start[0] <= e).
__device__ __forceinline__ int lds_find(const int32_t* start, int count, int32_t e) {
    int lo = 0;
    int hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= e) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Largest segment index k in [k0, n_segs) with start[k] <= e, by a uniform
// binary search over the kernel arguments (start[k0] <= e).
__device__ __forceinline__ int arg_find(KCopy a, int k0, int32_t e) {
    int lo = k0;
    int hi = a->n_segs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a->start[mid] <= e) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <bool PACK>
__global__ __launch_bounds__(kBlock) void bucket_copy_kernel(CopyArgs) {
    __shared__ int32_t s_start[kCopyMaxSegs + 1];   // the staged segments' starts, then the last one's end
    __shared__ char* s_ten[kCopyMaxSegs];           // this rank's tensor address at each staged start

    const KCopy a = copy_args();
    const int tid = threadIdx.x;
    const int rank = blockIdx.y;
    const int P = gridDim.y;
    char* const bucket = a->bucket[rank];
    const int es = a->es;
    const int ve = 16 / es;   // elements per 16-byte vector
    const int32_t len = a->len;
    const int32_t lo = static_cast<int32_t>(blockIdx.x) * a->tile_elems;
    const int32_t hi = lo + a->tile_elems < len ? lo + a->tile_elems : len;
    const int32_t tile_bytes = (hi - lo) * es;

    // The segment holding element lo (the same search in every lane).
    const int f = arg_find(a, 0, lo);
    const int32_t f_end = f + 1 < a->n_segs ? a->start[f + 1] : len;

    // Most tiles lie inside one segment (tensors are long against a tile):
    // then every vector maps to that tensor at a uniform offset, with no
    // staging and no per-lane search.
    if (f_end >= hi) {
        char* const ten = a->piece[f * P + rank] + static_cast<int64_t>(lo - a->start[f]) * es;
        const bool aligned = (reinterpret_cast<uintptr_t>(ten) & 15u) == 0;   // uniform
        u32x4 x[kVecPerLane];
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            const int32_t d = (u * kBlock + tid) * ve;   // element offset in the tile
            if (lo + d + ve > hi) continue;
            const char* src = PACK ? ten + static_cast<int64_t>(d) * es : bucket + static_cast<int64_t>(lo + d) * es;
            if (!PACK || aligned) {
                x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
            } else {
                x[u] = load_elems(src, es);
            }
        }
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            const int32_t d = (u * kBlock + tid) * ve;
            if (lo + d + ve > hi) continue;
            if (PACK) {
                store16_tile(bucket + static_cast<int64_t>(lo) * es, tile_bytes, d * es, x[u]);
            } else if (aligned) {
                __builtin_nontemporal_store(x[u], reinterpret_cast<u32x4*>(ten + static_cast<int64_t>(d) * es));
            } else {
                store_elems_nt(ten + static_cast<int64_t>(d) * es, x[u], es);
            }
        }
        // A partial last vector (the range's end): element by element.
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            const int32_t d = (u * kBlock + tid) * ve;
            if (lo + d >= hi || lo + d + ve <= hi) continue;
            for (int32_t e = lo + d; e < hi; ++e) {
                char* pb = bucket + static_cast<int64_t>(e) * es;
                char* pt = ten + static_cast<int64_t>(e - lo) * es;
                if (PACK) copy_elem(pb, pt, es); else copy_elem(pt, pb, es);
            }
        }
        return;
    }

    // Several segments overlap the tile: f .. g, at most n_segs of them,
    // fewer than the workgroup's lanes.  Stage them in LDS.
    const int g = arg_find(a, f, hi - 1);
    const int count = g - f + 1;
    if (tid < count) {
        const int k = f + tid;
        s_start[tid] = a->start[k];
        s_ten[tid] = a->piece[k * P + rank];
    }
    if (tid == 0) s_start[count] = g + 1 < a->n_segs ? a->start[g + 1] : len;
    __syncthreads();

    // Vectors inside one segment: every load first, then every store.  The
    // bucket side is always 16-byte aligned; the tensor side moves as one
    // 16-byte access when aligned, else element by element.
    u32x4 x[kVecPerLane];
    char* tn[kVecPerLane];
    int cls[kVecPerLane];   // 0 nothing here, 1 aligned, 2 misaligned tensor, 3 across segments
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) {
        const int32_t e0 = lo + (u * kBlock + tid) * ve;
        const int32_t e1 = e0 + ve;
        cls[u] = 0;
        tn[u] = nullptr;
        if (e0 < hi) {
            cls[u] = 3;
            if (e1 <= hi) {
                const int s = lds_find(s_start, count, e0);
                if (e1 <= s_start[s + 1]) {
                    tn[u] = s_ten[s] + static_cast<int64_t>(e0 - s_start[s]) * es;
                    cls[u] = (reinterpret_cast<uintptr_t>(tn[u]) & 15u) == 0 ? 1 : 2;
                }
            }
        }
        const char* bk = bucket + static_cast<int64_t>(e0) * es;
        if (cls[u] == 1) {
            x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(PACK ? tn[u] : bk));
        } else if (cls[u] == 2) {
            if (PACK) {
                x[u] = load_elems(tn[u], es);
            } else {
                x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bk));
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) {
        const int32_t d = (u * kBlock + tid) * ve;   // element offset in the tile
        if (cls[u] == 1) {
            if (PACK) {
                store16_tile(bucket + static_cast<int64_t>(lo) * es, tile_bytes, d * es, x[u]);
            } else {
                __builtin_nontemporal_store(x[u], reinterpret_cast<u32x4*>(tn[u]));
            }
        } else if (cls[u] == 2) {
            if (PACK) {
                store16_tile(bucket + static_cast<int64_t>(lo) * es, tile_bytes, d * es, x[u]);
            } else {
                store_elems_nt(tn[u], x[u], es);
            }
        }
    }

    // Vectors across a segment boundary, or cut by the range's end: element
    // by element.
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) {
        if (cls[u] != 3) continue;
        const int32_t e0 = lo + (u * kBlock + tid) * ve;
        const int32_t e1 = e0 + ve < hi ? e0 + ve : hi;
        int s = lds_find(s_start, count, e0);
        for (int32_t e = e0; e < e1; ++e) {
            while (e >= s_start[s + 1]) ++s;
            char* pb = bucket + static_cast<int64_t>(e) * es;
            char* pt = s_ten[s] + static_cast<int64_t>(e - s_start[s]) * es;
            if (PACK) copy_elem(pb, pt, es); else copy_elem(pt, pb, es);
        }
    }
}

// Static LDS of a kernel; if the runtime cannot say, a bound above what the
// staged-segment arrays take.
unsigned static_lds(const void* fn) {
    hipFuncAttributes at{};
    if (hipFuncGetAttributes(&at, fn) != hipSuccess) return 2048u;
    return static_cast<unsigned>(at.sharedSizeBytes);
}

}  // namespace

int64_t copy_tile_elems(int elem_bytes) { return static_cast<int64_t>(kBlock) * kVecPerLane * (16 / elem_bytes); }

int launch_bucket_copy(const CopyLaunch& l, const char** msg) {
    if (l.len <= 0) return 0;
    CopyArgs a{};
    for (int r = 0; r < l.P; ++r) a.bucket[r] = static_cast<char*>(l.bucket[r]);
    for (int k = 0; k < l.n_segs; ++k) {
        a.start[k] = l.start[k];
        for (int r = 0; r < l.P; ++r) a.piece[k * l.P + r] = static_cast<char*>(l.piece[k * l.P + r]);
    }
    a.n_segs = l.n_segs;
    a.len = l.len;
    a.es = l.elem_bytes;
    a.tile_elems = static_cast<int32_t>(copy_tile_elems(l.elem_bytes));
    const int64_t tiles = (static_cast<int64_t>(l.len) + a.tile_elems - 1) / a.tile_elems;

    const void* fn = l.pack ? reinterpret_cast<const void*>(&bucket_copy_kernel<true>)
                            : reinterpret_cast<const void*>(&bucket_copy_kernel<false>);
    // The kernel's own LDS (the staged segments), as the compiler laid it
    // out, counts against the per-CU share.
    static const unsigned own_lds[2] = {static_lds(reinterpret_cast<const void*>(&bucket_copy_kernel<false>)),
                                        static_lds(reinterpret_cast<const void*>(&bucket_copy_kernel<true>))};
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(l.P)),
                                         dim3(kBlock), args, lds_reserve(wg_per_cu_for(DDP_KF_BUCKET_COPY, l.pack ? kPackWgPerCu : kUnpackWgPerCu),
                                                           own_lds[l.pack ? 1 : 0]),
                                         static_cast<hipStream_t>(l.stream));
    if (e != hipSuccess) {
        *msg = "hipLaunchKernel(bucket_copy)";
        return static_cast<int>(e);
    }
    return 0;
}

}  // namespace ddp
