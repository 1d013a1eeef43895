// bucket_copy.hip -- gather a bucket out of ragged gradient tensors (pack)
// and scatter it back (unpack), all P ranks in one launch, for gfx950.
//
// DDP packs gradients into fixed-size buckets before the all-reduce and
// every rank fills them in the same order ("Distributed Training", "Data
// parallelism and all-reduce"; FSDP's flattened units, "Sharded data
// parallelism").  The segment table of a bucket says which piece of which
// tensor occupies which range of the bucket.
//
// A pure copy: bound by HBM bandwidth, 2 * bucket bytes per rank.  One
// workgroup per (tile of the bucket, rank), as many workgroups as tiles, so
// that the dispatcher keeps every CU busy.  One uniform binary search in
// the segment table finds the segment holding the tile's first element.
// Most tiles lie inside that one segment (tensors are long against a tile):
// every vector then maps to the tensor at a uniform offset and the tile
// moves with no further lookup.  Otherwise the workgroup stages the
// overlapping segments in LDS, so that each lane finds the segment of each
// of its vectors with a short binary search in LDS instead of a chain of
// dependent global loads.  A vector (16 bytes on the bucket side, always
// aligned) that lies inside one segment moves as one 16-byte access on the
// bucket side and, on the tensor side, as one 16-byte access when the
// tensor address is aligned, else as element-size accesses; a lane issues
// all of those loads before its first store, so kVecPerLane vectors per
// lane are in flight.  Vectors across a segment boundary move element by
// element afterwards.  Pack stores the bucket with device-scope buffer
// stores, unpack stores the tensors non-temporally; each measured fastest
// of the store policies tried (ordinary, non-temporal, device scope).
// Every bucket element is written exactly once (the segments tile the
// bucket), so no synchronisation between workgroups is needed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ddp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kVecPerLane = 2;   // 16-byte vectors per lane and tile

struct CopyArgs {
    const ddp_segment* segs;
    int64_t n_segs;
    const void* const* tensors;   // [P * n_tensors], rank-major
    int32_t n_tensors;
    int32_t es;                   // element bytes, 2 or 4
    void* bucket[kMaxRanks];
    int64_t bucket_len;
    int64_t tile_elems;           // elements per tile (multiple of 16 / es)
    int64_t tiles;
};

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
__device__ __forceinline__ void store16_tile(char* tile_base, int64_t tile_bytes, int64_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(
        v, __builtin_amdgcn_make_buffer_rsrc(tile_base, 0, static_cast<int>(tile_bytes), 0x00020000),
        static_cast<uint32_t>(off), 0, 16);
}

// Largest index g in [0, count) with dst[g] <= e (dst sorted ascending,
// dst[0] <= e).
__device__ __forceinline__ int lds_find(const int64_t* dst, int count, int64_t e) {
    int lo = 0;
    int hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (dst[mid] <= e) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <bool PACK>
__global__ __launch_bounds__(kBlock) void bucket_copy_kernel(CopyArgs a) {
    __shared__ int64_t s_dst[kBlock];
    __shared__ int64_t s_len[kBlock];
    __shared__ char* s_ten[kBlock];

    const int tid = threadIdx.x;
    const int rank = blockIdx.y;
    char* const bucket = static_cast<char*>(a.bucket[rank]);
    const void* const* tensors = a.tensors + static_cast<int64_t>(rank) * a.n_tensors;
    const int es = a.es;
    const int ve = 16 / es;   // elements per 16-byte vector
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * a.tile_elems;
    const int64_t hi = lo + a.tile_elems < a.bucket_len ? lo + a.tile_elems : a.bucket_len;

    // First segment holding element lo (the same search in every lane).
    int64_t f = 0;
    {
        int64_t l = 0;
        int64_t h = a.n_segs - 1;
        while (l < h) {
            const int64_t mid = (l + h + 1) >> 1;
            if (a.segs[mid].dst_off <= lo) l = mid; else h = mid - 1;
        }
        f = l;
    }

    // Most tiles lie inside one segment (tensors are long against a tile):
    // then every vector maps to that tensor at a uniform offset, with no
    // staging and no per-lane search.
    {
        const ddp_segment sg = a.segs[f];
        if (sg.dst_off + sg.len >= hi) {
            const char* ten = static_cast<const char*>(tensors[sg.tensor]) + (sg.src_off + (lo - sg.dst_off)) * es;
            const bool aligned = (reinterpret_cast<uintptr_t>(ten) & 15u) == 0;   // uniform
            u32x4 x[kVecPerLane];
#pragma unroll
            for (int u = 0; u < kVecPerLane; ++u) {
                const int64_t d = static_cast<int64_t>(u * kBlock + tid) * ve;   // element offset in the tile
                if (lo + d + ve > hi) continue;
                const char* src = PACK ? ten + d * es : bucket + (lo + d) * es;
                if (!PACK || aligned) {
                    x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
                } else {
                    x[u] = load_elems(src, es);
                }
            }
#pragma unroll
            for (int u = 0; u < kVecPerLane; ++u) {
                const int64_t d = static_cast<int64_t>(u * kBlock + tid) * ve;
                if (lo + d + ve > hi) continue;
                if (PACK) {
                    store16_tile(bucket + lo * es, (hi - lo) * es, d * es, x[u]);
                } else if (aligned) {
                    __builtin_nontemporal_store(x[u], reinterpret_cast<u32x4*>(const_cast<char*>(ten) + d * es));
                } else {
                    store_elems_nt(const_cast<char*>(ten) + d * es, x[u], es);
                }
            }
            // A partial last vector (the bucket's end): element by element.
#pragma unroll
            for (int u = 0; u < kVecPerLane; ++u) {
                const int64_t d = static_cast<int64_t>(u * kBlock + tid) * ve;
                if (lo + d >= hi || lo + d + ve <= hi) continue;
                for (int64_t e = lo + d; e < hi; ++e) {
                    char* pb = bucket + e * es;
                    char* pt = const_cast<char*>(ten) + (e - lo) * es;
                    if (PACK) copy_elem(pb, pt, es); else copy_elem(pt, pb, es);
                }
            }
            return;
        }
    }

    while (true) {
        const int64_t k = f + tid;
        const bool valid = k < a.n_segs && a.segs[k].dst_off < hi;
        if (valid) {
            const ddp_segment sg = a.segs[k];
            s_dst[tid] = sg.dst_off;
            s_len[tid] = sg.len;
            s_ten[tid] = static_cast<char*>(const_cast<void*>(tensors[sg.tensor])) + sg.src_off * es;
        }
        const int count = __syncthreads_count(valid);   // valid lanes form a prefix
        const int64_t cov_lo = s_dst[0] > lo ? s_dst[0] : lo;
        const int64_t last_end = s_dst[count - 1] + s_len[count - 1];
        const int64_t cov_hi = last_end < hi ? last_end : hi;

        // Vectors inside one segment: every load first, then every store.
        // The bucket side is always 16-byte aligned; the tensor side moves
        // as one 16-byte access when aligned, else element by element.
        u32x4 x[kVecPerLane];
        char* tn[kVecPerLane];
        int cls[kVecPerLane];   // 0 nothing here, 1 aligned, 2 misaligned tensor, 3 across segments
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            const int64_t e0 = lo + static_cast<int64_t>(u * kBlock + tid) * ve;
            const int64_t e1 = e0 + ve;
            cls[u] = 0;
            tn[u] = nullptr;
            if (e0 < cov_hi && e1 > cov_lo) {
                cls[u] = 3;
                if (e0 >= cov_lo && e1 <= cov_hi) {
                    const int g = lds_find(s_dst, count, e0);
                    if (e1 <= s_dst[g] + s_len[g]) {
                        tn[u] = s_ten[g] + (e0 - s_dst[g]) * es;
                        cls[u] = (reinterpret_cast<uintptr_t>(tn[u]) & 15u) == 0 ? 1 : 2;
                    }
                }
            }
            const char* bk = bucket + e0 * es;
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
            const int64_t d = static_cast<int64_t>(u * kBlock + tid) * ve;   // element offset in the tile
            if (cls[u] == 1) {
                if (PACK) {
                    store16_tile(bucket + lo * es, (hi - lo) * es, d * es, x[u]);
                } else {
                    __builtin_nontemporal_store(x[u], reinterpret_cast<u32x4*>(tn[u]));
                }
            } else if (cls[u] == 2) {
                if (PACK) {
                    store16_tile(bucket + lo * es, (hi - lo) * es, d * es, x[u]);
                } else {
                    store_elems_nt(tn[u], x[u], es);
                }
            }
        }

        // Vectors across a segment boundary, or partly covered by this
        // round's segments: element by element.
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            if (cls[u] != 3) continue;
            const int64_t e0 = lo + static_cast<int64_t>(u * kBlock + tid) * ve;
            const int64_t b = e0 > cov_lo ? e0 : cov_lo;
            const int64_t e1 = e0 + ve < cov_hi ? e0 + ve : cov_hi;
            int g = lds_find(s_dst, count, b);
            for (int64_t e = b; e < e1; ++e) {
                while (e >= s_dst[g] + s_len[g]) ++g;
                char* pb = bucket + e * es;
                char* pt = s_ten[g] + (e - s_dst[g]) * es;
                if (PACK) copy_elem(pb, pt, es); else copy_elem(pt, pb, es);
            }
        }
        __syncthreads();   // LDS is restaged below
        if (count < kBlock || last_end >= hi) break;
        f += count;
    }
}

// Static LDS of a kernel; if the runtime cannot say, a bound above what the
// staged-segment arrays take (256 entries of 24 bytes).
unsigned static_lds(const void* fn) {
    hipFuncAttributes at{};
    if (hipFuncGetAttributes(&at, fn) != hipSuccess) return 8192u;
    return static_cast<unsigned>(at.sharedSizeBytes);
}

}  // namespace

int launch_bucket_copy(const CopyLaunch& l, const char** msg) {
    if (l.bucket_len <= 0) return 0;
    CopyArgs a{};
    a.segs = l.segs;
    a.n_segs = l.n_segs;
    a.tensors = l.tensors;
    a.n_tensors = l.n_tensors;
    a.es = l.elem_bytes;
    for (int r = 0; r < l.P; ++r) a.bucket[r] = l.bucket[r];
    a.bucket_len = l.bucket_len;
    a.tile_elems = static_cast<int64_t>(kBlock) * kVecPerLane * (16 / l.elem_bytes);
    a.tiles = (l.bucket_len + a.tile_elems - 1) / a.tile_elems;

    if (a.tiles > 0x7fffffff) {
        *msg = "bucket too long for one launch";
        return static_cast<int>(hipErrorInvalidValue);
    }
    const void* fn = l.pack ? reinterpret_cast<const void*>(&bucket_copy_kernel<true>)
                            : reinterpret_cast<const void*>(&bucket_copy_kernel<false>);
    // The kernel's own LDS (the staged segments), as the compiler laid it
    // out, counts against the per-CU share.
    static const unsigned own_lds[2] = {static_lds(reinterpret_cast<const void*>(&bucket_copy_kernel<false>)),
                                        static_lds(reinterpret_cast<const void*>(&bucket_copy_kernel<true>))};
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(a.tiles), static_cast<unsigned>(l.P)),
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
