// api.cpp -- the C ABI declared in include/ddp_allreduce.h.
//
// Everything here runs on the host: argument validation (complete before
// any device work is enqueued), the bucket plan, error reporting, and the
// hand-off to the kernel launchers.  No HIP call is made before validation
// succeeds, so every error path can be exercised on a machine without a GPU.
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "launch.h"
#include "launch_copy.h"
#include "launch_multi.h"
#include "launch_step.h"

namespace {

thread_local std::string g_last_error;

// ddp_set_wg_per_cu: one cap per kernel family, -1 = the built-in choice.
constexpr int kFamilies = DDP_KF_STEP + 1;
std::atomic<int> g_wg_override[kFamilies] = {{-1}, {-1}, {-1}, {-1}, {-1}, {-1}, {-1}, {-1}};

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return DDP_OK;
}

bool valid_dtype(int d) { return d == DDP_F32 || d == DDP_BF16; }
int elem_bytes(int d) { return d == DDP_BF16 ? 2 : 4; }

struct Buf {
    uintptr_t lo;
    uintptr_t hi;   // one past the end
    int es;
    const char* what;
    int index;
};

// Two buffers may be disjoint or alias exactly (same start, same element
// size, same length); anything else is a partial overlap.
int check_overlaps(const std::vector<Buf>& bufs) {
    for (size_t i = 0; i < bufs.size(); ++i) {
        for (size_t j = i + 1; j < bufs.size(); ++j) {
            const Buf& a = bufs[i];
            const Buf& b = bufs[j];
            if (a.lo >= a.hi || b.lo >= b.hi) continue;
            const bool overlap = a.lo < b.hi && b.lo < a.hi;
            if (!overlap) continue;
            const bool exact = a.lo == b.lo && a.hi == b.hi && a.es == b.es;
            if (!exact) {
                return fail(DDP_E_OVERLAP, "%s[%d] and %s[%d] overlap without aliasing exactly", a.what,
                            a.index, b.what, b.index);
            }
        }
    }
    return DDP_OK;
}

// Longest buffer a call accepts, in elements: 2^40 (4 TiB of float32, far
// beyond any device), so that byte extents and pointer ends cannot wrap.
constexpr int64_t kMaxElems = int64_t(1) << 40;

int check_length(int64_t n, const char* what) {
    if (n < 0) return fail(DDP_E_ARG, "%s = %lld is negative", what, static_cast<long long>(n));
    if (n > kMaxElems)
        return fail(DDP_E_ARG, "%s = %lld is over 2^40 elements", what, static_cast<long long>(n));
    return DDP_OK;
}

int check_ranks(int32_t P) {
    if (P < 1 || P > DDP_MAX_RANKS) return fail(DDP_E_ARG, "P = %d outside 1..%d", P, DDP_MAX_RANKS);
    return DDP_OK;
}

int check_ptr_array(const void* const* arr, int32_t P, const char* what) {
    if (arr == nullptr) return fail(DDP_E_ARG, "%s is NULL", what);
    for (int r = 0; r < P; ++r) {
        if (arr[r] == nullptr) return fail(DDP_E_ARG, "%s[%d] is NULL", what, r);
        if (reinterpret_cast<uintptr_t>(arr[r]) & 15u)
            return fail(DDP_E_ALIGN, "%s[%d] is not 16-byte aligned", what, r);
    }
    return DDP_OK;
}

int hip_fail(int code, const char* msg) {
    return fail(DDP_E_HIP, "HIP error %d in %s", code, msg ? msg : "?");
}

// Shared validation of the reduction calls.
int validate_reduce(int op, int32_t P, int32_t chunking, const void* const* in, int in_dtype,
                    void* const* out, int out_dtype, int64_t n, bool out_required) {
    if (op != DDP_SUM && op != DDP_MEAN) return fail(DDP_E_ARG, "unknown reduce op %d", op);
    int s = check_ranks(P);
    if (s) return s;
    if (chunking < 1) return fail(DDP_E_ARG, "chunking = %d, must be >= 1", chunking);
    if (int e = check_length(n, "n")) return e;
    if (!valid_dtype(in_dtype)) return fail(DDP_E_ARG, "unknown input dtype %d", in_dtype);
    if (!valid_dtype(out_dtype)) return fail(DDP_E_ARG, "unknown output dtype %d", out_dtype);
    if ((s = check_ptr_array(in, P, "rank_in"))) return s;
    if (out_required || out != nullptr) {
        if ((s = check_ptr_array(const_cast<const void* const*>(out), P, "rank_out"))) return s;
    }
    return DDP_OK;
}

void add_rank_bufs(std::vector<Buf>& bufs, const void* const* arr, int32_t P, int64_t n, int es,
                   const char* what) {
    for (int r = 0; r < P; ++r) {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(arr[r]);
        bufs.push_back({lo, lo + static_cast<uintptr_t>(n) * es, es, what, r});
    }
}

uint64_t fnv1a(uint64_t h, const void* data, size_t len) {
    const unsigned char* p = static_cast<const unsigned char*>(data);
    for (size_t i = 0; i < len; ++i) {
        h ^= p[i];
        h *= 1099511628211ull;
    }
    return h;
}

// Buckets of E elements laid end to end in every rank buffer (the last one
// may be shorter), each all-reduced as its own ring.  Consecutive full
// buckets go out as one ring over all of them when that ring adds in the
// same order: with C a multiple of P and E = C * L, chunk k * C + j of the
// joint ring covers the elements of bucket k's chunk j and starts at rank
// (k * C + j) mod P = j mod P, where bucket k's chunk j starts.  The
// partial last bucket rides in the same launch as a second segment with its
// own chunks when the whole fits one launch; otherwise it, and every bucket
// when the full ones do not form one ring, gets a call of its own.
// One ring call of a bucketed all-reduce: elements [first, first + count)
// with `chunking` chunks, and optionally a second segment from `seg2` on.
struct BucketPart {
    int64_t first;
    int64_t count;
    int chunking;
    int64_t seg2;
    int seg2_chunking;
};

std::vector<BucketPart> bucket_parts(const ddp::RingLaunch& l, int64_t E) {
    std::vector<BucketPart> parts;
    const int64_t full = l.n / E;
    const int64_t tail = l.n - full * E;
    const bool joint = full > 1 && l.chunking % l.P == 0 && E % l.chunking == 0 && full * l.chunking <= INT32_MAX;
    // The joint ring (or a single full bucket) and the partial last bucket in
    // one launch, each with its own chunks, when both take the vector path
    // and no tile straddles them.
    const int64_t tile = ddp::ring_tile_elems(l);
    const int64_t first_chunks = joint ? full * l.chunking : l.chunking;
    if (l.mode == ddp::kAllReduce && (joint || full == 1) && tail > 0 && l.n <= ddp::kMaxLaunchElems &&
        (full * E) % tile == 0 &&
        (E + l.chunking - 1) / l.chunking >= tile && (tail + l.chunking - 1) / l.chunking >= tile) {
        parts.push_back({0, l.n, static_cast<int>(first_chunks), full * E, l.chunking});
        return parts;
    }
    if (joint) {
        parts.push_back({0, full * E, static_cast<int>(full * l.chunking), 0, 0});
    } else {
        for (int64_t k = 0; k < full; ++k) parts.push_back({k * E, E, l.chunking, 0, 0});
    }
    if (tail > 0) parts.push_back({full * E, tail, l.chunking, 0, 0});
    return parts;
}

int launch_buckets(const ddp::RingLaunch& l, int64_t E, const char** msg) {
    const int ies = l.in_bf16 ? 2 : 4;
    const int oes = l.out_bf16 ? 2 : 4;
    for (const BucketPart& p : bucket_parts(l, E)) {
        ddp::RingLaunch b = l;
        for (int r = 0; r < l.P; ++r) {
            b.in[r] = l.in[r] ? static_cast<const char*>(l.in[r]) + p.first * ies : nullptr;
            b.out[r] = l.out[r] ? static_cast<char*>(l.out[r]) + p.first * oes : nullptr;
        }
        if (l.w) b.w = l.w + p.first;
        if (l.v) b.v = l.v + p.first;
        b.n = p.count;
        b.chunking = p.chunking;
        b.seg2 = p.seg2;
        b.seg2_chunking = p.seg2_chunking;
        if (const int e = ddp::launch_ring_reduce(b, msg)) return e;
    }
    return 0;
}

// The stepwise ring over every bucket: the same parts as launch_buckets
// (whole buckets as one ring where that keeps every chunk), each part its
// 2(P-1) launches; the send counters keep adding up across parts.
int launch_step_buckets(const ddp::StepLaunch& l, int64_t E, const char** msg) {
    ddp::RingLaunch shape{};
    shape.mode = ddp::kReduceScatter;
    shape.P = l.P;
    shape.chunking = l.chunking;
    shape.n = l.n;
    for (const BucketPart& p : bucket_parts(shape, E)) {
        ddp::StepLaunch b = l;
        for (int r = 0; r < l.P; ++r) b.buf[r] = l.buf[r] + p.first;
        b.n = p.count;
        b.chunking = p.chunking;
        if (const int e = ddp::launch_ring_stepwise(b, msg)) return e;
    }
    return 0;
}

int check_bucket_elems(int64_t E, int in_dtype, int out_dtype) {
    if (E < 1) return fail(DDP_E_ARG, "bucket_elems = %lld, must be >= 1", static_cast<long long>(E));
    if (E > kMaxElems) return fail(DDP_E_ARG, "bucket_elems is over 2^40");
    if ((E * elem_bytes(in_dtype)) % 16 != 0 || (E * elem_bytes(out_dtype)) % 16 != 0)
        return fail(DDP_E_ALIGN, "bucket_elems = %lld does not keep every bucket 16-byte aligned",
                    static_cast<long long>(E));
    return DDP_OK;
}

}  // namespace

namespace ddp {
int wg_per_cu_override(int family) {
    return family >= 0 && family < kFamilies ? g_wg_override[family].load(std::memory_order_relaxed) : -1;
}
}  // namespace ddp

extern "C" {

const char* ddp_last_error(void) { return g_last_error.c_str(); }

int ddp_set_wg_per_cu(ddp_kernel_family family, int32_t wg_per_cu) {
    const int f = static_cast<int>(family);
    if (f < 0 || f >= kFamilies) return fail(DDP_E_ARG, "unknown kernel family %d", f);
    if (!(wg_per_cu == -1 || wg_per_cu == 0 || (wg_per_cu >= 2 && wg_per_cu <= 64)))
        return fail(DDP_E_ARG, "wg_per_cu = %d: expected -1, 0 or 2..64", wg_per_cu);
    g_wg_override[f].store(wg_per_cu, std::memory_order_relaxed);
    return ok();
}

int ddp_bucket_plan(const int64_t* numels, int32_t n_tensors, ddp_dtype dtype, int64_t bucket_bytes,
                    ddp_segment* segs, int64_t segs_cap, int64_t* n_segs, int32_t* n_buckets,
                    int64_t* total_elems, uint64_t* fingerprint) {
    if (n_tensors < 0) return fail(DDP_E_ARG, "n_tensors = %d is negative", n_tensors);
    if (n_tensors > 0 && numels == nullptr) return fail(DDP_E_ARG, "numels is NULL");
    if (!valid_dtype(dtype)) return fail(DDP_E_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (bucket_bytes <= 0 || bucket_bytes % 16 != 0)
        return fail(DDP_E_ARG, "bucket_bytes = %lld must be a positive multiple of 16",
                    static_cast<long long>(bucket_bytes));
    if (n_segs == nullptr) return fail(DDP_E_ARG, "n_segs is NULL");
    if (segs_cap < 0) return fail(DDP_E_ARG, "segs_cap is negative");
    const int64_t es = elem_bytes(dtype);
    const int64_t E = bucket_bytes / es;

    int64_t total = 0;
    for (int32_t t = 0; t < n_tensors; ++t) {
        if (numels[t] < 0) return fail(DDP_E_ARG, "numels[%d] is negative", t);
        if (numels[t] > INT64_MAX / 4 - total) return fail(DDP_E_ARG, "total element count overflows");
        total += numels[t];
    }
    const int64_t buckets = (total + E - 1) / E;
    if (buckets > INT32_MAX) return fail(DDP_E_ARG, "more than 2^31-1 buckets");

    // Reverse parameter order; the flat range is cut every E elements.
    int64_t count = 0;
    int64_t flat = 0;
    for (int32_t t = n_tensors - 1; t >= 0; --t) {
        int64_t remaining = numels[t];
        int64_t src = 0;
        while (remaining > 0) {
            const int64_t b = flat / E;
            const int64_t off = flat - b * E;
            const int64_t take = remaining < E - off ? remaining : E - off;
            if (segs != nullptr && count < segs_cap) {
                ddp_segment& s = segs[count];
                s.tensor = t;
                s.bucket = static_cast<int32_t>(b);
                s.src_off = src;
                s.dst_off = off;
                s.len = take;
            }
            ++count;
            src += take;
            flat += take;
            remaining -= take;
        }
    }
    *n_segs = count;
    if (n_buckets) *n_buckets = static_cast<int32_t>(buckets);
    if (total_elems) *total_elems = total;
    if (fingerprint) {
        uint64_t h = 14695981039346656037ull;
        const int32_t d = dtype;
        h = fnv1a(h, &d, sizeof d);
        h = fnv1a(h, &bucket_bytes, sizeof bucket_bytes);
        h = fnv1a(h, &n_tensors, sizeof n_tensors);
        if (n_tensors > 0) h = fnv1a(h, numels, sizeof(int64_t) * static_cast<size_t>(n_tensors));
        *fingerprint = h;
    }
    if (segs != nullptr && count > segs_cap)
        return fail(DDP_E_PLAN, "segment capacity %lld < %lld needed", static_cast<long long>(segs_cap),
                    static_cast<long long>(count));
    return ok();
}

// Pack and unpack: every argument is checked on the host before anything
// is launched, the segment table included, and the kernels read nothing but
// what was checked (the table travels in the kernel arguments).
static int bucket_copy(bool pack, int32_t P, ddp_dtype dtype, const ddp_segment* segs, int64_t n_segs,
                       const int64_t* numels, int32_t n_tensors, const void* const* tensor_ptrs,
                       const void* const* rank_bucket, int64_t bucket_len, void* stream) {
    int s = check_ranks(P);
    if (s) return s;
    if (!valid_dtype(dtype)) return fail(DDP_E_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (int e = check_length(bucket_len, "bucket_len")) return e;
    if (n_segs < 0) return fail(DDP_E_ARG, "n_segs is negative");
    if (n_tensors < 1) return fail(DDP_E_ARG, "n_tensors = %d, must be >= 1", n_tensors);
    if (numels == nullptr) return fail(DDP_E_ARG, "numels is NULL");
    for (int32_t t = 0; t < n_tensors; ++t)
        if (numels[t] < 0 || numels[t] > kMaxElems) return fail(DDP_E_ARG, "numels[%d] outside 0..2^40", t);
    if ((s = check_ptr_array(rank_bucket, P, "rank_bucket"))) return s;
    const int es = elem_bytes(dtype);

    // The segments must tile [0, bucket_len) in order, all with one bucket
    // index, each a non-empty piece inside its tensor.
    if (n_segs > 0 && segs == nullptr) return fail(DDP_E_ARG, "segs is NULL");
    if (bucket_len > 0 && n_segs == 0) return fail(DDP_E_PLAN, "a non-empty bucket needs segments");
    int64_t pos = 0;
    for (int64_t k = 0; k < n_segs; ++k) {
        const ddp_segment& g = segs[k];
        if (g.bucket != segs[0].bucket)
            return fail(DDP_E_PLAN, "segment %lld belongs to bucket %d, segment 0 to bucket %d",
                        static_cast<long long>(k), g.bucket, segs[0].bucket);
        if (g.tensor < 0 || g.tensor >= n_tensors)
            return fail(DDP_E_PLAN, "segment %lld names tensor %d of %d", static_cast<long long>(k), g.tensor,
                        n_tensors);
        if (g.len < 1) return fail(DDP_E_PLAN, "segment %lld is empty", static_cast<long long>(k));
        if (g.dst_off != pos)
            return fail(DDP_E_PLAN, "segment %lld starts at %lld, the previous one ends at %lld",
                        static_cast<long long>(k), static_cast<long long>(g.dst_off), static_cast<long long>(pos));
        if (g.src_off < 0 || g.len > numels[g.tensor] || g.src_off > numels[g.tensor] - g.len)
            return fail(DDP_E_PLAN, "segment %lld reads [%lld, %lld) of tensor %d, which holds %lld elements",
                        static_cast<long long>(k), static_cast<long long>(g.src_off),
                        static_cast<long long>(g.src_off + g.len), g.tensor,
                        static_cast<long long>(numels[g.tensor]));
        if (g.len > bucket_len - pos)
            return fail(DDP_E_PLAN, "segment %lld ends past the bucket's %lld elements", static_cast<long long>(k),
                        static_cast<long long>(bucket_len));
        pos += g.len;
    }
    if (pos != bucket_len)
        return fail(DDP_E_PLAN, "the segments cover %lld of the bucket's %lld elements", static_cast<long long>(pos),
                    static_cast<long long>(bucket_len));
    if (bucket_len == 0) return ok();

    // The tensors the segments touch: non-null, aligned to the element size.
    if (tensor_ptrs == nullptr) return fail(DDP_E_ARG, "tensor_ptrs is NULL");
    for (int64_t k = 0; k < n_segs; ++k) {
        for (int r = 0; r < P; ++r) {
            const void* t = tensor_ptrs[static_cast<int64_t>(r) * n_tensors + segs[k].tensor];
            if (t == nullptr) return fail(DDP_E_ARG, "tensor_ptrs[rank %d, tensor %d] is NULL", r, segs[k].tensor);
            if (reinterpret_cast<uintptr_t>(t) % es)
                return fail(DDP_E_ALIGN, "tensor_ptrs[rank %d, tensor %d] is not aligned to its element size", r,
                            segs[k].tensor);
        }
    }

    // What the copy writes must overlap nothing it reads or writes
    // elsewhere: the buckets are pairwise disjoint, no tensor piece
    // overlaps a bucket, and unpack's pieces (its destinations) are
    // pairwise disjoint.
    std::vector<Buf> bufs;
    add_rank_bufs(bufs, rank_bucket, P, bucket_len, es, "rank_bucket");
    for (size_t i = 0; i < bufs.size(); ++i)
        for (size_t j = i + 1; j < bufs.size(); ++j)
            if (bufs[i].lo < bufs[j].hi && bufs[j].lo < bufs[i].hi)
                return fail(DDP_E_OVERLAP, "rank_bucket[%d] and rank_bucket[%d] overlap", bufs[i].index,
                            bufs[j].index);
    std::vector<std::pair<uintptr_t, uintptr_t>> pieces;
    pieces.reserve(static_cast<size_t>(n_segs) * P);
    for (int64_t k = 0; k < n_segs; ++k) {
        for (int r = 0; r < P; ++r) {
            const uintptr_t t =
                reinterpret_cast<uintptr_t>(tensor_ptrs[static_cast<int64_t>(r) * n_tensors + segs[k].tensor]);
            const uintptr_t lo = t + static_cast<uintptr_t>(segs[k].src_off) * es;
            const uintptr_t hi = lo + static_cast<uintptr_t>(segs[k].len) * es;
            for (const Buf& b : bufs)
                if (lo < b.hi && b.lo < hi)
                    return fail(DDP_E_OVERLAP, "rank %d's piece of tensor %d overlaps rank_bucket[%d]", r,
                                segs[k].tensor, b.index);
            pieces.push_back({lo, hi});
        }
    }
    if (!pack) {
        std::sort(pieces.begin(), pieces.end());
        for (size_t i = 1; i < pieces.size(); ++i)
            if (pieces[i].first < pieces[i - 1].second)
                return fail(DDP_E_OVERLAP, "two tensor pieces that unpack writes overlap");
    }

    // Launches over consecutive ranges [A, B) of the bucket, each holding at
    // most copy_segments_per_launch(P) segments.  Every range but the last
    // ends on a 16-byte boundary of the bucket; the first segment of a
    // range may have begun in the previous one.
    const int per_launch = ddp::copy_segments_per_launch(P);
    const int64_t ve = 16 / es;
    int64_t A = 0;
    int64_t f = 0;   // the segment holding element A
    while (A < bucket_len) {
        int64_t B = bucket_len;
        if (n_segs - f > per_launch || bucket_len - A > ddp::kCopyMaxLaunchElems) {
            int64_t lim = A + ddp::kCopyMaxLaunchElems;
            if (f + per_launch < n_segs && segs[f + per_launch].dst_off < lim) lim = segs[f + per_launch].dst_off;
            // lim >= A + per_launch (segments are non-empty) and per_launch
            // > ve, so the vector boundary below lies past A.
            B = lim / ve * ve;
            if (B <= A) return fail(DDP_E_PLAN, "internal: empty copy range");
        }
        ddp::CopyLaunch l{};
        l.P = P;
        l.elem_bytes = es;
        l.pack = pack ? 1 : 0;
        l.len = static_cast<int32_t>(B - A);
        for (int r = 0; r < P; ++r) l.bucket[r] = static_cast<char*>(const_cast<void*>(rank_bucket[r])) + A * es;
        int n = 0;
        for (int64_t k = f; k < n_segs && segs[k].dst_off < B; ++k, ++n) {
            const int64_t first = segs[k].dst_off > A ? segs[k].dst_off : A;
            l.start[n] = static_cast<int32_t>(first - A);
            const int64_t src = segs[k].src_off + (first - segs[k].dst_off);
            for (int r = 0; r < P; ++r)
                l.piece[n * P + r] = static_cast<char*>(const_cast<void*>(
                                         tensor_ptrs[static_cast<int64_t>(r) * n_tensors + segs[k].tensor])) +
                                     src * es;
        }
        if (n < 1 || n > per_launch) return fail(DDP_E_PLAN, "internal: %d segments in one copy launch", n);
        l.n_segs = n;
        l.stream = stream;
        const char* msg = nullptr;
        const int e = ddp::launch_bucket_copy(l, &msg);
        if (e != 0) return hip_fail(e, msg);
        A = B;
        while (f < n_segs && segs[f].dst_off + segs[f].len <= A) ++f;
    }
    return ok();
}

int ddp_bucket_pack(int32_t P, ddp_dtype dtype, const ddp_segment* segs, int64_t n_segs, const int64_t* numels,
                    int32_t n_tensors, const void* const* tensor_ptrs, void* const* rank_bucket,
                    int64_t bucket_len, void* stream) {
    return bucket_copy(true, P, dtype, segs, n_segs, numels, n_tensors, tensor_ptrs,
                       const_cast<const void* const*>(rank_bucket), bucket_len, stream);
}

int ddp_bucket_unpack(int32_t P, ddp_dtype dtype, const ddp_segment* segs, int64_t n_segs, const int64_t* numels,
                      int32_t n_tensors, void* const* tensor_ptrs, const void* const* rank_bucket,
                      int64_t bucket_len, void* stream) {
    return bucket_copy(false, P, dtype, segs, n_segs, numels, n_tensors, const_cast<const void* const*>(tensor_ptrs),
                       rank_bucket, bucket_len, stream);
}

int allreduce_ring_emulated(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_in,
                            ddp_dtype in_dtype, void* const* rank_out, ddp_dtype out_dtype, int64_t n,
                            void* stream) {
    int s = validate_reduce(op, P, chunking, rank_in, in_dtype, rank_out, out_dtype, n, true);
    if (s) return s;
    std::vector<Buf> bufs;
    add_rank_bufs(bufs, rank_in, P, n, elem_bytes(in_dtype), "rank_in");
    add_rank_bufs(bufs, const_cast<const void* const*>(rank_out), P, n, elem_bytes(out_dtype), "rank_out");
    if ((s = check_overlaps(bufs))) return s;
    if (n == 0) return ok();

    ddp::RingLaunch l{};
    l.P = P;
    l.chunking = chunking;
    l.op = op;
    l.in_bf16 = in_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    l.sgd = 0;
    l.write_out = 1;
    for (int r = 0; r < P; ++r) {
        l.in[r] = rank_in[r];
        l.out[r] = rank_out[r];
    }
    l.n = n;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = ddp::launch_ring_reduce(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

int allreduce_ring_buckets(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_in,
                           ddp_dtype in_dtype, void* const* rank_out, ddp_dtype out_dtype, int64_t n,
                           int64_t bucket_elems, void* stream) {
    int s = validate_reduce(op, P, chunking, rank_in, in_dtype, rank_out, out_dtype, n, true);
    if (s) return s;
    if ((s = check_bucket_elems(bucket_elems, in_dtype, out_dtype))) return s;
    std::vector<Buf> bufs;
    add_rank_bufs(bufs, rank_in, P, n, elem_bytes(in_dtype), "rank_in");
    add_rank_bufs(bufs, const_cast<const void* const*>(rank_out), P, n, elem_bytes(out_dtype), "rank_out");
    if ((s = check_overlaps(bufs))) return s;
    if (n == 0) return ok();

    ddp::RingLaunch l{};
    l.P = P;
    l.chunking = chunking;
    l.op = op;
    l.in_bf16 = in_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    l.sgd = 0;
    l.write_out = 1;
    for (int r = 0; r < P; ++r) {
        l.in[r] = rank_in[r];
        l.out[r] = rank_out[r];
    }
    l.n = n;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = launch_buckets(l, bucket_elems, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

int ddp_buckets_launch_count(int32_t P, int32_t chunking, ddp_dtype in_dtype, ddp_dtype out_dtype,
                             int32_t sgd, int64_t n, int64_t bucket_elems, int64_t* launches) {
    int s = check_ranks(P);
    if (s) return s;
    if (chunking < 1) return fail(DDP_E_ARG, "chunking = %d, must be >= 1", chunking);
    if ((s = check_length(n, "n"))) return s;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(DDP_E_ARG, "unknown dtype");
    if ((s = check_bucket_elems(bucket_elems, in_dtype, out_dtype))) return s;
    if (launches == nullptr) return fail(DDP_E_ARG, "launches is NULL");
    ddp::RingLaunch l{};
    l.P = P;
    l.chunking = chunking;
    l.in_bf16 = in_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    l.sgd = sgd != 0;
    l.n = n;
    int64_t count = 0;
    if (n > 0)
        for (const BucketPart& p : bucket_parts(l, bucket_elems))
            count += (p.count + ddp::kMaxLaunchElems - 1) / ddp::kMaxLaunchElems;
    *launches = count;
    return ok();
}

namespace {

// The fused optimizer step; write_out: 0 nothing, 1 the reduced gradient,
// 2 the updated weights, into rank_out.  bucket_elems = 0: the buffers are
// one bucket.
int fused_sgd(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_grad,
              ddp_dtype grad_dtype, int64_t n, float* master_w, float* momentum, float lr, float mu,
              void* const* rank_grad_out, ddp_dtype out_dtype, int write_out, void* stream,
              int64_t bucket_elems = 0) {
    int s = validate_reduce(op, P, chunking, rank_grad, grad_dtype, rank_grad_out, out_dtype, n, false);
    if (s) return s;
    if (bucket_elems != 0 && (s = check_bucket_elems(bucket_elems, grad_dtype, out_dtype))) return s;
    if (master_w == nullptr || momentum == nullptr) return fail(DDP_E_ARG, "master_w or momentum is NULL");
    if ((reinterpret_cast<uintptr_t>(master_w) | reinterpret_cast<uintptr_t>(momentum)) & 15u)
        return fail(DDP_E_ALIGN, "master_w or momentum is not 16-byte aligned");
    if (!std::isfinite(lr) || !std::isfinite(mu))
        return fail(DDP_E_ARG, "lr and mu must be finite");
    std::vector<Buf> bufs;
    add_rank_bufs(bufs, rank_grad, P, n, elem_bytes(grad_dtype), "rank_grad");
    if (rank_grad_out)
        add_rank_bufs(bufs, const_cast<const void* const*>(rank_grad_out), P, n, elem_bytes(out_dtype),
                      "rank_grad_out");
    if ((s = check_overlaps(bufs))) return s;
    // The optimizer state may not alias anything, not even exactly.
    const uintptr_t wl = reinterpret_cast<uintptr_t>(master_w);
    const uintptr_t vl = reinterpret_cast<uintptr_t>(momentum);
    const uintptr_t bytes = static_cast<uintptr_t>(n) * 4;
    if (n > 0) {
        if (wl < vl + bytes && vl < wl + bytes) return fail(DDP_E_OVERLAP, "master_w and momentum overlap");
        for (const Buf& b : bufs) {
            if (b.lo < wl + bytes && wl < b.hi)
                return fail(DDP_E_OVERLAP, "master_w overlaps %s[%d]", b.what, b.index);
            if (b.lo < vl + bytes && vl < b.hi)
                return fail(DDP_E_OVERLAP, "momentum overlaps %s[%d]", b.what, b.index);
        }
    }
    if (n == 0) return ok();

    ddp::RingLaunch l{};
    l.P = P;
    l.chunking = chunking;
    l.op = op;
    l.in_bf16 = grad_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    l.sgd = 1;
    l.write_out = rank_grad_out != nullptr ? write_out : 0;
    for (int r = 0; r < P; ++r) {
        l.in[r] = rank_grad[r];
        l.out[r] = rank_grad_out ? rank_grad_out[r] : nullptr;
    }
    l.w = master_w;
    l.v = momentum;
    l.lr = lr;
    l.mu = mu;
    l.n = n;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = bucket_elems != 0 ? launch_buckets(l, bucket_elems, &msg) : ddp::launch_ring_reduce(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

}  // namespace

int allreduce_fused_sgd_buckets(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_grad,
                                ddp_dtype grad_dtype, int64_t n, int64_t bucket_elems, float* master_w,
                                float* momentum, float lr, float mu, void* const* rank_grad_out,
                                ddp_dtype out_dtype, void* stream) {
    if (bucket_elems == 0) return fail(DDP_E_ARG, "bucket_elems = 0, must be >= 1");
    return fused_sgd(op, P, chunking, rank_grad, grad_dtype, n, master_w, momentum, lr, mu, rank_grad_out,
                     out_dtype, 1, stream, bucket_elems);
}

int zero1_sgd_step_buckets(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_grad,
                           ddp_dtype grad_dtype, int64_t n, int64_t bucket_elems, float* master_w,
                           float* momentum, float lr, float mu, void* const* rank_param_out,
                           ddp_dtype param_dtype, void* stream) {
    if (rank_param_out == nullptr) return fail(DDP_E_ARG, "rank_param_out is NULL");
    if (bucket_elems == 0) return fail(DDP_E_ARG, "bucket_elems = 0, must be >= 1");
    return fused_sgd(op, P, chunking, rank_grad, grad_dtype, n, master_w, momentum, lr, mu, rank_param_out,
                     param_dtype, 2, stream, bucket_elems);
}

int allreduce_fused_sgd(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_grad,
                        ddp_dtype grad_dtype, int64_t n, float* master_w, float* momentum, float lr,
                        float mu, void* const* rank_grad_out, ddp_dtype out_dtype, void* stream) {
    return fused_sgd(op, P, chunking, rank_grad, grad_dtype, n, master_w, momentum, lr, mu, rank_grad_out,
                     out_dtype, 1, stream);
}

int zero1_sgd_step_emulated(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_grad,
                            ddp_dtype grad_dtype, int64_t n, float* master_w, float* momentum, float lr,
                            float mu, void* const* rank_param_out, ddp_dtype param_dtype, void* stream) {
    if (rank_param_out == nullptr) return fail(DDP_E_ARG, "rank_param_out is NULL");
    return fused_sgd(op, P, chunking, rank_grad, grad_dtype, n, master_w, momentum, lr, mu, rank_param_out,
                     param_dtype, 2, stream);
}

}  // extern "C"

namespace {

// reducescatter_ring_emulated (bucket_elems 0) and reducescatter_ring_buckets.
int reduce_scatter_call(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_in,
                        ddp_dtype in_dtype, void* const* rank_out, ddp_dtype out_dtype, int64_t n,
                        int64_t bucket_elems, void* stream) {
    int s = validate_reduce(op, P, chunking, rank_in, in_dtype, rank_out, out_dtype, n, true);
    if (s) return s;
    if (bucket_elems != 0 && (s = check_bucket_elems(bucket_elems, in_dtype, out_dtype))) return s;
    std::vector<Buf> bufs;
    add_rank_bufs(bufs, rank_in, P, n, elem_bytes(in_dtype), "rank_in");
    add_rank_bufs(bufs, const_cast<const void* const*>(rank_out), P, n, elem_bytes(out_dtype), "rank_out");
    if ((s = check_overlaps(bufs))) return s;
    if (n == 0) return ok();

    ddp::RingLaunch l{};
    l.mode = ddp::kReduceScatter;
    l.P = P;
    l.chunking = chunking;
    l.op = op;
    l.in_bf16 = in_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    for (int r = 0; r < P; ++r) {
        l.in[r] = rank_in[r];
        l.out[r] = rank_out[r];
    }
    l.n = n;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = bucket_elems != 0 ? launch_buckets(l, bucket_elems, &msg) : ddp::launch_ring_reduce(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

// allgather_ring_emulated (bucket_elems 0) and allgather_ring_buckets.
int all_gather_call(int32_t P, int32_t chunking, void* const* rank_buf, ddp_dtype dtype, int64_t n,
                    int64_t bucket_elems, void* stream) {
    int s = check_ranks(P);
    if (s) return s;
    if (chunking < 1) return fail(DDP_E_ARG, "chunking = %d, must be >= 1", chunking);
    if (int e = check_length(n, "n")) return e;
    if (!valid_dtype(dtype)) return fail(DDP_E_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (bucket_elems != 0 && (s = check_bucket_elems(bucket_elems, dtype, dtype))) return s;
    if ((s = check_ptr_array(const_cast<const void* const*>(rank_buf), P, "rank_buf"))) return s;
    std::vector<Buf> bufs;
    add_rank_bufs(bufs, const_cast<const void* const*>(rank_buf), P, n, elem_bytes(dtype), "rank_buf");
    for (size_t i = 0; i < bufs.size(); ++i)
        for (size_t j = i + 1; j < bufs.size(); ++j)
            if (n > 0 && bufs[i].lo < bufs[j].hi && bufs[j].lo < bufs[i].hi)
                return fail(DDP_E_OVERLAP, "rank_buf[%d] and rank_buf[%d] overlap", bufs[i].index,
                            bufs[j].index);
    if (n == 0) return ok();

    ddp::RingLaunch l{};
    l.mode = ddp::kAllGather;
    l.P = P;
    l.chunking = chunking;
    l.in_bf16 = dtype == DDP_BF16;
    l.out_bf16 = dtype == DDP_BF16;
    for (int r = 0; r < P; ++r) l.out[r] = rank_buf[r];
    l.n = n;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = bucket_elems != 0 ? launch_buckets(l, bucket_elems, &msg) : ddp::launch_ring_reduce(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

// allreduce_ring_stepwise (bucket_elems 0) and allreduce_ring_stepwise_buckets.
int stepwise_call(ddp_reduce_op op, int32_t P, int32_t chunking, void* const* rank_buf, ddp_dtype dtype,
                  int64_t n, int64_t bucket_elems, uint64_t* sent_dev, void* stream) {
    if (op != DDP_SUM && op != DDP_MEAN) return fail(DDP_E_ARG, "unknown reduce op %d", op);
    int s = check_ranks(P);
    if (s) return s;
    if (chunking < 1) return fail(DDP_E_ARG, "chunking = %d, must be >= 1", chunking);
    if (int e = check_length(n, "n")) return e;
    if (!valid_dtype(dtype)) return fail(DDP_E_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (dtype != DDP_F32)
        return fail(DDP_E_UNSUPPORTED, "the stepwise ring keeps partial sums in the rank buffers, "
                                       "which must therefore be float32");
    if (bucket_elems != 0 && (s = check_bucket_elems(bucket_elems, dtype, dtype))) return s;
    if ((s = check_ptr_array(const_cast<const void* const*>(rank_buf), P, "rank_buf"))) return s;
    std::vector<Buf> bufs;
    add_rank_bufs(bufs, const_cast<const void* const*>(rank_buf), P, n, 4, "rank_buf");
    if (sent_dev != nullptr) {
        if (reinterpret_cast<uintptr_t>(sent_dev) & 7u) return fail(DDP_E_ALIGN, "sent is not 8-byte aligned");
        const uintptr_t lo = reinterpret_cast<uintptr_t>(sent_dev);
        bufs.push_back({lo, lo + static_cast<uintptr_t>(P) * 8, 8, "sent", 0});
    }
    for (size_t i = 0; i < bufs.size(); ++i)
        for (size_t j = i + 1; j < bufs.size(); ++j)
            if (n > 0 && bufs[i].lo < bufs[j].hi && bufs[j].lo < bufs[i].hi)
                return fail(DDP_E_OVERLAP, "%s[%d] and %s[%d] overlap", bufs[i].what, bufs[i].index,
                            bufs[j].what, bufs[j].index);
    if (n == 0) return ok();

    ddp::StepLaunch l{};
    l.P = P;
    l.chunking = chunking;
    l.op = op;
    for (int r = 0; r < P; ++r) l.buf[r] = static_cast<float*>(rank_buf[r]);
    l.sent = sent_dev;
    l.n = n;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = bucket_elems != 0 ? launch_step_buckets(l, bucket_elems, &msg) : ddp::launch_ring_stepwise(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

}  // namespace

extern "C" {

int reducescatter_ring_emulated(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_in,
                                ddp_dtype in_dtype, void* const* rank_out, ddp_dtype out_dtype, int64_t n,
                                void* stream) {
    return reduce_scatter_call(op, P, chunking, rank_in, in_dtype, rank_out, out_dtype, n, 0, stream);
}

int reducescatter_ring_buckets(ddp_reduce_op op, int32_t P, int32_t chunking, const void* const* rank_in,
                               ddp_dtype in_dtype, void* const* rank_out, ddp_dtype out_dtype, int64_t n,
                               int64_t bucket_elems, void* stream) {
    if (bucket_elems == 0) return fail(DDP_E_ARG, "bucket_elems = 0, must be >= 1");
    return reduce_scatter_call(op, P, chunking, rank_in, in_dtype, rank_out, out_dtype, n, bucket_elems, stream);
}

int allgather_ring_emulated(int32_t P, int32_t chunking, void* const* rank_buf, ddp_dtype dtype, int64_t n,
                            void* stream) {
    return all_gather_call(P, chunking, rank_buf, dtype, n, 0, stream);
}

int allgather_ring_buckets(int32_t P, int32_t chunking, void* const* rank_buf, ddp_dtype dtype, int64_t n,
                           int64_t bucket_elems, void* stream) {
    if (bucket_elems == 0) return fail(DDP_E_ARG, "bucket_elems = 0, must be >= 1");
    return all_gather_call(P, chunking, rank_buf, dtype, n, bucket_elems, stream);
}

int allreduce_ring_stepwise(ddp_reduce_op op, int32_t P, int32_t chunking, void* const* rank_buf,
                            ddp_dtype dtype, int64_t n, uint64_t* sent_dev, void* stream) {
    return stepwise_call(op, P, chunking, rank_buf, dtype, n, 0, sent_dev, stream);
}

int allreduce_ring_stepwise_buckets(ddp_reduce_op op, int32_t P, int32_t chunking, void* const* rank_buf,
                                    ddp_dtype dtype, int64_t n, int64_t bucket_elems, uint64_t* sent_dev,
                                    void* stream) {
    if (bucket_elems == 0) return fail(DDP_E_ARG, "bucket_elems = 0, must be >= 1");
    return stepwise_call(op, P, chunking, rank_buf, dtype, n, bucket_elems, sent_dev, stream);
}

int allreduce_tree_emulated(ddp_reduce_op op, int32_t P, int32_t branching, const void* const* rank_in,
                            ddp_dtype in_dtype, void* const* rank_out, ddp_dtype out_dtype, int64_t n,
                            void* stream) {
    if (branching < 1) return fail(DDP_E_ARG, "branching = %d, must be >= 1", branching);
    int s = validate_reduce(op, P, 1, rank_in, in_dtype, rank_out, out_dtype, n, true);
    if (s) return s;
    std::vector<Buf> bufs;
    add_rank_bufs(bufs, rank_in, P, n, elem_bytes(in_dtype), "rank_in");
    add_rank_bufs(bufs, const_cast<const void* const*>(rank_out), P, n, elem_bytes(out_dtype), "rank_out");
    if ((s = check_overlaps(bufs))) return s;
    if (n == 0) return ok();

    ddp::RingLaunch l{};
    l.mode = ddp::kTree;
    l.P = P;
    l.chunking = 1;
    l.op = op;
    l.in_bf16 = in_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    l.write_out = 1;
    // b-ary heap: the parent of rank c >= 1 is (c - 1) / b.
    for (int c = 1; c < P; ++c) l.parents |= static_cast<uint64_t>((c - 1) / branching) << (4 * c);
    for (int r = 0; r < P; ++r) {
        l.in[r] = rank_in[r];
        l.out[r] = rank_out[r];
    }
    l.n = n;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = ddp::launch_ring_reduce(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

namespace {

// Fold-register parent of register c >= 1 of a two-level strategy: the
// registers are node blocks of Lr in the global order.  Within a block, a
// tree links peer l to peer (l - 1) / b; a ring or centralized level links
// every peer to the block's first register (a left fold from it).  A
// block's first register is linked the same way to the first registers of
// the other blocks.
int level_parent(int c, int Lr, ddp_strategy local, int32_t local_param, ddp_strategy global,
                 int32_t global_param) {
    const int gi = c / Lr;
    const int li = c % Lr;
    if (li > 0) return gi * Lr + (local == DDP_STRATEGY_TREE ? (li - 1) / local_param : 0);
    return (global == DDP_STRATEGY_TREE ? (gi - 1) / global_param : 0) * Lr;
}

int check_strategy(ddp_strategy st, int32_t param, const char* level) {
    switch (st) {
        case DDP_STRATEGY_RING:
            if (param < 0) return fail(DDP_E_ARG, "%s ring chunk count %d is negative", level, param);
            return DDP_OK;
        case DDP_STRATEGY_TREE:
            if (param < 1) return fail(DDP_E_ARG, "%s tree branching %d, must be >= 1", level, param);
            return DDP_OK;
        case DDP_STRATEGY_CENTRALIZED:
            return DDP_OK;
        default:
            return fail(DDP_E_ARG, "unknown %s strategy %d", level, static_cast<int>(st));
    }
}

}  // namespace

}  // extern "C"

namespace {

// The two-level fold over every bucket of a flat buffer.  A ring level's
// chunk j starts at member j mod M, so consecutive full buckets form one
// ring at that level, with the same chunks and start members, when the
// level's chunking is a multiple of M and the bucket length a multiple of
// the chunking; levels of fixed order (trees, centralized) always do.  When
// both levels allow it the full buckets go out as one launch sequence with
// both chunkings scaled by their count; otherwise each bucket is its own.
int launch_tree_buckets(const ddp::RingLaunch& l, int64_t E, int local_members, int global_members,
                        const char** msg) {
    const int64_t full = l.n / E;
    const int64_t tail = l.n - full * E;
    auto joins = [&](int chunking, int members) {
        return chunking == 0 || (chunking % members == 0 && E % chunking == 0 && full * chunking <= INT32_MAX);
    };
    const bool joint = full > 1 && joins(l.local_chunking, local_members) && joins(l.global_chunking, global_members);
    const int ies = l.in_bf16 ? 2 : 4;
    const int oes = l.out_bf16 ? 2 : 4;
    auto launch = [&](int64_t first, int64_t count, int64_t scale) {
        ddp::RingLaunch b = l;
        for (int r = 0; r < l.P; ++r) {
            b.in[r] = static_cast<const char*>(l.in[r]) + first * ies;
            b.out[r] = static_cast<char*>(l.out[r]) + first * oes;
        }
        b.n = count;
        b.local_chunking = static_cast<int>(l.local_chunking * scale);
        b.global_chunking = static_cast<int>(l.global_chunking * scale);
        return ddp::launch_ring_reduce(b, msg);
    };
    if (joint) {
        if (const int e = launch(0, full * E, full)) return e;
    } else {
        for (int64_t k = 0; k < full; ++k)
            if (const int e = launch(k * E, E, 1)) return e;
    }
    return tail > 0 ? launch(full * E, tail, 1) : 0;
}

// allreduce_hierarchical_emulated (bucket_elems 0) and allreduce_hierarchical_buckets.
int hierarchical_call(ddp_reduce_op op, int32_t nodes, int32_t local_ranks, ddp_strategy local_strategy,
                      int32_t local_param, ddp_strategy global_strategy, int32_t global_param,
                      const void* const* rank_in, ddp_dtype in_dtype, void* const* rank_out, ddp_dtype out_dtype,
                      int64_t n, int64_t bucket_elems, void* stream) {
    if (nodes < 1 || local_ranks < 1 || nodes > DDP_MAX_RANKS || local_ranks > DDP_MAX_RANKS ||
        nodes * local_ranks > DDP_MAX_RANKS)
        return fail(DDP_E_ARG, "nodes = %d x local_ranks = %d, need both >= 1 and a product <= %d", nodes,
                    local_ranks, DDP_MAX_RANKS);
    int s = check_strategy(local_strategy, local_param, "local");
    if (s) return s;
    if ((s = check_strategy(global_strategy, global_param, "global"))) return s;
    const int P = nodes * local_ranks;
    if ((s = validate_reduce(op, P, 1, rank_in, in_dtype, rank_out, out_dtype, n, true))) return s;
    if (bucket_elems != 0 && (s = check_bucket_elems(bucket_elems, in_dtype, out_dtype))) return s;
    std::vector<Buf> bufs;
    add_rank_bufs(bufs, rank_in, P, n, elem_bytes(in_dtype), "rank_in");
    add_rank_bufs(bufs, const_cast<const void* const*>(rank_out), P, n, elem_bytes(out_dtype), "rank_out");
    if ((s = check_overlaps(bufs))) return s;
    if (n == 0) return ok();

    ddp::RingLaunch l{};
    l.mode = ddp::kTree;
    l.P = P;
    l.chunking = 1;
    l.op = op;
    l.in_bf16 = in_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    l.write_out = 1;
    l.groups = nodes;
    if (local_strategy == DDP_STRATEGY_RING) l.local_chunking = local_param > 0 ? local_param : local_ranks;
    if (global_strategy == DDP_STRATEGY_RING) l.global_chunking = global_param > 0 ? global_param : nodes;
    for (int c = 1; c < P; ++c)
        l.parents |= static_cast<uint64_t>(
                         level_parent(c, local_ranks, local_strategy, local_param, global_strategy, global_param))
                     << (4 * c);
    for (int r = 0; r < P; ++r) {
        l.in[r] = rank_in[r];
        l.out[r] = rank_out[r];
    }
    l.n = n;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = bucket_elems != 0 ? launch_tree_buckets(l, bucket_elems, local_ranks, nodes, &msg)
                                    : ddp::launch_ring_reduce(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

}  // namespace

extern "C" {

int allreduce_hierarchical_emulated(ddp_reduce_op op, int32_t nodes, int32_t local_ranks,
                                    ddp_strategy local_strategy, int32_t local_param,
                                    ddp_strategy global_strategy, int32_t global_param,
                                    const void* const* rank_in, ddp_dtype in_dtype, void* const* rank_out,
                                    ddp_dtype out_dtype, int64_t n, void* stream) {
    return hierarchical_call(op, nodes, local_ranks, local_strategy, local_param, global_strategy, global_param,
                             rank_in, in_dtype, rank_out, out_dtype, n, 0, stream);
}

int allreduce_hierarchical_buckets(ddp_reduce_op op, int32_t nodes, int32_t local_ranks,
                                   ddp_strategy local_strategy, int32_t local_param,
                                   ddp_strategy global_strategy, int32_t global_param,
                                   const void* const* rank_in, ddp_dtype in_dtype, void* const* rank_out,
                                   ddp_dtype out_dtype, int64_t n, int64_t bucket_elems, void* stream) {
    if (bucket_elems == 0) return fail(DDP_E_ARG, "bucket_elems = 0, must be >= 1");
    return hierarchical_call(op, nodes, local_ranks, local_strategy, local_param, global_strategy, global_param,
                             rank_in, in_dtype, rank_out, out_dtype, n, bucket_elems, stream);
}

int ddp_multi_plan(const int64_t* numels, int32_t n_tensors, int32_t P, ddp_dtype in_dtype,
                   ddp_dtype out_dtype, const void* const* align_to, ddp_tensor_tiles* tiles,
                   int64_t* total_tiles, int64_t* tile_elems) {
    int s = check_ranks(P);
    if (s) return s;
    if (n_tensors < 1) return fail(DDP_E_ARG, "n_tensors = %d, must be >= 1", n_tensors);
    if (numels == nullptr || tiles == nullptr || total_tiles == nullptr || tile_elems == nullptr)
        return fail(DDP_E_ARG, "NULL pointer argument");
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(DDP_E_ARG, "unknown dtype");
    const int64_t tile = ddp::multi_tile_elems(P, in_dtype == DDP_BF16, out_dtype == DDP_BF16);
    const int ies = elem_bytes(in_dtype);
    const int small = ies < elem_bytes(out_dtype) ? ies : elem_bytes(out_dtype);
    // A lead must move every stream by whole 16-byte vectors: inputs,
    // outputs and float32 optimizer state.
    const int64_t lead_step = 16 / small > 4 ? 16 / small : 4;
    int64_t next = 0;
    for (int32_t t = 0; t < n_tensors; ++t) {
        if (numels[t] < 0) return fail(DDP_E_ARG, "numels[%d] is negative", t);
        if (numels[t] > (int64_t(1) << 29))
            return fail(DDP_E_UNSUPPORTED, "numels[%d] = %lld is over 2^29 elements", t,
                        static_cast<long long>(numels[t]));
        int64_t lead = 0;
        if (align_to != nullptr && numels[t] > 0) {
            const uintptr_t a = reinterpret_cast<uintptr_t>(align_to[t]);
            if (a % 16 == 0 && a % 128 != 0) {
                const int64_t l = static_cast<int64_t>((128 - a % 128) / ies);
                if (l % lead_step == 0) lead = l < numels[t] ? l : numels[t];
            }
        }
        tiles[t].numel = numels[t];
        tiles[t].first_tile = static_cast<int32_t>(next);
        tiles[t].lead = static_cast<int32_t>(lead);
        next += lead > 0 ? 1 + (numels[t] - lead + tile - 1) / tile : (numels[t] + tile - 1) / tile;
        if (next > INT32_MAX) return fail(DDP_E_UNSUPPORTED, "the plan needs over 2^31 - 1 tiles");
    }
    *total_tiles = next;
    *tile_elems = tile;
    return ok();
}

int ddp_multi_block_map(const ddp_tensor_tiles* tiles, int32_t n_tensors, int64_t total_tiles,
                        int32_t* block_first, int64_t cap, int64_t* n_blocks) {
    if (n_tensors < 1) return fail(DDP_E_ARG, "n_tensors = %d, must be >= 1", n_tensors);
    if (tiles == nullptr || n_blocks == nullptr) return fail(DDP_E_ARG, "NULL pointer argument");
    if (total_tiles < 0 || total_tiles > INT32_MAX) return fail(DDP_E_ARG, "total_tiles out of range");
    if (tiles[0].first_tile != 0) return fail(DDP_E_PLAN, "the plan does not start at tile 0");
    for (int32_t t = 1; t < n_tensors; ++t)
        if (tiles[t].first_tile < tiles[t - 1].first_tile || tiles[t].first_tile > total_tiles)
            return fail(DDP_E_PLAN, "first_tile of tensor %d out of order", t);
    const int64_t nb = (total_tiles + ddp::kMultiBlockTiles - 1) / ddp::kMultiBlockTiles;
    *n_blocks = nb;
    if (block_first == nullptr) return ok();
    if (cap < nb)
        return fail(DDP_E_PLAN, "block map capacity %lld < %lld needed", static_cast<long long>(cap),
                    static_cast<long long>(nb));
    // Entry k: the largest t with first_tile <= k * kMultiBlockTiles (the
    // tensor holding that tile; tensors without tiles give way to the next).
    int32_t t = 0;
    for (int64_t k = 0; k < nb; ++k) {
        const int64_t tile = k * ddp::kMultiBlockTiles;
        while (t + 1 < n_tensors && tiles[t + 1].first_tile <= tile) ++t;
        block_first[k] = t;
    }
    return ok();
}

namespace {

int validate_multi(ddp_reduce_op op, int32_t P, int32_t chunking, int32_t n_tensors,
                   const ddp_tensor_tiles* tiles_dev, int64_t total_tiles, int64_t tile_elems,
                   const void* const* in_ptrs_dev, ddp_dtype in_dtype, ddp_dtype out_dtype) {
    if (op != DDP_SUM && op != DDP_MEAN) return fail(DDP_E_ARG, "unknown reduce op %d", op);
    int s = check_ranks(P);
    if (s) return s;
    if (chunking < 1) return fail(DDP_E_ARG, "chunking = %d, must be >= 1", chunking);
    if (n_tensors < 1) return fail(DDP_E_ARG, "n_tensors = %d, must be >= 1", n_tensors);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(DDP_E_ARG, "unknown dtype");
    if (total_tiles < 0 || total_tiles > INT32_MAX) return fail(DDP_E_ARG, "total_tiles out of range");
    if (tiles_dev == nullptr || in_ptrs_dev == nullptr) return fail(DDP_E_ARG, "NULL table");
    if (tile_elems != ddp::multi_tile_elems(P, in_dtype == DDP_BF16, out_dtype == DDP_BF16))
        return fail(DDP_E_PLAN, "tile_elems does not match this P and these dtypes");
    return DDP_OK;
}

}  // namespace

int allreduce_multi_fused_sgd(ddp_reduce_op op, int32_t P, int32_t chunking, int32_t n_tensors,
                              const ddp_tensor_tiles* tiles_dev, int64_t total_tiles, int64_t tile_elems,
                              const int32_t* block_first_dev, const void* const* in_ptrs_dev, ddp_dtype grad_dtype, float* const* w_ptrs_dev,
                              float* const* v_ptrs_dev, float lr, float mu, void* const* out_ptrs_dev,
                              ddp_dtype out_dtype, void* stream) {
    int s = validate_multi(op, P, chunking, n_tensors, tiles_dev, total_tiles, tile_elems, in_ptrs_dev, grad_dtype,
                           out_dtype);
    if (s) return s;
    if (w_ptrs_dev == nullptr || v_ptrs_dev == nullptr) return fail(DDP_E_ARG, "NULL weight or momentum table");
    if (!std::isfinite(lr) || !std::isfinite(mu))
        return fail(DDP_E_ARG, "lr and mu must be finite");
    if (total_tiles == 0) return ok();

    ddp::MultiLaunch l{};
    l.P = P;
    l.chunking = chunking;
    l.op = op;
    l.in_bf16 = grad_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    l.T = n_tensors;
    l.tiles = tiles_dev;
    l.block_first = block_first_dev;
    l.in = in_ptrs_dev;
    l.out = out_ptrs_dev;
    l.w = w_ptrs_dev;
    l.v = v_ptrs_dev;
    l.lr = lr;
    l.mu = mu;
    l.sgd = 1;
    l.total_tiles = total_tiles;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = ddp::launch_multi_ring(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

int allreduce_multi_ring_emulated(ddp_reduce_op op, int32_t P, int32_t chunking, int32_t n_tensors,
                                  const ddp_tensor_tiles* tiles_dev, int64_t total_tiles, int64_t tile_elems,
                                  const int32_t* block_first_dev, const void* const* in_ptrs_dev, ddp_dtype in_dtype, void* const* out_ptrs_dev,
                                  ddp_dtype out_dtype, void* stream) {
    int s = validate_multi(op, P, chunking, n_tensors, tiles_dev, total_tiles, tile_elems, in_ptrs_dev, in_dtype,
                           out_dtype);
    if (s) return s;
    if (out_ptrs_dev == nullptr) return fail(DDP_E_ARG, "NULL table");
    if (total_tiles == 0) return ok();

    ddp::MultiLaunch l{};
    l.P = P;
    l.chunking = chunking;
    l.op = op;
    l.in_bf16 = in_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    l.T = n_tensors;
    l.tiles = tiles_dev;
    l.block_first = block_first_dev;
    l.in = in_ptrs_dev;
    l.out = out_ptrs_dev;
    l.total_tiles = total_tiles;
    l.stream = stream;
    const char* msg = nullptr;
    const int e = ddp::launch_multi_ring(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

static_assert(DDP_NOALLOC_SCRATCH_BYTES == ddp::kNoAllocScratchBytes, "scratch size in the header");

namespace {

static constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The allocation-free call's host staging area, a static array held by one
// call at a time (calls from several threads take turns).  Its contents are
// copied out of host memory before each call returns.
alignas(256) static unsigned char g_noalloc_stage[DDP_NOALLOC_SCRATCH_BYTES];
static std::mutex g_noalloc_mutex;
// What the last call copied into a scratch area, and on which device: a
// call whose tables are the same bytes on the same device skips its copy
// (the area keeps the last call's tables, and calls on one GPU are ordered
// by contract), so a loop over the same tensors costs one launch per call.
alignas(256) static unsigned char g_noalloc_last[DDP_NOALLOC_SCRATCH_BYTES];
static size_t g_noalloc_last_bytes = 0;
static void* g_noalloc_last_area = nullptr;
// Per device: a call was captured into a graph there.  Its replays rewrite
// the area whenever they run, so the last copy is no longer known and no
// later call on that device skips its copy.
static bool g_noalloc_captured[ddp::kMaxScratchDevices] = {};

}  // namespace

int allreduce_multi_ring_noalloc(ddp_reduce_op op, int32_t P, int32_t chunking, int32_t n_tensors,
                                 const int64_t* numels, const void* const* in_ptrs, ddp_dtype in_dtype,
                                 void* const* out_ptrs, ddp_dtype out_dtype, void* stream) {
    if (op != DDP_SUM && op != DDP_MEAN) return fail(DDP_E_ARG, "unknown reduce op %d", op);
    int s = check_ranks(P);
    if (s) return s;
    if (chunking < 1) return fail(DDP_E_ARG, "chunking = %d, must be >= 1", chunking);
    if (n_tensors < 1) return fail(DDP_E_ARG, "n_tensors = %d, must be >= 1", n_tensors);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(DDP_E_ARG, "unknown dtype");
    if (numels == nullptr || in_ptrs == nullptr || out_ptrs == nullptr)
        return fail(DDP_E_ARG, "NULL pointer argument");
    const int ies = elem_bytes(in_dtype);
    const int oes = elem_bytes(out_dtype);
    const int64_t T = n_tensors;
    // Sizes first, so that a request beyond the scratch area is refused
    // before anything else is read or written.
    const size_t ptr_bytes = static_cast<size_t>(P) * static_cast<size_t>(T) * sizeof(void*);
    const size_t tiles_bytes = static_cast<size_t>(T) * sizeof(ddp_tensor_tiles);
    if (tiles_bytes + 2 * ptr_bytes > static_cast<size_t>(DDP_NOALLOC_SCRATCH_BYTES))
        return fail(DDP_E_UNSUPPORTED,
                    "%d tensors x %d ranks need %zu bytes of tables, over the %d-byte scratch area", n_tensors,
                    P, tiles_bytes + 2 * ptr_bytes, DDP_NOALLOC_SCRATCH_BYTES);
    std::vector<Buf> bufs;
    for (int64_t t = 0; t < T; ++t) {
        if ((s = check_length(numels[t], "numels[t]"))) return s;
        if (numels[t] > (int64_t(1) << 29))
            return fail(DDP_E_UNSUPPORTED, "numels[%lld] = %lld is over 2^29 elements", static_cast<long long>(t),
                        static_cast<long long>(numels[t]));
        for (int r = 0; r < P; ++r) {
            const void* a = in_ptrs[r * T + t];
            const void* b = out_ptrs[r * T + t];
            if (numels[t] > 0 && (a == nullptr || b == nullptr))
                return fail(DDP_E_ARG, "rank %d's pointer of tensor %lld is NULL", r, static_cast<long long>(t));
            if ((reinterpret_cast<uintptr_t>(a) % ies) || (reinterpret_cast<uintptr_t>(b) % oes))
                return fail(DDP_E_ALIGN, "rank %d's tensor %lld is not aligned to its element size", r,
                            static_cast<long long>(t));
            if (numels[t] == 0) continue;
            const uintptr_t ia = reinterpret_cast<uintptr_t>(a);
            const uintptr_t ib = reinterpret_cast<uintptr_t>(b);
            bufs.push_back({ia, ia + static_cast<uintptr_t>(numels[t]) * ies, ies, "in", r});
            // In place (output = input, same element size) is the one alias.
            if (ib != ia || oes != ies)
                bufs.push_back({ib, ib + static_cast<uintptr_t>(numels[t]) * oes, oes, "out", r});
        }
    }
    // Every other pair of buffers must be disjoint: sorted by start, each
    // must begin at or after the furthest end seen so far.
    std::sort(bufs.begin(), bufs.end(), [](const Buf& x, const Buf& y) { return x.lo < y.lo; });
    uintptr_t reach = 0;
    for (size_t i = 0; i < bufs.size(); ++i) {
        if (i > 0 && bufs[i].lo < reach)
            return fail(DDP_E_OVERLAP, "a %s buffer of rank %d overlaps another tensor's buffer", bufs[i].what,
                        bufs[i].index);
        reach = std::max(reach, bufs[i].hi);
    }

    // Tables, laid out in the host stage as they will sit in the scratch
    // area: plan | block map | input pointers | output pointers.
    std::lock_guard<std::mutex> lock(g_noalloc_mutex);
    unsigned char* stage = g_noalloc_stage;
    auto* tiles = reinterpret_cast<ddp_tensor_tiles*>(stage);
    int64_t total_tiles = 0, tile_elems = 0;
    if ((s = ddp_multi_plan(numels, n_tensors, P, in_dtype, out_dtype, in_ptrs, tiles, &total_tiles, &tile_elems)))
        return s;
    if (total_tiles == 0) return ok();
    const size_t map_off = align_up(tiles_bytes, 256);
    const int64_t n_blocks = (total_tiles + ddp::kMultiBlockTiles - 1) / ddp::kMultiBlockTiles;
    const size_t in_off = align_up(map_off + static_cast<size_t>(n_blocks) * sizeof(int32_t), 256);
    const size_t out_off = align_up(in_off + ptr_bytes, 256);
    const size_t total_bytes = out_off + ptr_bytes;
    if (total_bytes > static_cast<size_t>(DDP_NOALLOC_SCRATCH_BYTES))
        return fail(DDP_E_UNSUPPORTED, "the tables need %zu bytes, over the %d-byte scratch area", total_bytes,
                    DDP_NOALLOC_SCRATCH_BYTES);
    int64_t nb = 0;
    if ((s = ddp_multi_block_map(tiles, n_tensors, total_tiles, reinterpret_cast<int32_t*>(stage + map_off), n_blocks,
                                 &nb)))
        return s;
    std::memcpy(stage + in_off, in_ptrs, ptr_bytes);
    std::memcpy(stage + out_off, out_ptrs, ptr_bytes);

    void* dev = nullptr;
    int ordinal = -1;
    bool capturing = false;
    const char* msg = nullptr;
    int e = ddp::noalloc_scratch(stream, &dev, &ordinal, &msg);
    if (e != 0) return hip_fail(e, msg);
    if ((e = ddp::stream_capturing(stream, &capturing, &msg)) != 0) return hip_fail(e, msg);
    if (capturing) g_noalloc_captured[ordinal] = true;
    unsigned char* d = static_cast<unsigned char*>(dev);
    // The area's bytes [0, known) are those of the host shadow; a run of
    // one fill launch's worth of bytes that the shadow already holds is not
    // written again (the tensors of a loop that alternates output buffers
    // change only the output pointer table).
    const size_t known = !g_noalloc_captured[ordinal] && g_noalloc_last_area == dev ? g_noalloc_last_bytes : 0;
    const size_t run = static_cast<size_t>(ddp::kFillWords) * sizeof(uint64_t);
    g_noalloc_last_area = nullptr;
    size_t pending = 0, pending_len = 0;    // consecutive runs that differ, written together
    for (size_t off = 0; off < total_bytes; off += run) {
        const size_t len = std::min(run, total_bytes - off);
        const bool held = off + len <= known && std::memcmp(g_noalloc_last + off, stage + off, len) == 0;
        if (!held) {
            if (pending_len == 0) pending = off;
            pending_len += len;
        }
        if ((held || off + len == total_bytes) && pending_len > 0) {
            if ((e = ddp::fill_scratch(d + pending, stage + pending, pending_len, stream, &msg)) != 0)
                return hip_fail(e, msg);
            pending_len = 0;
        }
    }
    std::memcpy(g_noalloc_last, stage, total_bytes);
    g_noalloc_last_bytes = std::max(total_bytes, known);
    g_noalloc_last_area = dev;

    ddp::MultiLaunch l{};
    l.P = P;
    l.chunking = chunking;
    l.op = op;
    l.in_bf16 = in_dtype == DDP_BF16;
    l.out_bf16 = out_dtype == DDP_BF16;
    l.T = n_tensors;
    l.tiles = reinterpret_cast<const ddp_tensor_tiles*>(d);
    l.block_first = reinterpret_cast<const int32_t*>(d + map_off);
    l.in = reinterpret_cast<const void* const*>(d + in_off);
    l.out = reinterpret_cast<void* const*>(d + out_off);
    l.total_tiles = total_tiles;
    l.stream = stream;
    e = ddp::launch_multi_ring(l, &msg);
    if (e != 0) return hip_fail(e, msg);
    return ok();
}

}  // extern "C"
