// ring_reduce_impl.h -- device code of the emulated ring all-reduce for
// CDNA4 (gfx950).  Included by the ring_reduce_*.hip translation units, each
// of which instantiates one (input type, output type) pair so that the
// kernels compile in parallel.
//
// P rank buffers of n elements sit in HBM.  For every element the kernel
// performs the additions a ring all-reduce over P devices performs -- the
// reduce-scatter carries the partial sum of a chunk from its start rank s
// through s+1, ..., s+P-1 (Burn collective blog, "Methods", Ring;
// "Distributed Training", "Sharded data parallelism": a ring all-reduce is
// a reduce-scatter followed by an all-gather) -- then applies Mean (Burn
// distributed guide, ReduceOperation), optionally one SGD-momentum step on
// float32 master weights (CS336 Lecture 8, "Data Parallelism (DDP)";
// "Distributed Training", "Mixed-Precision Training"), and writes the
// result -- the reduced gradient, or after the step the updated weights
// (ZeRO stage 1, "Distributed Training", "Sharded data parallelism") -- to
// every rank (the all-gather).
//
// The work is bound by HBM bandwidth: per element it reads P inputs, writes
// P outputs and does P-1 float32 additions.  The design follows from that:
//   * one one-wave workgroup (64 lanes) per tile and as many workgroups as
//     tiles, with the number resident per CU capped (launch.h): this mix of
//     reads and writes streams fastest with few waves per CU, and the
//     dispatcher balances tiles over the CUs and XCDs as they free up.  For
//     bf16 -> float32 every workgroup first pauses 256-1024 clocks,
//     which acts as a fraction of a workgroup below the cap;
//   * each lane loads U vectors of V elements from each of the P ranks (P*U
//     loads in flight) with non-temporal hints, folds them in registers and
//     stores the result with device-scope buffer stores.  Every lane store is
//     16 bytes wide when the output or the momentum state is float32 (V = 4),
//     so a wave writes 1 KiB contiguous per instruction; bf16 -> bf16 moves 8
//     elements per lane.  The data is touched once: tiles staged in LDS
//     through direct global-to-LDS loads measured slower for float32 and
//     level for bf16 -> float32, so tiles stay in registers;
//   * addresses are a per-rank base in SGPRs plus one 32-bit lane offset
//     shared by all ranks (the host splits buffers over 2^29 elements into
//     several launches), which keeps VGPRs for data;
//   * the reduce-scatter start rank s is uniform over a tile except where a
//     chunk boundary falls inside it, so the lanes load rank (s + k) mod P
//     into register k -- the rotation happens in the scalar pointer loads --
//     and one fixed fold serves every start rank.  Chunks are at least a
//     tile long on this path, so a tile holds at most two start ranks; the
//     second order is the same registers folded from k = 1, selected per
//     element.  Chunks shorter than a tile go to a one-element-per-lane
//     kernel.  The tile's chunk comes from 32-bit scalar arithmetic on a
//     divisor map the host builds per launch; a launch of several buckets
//     may end in a second segment (the last, partial bucket) with a map of
//     its own, chosen per tile by one comparison;
//   * bf16 inputs are widened exactly (a shift) inside the fold, float32
//     accumulation throughout, no FMA contraction, subnormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ddp {
namespace rr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = kRingBlock;

// Which chunk a launch-local element t belongs to, in 32-bit arithmetic:
// q = floor((t + off) / d) chunks after the launch's first one, whose index
// modulo the level's member count is `first`.  The host picks d and off so
// that t + off < 2^31 for every element of the launch (chunk_map in
// ring_reduce.hip): d is the chunk length, or 2^30 where a chunk is longer
// than that (a launch then holds at most one chunk boundary, which the
// shifted origin keeps in place).
struct ChunkMap {
    uint32_t d;          // divisor
    uint32_t m;          // floor((2^32 - 1) / d)
    uint32_t off;        // launch-local origin shift
    uint32_t first;      // first chunk of the launch, modulo the member count
    uint32_t members;    // the level's member count M
    uint32_t members_m;  // floor((2^32 - 1) / M)
};

struct RingArgs {
    // Rank r's buffers, already offset to this launch's first element, at
    // r and again at r + P: the P ranks from any start s are the P
    // consecutive entries from s, one scalar load.
    const void* in[2 * kMaxRanks];
    void* out[2 * kMaxRanks];
    float* w;
    float* v;
    float lr;
    float mu;
    ChunkMap ring;       // the ring's chunks (ring modes); the ring within the nodes (tree modes)
    uint32_t n;          // elements in this launch (< 2^29)
    uint32_t n_vec;      // elements covered by whole lane vectors
    int32_t mean;
    int32_t write_out;   // with SGD: 0 nothing, 1 the reduced gradient, 2 the updated weights
    uint64_t parents;    // tree strategies: 4 bits per fold register c >= 1, its parent register
    ChunkMap global;     // two-level strategies: the chunks of the ring over the nodes;
                         // ring all-reduce with a second segment: that segment's chunks
    int32_t groups;      // two-level strategies: G nodes of group_size ranks, node-major
    int32_t group_size;
    uint32_t seg2;       // ring all-reduce: the first element of a second segment -- a ring of
                         // its own, chunked by `global` from there -- or 2^32 - 1 for none
};

__device__ __forceinline__ u32x4 load16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Result stores go through a buffer resource over the destination (base in
// SGPRs, a 32-bit lane offset), because the buffer form carries a cache
// policy: device scope (sc1) without the non-temporal hint measured 2-3%
// faster than non-temporal stores for the all-reduce's 8-in/8-out pattern
// at the occupancy the launches use, and about 6% faster than ordinary
// stores.  The hardware drops stores at or beyond
// `bytes` from the base.
constexpr int kBufferWord3 = 0x00020000;   // gfx9 raw buffer: 32-bit format, no swizzle
constexpr int kStoreDeviceScope = 16;      // cache-policy operand of the store: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufferWord3);
}
__device__ __forceinline__ void store16(void* base, uint32_t bytes, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, buffer_over(base, bytes), off, 0, kStoreDeviceScope);
}
__device__ __forceinline__ void store8(void* base, uint32_t bytes, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, buffer_over(base, bytes), off, 0, kStoreDeviceScope);
}

// Element e of a 16-byte vector as float32.  A bf16 value is the upper half
// of a float32, so widening is exact; element 2k sits in the low half of
// word k.
template <bool BF16>
__device__ __forceinline__ float elem(const u32x4& x, int e) {
    if constexpr (BF16) {
        const uint32_t w = x[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
        return __uint_as_float(x[e]);
    }
}

// float32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet bit
// forced) so that rounding cannot turn it into infinity.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Mean: one division by P, correctly rounded.  For P a power of two the
// product with 2^-k is the exact quotient rounded once, i.e. the same value.
// Otherwise the quotient is taken in double and rounded to float: rounding a
// quotient of two floats first to 53 and then to 24 bits gives the correctly
// rounded result because 53 >= 2 * 24 + 2 (Figueroa, "When is double
// rounding innocuous?", SIGNUM Newsletter 30(3), 1995).
template <int P>
__device__ __forceinline__ float mean_of(float s) {
    if constexpr ((P & (P - 1)) == 0) {
        return s * (1.0f / static_cast<float>(P));
    } else {
        return static_cast<float>(static_cast<double>(s) / static_cast<double>(P));
    }
}

__device__ __forceinline__ void momentum_step(float g, float& w, float& v, float lr, float mu) {
#pragma clang fp contract(off)
    float vn = mu * v;
    vn = vn + g;
    const float step = lr * vn;
    w = w - step;
    v = vn;
}

// The kernel reads its arguments straight from the kernarg segment (address
// space 4).  A uniform index into the rank-pointer arrays then compiles to a
// scalar load, with no private copy of the argument block.
typedef const __attribute__((address_space(4))) RingArgs* KArgs;

// The tree strategies' arguments: the ring's, then the input pointers in
// fold order for every pair of level start ranks.  Row s_g * group_size +
// s_l holds the P ranks that the fold registers take when the local order
// starts at peer s_l and the global order at node s_g (level_ranks), so
// that a tile reads its P pointers with one scalar load, as the ring's
// tiles do, instead of deriving the order first.  The host fills the P
// rows of the launch (G * group_size = P).
struct TreeArgs {
    RingArgs ring;
    const void* order_in[kMaxRanks * kMaxRanks];
};
typedef const __attribute__((address_space(4))) TreeArgs* KTree;

__device__ __forceinline__ KArgs kernel_args() {
    return (KArgs)(__builtin_amdgcn_kernarg_segment_ptr());
}

// ---- the fold -------------------------------------------------------------
//
// x[k] holds rank (s + k) mod P, s the chunk's start rank, so the ring's
// order is the fixed fold ((x[0] + x[1]) + x[2]) + ... + x[P-1].  SHIFT
// folds the same registers as if the start rank were s + SHIFT:
// ((x[SHIFT] + x[SHIFT+1]) + ...), indices mod P.

template <int P, int SHIFT, bool BF16, int U, int V>
__device__ __forceinline__ void fold(const u32x4 (&x)[P][U], float (&acc)[U][V]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float s = elem<BF16>(x[SHIFT % P][u], e);
#pragma unroll
            for (int k = 1; k < P; ++k) s = s + elem<BF16>(x[(SHIFT + k) % P][u], e);
            acc[u][e] = s;
        }
    }
}

__device__ __forceinline__ int rank_at(int s, int k, int P) {
    const int r = s + k;
    return r >= P ? r - P : r;
}

// Chunks from the launch's first one to the one holding launch-local
// element t, and t's position within it (`rem`), for x = t + c.off < 2^31:
// the high half of x * m is floor(x / d) or one less -- x * m / 2^32 lies in
// (x / d - 2x / 2^32, x / d) -- so one comparison makes it exact.  With t
// uniform over a wave these are a handful of scalar instructions between a
// tile's start and its first load.
__device__ __forceinline__ uint32_t chunk_steps(uint32_t t, const __attribute__((address_space(4))) ChunkMap& c,
                                                uint32_t& rem) {
    const uint32_t x = t + c.off;
    uint32_t q = __umulhi(x, c.m);
    uint32_t r = x - q * c.d;
    if (r >= c.d) {
        ++q;
        r -= c.d;
    }
    rem = r;
    return q;
}

// The member (rank, or node, or peer) at which element t's chunk starts its
// ring, for a level of M members.
template <int M>
__device__ __forceinline__ int chunk_start(uint32_t t, const __attribute__((address_space(4))) ChunkMap& c) {
    uint32_t r;
    return static_cast<int>((c.first + chunk_steps(t, c, r)) % static_cast<uint32_t>(M));
}
// x mod M for the level's run-time member count, by the same
// multiply-high as chunk_steps (x < 2^31 + 16).
__device__ __forceinline__ int mod_members(uint32_t x, const __attribute__((address_space(4))) ChunkMap& c) {
    const uint32_t q = __umulhi(x, c.members_m);
    uint32_t r = x - q * c.members;
    if (r >= c.members) r -= c.members;
    return static_cast<int>(r);
}
__device__ __forceinline__ int chunk_start_rt(uint32_t t, const __attribute__((address_space(4))) ChunkMap& c) {
    uint32_t r;
    return mod_members(c.first + chunk_steps(t, c, r), c);
}

// The start member of the chunk holding tile element t0, and the first
// launch-local element of the next chunk.
template <int M>
__device__ __forceinline__ int tile_chunk(uint32_t t0, const __attribute__((address_space(4))) ChunkMap& c,
                                          uint32_t& next) {
    uint32_t r;
    const uint32_t q = chunk_steps(t0, c, r);
    next = t0 + (c.d - r);
    return static_cast<int>((c.first + q) % static_cast<uint32_t>(M));
}

// Holds a uniform value in SGPRs from this point of the program on.  Placed
// right after a tile's loads are issued, it makes the scalar loads of the
// kernel arguments the stores need (output bases, sizes, flags) go out and
// return while the tile's data is in flight; left to itself the compiler
// sinks them to their first use, which puts their round trips between the
// data arriving and the results leaving.
template <typename T>
__device__ __forceinline__ void pin_sgpr(T v) {
    asm volatile("" ::"s"(v));
}

// Every output rank receives the same value, so the order of the P stores
// is free.  Each wave starts at a different rank (its wave index mod P):
// the waves in flight then write to all P output streams at once instead
// of all to the same one (measured about 2% faster than a common order).
__device__ __forceinline__ int store_rotation(int P) {
    const int wave = static_cast<int>(blockIdx.x * (kBlock / 64) + threadIdx.x / 64);
    return __builtin_amdgcn_readfirstlane(wave % P);
}

// The P output bases in store order, dst[q] = rank (rot + q) mod P, and
// the P input bases in fold order, src[k] = rank (s + k) mod P: P
// consecutive entries of the doubled pointer tables, read with one scalar
// load each before the first store or load needs them.
template <int P>
__device__ __forceinline__ void rotated_outs(KArgs a, int rot, char* (&dst)[P]) {
#pragma unroll
    for (int q = 0; q < P; ++q) dst[q] = static_cast<char*>(a->out[rot + q]);
}

template <int P>
__device__ __forceinline__ void rotated_ins(KArgs a, int s, const char* (&src)[P]) {
#pragma unroll
    for (int k = 0; k < P; ++k) src[k] = static_cast<const char*>(a->in[s + k]);
}

// ---- one element per lane: tails and chunks shorter than a tile ----------

// The start rank of element i of a ring all-reduce launch: its chunk in
// the first segment, or in the second one (a ring of its own from seg2).
template <int P>
__device__ __forceinline__ int ring_start_rank(KArgs a, uint32_t i) {
    const uint32_t seg2 = a->seg2;
    return i < seg2 ? chunk_start<P>(i, a->ring) : chunk_start<P>(i - seg2, a->global);
}

template <int P, bool INB, bool OUTB, bool SGD>
__device__ __forceinline__ void process_element(KArgs a, uint32_t i) {
#pragma clang fp contract(off)
    const int s = ring_start_rank<P>(a, i);
    float g;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const void* p = a->in[rank_at(s, k, P)];   // per-lane pointer choice
        float xk;
        if constexpr (INB) {
            xk = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
        } else {
            xk = static_cast<const float*>(p)[i];
        }
        g = k == 0 ? xk : g + xk;
    }
    if (a->mean) g = mean_of<P>(g);
    if constexpr (SGD) {
        float w = a->w[i];
        float v = a->v[i];
        momentum_step(g, w, v, a->lr, a->mu);
        a->w[i] = w;
        a->v[i] = v;
        if (!a->write_out) return;
        if (a->write_out == 2) g = w;
    }
#pragma unroll
    for (int r = 0; r < P; ++r) {
        if constexpr (OUTB) {
            static_cast<uint16_t*>(a->out[r])[i] = static_cast<uint16_t>(bf16_bits(g));
        } else {
            static_cast<float*>(a->out[r])[i] = g;
        }
    }
}

// ---- the vector path ------------------------------------------------------

template <int W>
__device__ __forceinline__ u32x4 load_lane(const void* p) {
    if constexpr (W == 4) {
        return load16(p);
    } else {
        const u32x2 h = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        return u32x4{h[0], h[1], 0u, 0u};
    }
}

// One tile = U rows of kBlock lane vectors of V elements per rank,
// processed by one workgroup.  FULL: the whole tile lies below n_vec.
template <int P, bool INB, bool OUTB, bool SGD, bool FULL>
__device__ __forceinline__ void process_tile(KArgs a, uint32_t t0, int s0, uint32_t next) {
#pragma clang fp contract(off)
    constexpr int U = ring_vectors_per_lane(P, SGD);
    constexpr int V = ring_lane_elems(INB, OUTB, SGD);
    constexpr uint32_t IES = INB ? 2 : 4;   // input element bytes
    constexpr uint32_t OES = OUTB ? 2 : 4;  // output element bytes
    constexpr int WIN = V * IES / 4;        // input words per lane vector (2 or 4)
    constexpr uint32_t TILE = static_cast<uint32_t>(kBlock) * U * V;
    const uint32_t tid = threadIdx.x;
    const uint32_t n_vec = a->n_vec;

    // Chunks are at least TILE long on this path, so the tile holds one
    // start rank, or two with the boundary at element `next` of the launch.
    const uint32_t last = FULL ? t0 + TILE - 1 : n_vec - 1;
    const bool straddle = next <= last;
    const char* src[P];
    rotated_ins<P>(a, s0, src);

    u32x4 x[P][U];
    float ws[U][V];
    float vs[U][V];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
        ok[u] = FULL || (i0 < n_vec);
        if (ok[u]) {
#pragma unroll
            for (int k = 0; k < P; ++k) x[k][u] = load_lane<WIN>(src[k] + i0 * IES);
            if constexpr (SGD) {
                static_assert(V == 4, "the momentum state moves as one 16-byte vector per lane");
                const u32x4 wq = load16(reinterpret_cast<const char*>(a->w) + i0 * 4u);
                const u32x4 vq = load16(reinterpret_cast<const char*>(a->v) + i0 * 4u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ws[u][e] = __uint_as_float(wq[e]);
                    vs[u][e] = __uint_as_float(vq[e]);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < P; ++k) x[k][u] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // What the stores need, fetched while the loads are in flight.
    const uint32_t n = a->n;
    const int32_t mean_flag = a->mean;
    const int32_t write_out = SGD ? a->write_out : 1;
    const float lr = SGD ? a->lr : 0.0f;
    const float mu = SGD ? a->mu : 0.0f;
    char* dst[P];
    rotated_outs<P>(a, store_rotation(P), dst);
    pin_sgpr(n);
    pin_sgpr(mean_flag);
    if constexpr (SGD) {
        pin_sgpr(write_out);
        pin_sgpr(lr);
        pin_sgpr(mu);
    }
    if (!SGD || write_out) {
#pragma unroll
        for (int q = 0; q < P; ++q) pin_sgpr(dst[q]);
    }

    float acc[U][V];
    fold<P, 0, INB, U, V>(x, acc);
    if (straddle) {
        float acc2[U][V];
        fold<P, 1, INB, U, V>(x, acc2);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i0 = t0 + (u * kBlock + tid) * V;
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (i0 + e >= next) acc[u][e] = acc2[u][e];
        }
    }

    const bool mean = mean_flag != 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
        float g[V];
#pragma unroll
        for (int e = 0; e < V; ++e) g[e] = mean ? mean_of<P>(acc[u][e]) : acc[u][e];
        if constexpr (SGD) {
            u32x4 wq, vq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                momentum_step(g[e], ws[u][e], vs[u][e], lr, mu);
                wq[e] = __float_as_uint(ws[u][e]);
                vq[e] = __float_as_uint(vs[u][e]);
            }
            store16(a->w, n * 4u, i0 * 4u, wq);
            store16(a->v, n * 4u, i0 * 4u, vq);
            if (!write_out) continue;
            if (write_out == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) g[e] = ws[u][e];
            }
        }
        if constexpr (OUTB && V == 8) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = bf16_bits(g[2 * k]) | (bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
            for (int q = 0; q < P; ++q) store16(dst[q], n * OES, i0 * OES, o);
        } else if constexpr (OUTB) {
            u32x2 o;
#pragma unroll
            for (int k = 0; k < 2; ++k) o[k] = bf16_bits(g[2 * k]) | (bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
            for (int q = 0; q < P; ++q) store8(dst[q], n * OES, i0 * OES, o);
        } else {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(g[e]);
#pragma unroll
            for (int q = 0; q < P; ++q) store16(dst[q], n * OES, i0 * OES, o);
        }
    }
}

// One tile per workgroup and as many workgroups as tiles: the hardware
// dispatcher hands tiles to whichever CU is free, which balances the load
// across CUs and XCDs better than fixed per-workgroup shares.
template <int P, bool INB, bool OUTB, bool SGD>
__global__ __launch_bounds__(kBlock) void ring_reduce_kernel(RingArgs) {
    constexpr uint32_t TILE =
        static_cast<uint32_t>(kBlock) * ring_vectors_per_lane(P, SGD) * ring_lane_elems(INB, OUTB, SGD);
    const KArgs a = kernel_args();
    const uint32_t t0 = blockIdx.x * TILE;
    const uint32_t n_vec = a->n_vec;
    // The tile's start rank, computed before the branch so that its argument
    // loads go out together with n_vec's.  A tile of a second segment (the
    // host keeps tiles from straddling its start) takes that segment's
    // chunks, counted from its start.
    const uint32_t seg2 = a->seg2;
    uint32_t next;
    int s0;
    if constexpr (INB && !OUTB && !SGD) {
        constexpr int kSleep = ring_start_sleep(P, INB, OUTB, SGD);
        if constexpr (kSleep > 0) __builtin_amdgcn_s_sleep(kSleep);
        // bf16 -> float32: the start pause (launch.h), then seg2, then the
        // segment's chunk map.  Without the pause this order measured 0.9%
        // faster on 100 MiB buckets than the one batch below, and level with
        // it; the one batch is 0.2-0.7% faster for every other instantiation
        // measured (float32, and bf16 with the optimizer step).
        if (t0 < seg2) {
            s0 = tile_chunk<P>(t0, a->ring, next);
        } else {
            s0 = tile_chunk<P>(t0 - seg2, a->global, next);
            next += seg2;
        }
    } else {
        // Both segments' chunk maps are read in the same batch as seg2 and
        // n_vec, and the tile selects one: no round trip waits for seg2.
        const uint32_t rd = a->ring.d, rm = a->ring.m, roff = a->ring.off, rfirst = a->ring.first;
        const uint32_t gd = a->global.d, gm = a->global.m, goff = a->global.off, gfirst = a->global.first;
        asm volatile("" ::"s"(seg2), "s"(n_vec), "s"(rd), "s"(rm), "s"(roff), "s"(rfirst), "s"(gd), "s"(gm),
                     "s"(goff), "s"(gfirst));
        const bool second = t0 >= seg2;
        const uint32_t d = second ? gd : rd;
        const uint32_t x = (second ? t0 - seg2 : t0) + (second ? goff : roff);
        uint32_t q = __umulhi(x, second ? gm : rm);
        uint32_t r = x - q * d;
        if (r >= d) {
            ++q;
            r -= d;
        }
        next = t0 + (d - r);
        s0 = static_cast<int>(((second ? gfirst : rfirst) + q) % static_cast<uint32_t>(P));
    }
    if (t0 + TILE <= n_vec) {
        process_tile<P, INB, OUTB, SGD, true>(a, t0, s0, next);
    } else if (t0 < n_vec) {
        process_tile<P, INB, OUTB, SGD, false>(a, t0, s0, next);
    }
    if (blockIdx.x == gridDim.x - 1) {
        const uint32_t i = n_vec + threadIdx.x;
        if (i < a->n) process_element<P, INB, OUTB, SGD>(a, i);
    }
}

// Chunks shorter than a tile (C large against n): one element per lane.
template <int P, bool INB, bool OUTB, bool SGD>
__global__ __launch_bounds__(kBlock) void ring_reduce_scalar_kernel(RingArgs) {
    const KArgs a = kernel_args();
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < a->n) process_element<P, INB, OUTB, SGD>(a, i);
}

// ---- the ring's two halves as separate passes ------------------------------
//
// Reduce-scatter: element i's finished reduction is written to its owner
// only, owner = (s + P - 1) mod P, the rank where the chunk's reduce-scatter
// ends -- in the rotated load order that is register P-1.  The owner's copy
// goes out with the fused kernel's device-scope buffer stores, which
// measured faster than ordinary stores both alone and followed by an
// all-gather.  All-gather: every rank other than the owner receives the
// owner's value.  Tiles that straddle a chunk
// boundary take the per-element path (at most C-1 tiles per call).

template <int P, bool INB, bool OUTB>
__device__ __forceinline__ void rs_element(KArgs a, uint32_t i) {
#pragma clang fp contract(off)
    const int s = chunk_start<P>(i, a->ring);
    float g;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const void* p = a->in[rank_at(s, k, P)];
        float xk;
        if constexpr (INB) {
            xk = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
        } else {
            xk = static_cast<const float*>(p)[i];
        }
        g = k == 0 ? xk : g + xk;
    }
    if (a->mean) g = mean_of<P>(g);
    void* o = a->out[rank_at(s, P - 1, P)];
    if constexpr (OUTB) {
        static_cast<uint16_t*>(o)[i] = static_cast<uint16_t>(bf16_bits(g));
    } else {
        static_cast<float*>(o)[i] = g;
    }
}

template <int P, int ES>
__device__ __forceinline__ void ag_element(KArgs a, uint32_t i) {
    const int s = chunk_start<P>(i, a->ring);
    const int o = rank_at(s, P - 1, P);
    if constexpr (ES == 2) {
        const uint16_t v = static_cast<const uint16_t*>(a->out[o])[i];
#pragma unroll
        for (int r = 0; r < P; ++r)
            if (r != o) static_cast<uint16_t*>(a->out[r])[i] = v;
    } else {
        const uint32_t v = static_cast<const uint32_t*>(a->out[o])[i];
#pragma unroll
        for (int r = 0; r < P; ++r)
            if (r != o) static_cast<uint32_t*>(a->out[r])[i] = v;
    }
}

template <int P, bool INB, bool OUTB, bool FULL>
__device__ __forceinline__ void rs_tile(KArgs a, uint32_t t0) {
#pragma clang fp contract(off)
    constexpr int U = ring_vectors_per_lane(P, false);
    constexpr int V = ring_lane_elems(INB, OUTB, false);
    constexpr uint32_t IES = INB ? 2 : 4;
    constexpr uint32_t OES = OUTB ? 2 : 4;
    constexpr int WIN = V * IES / 4;
    constexpr uint32_t TILE = static_cast<uint32_t>(kBlock) * U * V;
    const uint32_t tid = threadIdx.x;
    const uint32_t n_vec = a->n_vec;
    const uint32_t last = FULL ? t0 + TILE - 1 : n_vec - 1;
    uint32_t next;
    const int s0 = tile_chunk<P>(t0, a->ring, next);
    if (next <= last) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i0 = t0 + (u * kBlock + tid) * V;
            if (FULL || i0 < n_vec) {
                for (int e = 0; e < V; ++e) rs_element<P, INB, OUTB>(a, i0 + e);
            }
        }
        return;
    }
    const char* src[P];
    rotated_ins<P>(a, s0, src);
    u32x4 x[P][U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
        ok[u] = FULL || (i0 < n_vec);
        if (ok[u]) {
#pragma unroll
            for (int k = 0; k < P; ++k) x[k][u] = load_lane<WIN>(src[k] + i0 * IES);
        } else {
#pragma unroll
            for (int k = 0; k < P; ++k) x[k][u] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    float acc[U][V];
    fold<P, 0, INB, U, V>(x, acc);
    char* const owner = static_cast<char*>(a->out[rank_at(s0, P - 1, P)]);
    const bool mean = a->mean != 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
        float g[V];
#pragma unroll
        for (int e = 0; e < V; ++e) g[e] = mean ? mean_of<P>(acc[u][e]) : acc[u][e];
        if constexpr (OUTB && V == 8) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = bf16_bits(g[2 * k]) | (bf16_bits(g[2 * k + 1]) << 16);
            store16(owner, a->n * OES, i0 * OES, o);
        } else if constexpr (OUTB) {
            u32x2 o;
#pragma unroll
            for (int k = 0; k < 2; ++k) o[k] = bf16_bits(g[2 * k]) | (bf16_bits(g[2 * k + 1]) << 16);
            store8(owner, a->n * OES, i0 * OES, o);
        } else {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(g[e]);
            store16(owner, a->n * OES, i0 * OES, o);
        }
    }
}

template <int P, int ES, bool FULL>
__device__ __forceinline__ void ag_tile(KArgs a, uint32_t t0) {
    constexpr int V = 16 / ES;
    constexpr uint32_t TILE = static_cast<uint32_t>(kBlock) * V;
    const uint32_t tid = threadIdx.x;
    const uint32_t n_vec = a->n_vec;
    const uint32_t i0 = t0 + tid * V;
    const uint32_t last = FULL ? t0 + TILE - 1 : n_vec - 1;
    uint32_t next;
    const int s0 = tile_chunk<P>(t0, a->ring, next);
    if (!FULL && i0 >= n_vec) return;
    if (next <= last) {
        for (int e = 0; e < V; ++e) ag_element<P, ES>(a, i0 + e);
        return;
    }
    const int o = rank_at(s0, P - 1, P);
    const u32x4 y = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a->out[o]) + i0 * ES);
    // the P-1 other ranks, starting at a rank that differs from wave to wave
    const int rot = P > 1 ? store_rotation(P - 1) : 0;
    char* dst[P > 1 ? P - 1 : 1];
#pragma unroll
    for (int q = 0; q < P - 1; ++q) dst[q] = static_cast<char*>(a->out[o + 1 + rank_at(rot, q, P - 1)]);
#pragma unroll
    for (int q = 0; q < P - 1; ++q) store16(dst[q], a->n * ES, i0 * ES, y);
}

template <int P, bool INB, bool OUTB>
__global__ __launch_bounds__(kBlock) void ring_rs_kernel(RingArgs) {
    constexpr uint32_t TILE =
        static_cast<uint32_t>(kBlock) * ring_vectors_per_lane(P, false) * ring_lane_elems(INB, OUTB, false);
    const KArgs a = kernel_args();
    const uint32_t t0 = blockIdx.x * TILE;
    const uint32_t n_vec = a->n_vec;
    if (t0 + TILE <= n_vec) {
        rs_tile<P, INB, OUTB, true>(a, t0);
    } else if (t0 < n_vec) {
        rs_tile<P, INB, OUTB, false>(a, t0);
    }
    if (blockIdx.x == gridDim.x - 1) {
        const uint32_t i = n_vec + threadIdx.x;
        if (i < a->n) rs_element<P, INB, OUTB>(a, i);
    }
}

template <int P, bool INB, bool OUTB>
__global__ __launch_bounds__(kBlock) void ring_rs_scalar_kernel(RingArgs) {
    const KArgs a = kernel_args();
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < a->n) rs_element<P, INB, OUTB>(a, i);
}

template <int P, int ES>
__global__ __launch_bounds__(kBlock) void ring_ag_kernel(RingArgs) {
    constexpr uint32_t TILE = static_cast<uint32_t>(kBlock) * (16 / ES);
    const KArgs a = kernel_args();
    const uint32_t t0 = blockIdx.x * TILE;
    const uint32_t n_vec = a->n_vec;
    if (t0 + TILE <= n_vec) {
        ag_tile<P, ES, true>(a, t0);
    } else if (t0 < n_vec) {
        ag_tile<P, ES, false>(a, t0);
    }
    if (blockIdx.x == gridDim.x - 1) {
        const uint32_t i = n_vec + threadIdx.x;
        if (i < a->n) ag_element<P, ES>(a, i);
    }
}

template <int P, int ES>
__global__ __launch_bounds__(kBlock) void ring_ag_scalar_kernel(RingArgs) {
    const KArgs a = kernel_args();
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < a->n) ag_element<P, ES>(a, i);
}

template <bool INB, bool OUTB, bool SCALAR>
const void* ring_rs_kernel_for(int P) {
    switch (P) {
#define DDP_CASE(p)                                                                       \
    case p:                                                                               \
        return SCALAR ? reinterpret_cast<const void*>(&ring_rs_scalar_kernel<p, INB, OUTB>) \
                      : reinterpret_cast<const void*>(&ring_rs_kernel<p, INB, OUTB>);
        DDP_CASE(1) DDP_CASE(2) DDP_CASE(3) DDP_CASE(4)
        DDP_CASE(5) DDP_CASE(6) DDP_CASE(7) DDP_CASE(8)
        DDP_CASE(9) DDP_CASE(10) DDP_CASE(11) DDP_CASE(12)
        DDP_CASE(13) DDP_CASE(14) DDP_CASE(15) DDP_CASE(16)
#undef DDP_CASE
        default:
            return nullptr;
    }
}

template <int ES, bool SCALAR>
const void* ring_ag_kernel_for(int P) {
    switch (P) {
#define DDP_CASE(p)                                                                 \
    case p:                                                                         \
        return SCALAR ? reinterpret_cast<const void*>(&ring_ag_scalar_kernel<p, ES>) \
                      : reinterpret_cast<const void*>(&ring_ag_kernel<p, ES>);
        DDP_CASE(1) DDP_CASE(2) DDP_CASE(3) DDP_CASE(4)
        DDP_CASE(5) DDP_CASE(6) DDP_CASE(7) DDP_CASE(8)
        DDP_CASE(9) DDP_CASE(10) DDP_CASE(11) DDP_CASE(12)
        DDP_CASE(13) DDP_CASE(14) DDP_CASE(15) DDP_CASE(16)
#undef DDP_CASE
        default:
            return nullptr;
    }
}

// ---- centralized, tree and two-level strategies ---------------------------
//
// The reduce runs along a tree over P fold registers (Burn collective blog,
// "Methods", Tree; Centralized is the tree whose root has every other member
// as a child): every register adds its children's partial sums to its own
// value in increasing child order, children before parents, and the root's
// value is broadcast.  The shape arrives as a parent table (4 bits per
// register); parents[c] < c, so walking the registers from the highest down
// finishes every child before its parent.  Register indices are
// compile-time; the shape only decides, with uniform branches, which of the
// P(P-1)/2 possible edges are taken.
//
// The same fold serves the two-level strategies (same blog, "Local strategy
// and global strategy", "Local ring downfall"): P = G nodes of Lr ranks,
// rank g*Lr + l being peer l of node g.  The registers hold node blocks in
// the global order, each block the node's peers in the local order; a local
// tree links the peers of a block, a ring or centralized level links them to
// the block's first register (a left fold from it), and the blocks' first
// registers are linked the same way at the global level.  A ring level
// rotates its order per chunk: its members start at (chunk mod members), so
// register k holds a rank that depends on the element's local and global
// chunk -- uniform over a tile except where a chunk boundary falls inside
// it.  Fixed orders pass chunk lengths beyond any index.  A single-level
// tree is the case G = 1.

// The rank held by each fold register when the local order starts at peer
// s_l and the global order at node s_g.
template <int P>
__device__ __forceinline__ void level_ranks(int G, int Lr, int s_l, int s_g, int (&rank)[P]) {
    int li = s_l;
    int gi = s_g;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        rank[k] = gi * Lr + li;
        li = li + 1 == Lr ? 0 : li + 1;
        if (++cnt == Lr) {
            cnt = 0;
            gi = gi + 1 == G ? 0 : gi + 1;
        }
    }
}

template <int P, bool BF16, int U, int V>
__device__ __forceinline__ void tree_fold(const u32x4 (&x)[P][U], uint64_t parents, float (&acc)[U][V]) {
#pragma clang fp contract(off)
    float part[P][U][V];
#pragma unroll
    for (int r = 0; r < P; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < V; ++e) part[r][u][e] = elem<BF16>(x[r][u], e);
#pragma unroll
    for (int p = P - 2; p >= 0; --p) {
#pragma unroll
        for (int c = p + 1; c < P; ++c) {
            if (static_cast<int>((parents >> (4 * c)) & 15u) == p) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int e = 0; e < V; ++e) part[p][u][e] = part[p][u][e] + part[c][u][e];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[u][e] = part[0][u][e];
}

template <int P, bool INB, bool OUTB>
__device__ __forceinline__ void tree_element(KArgs a, uint32_t i) {
#pragma clang fp contract(off)
    const int G = a->groups;
    const int Lr = a->group_size;
    int rank[P];
    level_ranks<P>(G, Lr, chunk_start_rt(i, a->ring), chunk_start_rt(i, a->global), rank);
    float part[P];
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const void* p = a->in[rank[k]];
        if constexpr (INB) {
            part[k] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
        } else {
            part[k] = static_cast<const float*>(p)[i];
        }
    }
    const uint64_t parents = a->parents;
#pragma unroll
    for (int p = P - 2; p >= 0; --p)
#pragma unroll
        for (int c = p + 1; c < P; ++c)
            if (static_cast<int>((parents >> (4 * c)) & 15u) == p) part[p] = part[p] + part[c];
    float g = part[0];
    if (a->mean) g = mean_of<P>(g);
#pragma unroll
    for (int r = 0; r < P; ++r) {
        if constexpr (OUTB) {
            static_cast<uint16_t*>(a->out[r])[i] = static_cast<uint16_t>(bf16_bits(g));
        } else {
            static_cast<float*>(a->out[r])[i] = g;
        }
    }
}

// Where a tree tile's chunks end at both levels, and its row of the order
// table.
struct TreeTileStart {
    uint32_t next_local;    // first element of the next local chunk
    uint32_t next_global;   // first element of the next global chunk
    int row;                // s_g * group_size + s_l
};

__device__ __forceinline__ TreeTileStart tree_tile_start(KArgs a, uint32_t t0) {
    uint32_t rl, rg;
    const uint32_t ql = chunk_steps(t0, a->ring, rl);
    const uint32_t qg = chunk_steps(t0, a->global, rg);
    TreeTileStart st;
    st.next_local = t0 + (a->ring.d - rl);
    st.next_global = t0 + (a->global.d - rg);
    st.row = mod_members(a->global.first + qg, a->global) * a->group_size + mod_members(a->ring.first + ql, a->ring);
    return st;
}

template <int P, bool INB, bool OUTB, bool FULL>
__device__ __forceinline__ void tree_tile(KArgs a, const void* const __attribute__((address_space(4)))* order,
                                          uint32_t t0, const TreeTileStart& st) {
#pragma clang fp contract(off)
    constexpr int U = ring_vectors_per_lane(P, false);
    constexpr int V = ring_lane_elems(INB, OUTB, false);
    constexpr uint32_t IES = INB ? 2 : 4;
    constexpr uint32_t OES = OUTB ? 2 : 4;
    constexpr int WIN = V * IES / 4;
    constexpr uint32_t TILE = static_cast<uint32_t>(kBlock) * U * V;
    const uint32_t tid = threadIdx.x;
    const uint32_t n_vec = a->n_vec;
    const uint32_t last = FULL ? t0 + TILE - 1 : n_vec - 1;
    if (st.next_local <= last || st.next_global <= last) {
        // a local or global chunk boundary inside the tile: element by element
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i0 = t0 + (u * kBlock + tid) * V;
            if (FULL || i0 < n_vec)
                for (int e = 0; e < V; ++e) tree_element<P, INB, OUTB>(a, i0 + e);
        }
        return;
    }
    const char* src[P];
#pragma unroll
    for (int k = 0; k < P; ++k) src[k] = static_cast<const char*>(order[st.row * P + k]);
    u32x4 x[P][U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
        ok[u] = FULL || (i0 < n_vec);
        if (ok[u]) {
#pragma unroll
            for (int k = 0; k < P; ++k)
                x[k][u] = load_lane<WIN>(src[k] + i0 * IES);
        } else {
#pragma unroll
            for (int r = 0; r < P; ++r) x[r][u] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // What the fold and the stores need, fetched while the loads are in
    // flight.  The parent table passes through an empty asm first, so that
    // the fold's edge tests (P(P-1)/2 of them) are not hoisted in front of
    // the loads.
    uint64_t parents = a->parents;
    asm volatile("" : "+s"(parents));
    const uint32_t n = a->n;
    const int32_t mean_flag = a->mean;
    char* dst[P];
    rotated_outs<P>(a, store_rotation(P), dst);
    pin_sgpr(parents);
    pin_sgpr(n);
    pin_sgpr(mean_flag);
#pragma unroll
    for (int q = 0; q < P; ++q) pin_sgpr(dst[q]);
    float acc[U][V];
    tree_fold<P, INB, U, V>(x, parents, acc);
    const bool mean = mean_flag != 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const uint32_t i0 = t0 + (u * kBlock + tid) * V;
        float g[V];
#pragma unroll
        for (int e = 0; e < V; ++e) g[e] = mean ? mean_of<P>(acc[u][e]) : acc[u][e];
        if constexpr (OUTB && V == 8) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = bf16_bits(g[2 * k]) | (bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
            for (int q = 0; q < P; ++q) store16(dst[q], n * OES, i0 * OES, o);
        } else if constexpr (OUTB) {
            u32x2 o;
#pragma unroll
            for (int k = 0; k < 2; ++k) o[k] = bf16_bits(g[2 * k]) | (bf16_bits(g[2 * k + 1]) << 16);
#pragma unroll
            for (int q = 0; q < P; ++q) store8(dst[q], n * OES, i0 * OES, o);
        } else {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(g[e]);
#pragma unroll
            for (int q = 0; q < P; ++q) store16(dst[q], n * OES, i0 * OES, o);
        }
    }
}

template <int P, bool INB, bool OUTB>
__global__ __launch_bounds__(kBlock) void tree_reduce_kernel(TreeArgs) {
    constexpr uint32_t TILE =
        static_cast<uint32_t>(kBlock) * ring_vectors_per_lane(P, false) * ring_lane_elems(INB, OUTB, false);
    const KTree ta = (KTree)(__builtin_amdgcn_kernarg_segment_ptr());
    const KArgs a = &ta->ring;
    const uint32_t t0 = blockIdx.x * TILE;
    const uint32_t n_vec = a->n_vec;
    // The tile's chunk ends and order row, computed before the branch so
    // that every argument they need goes out together with n_vec.
    const TreeTileStart st = tree_tile_start(a, t0);
    pin_sgpr(st.next_local);
    pin_sgpr(st.next_global);
    pin_sgpr(st.row);
    if (t0 + TILE <= n_vec) {
        tree_tile<P, INB, OUTB, true>(a, ta->order_in, t0, st);
    } else if (t0 < n_vec) {
        tree_tile<P, INB, OUTB, false>(a, ta->order_in, t0, st);
    }
    if (blockIdx.x == gridDim.x - 1) {
        const uint32_t i = n_vec + threadIdx.x;
        if (i < a->n) tree_element<P, INB, OUTB>(a, i);
    }
}

// Local or global chunks shorter than a tile: one element per lane.
template <int P, bool INB, bool OUTB>
__global__ __launch_bounds__(kBlock) void tree_reduce_scalar_kernel(TreeArgs) {
    const KArgs a = &((KTree)(__builtin_amdgcn_kernarg_segment_ptr()))->ring;
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < a->n) tree_element<P, INB, OUTB>(a, i);
}

template <bool INB, bool OUTB, bool SCALAR>
const void* tree_kernel_for(int P) {
    switch (P) {
#define DDP_CASE(p)                                                                           \
    case p:                                                                                   \
        return SCALAR ? reinterpret_cast<const void*>(&tree_reduce_scalar_kernel<p, INB, OUTB>) \
                      : reinterpret_cast<const void*>(&tree_reduce_kernel<p, INB, OUTB>);
        DDP_CASE(1) DDP_CASE(2) DDP_CASE(3) DDP_CASE(4)
        DDP_CASE(5) DDP_CASE(6) DDP_CASE(7) DDP_CASE(8)
        DDP_CASE(9) DDP_CASE(10) DDP_CASE(11) DDP_CASE(12)
        DDP_CASE(13) DDP_CASE(14) DDP_CASE(15) DDP_CASE(16)
#undef DDP_CASE
        default:
            return nullptr;
    }
}

template <bool INB, bool OUTB, bool SGD, bool SCALAR>
const void* ring_kernel_for(int P) {
    switch (P) {
#define DDP_CASE(p)                                                                                  \
    case p:                                                                                          \
        return SCALAR ? reinterpret_cast<const void*>(&ring_reduce_scalar_kernel<p, INB, OUTB, SGD>) \
                      : reinterpret_cast<const void*>(&ring_reduce_kernel<p, INB, OUTB, SGD>);
        DDP_CASE(1) DDP_CASE(2) DDP_CASE(3) DDP_CASE(4)
        DDP_CASE(5) DDP_CASE(6) DDP_CASE(7) DDP_CASE(8)
        DDP_CASE(9) DDP_CASE(10) DDP_CASE(11) DDP_CASE(12)
        DDP_CASE(13) DDP_CASE(14) DDP_CASE(15) DDP_CASE(16)
#undef DDP_CASE
        default:
            return nullptr;
    }
}

}  // namespace rr
}  // namespace ddp

// Defines ddp::ring_kernel_<name>(P, sgd, scalar),
// ddp::ring_rs_kernel_<name>(P, scalar) and ddp::tree_kernel_<name>(P, scalar) for
// one type pair.
#define DDP_RING_TYPE_PAIR(name, INB, OUTB)                                              \
    namespace ddp {                                                                      \
    const void* ring_kernel_##name(int P, int sgd, int scalar) {                         \
        if (sgd) return scalar ? rr::ring_kernel_for<INB, OUTB, true, true>(P)           \
                               : rr::ring_kernel_for<INB, OUTB, true, false>(P);         \
        return scalar ? rr::ring_kernel_for<INB, OUTB, false, true>(P)                   \
                      : rr::ring_kernel_for<INB, OUTB, false, false>(P);                 \
    }                                                                                    \
    const void* ring_rs_kernel_##name(int P, int scalar) {                               \
        return scalar ? rr::ring_rs_kernel_for<INB, OUTB, true>(P)                       \
                      : rr::ring_rs_kernel_for<INB, OUTB, false>(P);                     \
    }                                                                                    \
    const void* tree_kernel_##name(int P, int scalar) {                                  \
        return scalar ? rr::tree_kernel_for<INB, OUTB, true>(P)                          \
                      : rr::tree_kernel_for<INB, OUTB, false>(P);                        \
    }                                                                                    \
    }
