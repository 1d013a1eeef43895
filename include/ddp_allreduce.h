/*
 * ddp_allreduce.h -- C ABI of the MI355X (gfx950) gradient all-reduce library.
 *
 * What it computes.  Data-parallel training gives every rank (one replica of
 * the model) the gradient of its own shard of the batch; an all-reduce then
 * combines the ranks' equal-size gradient tensors elementwise so that every
 * rank holds the same sum or mean ("Distributed Training",
 * computervisiononline.com/explains/distributed-training, section "Data
 * parallelism and all-reduce"; CS336 "Lecture 8 - Parallelism", rd.me/cs336/
 * lec8, "Collective Operations").  The reduction is ReduceOperation Sum or
 * Mean (Burn distributed guide, pgsm.cn/news/420861, reduction configuration
 * section).  The order of the floating-point additions is that of a ring
 * (Burn collective blog, cielbird.github.io/blog/burn-distributed, "Methods",
 * Ring): a reduce-scatter followed by an all-gather.
 *
 * How it runs.  All P ranks live on one GPU as P buffers in HBM, and one
 * kernel performs, for every element, exactly the additions the ring would
 * perform over P GPUs, in the same order, then writes the result to every
 * rank's output.  The order is fixed as follows: with C chunks of length
 * L = ceil(n / C), element i belongs to chunk j = floor(i / L), whose ring
 * starts at rank s = j mod P and travels r -> r + 1, so
 *     result[i] = (((x_s[i] + x_{s+1}[i]) + x_{s+2}[i]) + ... + x_{s+P-1}[i])
 * (rank indices mod P), every addition a float32 addition rounded to
 * nearest even.  Mean then divides by P once, correctly rounded.  bf16
 * inputs are widened to float32 exactly before the first addition; bf16
 * outputs are rounded to nearest even, NaN kept quiet.  No FMA contraction
 * and no flushing of subnormals anywhere.
 *
 * Conventions shared by every call.
 *   - Device memory is owned by the caller (allocated through PyTorch or
 *     hipMalloc).  The library allocates no device memory and keeps no
 *     device state between calls.
 *   - "Host array of device pointers" means a plain C array in host memory
 *     whose entries are device addresses; it is read during the call only.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     Device work is enqueued on it and the call returns before it runs: the
 *     caller keeps every buffer alive and unmodified until the stream reaches
 *     that point (the pages' CollectiveTensor must be resolved before use;
 *     here resolving means synchronizing the stream or an event on it).
 *   - Every call validates its arguments before launching anything and
 *     returns a ddp_status; on any error nothing has been enqueued.  The
 *     library never aborts and never prints; ddp_last_error() gives a message
 *     for the calling thread's most recent failure.
 *   - Element counts (n, bucket_len) are 0..2^40; larger ones are rejected
 *     with DDP_E_ARG.
 *   - Device buffers named in host arrays (rank buffers, bucket buffers,
 *     master weights, momentum) must be 16-byte aligned.  For full speed
 *     they should start on 128-byte boundaries: a workgroup's tile starts
 *     at a multiple of the tile length from each launch's first element, so
 *     a buffer that starts inside a 128-byte line has every wave access
 *     touch one more line, and every wave store leave two lines partly
 *     written (measured 19% slower for gradient rows 32 bytes into a line,
 *     8-11% for the fused step's momentum).  The tensors of
 *     pack/unpack need only their element type's alignment; pack/unpack take
 *     their segment table and tensor addresses as host arrays and check
 *     them.  The multi-tensor calls read device tables (the tile plan and
 *     the tensors' addresses) that the library cannot read on the host:
 *     their contents are the caller's responsibility.
 *   - Two buffers of one call named in host arrays may either be disjoint or
 *     start at the same address with the same element size (exact aliasing,
 *     e.g. an in-place all-reduce); any other overlap is rejected.
 */
#ifndef DDP_ALLREDUCE_H
#define DDP_ALLREDUCE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest number of emulated ranks a call accepts. */
#define DDP_MAX_RANKS 16

typedef enum ddp_status {
    DDP_OK = 0,
    DDP_E_ARG = -1,          /* invalid argument (P, chunking, n, null pointer, enum) */
    DDP_E_UNSUPPORTED = -2,  /* valid but unsupported combination */
    DDP_E_ALIGN = -3,        /* a device buffer is not 16-byte aligned */
    DDP_E_OVERLAP = -4,      /* two buffers overlap other than by exact aliasing */
    DDP_E_PLAN = -5,         /* bucket plan inconsistent or capacity too small */
    DDP_E_HIP = -6           /* the HIP runtime reported an error */
} ddp_status;

/* ReduceOperation of the Burn distributed guide (reduction configuration
 * section): Sum adds the ranks' tensors, Mean gives every replica the
 * average (torch's ReduceOp.SUM / AVG in CS336 Lecture 8). */
typedef enum ddp_reduce_op { DDP_SUM = 0, DDP_MEAN = 1 } ddp_reduce_op;

/* Element types.  Accumulation is always float32. */
typedef enum ddp_dtype { DDP_F32 = 0, DDP_BF16 = 1 } ddp_dtype;

/* One piece of one tensor inside one bucket, in elements: elements
 * [src_off, src_off + len) of tensor `tensor` (flattened in C order) occupy
 * [dst_off, dst_off + len) of bucket `bucket`. */
typedef struct ddp_segment {
    int32_t tensor;
    int32_t bucket;
    int64_t src_off;
    int64_t dst_off;
    int64_t len;
} ddp_segment;

/* One tensor of a multi-tensor all-reduce (from ddp_multi_plan): its
 * element count, the index of its first tile in the launch, and `lead`:
 * 0, or the length of a short first tile [0, lead) after which every tile
 * starts on a 128-byte boundary of the address the plan was aligned to. */
typedef struct ddp_tensor_tiles {
    int64_t numel;
    int32_t first_tile;
    int32_t lead;
} ddp_tensor_tiles;

/*
 * ddp_bucket_plan -- host only, no device work.
 *
 * Plans fixed-size gradient buckets as DDP does ("Distributed Training",
 * "Data parallelism and all-reduce": gradients packed into buckets, filled
 * in the reverse order of the model's parameters, every rank reducing the
 * buckets in the same order).  Tensors are laid end to end in reverse
 * parameter order and the flat range is cut every E = bucket_bytes /
 * sizeof(dtype) elements, so every bucket but the last holds exactly E
 * elements and a tensor may straddle buckets.  Zero-size tensors produce no
 * segment.
 *
 *   numels       host array [n_tensors], element counts in parameter order
 *   dtype        element type (sets the element size)
 *   bucket_bytes bucket capacity in bytes; a positive multiple of 16
 *   segs         host array [segs_cap] to receive the segments, in bucket
 *                order and by increasing dst_off within a bucket; may be NULL
 *                to query the count only
 *   n_segs       out: number of segments (always written on DDP_OK and on
 *                DDP_E_PLAN for a too-small capacity)
 *   n_buckets    out: number of buckets (may be NULL)
 *   total_elems  out: sum of numels (may be NULL)
 *   fingerprint  out: 64-bit FNV-1a hash of (dtype, bucket_bytes, numels);
 *                equal on every rank that planned the same parameter list
 *                (may be NULL)
 * Errors: DDP_E_ARG (negative counts, NULL numels with n_tensors > 0, bad
 * dtype, bucket_bytes not a positive multiple of 16, more than 2^31-1
 * buckets), DDP_E_PLAN (segs_cap too small; *n_segs holds the need).
 */
int ddp_bucket_plan(const int64_t* numels, int32_t n_tensors, ddp_dtype dtype,
                    int64_t bucket_bytes, ddp_segment* segs, int64_t segs_cap,
                    int64_t* n_segs, int32_t* n_buckets, int64_t* total_elems,
                    uint64_t* fingerprint);

/*
 * ddp_bucket_pack / ddp_bucket_unpack -- device copies, all P ranks per
 * launch.
 *
 * Pack gathers every rank's pieces of one bucket out of its separately
 * allocated gradient tensors into that rank's flat bucket buffer; unpack
 * scatters a bucket back into the tensors.  ("Distributed Training": DDP
 * packs gradients into buckets that every rank fills in the same order;
 * FSDP flattens a unit's parameters into one tensor, "Sharded data
 * parallelism".)  Bit-exact copies.
 *
 * Every argument, the segment table included, is checked on the host
 * before anything is launched, and the kernels read only what was checked:
 * the library copies the table into the launches' kernel arguments.  A
 * bucket whose segments do not fit one launch's arguments (more than
 * min(128, 880 / P) segments) goes out as several launches over
 * consecutive ranges of the bucket, all on `stream`.
 *
 *   P            number of ranks, 1..DDP_MAX_RANKS
 *   dtype        element type of tensors and buckets
 *   segs         HOST array [n_segs]: the segments of this one bucket, as
 *                ddp_bucket_plan returns them: one bucket index, in order,
 *                tiling [0, bucket_len) exactly (segment k starts where
 *                segment k - 1 ends), each non-empty and inside its tensor
 *                (src_off + len <= numels[tensor])
 *   n_segs       number of segments, >= 0 (0 only with bucket_len = 0)
 *   numels       HOST array [n_tensors]: element count of every tensor
 *   n_tensors    number of tensors per rank, >= 1
 *   tensor_ptrs  HOST array [P * n_tensors] of device pointers, rank-major:
 *                entry r * n_tensors + t is rank r's tensor t (contiguous,
 *                numels[t] elements, aligned to the element size).  Only
 *                the tensors the segments name are read (and checked).
 *   rank_bucket  HOST array [P] of device pointers to the bucket buffers
 *                (bucket_len elements each, 16-byte aligned, pairwise
 *                disjoint)
 *   bucket_len   elements in this bucket, >= 0 (0: nothing is launched)
 * Host arrays are read during the call only.
 * Errors: DDP_E_PLAN (the segments do not tile the bucket in order, name a
 * tensor outside 0..n_tensors-1, are empty, mix bucket indices, or read
 * past a tensor's numels); DDP_E_ARG (counts, NULL pointers, dtype);
 * DDP_E_ALIGN (a bucket not 16-byte aligned, a tensor not aligned to its
 * element size); DDP_E_OVERLAP (buckets that overlap, a tensor piece that
 * overlaps a bucket, or for unpack two tensor pieces that overlap);
 * DDP_E_HIP.  On any error nothing has been launched.
 */
int ddp_bucket_pack(int32_t P, ddp_dtype dtype, const ddp_segment* segs,
                    int64_t n_segs, const int64_t* numels, int32_t n_tensors,
                    const void* const* tensor_ptrs, void* const* rank_bucket,
                    int64_t bucket_len, void* stream);

int ddp_bucket_unpack(int32_t P, ddp_dtype dtype, const ddp_segment* segs,
                      int64_t n_segs, const int64_t* numels, int32_t n_tensors,
                      void* const* tensor_ptrs, const void* const* rank_bucket,
                      int64_t bucket_len, void* stream);

/*
 * allreduce_ring_emulated -- the all-reduce of P rank buffers of n elements
 * in the chunked ring order described at the top of this header.
 *
 * Every rank contributes a tensor of the same size and every rank receives
 * the result ("Distributed Training", "Data parallelism and all-reduce");
 * the ring is a reduce-scatter followed by an all-gather (the same page,
 * "Sharded data parallelism", on the ring's communication volume).
 *
 *   op        DDP_SUM or DDP_MEAN
 *   P         number of ranks, 1..DDP_MAX_RANKS
 *   chunking  number of ring chunks C >= 1 (C = P is the textbook ring)
 *   rank_in   host array [P] of device pointers, n elements of in_dtype each
 *   in_dtype  DDP_F32 or DDP_BF16
 *   rank_out  host array [P] of device pointers, n elements of out_dtype
 *             each; rank_out[r] may equal rank_in[r] when the element sizes
 *             match (in-place all-reduce)
 *   out_dtype DDP_F32 or DDP_BF16
 *   n         elements per rank, >= 0 (0: nothing is launched)
 * One launch per 2^29 elements, for every pair of element types: each
 * element is read from the P inputs, folded and written to the P outputs
 * in one pass.
 * Errors: DDP_E_ARG, DDP_E_ALIGN, DDP_E_OVERLAP, DDP_E_HIP.
 */
int allreduce_ring_emulated(ddp_reduce_op op, int32_t P, int32_t chunking,
                            const void* const* rank_in, ddp_dtype in_dtype,
                            void* const* rank_out, ddp_dtype out_dtype,
                            int64_t n, void* stream);

/*
 * allreduce_fused_sgd -- the same all-reduce, followed in the same kernel by
 * one SGD-with-momentum step on a float32 master copy of the weights.
 *
 * After the all-reduce every replica holds the same gradient and takes the
 * same local optimizer step (CS336 Lecture 8, "Data Parallelism (DDP)");
 * mixed precision keeps float32 master weights and accumulates in float32
 * ("Distributed Training", Related, "Mixed-Precision Training").  Since the
 * replicas are identical, one copy of (w, v) stands for all of them.  With
 * g the reduced gradient in float32 (after the Mean division, before any
 * output rounding), each element does, with one rounding per operation:
 *     v = mu * v;  v = v + g;  w = w - lr * v
 * (heavy-ball momentum, no dampening, no Nesterov, no weight decay).
 *
 *   rank_grad      host array [P] of device pointers, n elements of grad_dtype
 *   master_w       device pointer, n floats, updated in place
 *   momentum       device pointer, n floats, updated in place
 *   lr, mu         learning rate and momentum factor (finite)
 *   rank_grad_out  host array [P] of device pointers to receive the reduced
 *                  gradient as out_dtype, or NULL to skip writing it
 *   other arguments as for allreduce_ring_emulated.  master_w and momentum
 *   must be disjoint from each other and from every gradient buffer.
 * Errors: DDP_E_ARG, DDP_E_ALIGN, DDP_E_OVERLAP, DDP_E_HIP.
 */
int allreduce_fused_sgd(ddp_reduce_op op, int32_t P, int32_t chunking,
                        const void* const* rank_grad, ddp_dtype grad_dtype,
                        int64_t n, float* master_w, float* momentum, float lr,
                        float mu, void* const* rank_grad_out,
                        ddp_dtype out_dtype, void* stream);

/*
 * allreduce_ring_buckets / allreduce_fused_sgd_buckets -- every bucket of
 * a flat gradient buffer in one call.
 *
 * DDP cuts the gradients into fixed-size buckets and every rank reduces
 * them in the same order ("Distributed Training", "Data parallelism and
 * all-reduce"); with the gradients kept as views of one flat buffer per
 * rank, bucket k is elements [k * E, min((k + 1) * E, n)) of it.  These
 * calls all-reduce every bucket of such buffers, each bucket exactly as
 * allreduce_ring_emulated (or allreduce_fused_sgd) reduces it on its own:
 * its own C chunks of ceil(len_k / C) elements, its own start ranks, the
 * same bits.  Fewer, longer launches use the memory system better than one
 * short launch per bucket (the same page, "Communication costs", on larger
 * messages): when C is a multiple of P and E a multiple of C, consecutive
 * full buckets are one ring with the same order of additions and go out as
 * one launch, which also carries the partial last bucket (with its own
 * chunks) when all n elements fit one launch (2^29), the full buckets end
 * on a whole workgroup tile and every chunk is at least a tile long; a
 * single full bucket shares a launch with the partial one on the same
 * size conditions, for any C; otherwise each bucket is its own launch.
 *
 *   bucket_elems  E >= 1, with E * element size a multiple of 16 bytes for
 *                 both element types (every bucket stays 16-byte aligned)
 *   n             elements per rank buffer (all its buckets), >= 0
 *   other arguments, layout, ownership and errors as for
 *   allreduce_ring_emulated and allreduce_fused_sgd; master_w and momentum
 *   hold n floats in the same bucket layout.
 * Errors: those of the single-bucket calls; DDP_E_ARG for bucket_elems < 1,
 * DDP_E_ALIGN for a bucket size that misaligns the buckets.
 */
int allreduce_ring_buckets(ddp_reduce_op op, int32_t P, int32_t chunking,
                           const void* const* rank_in, ddp_dtype in_dtype,
                           void* const* rank_out, ddp_dtype out_dtype,
                           int64_t n, int64_t bucket_elems, void* stream);

int allreduce_fused_sgd_buckets(ddp_reduce_op op, int32_t P, int32_t chunking,
                                const void* const* rank_grad, ddp_dtype grad_dtype,
                                int64_t n, int64_t bucket_elems, float* master_w,
                                float* momentum, float lr, float mu,
                                void* const* rank_grad_out, ddp_dtype out_dtype,
                                void* stream);

/*
 * zero1_sgd_step_emulated -- one ZeRO stage 1 step: the optimizer state is
 * sharded over the ranks and the updated parameters go to every rank.
 *
 * Stage 1 partitions the 32-bit master weights and the optimizer's moments
 * across the data-parallel ranks, each rank updating only its partition;
 * each parameter belongs to one rank, whose optimizer updates it, and the
 * updated parameters are then sent to all ranks ("Distributed Training",
 * "Sharded data parallelism: ZeRO and FSDP").  Here the partition is the
 * ring's own: element i belongs to the owner of its chunk, where the
 * reduce-scatter ends.  In one pass, for every element: the reduce-scatter
 * in ring order (the same float32 value, Mean applied, as
 * allreduce_ring_emulated), the owner's momentum step
 *     v = mu * v;  v = v + g;  w = w - lr * v
 * on its shard of master_w and momentum (one rounding per operation), and
 * the all-gather of the updated weight, rounded to param_dtype (bf16:
 * nearest even), into every rank's parameter buffer.  master_w and
 * momentum hold the union of the P shards.  The update equals that of
 * allreduce_fused_sgd bit for bit: stage 1 only partitions the state.
 *
 *   rank_grad        host array [P] of device pointers, n elements of grad_dtype
 *   master_w         device pointer, n floats, updated in place
 *   momentum         device pointer, n floats, updated in place
 *   lr, mu           learning rate and momentum factor (finite)
 *   rank_param_out   host array [P] of device pointers, n elements of
 *                    param_dtype, receiving the updated parameters; entry r
 *                    may be rank_grad[r] itself (exact aliasing)
 *   other arguments as for allreduce_ring_emulated.  master_w and momentum
 *   must be disjoint from each other and from every other buffer.
 * Errors: DDP_E_ARG (also for a NULL rank_param_out), DDP_E_ALIGN,
 * DDP_E_OVERLAP, DDP_E_HIP.
 */
int zero1_sgd_step_emulated(ddp_reduce_op op, int32_t P, int32_t chunking,
                            const void* const* rank_grad, ddp_dtype grad_dtype,
                            int64_t n, float* master_w, float* momentum, float lr,
                            float mu, void* const* rank_param_out,
                            ddp_dtype param_dtype, void* stream);

/*
 * ddp_buckets_launch_count -- host only, no device work: how many kernel
 * launches one of the bucketed calls above (or zero1_sgd_step_buckets)
 * enqueues for these arguments, by the rule stated above.  For callers
 * that size launch-time budgets or time the kernel per launch.
 *
 *   P, chunking, in_dtype, out_dtype, n, bucket_elems   as for the call
 *                (out_dtype: the output or parameter type, or the gradient
 *                type when nothing is written)
 *   sgd          nonzero for the fused optimizer calls
 *   launches     out: the number of launches (0 for n = 0)
 * Errors: DDP_E_ARG, DDP_E_ALIGN, as for the calls.
 */
int ddp_buckets_launch_count(int32_t P, int32_t chunking, ddp_dtype in_dtype,
                             ddp_dtype out_dtype, int32_t sgd, int64_t n,
                             int64_t bucket_elems, int64_t* launches);

/*
 * zero1_sgd_step_buckets -- zero1_sgd_step_emulated over every bucket of a
 * flat gradient buffer in one call, each bucket exactly as
 * zero1_sgd_step_emulated steps it on its own (its own ring, chunks and
 * owners), launched as allreduce_ring_buckets launches its buckets.  ZeRO
 * flattens the parameters of a partition into one buffer ("Distributed
 * Training", "Sharded data parallelism: ZeRO and FSDP").
 *
 *   bucket_elems  as for allreduce_ring_buckets
 *   other arguments, layout, ownership and errors as for
 *   zero1_sgd_step_emulated and allreduce_ring_buckets.
 */
int zero1_sgd_step_buckets(ddp_reduce_op op, int32_t P, int32_t chunking,
                           const void* const* rank_grad, ddp_dtype grad_dtype,
                           int64_t n, int64_t bucket_elems, float* master_w,
                           float* momentum, float lr, float mu,
                           void* const* rank_param_out, ddp_dtype param_dtype,
                           void* stream);

/*
 * reducescatter_ring_emulated -- the first half of the ring on its own.
 *
 * Every rank ends holding the finished reduction of the chunks it owns
 * ("Distributed Training", "Sharded data parallelism": FSDP reduce-scatters
 * gradients so that each rank keeps its shard; CS336 Lecture 8, "Collective
 * Operations": each rank receives a unique chunk of the reduced tensor).
 * The chunk that starts its ring at rank s is owned by rank (s + P - 1) mod P,
 * where its reduce-scatter ends.  For every element i the call writes the
 * reduction (the same value, bit for bit, that allreduce_ring_emulated
 * produces, Mean applied) to rank_out[owner(i)][i] only; every other
 * element of every rank_out buffer is left untouched.  (In a real ring the
 * other ranks would hold partial sums there.)
 *
 * Arguments, layout, ownership and errors as for allreduce_ring_emulated.
 * reducescatter_ring_emulated followed by allgather_ring_emulated on
 * rank_out equals allreduce_ring_emulated bit for bit.
 */
int reducescatter_ring_emulated(ddp_reduce_op op, int32_t P, int32_t chunking,
                                const void* const* rank_in, ddp_dtype in_dtype,
                                void* const* rank_out, ddp_dtype out_dtype,
                                int64_t n, void* stream);

/*
 * allgather_ring_emulated -- the second half of the ring on its own.
 *
 * Gives every rank the complete tensor (CS336 Lecture 8, "Collective
 * Operations"; FSDP all-gathers a unit's parameters, "Distributed Training",
 * "Sharded data parallelism").  With the chunk ownership of
 * reducescatter_ring_emulated (chunk length ceil(n / C), chunk j owned by
 * rank (j + P - 1) mod P), every element i is copied bit for bit from
 * rank_buf[owner(i)][i] into the same position of every other rank's
 * buffer.
 *
 *   P         number of ranks, 1..DDP_MAX_RANKS (P = 1: nothing to do)
 *   chunking  C >= 1
 *   rank_buf  host array [P] of device pointers, n elements of dtype each,
 *             16-byte aligned, pairwise disjoint
 *   dtype     DDP_F32 or DDP_BF16 (only the element size matters)
 *   n         elements per rank, >= 0
 * Errors: DDP_E_ARG, DDP_E_ALIGN, DDP_E_OVERLAP, DDP_E_HIP.
 */
int allgather_ring_emulated(int32_t P, int32_t chunking, void* const* rank_buf,
                            ddp_dtype dtype, int64_t n, void* stream);

/*
 * reducescatter_ring_buckets / allgather_ring_buckets -- the two halves over
 * every bucket of a flat buffer in one call.
 *
 * Bucket k is elements [k * E, min((k + 1) * E, n)) of every rank buffer,
 * as for allreduce_ring_buckets ("Distributed Training", "Data parallelism
 * and all-reduce"; FSDP reduce-scatters gradients and all-gathers
 * parameters unit by unit, same page, "Sharded data parallelism").  Each
 * bucket is reduce-scattered (all-gathered) exactly as the single-bucket
 * call does it: its own C chunks of ceil(len_k / C) elements, its own
 * owners, the same bits, untouched elements left untouched.  When C is a
 * multiple of P and E a multiple of C, consecutive full buckets are one
 * ring of (full buckets x C) chunks with the same chunks and owners and go
 * out as one launch sequence; otherwise each bucket is its own.
 *
 *   bucket_elems  E >= 1, with E * element size a multiple of 16 bytes for
 *                 every element type of the call
 *   n             elements per rank buffer (all its buckets), >= 0
 *   other arguments, layout, ownership and errors as for
 *   reducescatter_ring_emulated and allgather_ring_emulated.
 * Errors: those of the single-bucket calls; DDP_E_ARG for bucket_elems < 1,
 * DDP_E_ALIGN for a bucket size that misaligns the buckets.
 */
int reducescatter_ring_buckets(ddp_reduce_op op, int32_t P, int32_t chunking,
                               const void* const* rank_in, ddp_dtype in_dtype,
                               void* const* rank_out, ddp_dtype out_dtype,
                               int64_t n, int64_t bucket_elems, void* stream);
int allgather_ring_buckets(int32_t P, int32_t chunking, void* const* rank_buf,
                           ddp_dtype dtype, int64_t n, int64_t bucket_elems,
                           void* stream);

/*
 * allreduce_ring_stepwise -- the same all-reduce, one ring step per launch.
 *
 * The ring as the pages describe it: peers pass slices of the tensor around
 * the ring (Burn collective blog, "Methods", Ring), P-1 reduce-scatter steps
 * then P-1 all-gather steps ("Distributed Training", "Sharded data
 * parallelism"; its "How to Apply It" prints the resulting traffic,
 * 2(W-1)/W model sizes per device).  Launch t of the reduce-scatter moves the
 * chunk that started at rank s from rank s+t to rank s+t+1, which adds it to
 * its own copy; the last one ends at the chunk's owner, which applies Mean;
 * the all-gather launches then copy the finished chunk around the ring.
 * The result is bit for bit that of allreduce_ring_emulated.
 *
 *   rank_buf  host array [P] of device pointers, n float32 each, in place:
 *             the inputs, and on completion every rank's result; 16-byte
 *             aligned, pairwise disjoint
 *   dtype     DDP_F32 only (partial sums live in the rank buffers and stay
 *             float32); DDP_BF16 returns DDP_E_UNSUPPORTED
 *   sent_dev  device array [P] of uint64, 8-byte aligned, or NULL; rank r's
 *             entry is increased by the number of elements rank r sends
 *             (the caller clears it first)
 *   other arguments as for allreduce_ring_emulated.  2(P-1) launches (more
 *   for n over 2^29).
 * Errors: DDP_E_ARG, DDP_E_UNSUPPORTED, DDP_E_ALIGN, DDP_E_OVERLAP, DDP_E_HIP.
 */
int allreduce_ring_stepwise(ddp_reduce_op op, int32_t P, int32_t chunking,
                            void* const* rank_buf, ddp_dtype dtype, int64_t n,
                            uint64_t* sent_dev, void* stream);

/*
 * allreduce_ring_stepwise_buckets -- the stepwise ring over every bucket of
 * a flat buffer in one call.
 *
 * Each bucket (as for allreduce_ring_buckets) goes through its own P-1
 * reduce-scatter and P-1 all-gather steps, with its own chunks, exactly as
 * allreduce_ring_stepwise runs it alone: the same bits and the same send
 * counts.  When C is a multiple of P and E a multiple of C, consecutive full
 * buckets are one ring of (full buckets x C) chunks whose step t moves every
 * chunk of every full bucket in one launch: 2(P-1) launches for the full
 * buckets together instead of 2(P-1) each.
 *
 *   bucket_elems  E >= 1, with 4 * E a multiple of 16 bytes
 *   other arguments, layout, ownership and errors as for
 *   allreduce_ring_stepwise (sent_dev accumulates over all buckets).
 * Errors: those of allreduce_ring_stepwise; DDP_E_ARG for bucket_elems < 1,
 * DDP_E_ALIGN for a bucket size that misaligns the buckets.
 */
int allreduce_ring_stepwise_buckets(ddp_reduce_op op, int32_t P, int32_t chunking,
                                    void* const* rank_buf, ddp_dtype dtype, int64_t n,
                                    int64_t bucket_elems, uint64_t* sent_dev,
                                    void* stream);

/*
 * allreduce_tree_emulated -- the all-reduce along a tree instead of a ring.
 *
 * The Tree strategy arranges the peers in a b-tree that reduces in parallel
 * (O(log_b N)); the Centralized strategy sends every tensor to a root that
 * aggregates and broadcasts the result (Burn collective blog, "Methods");
 * both are a reduce followed by a broadcast (same page, "Local ring
 * downfall").  The tree is the b-ary heap over the ranks: rank 0 is the root
 * and the children of rank i are ranks b*i+1 ... b*i+b.  Every rank adds its
 * children's partial sums to its own value in increasing child order, after
 * all of them have arrived; the root applies Mean; every rank receives the
 * root's value.  Partial sums are float32.  branching >= P-1 makes every
 * rank a child of the root: the Centralized strategy, whose additions run
 * in rank order (the same order as allreduce_ring_emulated with one chunk).
 *
 *   branching  b >= 1 (b = 1 is a chain)
 *   other arguments, layout, ownership and errors as for
 *   allreduce_ring_emulated (there is no chunking: the tree's order is the
 *   same for every element).
 */
int allreduce_tree_emulated(ddp_reduce_op op, int32_t P, int32_t branching,
                            const void* const* rank_in, ddp_dtype in_dtype,
                            void* const* rank_out, ddp_dtype out_dtype,
                            int64_t n, void* stream);

/* The strategies of one level of a two-level all-reduce (Burn collective
 * blog, "Methods"). */
typedef enum ddp_strategy {
    DDP_STRATEGY_RING = 0,         /* parameter: chunk count C >= 1, 0 = the level's member count */
    DDP_STRATEGY_TREE = 1,         /* parameter: branching factor b >= 1 */
    DDP_STRATEGY_CENTRALIZED = 2   /* parameter ignored */
} ddp_strategy;

/*
 * allreduce_hierarchical_emulated -- the all-reduce split over two levels,
 * each with its own strategy (Burn collective blog, "Local strategy and
 * global strategy" and "Local ring downfall").
 *
 * The P = nodes * local_ranks ranks form `nodes` nodes of `local_ranks`
 * peers, numbered node-major: rank g * local_ranks + l is peer l of node g.
 * With a Tree or Centralized local strategy the steps are a local reduce to
 * peer 0 of every node, a global all-reduce among those peers, and a local
 * broadcast; with a Ring local strategy the local reduce is a local ring
 * all-reduce (a ring cannot be split into a reduce and a broadcast), after
 * which peer 0 holds the same node sum.  Each level sums in the order of its
 * single-level strategy over its members (the node's peers in peer order;
 * the nodes in node order):
 *   Ring: C chunks of length ceil(n / C); the chunk holding element i
 *     starts at member (chunk mod m) and adds the members in ring order
 *     (as allreduce_ring_emulated over m members);
 *   Tree: the b-ary heap of allreduce_tree_emulated over the members;
 *   Centralized: the root adds the other members in order.
 * Mean divides the global sum once by P (all ranks), correctly rounded;
 * every rank receives the result.  Partial sums are float32 throughout.
 * One node is the local strategy alone over P ranks; one peer per node is
 * the global strategy alone.
 *
 *   nodes, local_ranks     >= 1 each, product <= DDP_MAX_RANKS
 *   local_strategy, local_param    the strategy within every node and its
 *                                  parameter (see ddp_strategy)
 *   global_strategy, global_param  the strategy over the nodes
 *   rank_in, in_dtype, rank_out, out_dtype, n, stream   as for
 *   allreduce_ring_emulated, with P = nodes * local_ranks
 * Errors: as for allreduce_ring_emulated; DDP_E_ARG also for an unknown
 * strategy, a negative ring parameter or a tree branching below 1.
 */
int allreduce_hierarchical_emulated(ddp_reduce_op op, int32_t nodes, int32_t local_ranks,
                                    ddp_strategy local_strategy, int32_t local_param,
                                    ddp_strategy global_strategy, int32_t global_param,
                                    const void* const* rank_in, ddp_dtype in_dtype,
                                    void* const* rank_out, ddp_dtype out_dtype,
                                    int64_t n, void* stream);

/*
 * allreduce_hierarchical_buckets -- the two-level all-reduce over every
 * bucket of a flat buffer in one call.
 *
 * Bucket k is elements [k * E, min((k + 1) * E, n)) of every rank buffer,
 * as for allreduce_ring_buckets ("Distributed Training", "Data parallelism
 * and all-reduce"), and each bucket is reduced exactly as
 * allreduce_hierarchical_emulated reduces it alone: its own chunks at each
 * ring level, the same bits.  A ring level's chunk j starts at member
 * j mod M (M its member count), so when every ring level's chunking is a
 * multiple of its M and E a multiple of that chunking, consecutive full
 * buckets are one two-level ring and go out as one launch sequence; levels
 * of fixed order (tree, centralized) never prevent it.  Otherwise each
 * bucket is its own.
 *
 *   bucket_elems  E >= 1, with E * element size a multiple of 16 bytes for
 *                 both element types
 *   other arguments, layout, ownership and errors as for
 *   allreduce_hierarchical_emulated.
 * Errors: those of allreduce_hierarchical_emulated; DDP_E_ARG for
 * bucket_elems < 1, DDP_E_ALIGN for a bucket size that misaligns the buckets.
 */
int allreduce_hierarchical_buckets(ddp_reduce_op op, int32_t nodes, int32_t local_ranks,
                                   ddp_strategy local_strategy, int32_t local_param,
                                   ddp_strategy global_strategy, int32_t global_param,
                                   const void* const* rank_in, ddp_dtype in_dtype,
                                   void* const* rank_out, ddp_dtype out_dtype,
                                   int64_t n, int64_t bucket_elems, void* stream);

/*
 * ddp_multi_plan -- host only: lay out the tiles of a multi-tensor
 * all-reduce.
 *
 * Without buckets every parameter's gradient is all-reduced on its own
 * (CS336 Lecture 8, "Data Parallelism (DDP)"), and small collectives use
 * the hardware badly ("Distributed Training", "Communication costs"); the
 * multi-tensor call below reduces all of them in one launch.  This plan
 * gives tensor t a run of tiles starting at tiles[t].first_tile, in the
 * order given.  Any order gives the same results; listing the tensors
 * smallest first (and the pointer tables in the same order) puts the
 * tiles of small tensors, which do the least work per tile, at the start
 * of the launch rather than in its tail (measured 1.6-2% faster on the
 * 161 ResNet-50 gradient tensors).
 *
 *
 * Tiles of a tensor start at its first element, so a tensor that starts
 * off a 128-byte line (a view into a larger buffer) has every wave access
 * straddle one line more than it covers, and its stores leave lines partly
 * written (measured 25% slower on the 161 ResNet-50 tensors as views of
 * arena rows).  With `align_to`, the address of each tensor (say rank 0's
 * input), a tensor whose address is 16-byte aligned but not on a line gets
 * a short first tile up to the next line (`lead` elements) when that keeps
 * every later tile's offsets 16-byte aligned for both element types and for
 * float32 optimizer state; the other ranks' copies should then sit at the
 * same offset within a line, as rows of one arena do.  The plan is then
 * specific to those addresses.
 *
 *   numels       host array [n_tensors], each 0 .. 2^29 elements
 *   P, in_dtype, out_dtype   as for the all-reduce (they set the tile size)
 *   align_to     host array [n_tensors] of addresses, or NULL (no short
 *                first tiles: the plan depends on the numels only)
 *   tiles        host array [n_tensors] to receive the plan
 *   total_tiles  out: tiles of all tensors (the launch's workgroups), at
 *                most 2^31 - 1
 *   tile_elems   out: elements per tile (pass it back to the all-reduce)
 * Errors: DDP_E_ARG (bad counts, pointers, P or dtypes), DDP_E_UNSUPPORTED
 * (a tensor over 2^29 elements: use the single-tensor call; over 2^31 - 1
 * tiles in all).
 */
int ddp_multi_plan(const int64_t* numels, int32_t n_tensors, int32_t P,
                   ddp_dtype in_dtype, ddp_dtype out_dtype, const void* const* align_to,
                   ddp_tensor_tiles* tiles, int64_t* total_tiles, int64_t* tile_elems);

/*
 * ddp_multi_block_map -- host only: an index into a multi-tensor plan, so
 * that a workgroup finds its tensor with one table read and a short search
 * instead of a binary search over the whole plan (8 dependent reads for
 * 161 tensors, 11 for 2,000).  Entry k is the tensor holding tile 64 k: the
 * largest t with tiles[t].first_tile <= 64 k.
 *
 *   tiles, n_tensors, total_tiles   a plan from ddp_multi_plan (host copy)
 *   block_first  host array [cap] to receive ceil(total_tiles / 64) entries;
 *                may be NULL to query the count only
 *   n_blocks     out: ceil(total_tiles / 64)
 * The kernels clamp every entry they read to [0, n_tensors), so a map of
 * another plan gives wrong tensors but no access outside the plan.
 * Errors: DDP_E_ARG (counts, NULL pointers), DDP_E_PLAN (first_tile not
 * starting at 0 or decreasing, or cap too small).
 */
int ddp_multi_block_map(const ddp_tensor_tiles* tiles, int32_t n_tensors,
                        int64_t total_tiles, int32_t* block_first, int64_t cap,
                        int64_t* n_blocks);

/*
 * allreduce_multi_ring_emulated -- n_tensors independent all-reduces in one
 * launch; tensor t gives, bit for bit, what allreduce_ring_emulated gives
 * for it alone (same P, op and chunking; its own chunk length
 * ceil(numel_t / C)).
 *
 *   tiles_dev    DEVICE array [n_tensors]: the plan of ddp_multi_plan for
 *                these tensors, P and dtypes (made with or without align_to;
 *                with, the tiles sit on lines of the addresses it was given,
 *                and the results are the same bits either way; the library
 *                does not read it on the host; any other table is undefined
 *                behaviour)
 *   total_tiles, tile_elems   the values ddp_multi_plan returned
 *                (tile_elems is checked against this call's tile size)
 *   block_first_dev  DEVICE array: the block map of ddp_multi_block_map for
 *                this plan, or NULL (then every workgroup searches the whole
 *                plan; the results are the same)
 *   in_ptrs_dev  DEVICE array [P * n_tensors] of device pointers,
 *                rank-major (entry r * n_tensors + t = rank r's tensor t)
 *   out_ptrs_dev DEVICE array [P * n_tensors] of device pointers, same
 *                layout; an output may be its input (in place)
 *   Tensors need only the alignment of their element type; 16-byte
 *   aligned ones move as 16-byte vectors.  Buffers of different tensors or
 *   ranks must not overlap (not checked: the tables live on the device).
 * Errors: DDP_E_ARG, DDP_E_PLAN (tile_elems mismatch), DDP_E_HIP.
 */
int allreduce_multi_ring_emulated(ddp_reduce_op op, int32_t P, int32_t chunking,
                                  int32_t n_tensors, const ddp_tensor_tiles* tiles_dev,
                                  int64_t total_tiles, int64_t tile_elems,
                                  const int32_t* block_first_dev,
                                  const void* const* in_ptrs_dev, ddp_dtype in_dtype,
                                  void* const* out_ptrs_dev, ddp_dtype out_dtype,
                                  void* stream);

/*
 * allreduce_multi_fused_sgd -- the multi-tensor all-reduce followed, in the
 * same launch, by one SGD-with-momentum step per tensor: the whole
 * per-parameter data-parallel step (CS336 Lecture 8, "Data Parallelism
 * (DDP)": every parameter's gradient is all-reduced with AVG, then every
 * rank runs optimizer.step() locally on identical gradients).  Tensor t is
 * reduced exactly as allreduce_multi_ring_emulated reduces it; with g its
 * reduced float32 gradient (Mean applied, before any output rounding) each
 * element then does, one rounding per operation,
 *     v = mu * v;  v = v + g;  w = w - lr * v
 * on the tensor's float32 master weights and momentum (one copy stands for
 * the identical replicas), as allreduce_fused_sgd does.
 *
 *   tiles_dev, total_tiles, tile_elems   the plan of ddp_multi_plan for these
 *                tensors, P, grad_dtype and out_dtype (out_dtype sets the
 *                tile size even when no gradient is written)
 *   block_first_dev  its block map (ddp_multi_block_map), or NULL
 *   in_ptrs_dev  DEVICE array [P * n_tensors] of gradient pointers,
 *                rank-major, elements of grad_dtype
 *   w_ptrs_dev, v_ptrs_dev   DEVICE arrays [n_tensors] of pointers to each
 *                tensor's float32 master weights and momentum, updated in
 *                place; they must not overlap any other buffer (not checked:
 *                the tables live on the device)
 *   lr, mu       learning rate and momentum factor (finite)
 *   out_ptrs_dev DEVICE array [P * n_tensors] receiving the reduced
 *                gradients as out_dtype, or NULL to skip writing them
 * Errors: DDP_E_ARG, DDP_E_PLAN (tile_elems mismatch), DDP_E_HIP.
 */
int allreduce_multi_fused_sgd(ddp_reduce_op op, int32_t P, int32_t chunking,
                              int32_t n_tensors, const ddp_tensor_tiles* tiles_dev,
                              int64_t total_tiles, int64_t tile_elems,
                              const int32_t* block_first_dev,
                              const void* const* in_ptrs_dev, ddp_dtype grad_dtype,
                              float* const* w_ptrs_dev, float* const* v_ptrs_dev,
                              float lr, float mu, void* const* out_ptrs_dev,
                              ddp_dtype out_dtype, void* stream);

/* Bytes of the per-GPU scratch area of allreduce_multi_ring_noalloc. */
#define DDP_NOALLOC_SCRATCH_BYTES (1 << 20)

/*
 * allreduce_multi_ring_noalloc -- allreduce_multi_ring_emulated for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  It takes host arrays and
 * builds the plan (ddp_multi_plan, tiles on rank 0's input lines), its block
 * map and the two pointer tables itself, in a scratch area of
 * DDP_NOALLOC_SCRATCH_BYTES that the library holds in device memory on every
 * GPU it runs on until the process ends; it calls no hipMalloc, hipFree or
 * other allocating device routine.  Results are, bit for bit, those of
 * allreduce_multi_ring_emulated on the same tensors (tensor t reduced alone,
 * in the ring order, with its own chunk length).
 *
 *   op, P, chunking      as for allreduce_multi_ring_emulated
 *   n_tensors            tensors per rank, >= 1
 *   numels               HOST array [n_tensors], each 0 .. 2^29 elements
 *   in_ptrs              HOST array [P * n_tensors] of device pointers,
 *                        rank-major (entry r * n_tensors + t = rank r's
 *                        tensor t), each aligned to its element size; may be
 *                        NULL where numels[t] = 0
 *   out_ptrs             HOST array [P * n_tensors], same layout, elements of
 *                        out_dtype; an output may be its own input when the
 *                        element types match (in place)
 *   stream               the stream to enqueue on (NULL: the null stream);
 *                        its GPU's scratch area is used
 * Host arrays are read during the call only.  Apart from the in-place alias,
 * every buffer must be disjoint from every other (checked).  The tables
 * (16 bytes per tensor, 2 * 8 * P bytes per tensor of pointers, 4 bytes per
 * 64 tiles of block map, each part rounded to 256 bytes) must fit the
 * scratch area: about 7,700 tensors at P = 8.
 *
 * Every call on one GPU shares that GPU's scratch area, which keeps the last
 * call's tables: a call writes its tables in, in stream order, with small
 * kernels that carry them in their arguments, then launches.  It writes
 * only the parts that differ from what the last call on that GPU wrote, so
 * the same tensors again write nothing and only launch.  Under HIP
 * graph capture the writes are captured with the launch, so every replay
 * rewrites the area with its own tables first; from a GPU's first captured
 * call on, no call on that GPU skips its writes (replays change the area
 * when they run).  Calls and replays on one stream follow each other
 * safely; calls that
 * overlap on one GPU (other streams, other threads' streams, replays on
 * other streams) race on the tables and give undefined results.  Nothing in the area needs clearing:
 * every byte a launch reads was written by its own call (or by an earlier
 * call with the same tables).
 * Errors: DDP_E_ARG (counts, NULL arrays or pointers, op, dtypes),
 * DDP_E_ALIGN, DDP_E_OVERLAP, DDP_E_UNSUPPORTED (a tensor over 2^29
 * elements; tables larger than the scratch area), DDP_E_HIP.  On any error
 * nothing has been enqueued.
 */
int allreduce_multi_ring_noalloc(ddp_reduce_op op, int32_t P, int32_t chunking,
                                 int32_t n_tensors, const int64_t* numels,
                                 const void* const* in_ptrs, ddp_dtype in_dtype,
                                 void* const* out_ptrs, ddp_dtype out_dtype,
                                 void* stream);

/* Kernel families whose launch shape ddp_set_wg_per_cu can override. */
typedef enum ddp_kernel_family {
    DDP_KF_RING = 0,            /* allreduce_ring_emulated */
    DDP_KF_RING_SGD = 1,        /* allreduce_fused_sgd, zero1_sgd_step_emulated */
    DDP_KF_TREE = 2,            /* allreduce_tree_emulated, allreduce_hierarchical_emulated */
    DDP_KF_REDUCE_SCATTER = 3,  /* reducescatter_ring_emulated */
    DDP_KF_ALL_GATHER = 4,      /* allgather_ring_emulated */
    DDP_KF_MULTI = 5,           /* allreduce_multi_ring_emulated, allreduce_multi_fused_sgd */
    DDP_KF_BUCKET_COPY = 6,     /* ddp_bucket_pack, ddp_bucket_unpack */
    DDP_KF_STEP = 7             /* allreduce_ring_stepwise */
} ddp_kernel_family;

/*
 * ddp_set_wg_per_cu -- host only, no device work.  A tuning knob, not part
 * of the method: results are the same bits at every setting.
 *
 * Every kernel here streams HBM with little arithmetic, and the mix of
 * reads and writes reaches its highest rate on MI355X with few resident
 * waves per CU.  Each launch therefore caps its resident workgroups per CU
 * (by reserving LDS it never touches) at a value chosen per kernel family,
 * rank count and element types from measurements.  This call overrides the
 * cap of one family for every later launch of the process (all threads):
 *
 *   family      the kernel family
 *   wg_per_cu   2..64: at most that many workgroups per CU; 0: no cap (the
 *               hardware's own occupancy); -1: the built-in choice again
 * Errors: DDP_E_ARG (unknown family, value outside -1, 0, 2..64).
 * Calls that race with launches on other threads are safe; which setting a
 * concurrent launch sees is unspecified.
 */
int ddp_set_wg_per_cu(ddp_kernel_family family, int32_t wg_per_cu);

/* Message describing the calling thread's most recent non-OK status
 * ("" if none).  The pointer stays valid until the thread's next call. */
const char* ddp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DDP_ALLREDUCE_H */
