/* A plain C caller of the library: plans buckets and exercises the
 * validation of the all-reduce entry points, with no GPU work (every call
 * below returns before any launch).  Built and run by
 * tests/test_c_program.py; prints one line per check and exits non-zero on
 * the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ddp_allreduce.h"

#define CHECK(cond, what)                                              \
    do {                                                               \
        if (!(cond)) {                                                 \
            printf("FAIL %s (last error: %s)\n", what, ddp_last_error()); \
            return 1;                                                  \
        }                                                              \
        printf("ok %s\n", what);                                       \
    } while (0)

int main(void) {
    /* Three tensors in parameter order; 16-element (64-byte) float buckets. */
    const int64_t numels[3] = {5, 7, 20};
    ddp_segment segs[8];
    int64_t n_segs = -1, total = -1;
    int32_t n_buckets = -1;
    uint64_t fp1 = 0, fp2 = 0;
    int s = ddp_bucket_plan(numels, 3, DDP_F32, 64, segs, 8, &n_segs, &n_buckets, &total, &fp1);
    CHECK(s == DDP_OK, "plan status");
    CHECK(total == 32 && n_buckets == 2, "plan totals");
    /* reverse parameter order: tensor 2 (20 elements) fills bucket 0 and
     * straddles into bucket 1, then tensor 1, then tensor 0 */
    CHECK(n_segs == 4, "plan segment count");
    CHECK(segs[0].tensor == 2 && segs[0].bucket == 0 && segs[0].src_off == 0 && segs[0].dst_off == 0 &&
              segs[0].len == 16, "segment 0");
    CHECK(segs[1].tensor == 2 && segs[1].bucket == 1 && segs[1].src_off == 16 && segs[1].dst_off == 0 &&
              segs[1].len == 4, "segment 1 (straddling)");
    CHECK(segs[2].tensor == 1 && segs[2].bucket == 1 && segs[2].dst_off == 4 && segs[2].len == 7, "segment 2");
    CHECK(segs[3].tensor == 0 && segs[3].bucket == 1 && segs[3].dst_off == 11 && segs[3].len == 5, "segment 3");
    s = ddp_bucket_plan(numels, 3, DDP_F32, 64, NULL, 0, &n_segs, NULL, NULL, &fp2);
    CHECK(s == DDP_OK && n_segs == 4 && fp1 == fp2, "count-only plan, same fingerprint");
    s = ddp_bucket_plan(numels, 3, DDP_F32, 48, NULL, 0, &n_segs, NULL, NULL, &fp2);
    CHECK(s == DDP_OK && fp1 != fp2, "another bucket size, another fingerprint");
    s = ddp_bucket_plan(numels, 3, DDP_F32, 60, NULL, 0, &n_segs, NULL, NULL, NULL);
    CHECK(s == DDP_E_ARG && strstr(ddp_last_error(), "multiple of 16") != NULL, "bucket bytes not a multiple of 16");

    /* Validation of the all-reduce: fake, never dereferenced addresses. */
    const void* in[2] = {(const void*)0x7f0000000000ull, (const void*)0x7f0000100000ull};
    void* out[2] = {(void*)0x7f0004000000ull, (void*)0x7f0004100000ull};
    CHECK(allreduce_ring_emulated(DDP_MEAN, 0, 2, in, DDP_F32, out, DDP_F32, 16, NULL) == DDP_E_ARG,
          "P = 0 rejected");
    CHECK(allreduce_ring_emulated(DDP_MEAN, 2, 0, in, DDP_F32, out, DDP_F32, 16, NULL) == DDP_E_ARG,
          "chunking = 0 rejected");
    const void* odd[2] = {(const void*)0x7f0000000000ull, (const void*)0x7f0000100004ull};
    CHECK(allreduce_ring_emulated(DDP_MEAN, 2, 2, odd, DDP_F32, out, DDP_F32, 16, NULL) == DDP_E_ALIGN,
          "misaligned rank buffer rejected");
    void* over[2] = {(void*)0x7f0000000010ull, (void*)0x7f0004100000ull};
    CHECK(allreduce_ring_emulated(DDP_MEAN, 2, 2, in, DDP_F32, over, DDP_F32, 1024, NULL) == DDP_E_OVERLAP,
          "partial overlap rejected");
    CHECK(allreduce_ring_emulated(DDP_MEAN, 2, 2, in, DDP_F32, out, DDP_F32, 0, NULL) == DDP_OK &&
              ddp_last_error()[0] == '\0', "n = 0 is a no-op");
    CHECK(allreduce_ring_buckets(DDP_SUM, 2, 2, in, DDP_F32, out, DDP_F32, 1024, 6, NULL) == DDP_E_ALIGN,
          "bucket size that misaligns the buckets rejected");
    CHECK(reducescatter_ring_buckets(DDP_SUM, 2, 2, in, DDP_F32, out, DDP_F32, 1024, 0, NULL) == DDP_E_ARG &&
              allgather_ring_buckets(2, 2, out, DDP_BF16, 1024, 4, NULL) == DDP_E_ALIGN &&
              allreduce_ring_stepwise_buckets(DDP_SUM, 2, 2, out, DDP_F32, 0, 4, NULL, NULL) == DDP_OK,
          "bucketed halves and stepwise ring validation");
    CHECK(allreduce_hierarchical_buckets(DDP_MEAN, 2, 1, DDP_STRATEGY_RING, 0, DDP_STRATEGY_TREE, 2, in, DDP_F32,
                                         out, DDP_F32, 1024, 6, NULL) == DDP_E_ALIGN,
          "bucketed two-level call validation");
    CHECK(ddp_set_wg_per_cu(DDP_KF_RING, 1) == DDP_E_ARG && ddp_set_wg_per_cu(DDP_KF_RING, -1) == DDP_OK,
          "occupancy knob validation");
    /* Pack and unpack check the segment table against the plan before
     * anything is launched: bucket 1 is segments 1..3 (tensor 2's last 4
     * elements, tensor 1, tensor 0), 16 elements. */
    const void* tens[2 * 3] = {(const void*)0x7f0010000000ull, (const void*)0x7f0010100000ull,
                               (const void*)0x7f0010200000ull, (const void*)0x7f0011000000ull,
                               (const void*)0x7f0011100000ull, (const void*)0x7f0011200000ull};
    void* bk[2] = {(void*)0x7f0020000000ull, (void*)0x7f0020100000ull};
    ddp_segment b1[3];
    memcpy(b1, segs + 1, sizeof b1);
    b1[1].tensor = 3;
    CHECK(ddp_bucket_pack(2, DDP_F32, b1, 3, numels, 3, tens, bk, 16, NULL) == DDP_E_PLAN,
          "pack: a segment naming a tensor past the list is rejected");
    memcpy(b1, segs + 1, sizeof b1);
    b1[2].src_off = 1;
    CHECK(ddp_bucket_pack(2, DDP_F32, b1, 3, numels, 3, tens, bk, 16, NULL) == DDP_E_PLAN,
          "pack: a segment reading past its tensor's end is rejected");
    memcpy(b1, segs + 1, sizeof b1);
    b1[1].dst_off = 5;
    CHECK(ddp_bucket_unpack(2, DDP_F32, b1, 3, numels, 3, (void* const*)tens, (const void* const*)bk, 16,
                            NULL) == DDP_E_PLAN, "unpack: segments that leave a gap are rejected");
    memcpy(b1, segs + 1, sizeof b1);
    CHECK(ddp_bucket_pack(2, DDP_F32, b1, 3, numels, 3, tens, bk, 17, NULL) == DDP_E_PLAN,
          "pack: segments that do not cover the bucket are rejected");
    b1[0].bucket = 0;
    CHECK(ddp_bucket_pack(2, DDP_F32, b1, 3, numels, 3, tens, bk, 16, NULL) == DDP_E_PLAN,
          "pack: segments of two buckets are rejected");
    /* The allocation-free multi-tensor call: host arrays, checked before any HIP call. */
    {
        const int64_t mn[2] = {100, 37};
        const int64_t big[2] = {((int64_t)1 << 29) + 1, 1};
        const void* mi[4] = {(const void*)0x7f0030000000ull, (const void*)0x7f0030100000ull,
                             (const void*)0x7f0030200000ull, (const void*)0x7f0030300000ull};
        void* mo[4] = {(void*)0x7f0031000000ull, (void*)0x7f0031100000ull, (void*)0x7f0031200000ull,
                       (void*)0x7f0031300000ull};
        void* mo_over[4] = {(void*)0x7f0030000040ull, (void*)0x7f0031100000ull, (void*)0x7f0031200000ull,
                            (void*)0x7f0031300000ull};
        const int64_t none[2] = {0, 0};
        const void* nulls[4] = {NULL, NULL, NULL, NULL};
        void* onulls[4] = {NULL, NULL, NULL, NULL};
        CHECK(allreduce_multi_ring_noalloc(DDP_MEAN, 2, 0, 2, mn, mi, DDP_F32, mo, DDP_F32, NULL) == DDP_E_ARG,
              "no-alloc: chunking 0 is rejected");
        CHECK(allreduce_multi_ring_noalloc(DDP_MEAN, 2, 2, 2, NULL, mi, DDP_F32, mo, DDP_F32, NULL) == DDP_E_ARG,
              "no-alloc: NULL numels is rejected");
        CHECK(allreduce_multi_ring_noalloc(DDP_MEAN, 2, 2, 2, big, mi, DDP_F32, mo, DDP_F32, NULL) ==
                  DDP_E_UNSUPPORTED, "no-alloc: a tensor over 2^29 elements is rejected");
        CHECK(allreduce_multi_ring_noalloc(DDP_MEAN, 2, 2, 2, mn, mi, DDP_F32, mo_over, DDP_F32, NULL) ==
                  DDP_E_OVERLAP, "no-alloc: an output inside another input is rejected");
        CHECK(allreduce_multi_ring_noalloc(DDP_MEAN, 2, 2, 2, none, nulls, DDP_F32, onulls, DDP_F32, NULL) ==
                  DDP_OK, "no-alloc: empty tensors launch nothing");
    }
    printf("all checks passed\n");
    return 0;
}
