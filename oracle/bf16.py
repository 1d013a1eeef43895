"""bfloat16 <-> float32 conversions written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bfloat16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits,
7 stored mantissa bits.  The pages name 16-bit gradients with an FP32 master
copy and FP32 accumulation ("Distributed Training", Related, "Mixed-Precision
Training"; "Sharded data parallelism" for 16-bit gradients beside 32-bit
weights).  They do not state the rounding; the reading here is IEEE
round-to-nearest, ties-to-even, with NaN kept quiet.

Parity status: pinned by the tests against hand cases (ties, the largest
finite value, overflow, signed zero, subnormals, NaN) and against a
definition check that compares distances to both neighbours in exact
arithmetic on random bit patterns.
"""

import numpy as np


def bf16_bits_to_f32(bits):
    """Widen bfloat16 bit patterns (uint16) to float32.  Exact: the bf16 bits
    become the upper 16 bits of the float32 and the lower 16 are zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits.

    For a finite x the two bfloat16 values that bracket it are its truncation
    toward zero and the next bfloat16 away from zero.  The nearer one is
    chosen, comparing distances in float64 where both are exact; on a tie the
    one with an even last mantissa bit wins.  Past the largest finite value
    the next value up is taken as 2**128, which turns the rounding into
    overflow to infinity exactly when IEEE rounding would.  NaN stays NaN with
    its sign and its quiet bit set.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    sign = u & np.uint32(0x80000000)
    mag = u & np.uint32(0x7FFFFFFF)
    is_nan = mag > np.uint32(0x7F800000)
    # Infinity and NaN take no part in the distance comparison below.
    mag_cmp = np.where(mag >= np.uint32(0x7F800000), np.uint32(0), mag)

    lo_mag = np.where(mag >= np.uint32(0x7F800000), mag,
                      mag & np.uint32(0xFFFF0000))     # truncation toward zero
    hi_mag = lo_mag + np.uint32(0x00010000)            # next bf16 away from zero
    ax = mag_cmp.view(np.float32).astype(np.float64)
    lo_val = np.where(mag >= np.uint32(0x7F800000), np.uint32(0), lo_mag) \
        .view(np.float32).astype(np.float64)
    # hi_mag == 0x7F800000 encodes infinity; its distance is taken to 2**128.
    hi_val = np.where(hi_mag == np.uint32(0x7F800000), 2.0 ** 128,
                      np.minimum(hi_mag, np.uint32(0x7F7F0000)).view(np.float32)
                      .astype(np.float64))
    d_lo = ax - lo_val
    d_hi = hi_val - ax
    lo_even = ((lo_mag >> np.uint32(16)) & np.uint32(1)) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    # Exact bf16 values (including zero and infinity) have d_lo == 0.
    take_hi &= d_lo != 0
    out_mag = np.where(take_hi, hi_mag, lo_mag)
    out = (sign | out_mag) >> np.uint32(16)
    nan_out = ((u >> np.uint32(16)) | np.uint32(0x0040))
    out = np.where(is_nan, nan_out, out)
    return out.astype(np.uint16)
