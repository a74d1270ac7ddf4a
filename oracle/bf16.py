"""bfloat16 as raw uint16 bit patterns (numpy has no bf16 dtype).

TEST INFRASTRUCTURE ONLY (see the package docstring).

bfloat16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits,
7 stored mantissa bits.  The compute dtype of the path is bf16 ("bitsandbytes
deep dive", section 8.3 / 8.5), so dequantized weights are produced as bf16 by
round-to-nearest-even of an fp32 value.
"""
import numpy as np

BITS = np.uint16     # storage of one value


def to_f32(u16):
    """Exact value of bf16 bit patterns as float32 (bits placed in the top half)."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(u16):
    """Exact value of bf16 bit patterns as float64."""
    return to_f32(u16).astype(np.float64)


def from_f32_rne(f32):
    """Round float32 values to bf16, nearest, ties to even; returns uint16 bits.

    Written from the definition, not from a bit trick: for a finite x the two
    bf16 neighbours are lo = x with its low 16 bits cleared (the truncation
    toward zero) and hi = the next bf16 away from zero.  Whichever is nearer to
    x wins; at an exact tie the one whose last stored mantissa bit is 0 wins.
    Distances are computed in float64, where the difference of two float32
    values is exact.  NaN stays NaN (quiet); infinities pass through.
    """
    x = np.asarray(f32, dtype=np.float32)
    bits = x.view(np.uint32)
    lo_bits = bits & np.uint32(0xFFFF0000)
    hi_bits = lo_bits + np.uint32(0x00010000)          # next magnitude up
    lo = lo_bits.view(np.float32).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        hi = hi_bits.view(np.float32).astype(np.float64)
        # past the largest finite bf16 the next grid point is 2^128 (which
        # then encodes as infinity): measure the distance to that point
        hi = np.where(np.isinf(hi), np.copysign(2.0 ** 128, hi), hi)
        xd = x.astype(np.float64)
        d_lo = np.abs(xd - lo)
        d_hi = np.abs(hi - xd)
    lo_even = ((lo_bits >> np.uint32(16)) & np.uint32(1)) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    out = np.where(take_hi, hi_bits, lo_bits) >> np.uint32(16)
    finite = np.isfinite(x)
    out = np.where(finite, out, (bits >> np.uint32(16)) | np.where(np.isnan(x), np.uint32(0x40), np.uint32(0)))
    return out.astype(np.uint16)
