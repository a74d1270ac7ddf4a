"""FP4 codebook for the same blockwise 4-bit scheme (the quant type "fp4").

TEST INFRASTRUCTURE ONLY (see the package docstring).

The level values are PARITY UNPINNED BY THE PAGES: the pages give none.  The
tests pin them to the E2M1 element's format parameters from the OCP MX
specification (tests/golden/e2m1_mx_element.json), not to a page; the
encoder, the scales and the packing are pinned as NF4's are.

"bitsandbytes deep dive" (aicoding.csdn.net), section 6.5 and section 8.1: the
quant type picks the codebook, i.e. what value each 4-bit code 0..15 stands
for; "fp4" is a floating-point-style layout of 16 codes, not a uniform integer
grid, and it is the configuration's default (section 8.1).  The page gives no
values.  Reading R13: the 4-bit float E2M1 -- one sign bit (bit 3), two
exponent bits (bits 2..1, bias 1) and one mantissa bit (bit 0), with
subnormals at exponent 0 and no infinities or NaNs, the element type of the
OCP Microscaling (MX) formats v1.0 -- normalised to [-1, 1] by its largest
magnitude 6, so that the block absmax maps to +-1 as NF4's does (section 5.2:
u = w / a lies in [-1, 1]).  The code of a level is its E2M1 bit pattern.

Encoding (reading R13, with R3's tie rule): the nearest level to u = w / a in
exact arithmetic; a tie goes to the lower level.  Ties cannot occur between
two distinct levels for bf16 weights (every adjacent pair of levels has a
member that is not a short binary fraction, so no product a * m of a bf16 a
and a midpoint m is a bf16 value); they occur only between +0 and -0, which
are the same level: w = 0 (of either sign) and the all-zero block encode as
+0 (code 0).  Code 8 (-0) decodes to -0 but is never produced.

Everything else is the NF4 scheme of oracle.nf4 with this table: blocks of
64, the block absmax, the double quantization of the scales (or the fp32
absmax without it), the packing, a_hat and w_hat = RNE_bf16(fl32(a_hat * c_q)).
"""
from fractions import Fraction

import numpy as np

from . import nf4

E2M1_BIAS = 1
E2M1_MAX = 6.0          # largest magnitude: exponent 3, mantissa 1 -> 2^(3-1) * 1.5


def e2m1_value(code):
    """Exact value of the 4-bit float E2M1 with bit pattern `code` (a Fraction).

    Sign bit 3; exponent e = bits 2..1; mantissa m = bit 0.  e = 0 is
    subnormal: (m / 2) * 2^(1 - bias); otherwise (1 + m / 2) * 2^(e - bias).
    """
    code = int(code)
    assert 0 <= code < 16
    s = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = Fraction(m, 2) * Fraction(2) ** (1 - E2M1_BIAS)
    else:
        mag = (1 + Fraction(m, 2)) * Fraction(2) ** (e - E2M1_BIAS)
    return s * mag


def fp4_levels_exact():
    """c[code] = e2m1(code) / 6 as exact Fractions, code 0..15 (code 8 is -0, equal to 0)."""
    return [e2m1_value(c) / Fraction(int(E2M1_MAX)) for c in range(16)]


def fp4_table():
    """The FP4 codebook c[0..15] in code order as float32 (each exact quotient rounded to nearest).

    The quotients are v/6 for v with at most two significant bits; rounding
    the float64 quotient to float32 is the correctly rounded float32 of the
    exact quotient here (checked against exact rational rounding in the
    tests).  Code 8 is -0.0, kept as a signed zero so that a_hat * c_8 = -0.
    """
    out = np.empty(16, dtype=np.float32)
    for c, q in enumerate(fp4_levels_exact()):
        v = np.float32(float(q))
        out[c] = np.float32(-0.0) if c == 8 else v
    return out


def sorted_codes():
    """The 15 distinct levels in ascending order, as codes: 15, 14, .., 9, 0, 1, .., 7.

    Zero appears once, as +0 (code 0).
    """
    return [15 - j for j in range(7)] + [j for j in range(8)]


def fp4_midpoints():
    """Decision thresholds between the 14 pairs of adjacent distinct levels, exact in float64."""
    c = fp4_table().astype(np.float64)
    s = c[sorted_codes()]
    return (s[:-1] + s[1:]) * 0.5


def fp4_codes(wb, a):
    """q = the code of the nearest level to u = w/a, ties to the lower level (zero -> +0).

    The nearest distinct level has ascending index idx = #{j : w > a * m_j}
    (the count of midpoints strictly below u, as for NF4); a * m_j is exact in
    float64 for bf16 a.  The code is then that level's E2M1 pattern.
    wb: [nblocks, 64] float64; a: [nblocks] float64 >= 0.  Returns uint8.
    """
    wb = np.asarray(wb, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    m = fp4_midpoints()
    thr = a[:, None, None] * m[None, None, :]
    idx = np.sum(wb[:, :, None] > thr, axis=2)
    q = np.asarray(sorted_codes(), dtype=np.uint8)[idx]
    q[a == 0.0, :] = 0
    return q


def quantize(W_u16, dtype="bf16"):
    """FP4 blockwise quantization with double-quantized scales -> (packed codes, q8, A2).

    The scales depend on the block absmax only, so q8 and A2 equal those of
    the NF4 quantization of the same weight (section 7: the constants are
    quantized after, and independently of, the codes).
    """
    wb16 = nf4.blocks(np.asarray(W_u16, dtype=nf4.codec(dtype).BITS))
    nb = wb16.shape[0]
    a = np.empty(nb, dtype=np.float64)
    codes = np.empty((nb, nf4.BLOCK), dtype=np.uint8)
    step = 1 << 14
    for s in range(0, nb, step):
        wb = nf4.codec(dtype).to_f64(wb16[s:s + step])
        a[s:s + step] = nf4.block_absmax(wb)
        codes[s:s + step] = fp4_codes(wb, a[s:s + step])
    A2 = nf4.superblock_absmax(a)
    q8 = np.empty(nb, dtype=np.uint8)
    for s in range(0, nb, step):
        e = min(nb, s + step)
        q8[s:e] = nf4.scale_codes(a[s:e], A2[s // nf4.SUPER: -(-e // nf4.SUPER)])
    return nf4.pack_nibbles(codes), q8, A2


def quantize_nodq(W_u16, dtype="bf16"):
    """FP4 codes with one fp32 absmax per block (double quantization off) -> (packed codes, absmax)."""
    wb16 = nf4.blocks(np.asarray(W_u16, dtype=nf4.codec(dtype).BITS))
    nb = wb16.shape[0]
    a = np.empty(nb, dtype=np.float32)
    codes = np.empty((nb, nf4.BLOCK), dtype=np.uint8)
    step = 1 << 14
    for s in range(0, nb, step):
        wb = nf4.codec(dtype).to_f64(wb16[s:s + step])
        ab = nf4.block_absmax(wb)
        a[s:s + step] = ab
        codes[s:s + step] = fp4_codes(wb, ab)
    return nf4.pack_nibbles(codes), a


def dequantize(packed, q8, A2, N, K, dtype="bf16"):
    """w_hat = RNE_16(fl32(a_hat * c_q)) with the FP4 table, shape [N, K], 16-bit bits of `dtype`."""
    return nf4.dequantize(packed, q8, A2, N, K, table=fp4_table(), dtype=dtype)


def dequantize_nodq(packed, absmax, N, K, dtype="bf16"):
    """w_hat with the stored fp32 block absmax and the FP4 table."""
    return nf4.dequantize_nodq(packed, absmax, N, K, table=fp4_table(), dtype=dtype)


def dequantize_rows(packed, q8, A2, K, rows, dtype="bf16"):
    """w_hat of selected rows (double-quantized scales) with the FP4 table."""
    return nf4.dequantize_rows(packed, q8, A2, K, rows, table=fp4_table(), dtype=dtype)
