"""NF4 blockwise quantization with double quantization of the block scales.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Parity status of each
function is stated in its docstring; every function here is pinned by a
``-m "not gpu"`` test in ``tests/test_oracle_nf4.py`` against something other
than itself (the pages' numbers, closed forms, brute force, library routines).
The one part the pages cannot pin is the interior of the NF4 table, which is
therefore PARITY UNPINNED BY THE PAGES: the page's formula was lost in
extraction, so the 14 interior values are pinned only to the construction
below (reading R1) and to its quantile invariants; the endpoints +-1, the exact
0 and every other function of this module are pinned by the pages or the
mathematics.

Notation follows "bitsandbytes deep dive" (aicoding.csdn.net), section 5.2:
a block B = {w_i}, a = max_i |w_i|, u_i = w_i / a, q_i = argmin_j |u_i - c_j|,
w_hat_i = a * c_{q_i}.  Storage is the nn.Linear weight layout [N = Dout,
K = Din], row-major, flattened row-major and cut into blocks of 64 (section
5.1); K must be a multiple of 64 so that no block straddles a row.
"""
from statistics import NormalDist

import numpy as np

from . import bf16, f16, f32

BLOCK = 64          # first-level block (section 5.1: default block size 64)
SUPER = 256         # first-level scales per fp32 second-level scale (section 7.2)
SUPER_ELEMS = BLOCK * SUPER
ZERO_CODE = 7       # index of the exact-zero codebook entry


# ----------------------------------------------------------------------------
# a1: the NF4 codebook
# ----------------------------------------------------------------------------
def codec(dtype):
    """The float format of a tensor (deep dive 8.3): "bf16" (the default compute dtype), "f16", or "f32"
    (binary32, where the dequantized weight keeps its fp32 product unrounded)."""
    return {"bf16": bf16, "f16": f16, "f32": f32}[dtype]


def nf4_delta():
    """Truncation probability of the outermost quantile (reading R1).

    The explainer page (section 3) builds the levels from equal-probability
    segments of N(0,1), one level per segment at its midpoint; with 16 levels
    the outermost midpoint is 1 - 1/32, and with 15 levels it is 1 - 1/30.  The
    positive half here uses 8 non-zero levels and the negative half 7, so the
    shared outer probability is the mean of those two midpoints.
    """
    return 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


def nf4_table_f64():
    """The 16 NF4 levels in float64, ascending (reading R1).

    "bitsandbytes deep dive" section 6.2: take representative points from the
    quantile function of N(0,1), normalise to [-1, 1], build the two halves
    asymmetrically and keep an exact 0.  Positive half: Phi^-1 at 8 probabilities
    evenly spaced from delta down toward 1/2 (1/2 itself excluded); negative
    half: -Phi^-1 at 7 such probabilities; plus 0; everything divided by
    Phi^-1(delta) so that the extreme levels are exactly -1 and +1.
    Phi^-1 is Python's statistics.NormalDist().inv_cdf (double precision).
    """
    inv = NormalDist().inv_cdf
    d = nf4_delta()
    pos = [inv(d - i * (d - 0.5) / 8.0) for i in range(8)]
    neg = [-inv(d - i * (d - 0.5) / 7.0) for i in range(7)]
    vals = np.array(sorted(pos + neg + [0.0]), dtype=np.float64)
    return vals / inv(d)


def nf4_table():
    """The NF4 codebook c[0..15] as float32 (round-to-nearest of the float64 levels)."""
    return nf4_table_f64().astype(np.float32)


def nf4_midpoints(table=None):
    """Decision thresholds m_j = (c_j + c_{j+1}) / 2, j = 0..14, exact in float64.

    With c_j float32 the sum of two of them and the halving are exact in
    float64, so these are the exact real midpoints of the float32 codebook.
    """
    c = (nf4_table() if table is None else np.asarray(table, np.float32)).astype(np.float64)
    return (c[:-1] + c[1:]) * 0.5


# ----------------------------------------------------------------------------
# a2: blocking and block absmax
# ----------------------------------------------------------------------------
def blocks(w):
    """View a [N, K] (or flat) weight as [n/64, 64] blocks of the row-major flattening."""
    w = np.asarray(w)
    assert w.size % BLOCK == 0, "element count must be a multiple of 64"
    if w.ndim == 2:
        assert w.shape[1] % BLOCK == 0, "K must be a multiple of 64"
    return w.reshape(-1, BLOCK)


def block_absmax(wb):
    """a_b = max_i |w_i| over each block (exact; section 5.2)."""
    return np.max(np.abs(np.asarray(wb, dtype=np.float64)), axis=1)


# ----------------------------------------------------------------------------
# a4: NF4 codes and packing
# ----------------------------------------------------------------------------
def nf4_codes(wb, a, table=None):
    """q = argmin_j |w/a - c_j| in exact arithmetic, ties to the lower index.

    Because c is ascending, the nearest level is the number of midpoints that
    u = w/a lies strictly above: q = #{j : w/a > m_j}.  A tie (u exactly on a
    midpoint) leaves u at the lower index.  With a > 0 this is the same as
    q = #{j : w > a*m_j}; a*m_j is exact in float64 whenever a has at most 27
    significant bits (bf16 inputs have 8), so the comparison is exact.
    An all-zero block (a = 0) has no defined u; it takes the zero code 7
    (reading: the block is reproduced exactly by a * c_7 = 0).
    wb: [nblocks, 64] float64; a: [nblocks] float64 >= 0.  Returns uint8 codes.
    """
    wb = np.asarray(wb, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    m = nf4_midpoints(table)
    thr = a[:, None, None] * m[None, None, :]            # [nb, 1, 15], exact
    q = np.sum(wb[:, :, None] > thr, axis=2).astype(np.uint8)
    q[a == 0.0, :] = ZERO_CODE
    return q


def pack_nibbles(codes):
    """Two 4-bit codes per byte: element 2i in bits 7..4, element 2i+1 in bits 3..0.

    The page only says two codes share one uint8 (section 5.2 / 8.2); the
    nibble order is a reading.
    """
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    assert c.size % 2 == 0 and np.all(c < 16)
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of pack_nibbles: [n/2] bytes -> [n] codes."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0x0F
    return out


# ----------------------------------------------------------------------------
# a3: double quantization of the block scales
# ----------------------------------------------------------------------------
def superblock_absmax(a):
    """A2_S = max of the block absmax values a_b over each group of 256 blocks.

    Groups are consecutive flat block indices [256 S, 256 S + 256); the last
    group is short when the block count is not a multiple of 256.  Returned as
    float32 (exact: every a_b of a bf16 weight is a bf16 value).
    """
    a = np.asarray(a, dtype=np.float64)
    ng = -(-a.size // SUPER)
    pad = np.zeros(ng * SUPER, dtype=np.float64)
    pad[: a.size] = a
    return pad.reshape(ng, SUPER).max(axis=1).astype(np.float32)


def scale_codes(a, A2):
    """8-bit code of each block scale: q8 = argmin_k |a/A2 - k/255|, ties to the lower k.

    Reading of section 7.2 ("first-level scale stored in 8 bits, one fp32
    second-level scale per 256"): a linear unsigned absmax code over [0, 255],
    the absmax idea of section 4.1 applied to non-negative values.
    Exact form: the nearest k is the number of half-way points (2k-1)/510 that
    a/A2 lies strictly above, q8 = #{k in 1..255 : 510 a > (2k-1) A2}; both
    products are exact in float64 (bf16-valued operands).  A2 = 0 gives 0.
    a: [nblocks] float64; A2: [ngroups] float32.  Returns uint8.
    """
    a = np.asarray(a, dtype=np.float64)
    A2b = np.repeat(np.asarray(A2, dtype=np.float64), SUPER)[: a.size]
    k = np.arange(1, 256, dtype=np.float64)
    q = np.sum(510.0 * a[:, None] > (2.0 * k[None, :] - 1.0) * A2b[:, None], axis=1)
    return q.astype(np.uint8)


def scale_dequant(q8, A2):
    """a_hat_b = fl32( fl32(A2_S / 255) * q8_b ): two IEEE float32 roundings (reading)."""
    q8 = np.asarray(q8, dtype=np.uint8)
    A2 = np.asarray(A2, dtype=np.float32)
    step = A2 / np.float32(255.0)                        # float32, correctly rounded
    stepb = np.repeat(step, SUPER)[: q8.size]
    return (stepb * q8.astype(np.float32)).astype(np.float32)


# ----------------------------------------------------------------------------
# a5: dequantization
# ----------------------------------------------------------------------------
def dequantize(packed, q8, A2, N, K, table=None, dtype="bf16"):
    """w_hat = RNE_16( fl32(a_hat_b * c_q) ) as uint16 bits, shape [N, K].

    Section 5.2: w_hat = a * c_q, with the scale itself recovered from its 8-bit
    code (section 7).  The product is taken in float32 and rounded once to the
    compute dtype (section 8.3: bf16, or fp16 with dtype="f16"); IEEE signed
    zeros are kept.
    """
    ahat = scale_dequant(q8, A2)
    return dequant_blocks(packed, ahat, table, dtype).reshape(N, K)


def dequant_blocks(packed, ahat, table=None, dtype="bf16"):
    """w_hat for whole blocks: packed [nb*32] bytes, ahat [nb] float32 -> [nb, 64] 16-bit bits."""
    c = nf4_table() if table is None else np.asarray(table, np.float32)
    codes = unpack_nibbles(packed).reshape(-1, BLOCK)
    ahat = np.asarray(ahat, dtype=np.float32)
    w32 = (ahat[:, None] * c[codes]).astype(np.float32)
    return codec(dtype).from_f32_rne(w32)


def dequant_blocks_f32(packed, ahat, table=None):
    """fl32(a_hat * c_q) for whole blocks as float32 [nb, 64]: the dequantized weight before any rounding to a
    16-bit compute dtype (section 5.2: w_hat = a * c_q, one IEEE float32 product; fp32 is one of the compute
    dtypes of section 8.3)."""
    c = nf4_table() if table is None else np.asarray(table, np.float32)
    codes = unpack_nibbles(packed).reshape(-1, BLOCK)
    ahat = np.asarray(ahat, dtype=np.float32)
    return (ahat[:, None] * c[codes]).astype(np.float32)


def dequantize_f32(packed, q8, A2, N, K, table=None):
    """fp32 w_hat [N, K] = fl32(a_hat * c_q) with the double-quantized scales."""
    return dequant_blocks_f32(packed, scale_dequant(q8, A2), table).reshape(N, K)


def dequantize_nodq_f32(packed, absmax, N, K, table=None):
    """fp32 w_hat [N, K] = fl32(a * c_q) with the stored fp32 block absmax."""
    return dequant_blocks_f32(packed, np.asarray(absmax, np.float32), table).reshape(N, K)


def dequantize_rows(packed, q8, A2, K, rows, table=None, dtype="bf16"):
    """w_hat of the selected rows of an [N, K] weight only (for sampled checks)."""
    rows = np.asarray(rows, dtype=np.int64)
    bpr = K // BLOCK
    bidx = (rows[:, None] * bpr + np.arange(bpr)[None, :]).reshape(-1)
    ahat = _ahat_of_blocks(q8, A2, bidx)
    pk = np.asarray(packed).reshape(-1, BLOCK // 2)[bidx].reshape(-1)
    return dequant_blocks(pk, ahat, table, dtype).reshape(rows.size, K)


def _ahat_of_blocks(q8, A2, bidx):
    """a_hat of an arbitrary set of flat block indices (same two roundings as scale_dequant)."""
    step = np.asarray(A2, dtype=np.float32)[bidx // SUPER] / np.float32(255.0)
    return (step * np.asarray(q8, dtype=np.uint8)[bidx].astype(np.float32)).astype(np.float32)


# ----------------------------------------------------------------------------
# a2..a4 composed: quantize a bf16 weight
# ----------------------------------------------------------------------------
def quantize(W_u16, table=None, dtype="bf16"):
    """Quantize a bf16 (or, with dtype="f16", fp16) weight [N, K] (uint16 bits) -> (packed codes, q8, A2).
    With dtype="f32" the weight is fp32 (uint32 bits); the steps are the same, since every threshold product
    a * m_j (24-bit a, 25-bit m_j) is still exact in float64.

    The codes are taken against the true block absmax a (the page encodes the
    weights first and only then re-quantizes the constants, section 7).
    Returns packed uint8 [N*K/2], q8 uint8 [N*K/64], A2 float32 [ceil(N*K/16384)].
    """
    wb16 = blocks(np.asarray(W_u16, dtype=codec(dtype).BITS))
    nb = wb16.shape[0]
    a = np.empty(nb, dtype=np.float64)
    codes = np.empty((nb, BLOCK), dtype=np.uint8)
    step = 1 << 14                     # blocks per pass: bounds the temporaries only
    for s in range(0, nb, step):
        wb = codec(dtype).to_f64(wb16[s:s + step])
        a[s:s + step] = block_absmax(wb)
        codes[s:s + step] = nf4_codes(wb, a[s:s + step], table)
    A2 = superblock_absmax(a)
    q8 = np.empty(nb, dtype=np.uint8)
    for s in range(0, nb, step):
        e = min(nb, s + step)           # step is a multiple of 256: groups stay whole
        q8[s:e] = scale_codes(a[s:e], A2[s // SUPER: -(-e // SUPER)])
    return pack_nibbles(codes), q8, A2


# ----------------------------------------------------------------------------
# Double quantization off: one fp32 absmax per block
# ----------------------------------------------------------------------------
def quantize_nodq(W_u16, table=None, dtype="bf16"):
    """Quantize a bf16 (or fp16) weight [N, K] without double quantization -> (packed codes, absmax).

    "bitsandbytes deep dive" 7.1 and 9.5: with double quantization off every
    block keeps its absmax as an fp32 constant (32 bits per 64 weights).  The
    codes are the same nearest-level codes as with it on (both are taken
    against the true block absmax).  Returns packed uint8 [N*K/2] and absmax
    float32 [N*K/64] (exact: the absmax of bf16 values is a bf16 value).
    """
    wb16 = blocks(np.asarray(W_u16, dtype=codec(dtype).BITS))
    nb = wb16.shape[0]
    a = np.empty(nb, dtype=np.float32)
    codes = np.empty((nb, BLOCK), dtype=np.uint8)
    step = 1 << 14
    for s in range(0, nb, step):
        wb = codec(dtype).to_f64(wb16[s:s + step])
        ab = block_absmax(wb)
        a[s:s + step] = ab
        codes[s:s + step] = nf4_codes(wb, ab, table)
    return pack_nibbles(codes), a


def dequantize_nodq(packed, absmax, N, K, table=None, dtype="bf16"):
    """w_hat = RNE_bf16( fl32(a_b * c_q) ) with the stored fp32 block absmax, shape [N, K].

    Section 5.2 (w_hat = a * c_q) with a kept exactly (section 7.1: no second
    quantization), rounded once to the bf16 compute dtype (section 8.3).
    """
    return dequant_blocks(packed, np.asarray(absmax, np.float32), table, dtype).reshape(N, K)


def dequantize_rows_nodq(packed, absmax, K, rows, table=None, dtype="bf16"):
    """w_hat of the selected rows of an [N, K] weight quantized without double quantization."""
    rows = np.asarray(rows, dtype=np.int64)
    bpr = K // BLOCK
    bidx = (rows[:, None] * bpr + np.arange(bpr)[None, :]).reshape(-1)
    pk = np.asarray(packed).reshape(-1, BLOCK // 2)[bidx].reshape(-1)
    return dequant_blocks(pk, np.asarray(absmax, np.float32)[bidx], table, dtype).reshape(rows.size, K)


def storage_bytes_nodq(N, K):
    """Bytes of (packed codes, fp32 block absmax) for an [N, K] weight."""
    n = N * K
    return n // 2, 4 * (n // BLOCK)


def bits_per_param_nodq(N, K):
    """Average stored bits per weight without double quantization: 4 + 32/64 = 4.5."""
    cb, ab = storage_bytes_nodq(N, K)
    return 8.0 * (cb + ab) / (N * K)


def storage_bytes(N, K):
    """Bytes of (packed codes, q8, A2) for an [N, K] weight."""
    n = N * K
    return n // 2, n // BLOCK, 4 * (-(-n // SUPER_ELEMS))


def bits_per_param(N, K):
    """Average stored bits per weight, 4 + 8/64 + 32/(64*256) when n divides by 16384."""
    cb, qb, ab = storage_bytes(N, K)
    return 8.0 * (cb + qb + ab) / (N * K)
