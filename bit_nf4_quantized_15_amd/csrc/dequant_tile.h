// In-register 4-bit dequantization for the fused GEMM kernels.
//
// A weight block (64 codes of one row) has one reconstructed scale
// a_hat = fl32(fl32(a2/255) * q8), so its 16 possible 16-bit values
// RNE_16(fl32(a_hat * c_j)) form a per-block table (c: the NF4 or the FP4
// codebook; 16-bit: the bf16 or fp16 compute dtype).  The table is kept as
// two 16-byte byte tables (low bytes, high bytes of the 16 entries) in 8
// VGPRs; v_perm_b32 looks up 4 codes at once in each 8-entry half, and an AND
// keeps the half that holds the code.  Every dequantized value is exactly the
// value that qlora_dequantize produces ("bitsandbytes deep dive" 5.2:
// w_hat = a * c_q).
#pragma once

#include "common.h"

namespace qlora {

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
    return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// fl32(a2 / 255): for every bf16-valued a2 (which every stored second-level
// scale is) the fp64 product with the double nearest 1/255 rounds to the same
// float as the correctly rounded quotient (the binary expansion of m/255 is
// periodic with period 8, so it never lies near a float rounding boundary).
__device__ __forceinline__ float scale_step(float a2) {
    return (float)((double)a2 * (1.0 / 255.0));
}

__device__ __forceinline__ float block_ahat(const uint8_t* __restrict__ q8, const float* __restrict__ a2,
                                            int64_t blk) {
    return scale_step(a2[blk >> 8]) * (float)q8[blk];
}

struct Nf4Tab {
    uint32_t lo[4];  // byte i of lo[q] = low byte of entry 4q + i
    uint32_t hi[4];  // byte i of hi[q] = high byte of entry 4q + i
};

template <int CB, int DT>
__device__ __forceinline__ Nf4Tab make_tab(float ahat) {
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = pack2<DT>(ahat * level<CB>(2 * j), ahat * level<CB>(2 * j + 1));
    Nf4Tab T;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        T.lo[q] = perm_b32(e[2 * q + 1], e[2 * q], 0x06040200u);
        T.hi[q] = perm_b32(e[2 * q + 1], e[2 * q], 0x07050301u);
    }
    return T;
}

// s1 holds 4 codes, one per byte, as lookup selectors: code c < 8 as c and
// code c >= 8 as 16 + (c - 8).  Returns the low and high bytes of their table
// entries, byte i for code i.  v_perm_b32 yields 0xFF for a selector byte >= 13,
// so looking up s1 in entries 0..7 and s1 ^ 0x10 in entries 8..15 leaves the hit
// in one half and 0xFF in the other, and AND merges them.
__device__ __forceinline__ void lut4(const Nf4Tab& T, uint32_t s1, uint32_t& lo, uint32_t& hi) {
    const uint32_t s2 = s1 ^ 0x10101010u;
    lo = perm_b32(T.lo[1], T.lo[0], s1) & perm_b32(T.lo[3], T.lo[2], s2);
    hi = perm_b32(T.hi[1], T.hi[0], s1) & perm_b32(T.hi[3], T.hi[2], s2);
}

// One dword of packed codes (8 consecutive weights, weight 2i in the high
// nibble of byte i) -> the 8 bf16 weights as 4 dwords (weight 2j in the low
// half of dword j), i.e. an MFMA bf16x8 operand in k order.
__device__ __forceinline__ u32x4_t deq8(const Nf4Tab& T, uint32_t d) {
    // selectors of the odd (low nibble) and even (high nibble) weights
    const uint32_t so = (d & 0x07070707u) | ((d << 1) & 0x10101010u);
    const uint32_t se = ((d >> 4) & 0x07070707u) | ((d >> 3) & 0x10101010u);
    uint32_t la, ha, lb, hb;
    lut4(T, perm_b32(so, se, 0x05010400u), la, ha);  // weights 0..3
    lut4(T, perm_b32(so, se, 0x07030602u), lb, hb);  // weights 4..7
    return u32x4_t{perm_b32(ha, la, 0x05010400u), perm_b32(ha, la, 0x07030602u),
                   perm_b32(hb, lb, 0x05010400u), perm_b32(hb, lb, 0x07030602u)};
}

// deq8 without the two selector interleaves: the 8 weights come out in the
// order 1, 3, 5, 7, 0, 2, 4, 6 (odd weights from the low nibbles, then even
// ones from the high nibbles).  A product that stages its other operand in the
// same order within every 8 consecutive k (x_order8) saves 2 of the 27 VALU.
// Its selectors mark the other half with bit 7 instead of bit 4 (any selector byte
// >= 13 yields 0xFF): a high nibble's top bit is bit 7 already, which saves one
// operation per 8 codes.
__device__ __forceinline__ void lut4_b7(const Nf4Tab& T, uint32_t s1, uint32_t& lo, uint32_t& hi) {
    const uint32_t s2 = s1 ^ 0x80808080u;
    lo = perm_b32(T.lo[1], T.lo[0], s1) & perm_b32(T.lo[3], T.lo[2], s2);
    hi = perm_b32(T.hi[1], T.hi[0], s1) & perm_b32(T.hi[3], T.hi[2], s2);
}

__device__ __forceinline__ u32x4_t deq8_oddeven(const Nf4Tab& T, uint32_t d) {
    const uint32_t so = (d & 0x07070707u) | ((d << 4) & 0x80808080u);
    const uint32_t se = ((d >> 4) & 0x07070707u) | (d & 0x80808080u);
    uint32_t lo, ho, le, he;
    lut4_b7(T, so, lo, ho);
    lut4_b7(T, se, le, he);
    return u32x4_t{perm_b32(ho, lo, 0x05010400u), perm_b32(ho, lo, 0x07030602u), perm_b32(he, le, 0x05010400u),
                   perm_b32(he, le, 0x07030602u)};
}

// 8 consecutive 16-bit elements (4 dwords, element 2j in the low half of dword
// j) reordered as 1, 3, 5, 7, 0, 2, 4, 6: the order of deq8_oddeven.
__device__ __forceinline__ u32x4_t x_order8(u32x4_t v) {
    return u32x4_t{perm_b32(v[1], v[0], 0x07060302u), perm_b32(v[3], v[2], 0x07060302u),
                   perm_b32(v[1], v[0], 0x05040100u), perm_b32(v[3], v[2], 0x05040100u)};
}

// The fused forward's lane halves dequantize the same two columns: lanes 0-31
// build the table of the first and lanes 32-63 that of the second, and
// v_permlane32_swap hands each half the other's, so every lane ends with both.
__device__ __forceinline__ void share_tabs(const Nf4Tab& mine, Nf4Tab& t0, Nf4Tab& t1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const auto l = __builtin_amdgcn_permlane32_swap(mine.lo[q], mine.lo[q], false, false);
        const auto h = __builtin_amdgcn_permlane32_swap(mine.hi[q], mine.hi[q], false, false);
        t0.lo[q] = l[0];
        t1.lo[q] = l[1];
        t0.hi[q] = h[0];
        t1.hi[q] = h[1];
    }
}

// Byte offset of 16-byte chunk `chunk` (0..7) of row `row` in an LDS tile of
// 64 bf16 per row.  The XOR swizzle spreads both the row-wise MFMA operand
// reads (16 consecutive rows, same chunk) and the column scatter of the
// transposed weight tile (rows 64 apart) over distinct banks.
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
    return (uint32_t)row * 128u + ((uint32_t)(chunk ^ ((row ^ (row >> 3) ^ (row >> 5)) & 7)) << 4);
}

}  // namespace qlora
