// In-register NF4 dequantization for the fused GEMM kernels.
//
// A weight block (64 codes of one row) has one reconstructed scale
// a_hat = fl32(fl32(a2/255) * q8), so its 16 possible bf16 values
// RNE_bf16(fl32(a_hat * c_j)) form a per-block table.  The table is kept as
// two 16-byte byte tables (low bytes, high bytes of the 16 bf16 entries) in 8
// VGPRs; v_perm_b32 looks up 4 codes at once in an 8-entry half, and a bitfield
// select picks the half.  Every dequantized value is exactly the bf16 that
// qlora_dequantize produces ("bitsandbytes deep dive" 5.2: w_hat = a * c_q).
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

__device__ __forceinline__ Nf4Tab make_tab(float ahat) {
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = pack_bf16x2(ahat * nf4_level(2 * j), ahat * nf4_level(2 * j + 1));
    Nf4Tab T;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        T.lo[q] = perm_b32(e[2 * q + 1], e[2 * q], 0x06040200u);
        T.hi[q] = perm_b32(e[2 * q + 1], e[2 * q], 0x07050301u);
    }
    return T;
}

// s holds 4 codes (0..15), one per byte; returns the low and high bytes of
// their table entries, byte i for code i.
__device__ __forceinline__ void lut4(const Nf4Tab& T, uint32_t s, uint32_t& lo, uint32_t& hi) {
    const uint32_t sel = s & 0x07070707u;
    // 0xFF in the bytes whose code is >= 8 (v_perm selector 12 -> 0x00, 13 -> 0xFF)
    const uint32_t m = perm_b32(0u, 0u, ((s >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
    const uint32_t l0 = perm_b32(T.lo[1], T.lo[0], sel);
    const uint32_t l1 = perm_b32(T.lo[3], T.lo[2], sel);
    const uint32_t h0 = perm_b32(T.hi[1], T.hi[0], sel);
    const uint32_t h1 = perm_b32(T.hi[3], T.hi[2], sel);
    lo = (m & l1) | (~m & l0);
    hi = (m & h1) | (~m & h0);
}

// One dword of packed codes (8 consecutive weights, weight 2i in the high
// nibble of byte i) -> the 8 bf16 weights as 4 dwords (weight 2j in the low
// half of dword j), i.e. an MFMA bf16x8 operand in k order.
__device__ __forceinline__ u32x4_t deq8(const Nf4Tab& T, uint32_t d) {
    uint32_t le, he, lo, ho;
    lut4(T, (d >> 4) & 0x0F0F0F0Fu, le, he);  // weights 0, 2, 4, 6
    lut4(T, d & 0x0F0F0F0Fu, lo, ho);         // weights 1, 3, 5, 7
    const uint32_t p0 = perm_b32(he, le, 0x05010400u);  // [w0 | w2]
    const uint32_t p1 = perm_b32(he, le, 0x07030602u);  // [w4 | w6]
    const uint32_t q0 = perm_b32(ho, lo, 0x05010400u);  // [w1 | w3]
    const uint32_t q1 = perm_b32(ho, lo, 0x07030602u);  // [w5 | w7]
    return u32x4_t{perm_b32(q0, p0, 0x05040100u), perm_b32(q0, p0, 0x07060302u),
                   perm_b32(q1, p1, 0x05040100u), perm_b32(q1, p1, 0x07060302u)};
}

// Same lookup, but returns the weights as [w0|w2], [w4|w6], [w1|w3], [w5|w7]
// (for kernels that scatter single bf16 values).
__device__ __forceinline__ u32x4_t deq8_evens_odds(const Nf4Tab& T, uint32_t d) {
    uint32_t le, he, lo, ho;
    lut4(T, (d >> 4) & 0x0F0F0F0Fu, le, he);
    lut4(T, d & 0x0F0F0F0Fu, lo, ho);
    return u32x4_t{perm_b32(he, le, 0x05010400u), perm_b32(he, le, 0x07030602u),
                   perm_b32(ho, lo, 0x05010400u), perm_b32(ho, lo, 0x07030602u)};
}

// Byte offset of 16-byte chunk `chunk` (0..7) of row `row` in an LDS tile of
// 64 bf16 per row.  The XOR swizzle spreads both the row-wise MFMA operand
// reads (16 consecutive rows, same chunk) and the column scatter of the
// transposed weight tile (rows 64 apart) over distinct banks.
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
    return (uint32_t)row * 128u + ((uint32_t)(chunk ^ ((row ^ (row >> 3) ^ (row >> 5)) & 7)) << 4);
}

}  // namespace qlora
