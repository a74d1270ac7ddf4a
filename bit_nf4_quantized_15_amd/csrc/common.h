// Internal helpers shared by the HIP kernels of libqlora (gfx950 only).
#pragma once

#include <algorithm>
#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora.h"

namespace qlora {

constexpr int kBlock = 64;                 // weights per first-level block
constexpr int kSuper = 256;                // blocks per second-level (fp32) scale
constexpr int kSuperElems = kBlock * kSuper;
constexpr int kZeroCode = 7;

// The 16 NF4 levels as IEEE binary32 bit patterns, ascending: Phi^-1 of
// 8 (positive half) and 7 (negative half) equal-probability points between
// 1/2 and delta = 1 - (1/32 + 1/30)/2, plus an exact 0, divided by
// Phi^-1(delta) and rounded to nearest float ("bitsandbytes deep dive",
// section 6.2: quantiles of N(0,1), normalised to [-1,1], asymmetric, exact 0).
constexpr uint32_t kNf4Bits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The 16 FP4 levels in code order: the 4-bit float E2M1 (bit 3 sign, bits
// 2..1 exponent with bias 1, bit 0 mantissa; magnitudes 0, 0.5, 1, 1.5, 2, 3,
// 4, 6) divided by 6 and rounded to nearest float; code 8 is -0 ("bitsandbytes
// deep dive", sections 6.5 and 8.1: fp4 is a floating-point-style codebook).
constexpr uint32_t kFp4Bits[16] = {
    0x00000000u, 0x3daaaaabu, 0x3e2aaaabu, 0x3e800000u, 0x3eaaaaabu, 0x3f000000u,
    0x3f2aaaabu, 0x3f800000u, 0x80000000u, 0xbdaaaaabu, 0xbe2aaaabu, 0xbe800000u,
    0xbeaaaaabu, 0xbf000000u, 0xbf2aaaabu, 0xbf800000u};

// Codebook selector of the kernels (the quant_type of qlora_nf4).
constexpr int kCbNf4 = 0;
constexpr int kCbFp4 = 1;

// Level of code j in codebook CB.
template <int CB>
__device__ __forceinline__ float level(int j) {
    return __uint_as_float(CB == kCbFp4 ? kFp4Bits[j] : kNf4Bits[j]);
}

// The distinct levels in ascending order, as codes: index i -> code.  NF4 is
// ascending already (16 levels); FP4 has 15 distinct levels (one zero, +0):
// codes 15, 14, .., 9 (negative, magnitude descending), then 0, 1, .., 7.
template <int CB>
__device__ __forceinline__ uint32_t code_of_sorted(uint32_t i) {
    if (CB == kCbFp4) return i >= 7u ? i - 7u : 15u - i;
    return i;
}
template <int CB>
constexpr int kDistinctLevels = CB == kCbFp4 ? 15 : 16;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two floats -> packed bf16x2 (lo in bits 15..0), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f = {lo, hi};
    bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

// The 16-bit compute dtype of a layer's tensors (the dtype field of qlora_nf4;
// "bitsandbytes deep dive" 8.3): bf16 (default) or IEEE fp16.
constexpr int kDtBf16 = 0;
constexpr int kDtF16 = 1;
// IEEE fp32 (deep dive 8.3's third compute dtype): the fp32 kernel family
// (gemm_f32.hip) and the quantizer only; with_cb_dt covers the 16-bit dtypes.
constexpr int kDtF32 = 2;

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Exact value of a 16-bit pattern of dtype DT.
template <int DT>
__device__ __forceinline__ float h16_to_f32(uint32_t b16) {
    if (DT == kDtF16) return (float)__builtin_bit_cast(_Float16, (uint16_t)b16);
    return bf16_bits_to_f32(b16);
}

// Two floats -> packed pair of dtype DT (lo in bits 15..0), round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if (DT == kDtF16) {
        f32x2_t f = {lo, hi};
        f16x2_t h = __builtin_convertvector(f, f16x2_t);
        return __builtin_bit_cast(uint32_t, h);
    }
    return pack_bf16x2(lo, hi);
}

// Host-side dispatch from the runtime codebook and dtype to template
// arguments: calls f(IntC<CB>{}, IntC<DT>{}).
template <int V>
using IntC = std::integral_constant<int, V>;
template <typename F>
inline void with_cb_dt(int cb, int dt, F&& f) {
    if (cb == kCbFp4) {
        if (dt == kDtF16) f(IntC<kCbFp4>{}, IntC<kDtF16>{});
        else f(IntC<kCbFp4>{}, IntC<kDtBf16>{});
    } else {
        if (dt == kDtF16) f(IntC<kCbNf4>{}, IntC<kDtF16>{});
        else f(IntC<kCbNf4>{}, IntC<kDtBf16>{});
    }
}
template <typename F>
inline void with_dt(int dt, F&& f) {
    if (dt == kDtF16) f(IntC<kDtF16>{});
    else f(IntC<kDtBf16>{});
}

// Round a float down (toward -inf) onto the bf16 grid; returned as a float.
__device__ __forceinline__ float f32_rd_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t t = u & 0xFFFF0000u;                       // truncation toward zero
    if ((u & 0x80000000u) && (u & 0x0000FFFFu)) t += 0x00010000u;  // negative: one step down
    return __uint_as_float(t);
}

// Report a launch error as a status.
inline qlora_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

// Launchers (one per translation unit).
// `cb` selects the codebook (kCbNf4, kCbFp4) of the codes the kernels read or
// write, `dt` the compute dtype (kDtBf16, kDtF16) of every 16-bit tensor
// (launch_quantize also takes kDtF32: an fp32 source weight).
qlora_status launch_quantize(const void* W, int64_t nblocks, uint8_t* codes, uint8_t* q8, float* a2, int cb,
                             int dt, hipStream_t s);
// up to kQuantBatchMax weights of one configuration (codebook, 16-bit dtype, with or
// without double quantization: all q8 null or none) in one launch
constexpr int kQuantBatchMax = 16;
qlora_status launch_quantize_batch(const void* const* W, const int64_t* nblocks, uint8_t* const* codes,
                                   uint8_t* const* q8, float* const* a2, int count, int cb, int dt, hipStream_t s);
qlora_status launch_dequantize(const uint8_t* codes, const uint8_t* q8, const float* a2, int cb, int dt,
                               int64_t nblocks, uint16_t* out, hipStream_t s);
qlora_status launch_dequantize_f32(const uint8_t* codes, const uint8_t* q8, const float* a2, int cb, int64_t nblocks,
                                   float* out, hipStream_t s);
qlora_status launch_merge(const uint8_t* codes, const uint8_t* q8, const float* a2, int cb, int dt, const uint16_t* A,
                          const uint16_t* B, int r, float s, uint16_t* out, int N, int K, hipStream_t st);
qlora_status launch_gemm_fwd(const uint16_t* x, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                             int dt, const uint16_t* t, const uint16_t* B, uint16_t* y, int M, int N, int K, int r,
                             hipStream_t s);
// Decode-size forward (1 <= M <= kGemvMaxM): the same dequantized weights as
// launch_gemm_fwd (results differ only in the order of the fp32 sums).
constexpr int kGemvMaxM = 16;
bool gemv_supported(int M, int N, int K, int r);
qlora_status launch_gemv_fwd(const uint16_t* x, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                             int dt, const uint16_t* t, const uint16_t* B, uint16_t* y, int M, int N, int K, int r,
                             hipStream_t s);
// The whole decode-size layer call in one launch: t = bf16(scale x A) (also
// stored to t_out when given) and y = x W_hat^T + t B.  ws holds the partial
// products of x A and their publication tags (gemv_linear_workspace bytes,
// 16-byte aligned; any initial contents).
size_t gemv_linear_workspace(int M, int N, int K, int r);
qlora_status launch_gemv_linear(const uint16_t* x, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                                int dt, const uint16_t* A, const uint16_t* B, float scale, uint16_t* y,
                                uint16_t* t_out, void* ws, int M, int N, int K, int r, hipStream_t s);
qlora_status launch_gemm_bwd_dx(const uint16_t* dy, const uint8_t* codes, const uint8_t* q8, const float* a2,
                                int cb, int dt, const uint16_t* u, const uint16_t* A, uint16_t* dx, int M, int N, int K, int r,
                                hipStream_t s);
// out [M, r] = bf16(scale * X [M, C] Y), Y given as Yt [r, C] or, with y_natural, as [C, r];
// ws: nt_ws_bytes(M, C, r) bytes
qlora_status launch_nt(const uint16_t* X, const uint16_t* Y, bool y_natural, void* ws, uint16_t* out, float scale,
                       int M, int C, int r, int dt, hipStream_t s);
// Any number of such products of one rank r and one layout of Y, up to 8 per launch (each
// with its own M, C, X, Y, out, scale and nt_ws_bytes(M, C, r) bytes of workspace)
struct NtDesc {
    const uint16_t* X;
    const uint16_t* Y;
    void* ws;
    uint16_t* out;
    float scale;
    int M, C;
};
qlora_status launch_nt_batch(const NtDesc* d, int count, bool y_natural, int r, int dt, hipStream_t s);
// out[d * ld_d + j * ld_j] = sum_m X [M, D][m, d] * S [M, r][m, j]; ws: tn_ws_bytes(M, D, r) bytes
qlora_status launch_tn(const uint16_t* X, const uint16_t* S, void* ws, float* out, int M, int D, int r,
                       int64_t ld_d, int64_t ld_j, int dt, hipStream_t s);
// two such contractions over the same M and r (dA and dB of a layer) in one launch;
// ws0 and ws1: tn_ws_bytes(M, D0, r) and tn_ws_bytes(M, D1, r) bytes
qlora_status launch_tn2(const uint16_t* X0, const uint16_t* S0, void* ws0, float* out0, int D0, int64_t ld_d0,
                        int64_t ld_j0, const uint16_t* X1, const uint16_t* S1, void* ws1, float* out1, int D1,
                        int64_t ld_d1, int64_t ld_j1, int M, int r, int dt, hipStream_t s);
// Any number of such contractions of one rank r, up to 16 per launch (each with its
// own M, D, operands, output and tn_ws_bytes(M, D, r) bytes of workspace)
struct TnDesc {
    const uint16_t* X;
    const uint16_t* S;
    void* ws;
    float* out;
    int M, D;
    int64_t ld_d, ld_j;
};
qlora_status launch_tn_batch(const TnDesc* d, int count, int r, int dt, hipStream_t s);
qlora_status launch_fill(float* out, int64_t count, float v, hipStream_t s);
qlora_status launch_expand_pooled(const uint16_t* A, int K, int r, int g, int dt, uint16_t* out, hipStream_t s);
qlora_status launch_pool_rows(const float* in, int K, int r, int g, float* out, hipStream_t s);

// fp32 compute dtype (gemm_f32.hip).  A contraction whose tile grid is small
// splits its reduction: `splits` partial sums of rows * cols fp32 each go to
// the caller's `part` buffer (plan_f32 gives the count the launch will use).
struct F32Plan {
    int splits, kchunk;
};
F32Plan plan_f32(int rows, int cols, int red);
constexpr int kF32LoraDown = 0;   // out [M, r] = scale * X [M, C] Y [C, r]
constexpr int kF32LoraDownT = 1;  // out [M, r] = scale * X [M, C] Y^T, Y [r, C]
constexpr int kF32Grad = 2;       // out [C, r] = scale * X^T Y, X [M, C], Y [M, r]
constexpr int kF32GradT = 3;      // out [r, C] = scale * X^T Y, X [M, r], Y [M, C]
qlora_status launch_f32_lora(int which, const float* X, const float* Y, int M, int C, int r, float scale, float* out,
                             float* part, hipStream_t s);
qlora_status launch_f32_fwd(const float* x, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                            const float* t, const float* B, float* y, int M, int N, int K, int r, float* part,
                            hipStream_t s);
qlora_status launch_f32_bwd_dx(const float* dy, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                               const float* u, const float* A, float* dx, int M, int N, int K, int r, float* part,
                               hipStream_t s);

}  // namespace qlora
