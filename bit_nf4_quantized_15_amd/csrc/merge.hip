// LoRA merge for deployment ("LoRA, QLoRA, QA-LoRA explained", section 2:
// W_eff = dequant(W4) + (alpha/r) A B; "bitsandbytes deep dive", section
// 12.10: merged in higher precision, optionally re-quantized afterwards).
//
// In the stored layout [N = Dout, K = Din], with A [K, r] and B [r, N]:
//   out[n, k] = RNE_bf16( fl32( w_hat[n, k] + fl32( s * acc[n, k] ) ) ),
//   acc[n, k] = the fp32 sum over j = 0 .. r-1, in that order, of A[k, j] B[j, n]
// (each product of two bf16 values is exact in fp32, so every step rounds
// once), s = fl32(alpha / r), w_hat = RNE_bf16(fl32(a_hat * c_code)).
//
// nf4_merge_kernel: a workgroup of 256 lanes owns a 64 x 64 output tile (rows
// n0 .. n0+63, one 64-column block k0 .. k0+63); lane (tn, tk) computes rows
// n0 + 4 tn .. +3 and columns k0 + 4 tk .. +3.  A's rows of the tile are staged
// transposed and B's columns as they are, both as fp32 in LDS; per j a lane
// reads 4 values of each with one 16-byte read (the 16 lanes of a row group
// read 256 contiguous bytes, the other operand is a broadcast).  HBM traffic:
// the codes and scales once, A and B once per tile, the bf16 output once.
#include "common.h"

namespace qlora {
namespace {

constexpr int kMT = 64;       // tile rows (n) and columns (k): one NF4 block of columns
constexpr int kMaxR = 128;

template <bool DQ, int CB, int DT>
__global__ __launch_bounds__(256) void nf4_merge_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ q8, const float* __restrict__ a2,
                                                        const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                        int r, float s, uint16_t* __restrict__ out, int N, int K) {
    __shared__ __attribute__((aligned(16))) float As[kMaxR][kMT];  // As[j][kk] = A[k0 + kk, j]
    __shared__ __attribute__((aligned(16))) float Bs[kMaxR][kMT];  // Bs[j][nn] = B[j, n0 + nn]
    const int tid = threadIdx.x;
    const int n0 = blockIdx.y * kMT, kb = blockIdx.x, k0 = kb * kMT;
    for (int i = tid; i < r * kMT; i += 256) {
        const int kk = i / r, j = i - kk * r;  // consecutive lanes read consecutive elements of A's rows
        As[j][kk] = h16_to_f32<DT>(A[(int64_t)(k0 + kk) * r + j]);
    }
    for (int i = tid; i < r * kMT; i += 256) {
        const int j = i / kMT, nn = i - j * kMT;
        Bs[j][nn] = n0 + nn < N ? h16_to_f32<DT>(B[(int64_t)j * N + n0 + nn]) : 0.0f;
    }
    __syncthreads();

    const int tn = tid >> 4, tk = tid & 15;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = 0.0f;
    for (int j = 0; j < r; ++j) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&As[j][4 * tk]);
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&Bs[j][4 * tn]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][e] = __fmaf_rn(b[i], a[e], acc[i][e]);  // exact product, one rounding
    }

    const int KB = K / kBlock;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = n0 + 4 * tn + i;
        if (n >= N) continue;
        const int64_t blk = (int64_t)n * KB + kb;
        const float ahat = DQ ? __fmul_rn(__fdiv_rn(a2[blk / kSuper], 255.0f), (float)q8[blk]) : a2[blk];
        // 4 codes: elements k0 + 4 tk .. +3 of row n, two bytes, element 2i in the high nibble
        const uint32_t pk = *reinterpret_cast<const uint16_t*>(codes + (blk * kBlock + 4 * tk) / 2);
        uint32_t o[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            const uint32_t byte = (pk >> (8 * e2)) & 0xFFu;
            float v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t code = h == 0 ? byte >> 4 : byte & 0xFu;
                const uint32_t wh = pack2<DT>(__fmul_rn(ahat, level<CB>((int)code)), 0.0f) & 0xFFFFu;
                const float corr = __fmul_rn(s, acc[i][2 * e2 + h]);
                v[h] = __fadd_rn(h16_to_f32<DT>(wh), corr);
            }
            o[e2] = pack2<DT>(v[0], v[1]);
        }
        *reinterpret_cast<uint2*>(out + (int64_t)n * K + k0 + 4 * tk) = uint2{o[0], o[1]};
    }
}

}  // namespace

qlora_status launch_merge(const uint8_t* codes, const uint8_t* q8, const float* a2, int cb, int dt, const uint16_t* A,
                          const uint16_t* B, int r, float s, uint16_t* out, int N, int K, hipStream_t st) {
    if (r < 1 || r > kMaxR) return QLORA_ERR_INVALID_ARG;
    const dim3 grid((unsigned)(K / kMT), (unsigned)((N + kMT - 1) / kMT));
    with_cb_dt(cb, dt, [&](auto cbc, auto dtc) {
        constexpr int CB = decltype(cbc)::value, DT = decltype(dtc)::value;
        if (q8)
            hipLaunchKernelGGL((nf4_merge_kernel<true, CB, DT>), grid, dim3(256), 0, st, codes, q8, a2, A, B, r, s, out,
                               N, K);
        else
            hipLaunchKernelGGL((nf4_merge_kernel<false, CB, DT>), grid, dim3(256), 0, st, codes, q8, a2, A, B, r, s,
                               out, N, K);
    });
    return launch_status();
}

}  // namespace qlora
