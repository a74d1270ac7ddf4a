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
// nf4_merge_kernel: a workgroup of 256 lanes owns a 128 x 128 output tile
// (rows n0 .. n0+127, columns k0 .. k0+127: two NF4 blocks of every row); lane
// (tn, tk) = (tid / 16, tid % 16) accumulates rows n0 + 8 tn .. +7 and columns
// k0 + 8 tk .. +7 in 64 registers.  The rank sum runs over j in chunks of 32:
// A's rows of the tile (transposed, As[j][k]) and B's columns (Bs[j][n]) are
// staged as fp32 in LDS, ranks past r as zeros (a +0 product leaves an fp32
// sum unchanged, so the padded sum equals the sum over j < r); per j a lane
// reads 8 + 8 values with four 16-byte reads (lanes of a row group share the
// B reads, lanes of a column group the A reads) for 64 FMAs.  HBM traffic: the
// codes and scales once, the output once; A and B come from L2.
#include "common.h"

namespace qlora {
namespace {

constexpr int kMT = 128;      // tile rows (n) and columns (k): two NF4 blocks of columns
constexpr int kMJ = 32;       // ranks per LDS chunk
constexpr int kMaxR = 128;

template <bool DQ, int CB, int DT>
__global__ __launch_bounds__(256) void nf4_merge_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ q8, const float* __restrict__ a2,
                                                        const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                        int r, float s, uint16_t* __restrict__ out, int N, int K) {
    __shared__ __attribute__((aligned(16))) float As[kMJ][kMT];  // As[j][kk] = A[k0 + kk, j0 + j]
    __shared__ __attribute__((aligned(16))) float Bs[kMJ][kMT];  // Bs[j][nn] = B[j0 + j, n0 + nn]
    const int tid = threadIdx.x;
    const int n0 = blockIdx.y * kMT, k0 = blockIdx.x * kMT;
    const int tn = tid >> 4, tk = tid & 15;

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;

    const int sc = tid & 127, sj = tid >> 7;  // staging: column (k or n) of the tile, first rank (0 or 1)
    for (int j0 = 0; j0 < r; j0 += kMJ) {
        if (j0 > 0) __syncthreads();          // every lane is done with the previous chunk
#pragma unroll
        for (int q = 0; q < kMJ / 2; ++q) {
            const int jj = sj + 2 * q, j = j0 + jj;
            const int k = k0 + sc, n = n0 + sc;
            As[jj][sc] = (j < r && k < K) ? h16_to_f32<DT>(A[(int64_t)k * r + j]) : 0.0f;
            Bs[jj][sc] = (j < r && n < N) ? h16_to_f32<DT>(B[(int64_t)j * N + n]) : 0.0f;
        }
        __syncthreads();
#pragma unroll 4
        for (int jj = 0; jj < kMJ; ++jj) {
            const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(&As[jj][8 * tk]);
            const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(&As[jj][8 * tk + 4]);
            const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(&Bs[jj][8 * tn]);
            const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(&Bs[jj][8 * tn + 4]);
            const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i][e] = __fmaf_rn(b[i], a[e], acc[i][e]);  // exact product, one rounding
        }
    }

    const int KB = K / kBlock;
    const int k = k0 + 8 * tk;              // this lane's 8 columns, all in block k / 64
    if (k >= K) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int n = n0 + 8 * tn + i;
        if (n >= N) continue;
        const int64_t blk = (int64_t)n * KB + k / kBlock;
        const float ahat = DQ ? __fmul_rn(__fdiv_rn(a2[blk / kSuper], 255.0f), (float)q8[blk]) : a2[blk];
        // 8 codes: elements k .. k+7 of row n, four bytes, element 2i in the high nibble of byte i
        const uint32_t pk = *reinterpret_cast<const uint32_t*>(codes + ((int64_t)n * K + k) / 2);
        uint32_t o[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
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
        *reinterpret_cast<u32x4_t*>(out + (int64_t)n * K + k) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
}

}  // namespace

qlora_status launch_merge(const uint8_t* codes, const uint8_t* q8, const float* a2, int cb, int dt, const uint16_t* A,
                          const uint16_t* B, int r, float s, uint16_t* out, int N, int K, hipStream_t st) {
    if (r < 1 || r > kMaxR) return QLORA_ERR_INVALID_ARG;
    const dim3 grid((unsigned)((K + kMT - 1) / kMT), (unsigned)((N + kMT - 1) / kMT));
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
