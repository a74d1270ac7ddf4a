// LoRA side-path kernels (MFMA v_mfma_f32_32x32x16_bf16, gfx950).
//
// The rank-r products of the layer ("bitsandbytes deep dive" 12.2:
// Y = XW + s X A B, A [Din, r], B [r, Dout], s = lora_alpha / r; the chain
// rule through the same graph for the backward, base frozen):
//   t  = s x A        [M, r]   (forward, kept for the backward)
//   u  = s dy B^T     [M, r]
//   dA = x^T u        [K, r]
//   dB = t^T dy       [r, N]
// All four stream one large operand (x or dy) once and are HBM bound.  The
// reductions are split over the long dimension for parallelism; partial sums
// go to a workspace and are added in a fixed order (deterministic results).
#include "common.h"
#include "lora_plan.h"

namespace qlora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16_t mfma32(bf16x8 a, bf16x8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive bf16 src[row*ld + c0 .. +7] (zero outside [0,nrows) x [0,ncols)).
template <bool VEC>
__device__ __forceinline__ bf16x8 load8_row(const uint16_t* __restrict__ src, int64_t ld, int row, int nrows, int c0,
                                           int ncols) {
    if (VEC) {
        if (row < nrows && c0 < ncols)
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4_t*>(src + (int64_t)row * ld + c0));
        return __builtin_bit_cast(bf16x8, u32x4_t{0u, 0u, 0u, 0u});
    }
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int a = c0 + 2 * i, b = a + 1;
        const uint32_t lo = (row < nrows && a < ncols) ? src[(int64_t)row * ld + a] : 0u;
        const uint32_t hi = (row < nrows && b < ncols) ? src[(int64_t)row * ld + b] : 0u;
        w[i] = lo | (hi << 16);
    }
    return __builtin_bit_cast(bf16x8, u32x4_t{w[0], w[1], w[2], w[3]});
}

// 8 bf16 down a column: src[(r0 + i)*ld + col], i = 0..7.
__device__ __forceinline__ bf16x8 load8_col(const uint16_t* __restrict__ src, int64_t ld, int r0, int nrows, int col,
                                           int ncols) {
    uint32_t w[4];
    const bool cok = col < ncols;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int a = r0 + 2 * i, b = a + 1;
        const uint32_t lo = (cok && a < nrows) ? src[(int64_t)a * ld + col] : 0u;
        const uint32_t hi = (cok && b < nrows) ? src[(int64_t)b * ld + col] : 0u;
        w[i] = lo | (hi << 16);
    }
    return __builtin_bit_cast(bf16x8, u32x4_t{w[0], w[1], w[2], w[3]});
}

// At[j, k] = A[k, j]
__global__ void transpose_kernel(const uint16_t* __restrict__ A, uint16_t* __restrict__ At, int K, int r) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)K * r) return;
    const int j = (int)(i / K), k = (int)(i - (int64_t)j * K);
    At[i] = A[(int64_t)k * r + j];
}

// part[split, m, j] = sum over c in the split's range of X[m, c] * Yt[j, c]
// One wave per (32-row tile, split); TQ 32-column tiles of j.
template <int TQ, bool VEC>
__global__ __launch_bounds__(64) void nt_partial_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Yt,
                                                        float* __restrict__ part, int M, int C, int r, int chunk) {
    const int lane = threadIdx.x, h = lane >> 5, l32 = lane & 31;
    const int m0 = blockIdx.x * 32;
    const int split = blockIdx.y;
    const int c_begin = split * chunk;
    const int c_end = min(C, c_begin + chunk);
    f32x16_t acc[TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][v] = 0.0f;
    for (int c = c_begin; c < c_end; c += 16) {
        const int cc = c + 8 * h;
        const bf16x8 a = load8_row<VEC>(X, C, m0 + l32, M, cc, c_end);
#pragma unroll
        for (int q = 0; q < TQ; ++q) {
            const bf16x8 b = load8_row<VEC>(Yt, C, 32 * q + l32, r, cc, c_end);
            acc[q] = mfma32(a, b, acc[q]);
        }
    }
    float* out = part + (int64_t)split * M * r;
#pragma unroll
    for (int q = 0; q < TQ; ++q) {
        const int j = 32 * q + l32;
        if (j >= r) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = m0 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (m < M) out[(int64_t)m * r + j] = acc[q][v];
        }
    }
}

// out[m, j] = bf16( s * sum_split part[split, m, j] )
__global__ void finalize_bf16_kernel(const float* __restrict__ part, int splits, int64_t count, float s,
                                     uint16_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    float acc = 0.0f;
    for (int p = 0; p < splits; ++p) acc += part[(int64_t)p * count + i];
    out[i] = (uint16_t)(pack_bf16x2(s * acc, 0.0f) & 0xFFFFu);
}

// part[split, p, q] = sum over m in the split's range of P[m, p] * Q[m, q]
// One wave per (32*TP x 32*TQ output tile, split).
template <int TP, int TQ>
__global__ __launch_bounds__(64) void tn_partial_kernel(const uint16_t* __restrict__ P, const uint16_t* __restrict__ Q,
                                                        float* __restrict__ part, int M, int Pd, int Qd, int chunk) {
    const int lane = threadIdx.x, h = lane >> 5, l32 = lane & 31;
    const int p0 = blockIdx.x * 32 * TP, q0 = blockIdx.y * 32 * TQ;
    const int split = blockIdx.z;
    const int m_begin = split * chunk;
    const int m_end = min(M, m_begin + chunk);
    f32x16_t acc[TP][TQ];
#pragma unroll
    for (int a = 0; a < TP; ++a)
#pragma unroll
        for (int b = 0; b < TQ; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
    for (int m = m_begin; m < m_end; m += 16) {
        const int mm = m + 8 * h;
        bf16x8 pa[TP], qb[TQ];
#pragma unroll
        for (int a = 0; a < TP; ++a) pa[a] = load8_col(P, Pd, mm, m_end, p0 + 32 * a + l32, Pd);
#pragma unroll
        for (int b = 0; b < TQ; ++b) qb[b] = load8_col(Q, Qd, mm, m_end, q0 + 32 * b + l32, Qd);
#pragma unroll
        for (int a = 0; a < TP; ++a)
#pragma unroll
            for (int b = 0; b < TQ; ++b) acc[a][b] = mfma32(pa[a], qb[b], acc[a][b]);
    }
    float* out = part + (int64_t)split * Pd * Qd;
#pragma unroll
    for (int a = 0; a < TP; ++a)
#pragma unroll
        for (int b = 0; b < TQ; ++b) {
            const int q = q0 + 32 * b + l32;
            if (q >= Qd) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int p = p0 + 32 * a + 8 * (v >> 2) + 4 * h + (v & 3);
                if (p < Pd) out[(int64_t)p * Qd + q] = acc[a][b][v];
            }
        }
}

// out[i] = sum_split part[split, i]   (fp32)
__global__ void reduce_f32_kernel(const float* __restrict__ part, int splits, int64_t count, float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    float acc = 0.0f;
    for (int p = 0; p < splits; ++p) acc += part[(int64_t)p * count + i];
    out[i] = acc;
}

__global__ void fill_f32_kernel(float* __restrict__ out, int64_t count, float v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) out[i] = v;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

qlora_status launch_transpose(const uint16_t* A, uint16_t* At, int K, int r, hipStream_t s) {
    hipLaunchKernelGGL(transpose_kernel, dim3(blocks_for((int64_t)K * r, 256)), dim3(256), 0, s, A, At, K, r);
    return launch_status();
}

qlora_status launch_nt(const uint16_t* X, const uint16_t* Yt, float* part, uint16_t* out, float scale, int M, int C,
                       int r, hipStream_t s) {
    const SplitPlan sp = plan_nt(M, C);
    const dim3 grid((unsigned)((M + 31) / 32), (unsigned)sp.splits);
    const bool vec = (C % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15u) == 0) &&
                     ((reinterpret_cast<uintptr_t>(Yt) & 15u) == 0);
    const int tq = (r + 31) / 32;
#define QL_NT(TQ)                                                                                              \
    if (vec) hipLaunchKernelGGL((nt_partial_kernel<TQ, true>), grid, dim3(64), 0, s, X, Yt, part, M, C, r, sp.chunk); \
    else hipLaunchKernelGGL((nt_partial_kernel<TQ, false>), grid, dim3(64), 0, s, X, Yt, part, M, C, r, sp.chunk);
    switch (tq) {
        case 1: QL_NT(1) break;
        case 2: QL_NT(2) break;
        case 3: QL_NT(3) break;
        default: QL_NT(4) break;
    }
#undef QL_NT
    const int64_t count = (int64_t)M * r;
    hipLaunchKernelGGL(finalize_bf16_kernel, dim3(blocks_for(count, 256)), dim3(256), 0, s, part, sp.splits, count,
                       scale, out);
    return launch_status();
}

qlora_status launch_tn(const uint16_t* P, const uint16_t* Q, float* part, float* out, int M, int Pd, int Qd,
                       hipStream_t s) {
    // the small dimension (r <= 128) is covered whole by one wave
    const SplitPlan sp = plan_tn(M, Pd, Qd);
    const int64_t count = (int64_t)Pd * Qd;
    if (Qd <= 128 && Qd <= Pd) {
        const int tq = (Qd + 31) / 32;
        const dim3 grid((unsigned)((Pd + 31) / 32), 1u, (unsigned)sp.splits);
#define QL_TN(TQ) hipLaunchKernelGGL((tn_partial_kernel<1, TQ>), grid, dim3(64), 0, s, P, Q, part, M, Pd, Qd, sp.chunk);
        switch (tq) {
            case 1: QL_TN(1) break;
            case 2: QL_TN(2) break;
            case 3: QL_TN(3) break;
            default: QL_TN(4) break;
        }
#undef QL_TN
    } else {
        const int tp = (Pd + 31) / 32;
        const dim3 grid(1u, (unsigned)((Qd + 31) / 32), (unsigned)sp.splits);
#define QL_TN(TP) hipLaunchKernelGGL((tn_partial_kernel<TP, 1>), grid, dim3(64), 0, s, P, Q, part, M, Pd, Qd, sp.chunk);
        switch (tp) {
            case 1: QL_TN(1) break;
            case 2: QL_TN(2) break;
            case 3: QL_TN(3) break;
            default: QL_TN(4) break;
        }
#undef QL_TN
    }
    hipLaunchKernelGGL(reduce_f32_kernel, dim3(blocks_for(count, 256)), dim3(256), 0, s, part, sp.splits, count, out);
    return launch_status();
}

qlora_status launch_fill(float* out, int64_t count, float v, hipStream_t s) {
    if (count > 0) hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(count, 256)), dim3(256), 0, s, out, count, v);
    return launch_status();
}

}  // namespace qlora
