// The fp32 compute dtype ("bitsandbytes deep dive", section 8.3: a 4-bit
// layer computes in fp32, bf16 or fp16).  Every floating-point tensor of the
// layer is binary32 and the dequantized weight is the fp32 product
// w_hat = fl32(a_hat * c_q) itself (section 5.2), with no 16-bit rounding.
//
// All six contractions of the layer run on one tiled kernel,
//   C[i, j] = sum_k A[i, k] B[k, j]  (+ a second reduction for the LoRA term),
// whose operands come in four layouts, each staged as a [16][128] fp32 tile
// of LDS, reduction index first:
//   kIMaj   plain, element (i, k) at p[i * ld + k]   (contiguous along k)
//   kKMaj   plain, element (i, k) at p[k * ld + i]   (contiguous along i)
//   kQIMaj  NF4/FP4 codes, code row i, column k: the forward's w_hat [N, K]
//           read as B[k][n] (reduction along a code row)
//   kQKMaj  codes, code row k, column i: dx's w_hat read as B[n][k]
//           (reduction across code rows)
// and the matrix cores take them as v_mfma_f32_32x32x2_f32 (a 256-lane
// workgroup owns a 128 x 128 tile, 2 x 2 waves of 64 x 64, four 32 x 32
// accumulators per wave; each 16-deep step is 8 MFMA k-pairs).  The tiles are
// double-buffered: the next step's global loads are issued before this
// step's MFMAs and stored after them, one barrier per step.
//
// Uses in the layer (s = alpha / r):
//   t  = s x A          A: x  kIMaj [M, K],  B: A  kKMaj [K, r]
//   y  = x w_hat^T + t B   A: x kIMaj, B: codes kQIMaj; then t kIMaj, B kKMaj
//   u  = s dy B^T       A: dy kIMaj [M, N],  B: B  kIMaj [r, N]
//   dx = dy w_hat + u A^T  A: dy kIMaj, B: codes kQKMaj; then u kIMaj, A kIMaj
//   dA = x^T u          A: x  kKMaj,         B: u  kKMaj
//   dB = t^T dy         A: t  kKMaj,         B: dy kKMaj
// Small grids split the first reduction over blockIdx.z into fp32 partial
// sums, added in split order by f32_reduce_kernel (deterministic); the
// second reduction then belongs to split 0.
#include "common.h"

namespace qlora {
namespace {

constexpr int kFT = 256;           // lanes per workgroup
constexpr int kFTile = 128;        // output tile rows and columns
constexpr int kFK = 16;            // reduction depth of one step
constexpr int kFLd = kFTile + 32;  // LDS row stride in floats: consecutive k rows sit 32 banks apart

constexpr int kIMaj = 0, kKMaj = 1, kQIMaj = 2, kQKMaj = 3;
constexpr int kNone = -1;

struct Opnd {
    const float* p;        // plain operands
    const uint8_t* codes;  // quantized operands: packed codes [rows, kw / 2], element 2i in the high nibble
    const uint8_t* q8;     // 8-bit block scale codes (NULL: a2 holds one fp32 absmax per block)
    const float* a2;       // fp32 scales: one per 256 blocks (with q8) or per block
    int64_t ld;            // plain: row stride in elements
    int ilen, klen;        // extents along the output index i and the reduction index k
    int kw;                // quantized: code row length (elements)
    int vec;               // plain: ld % 4 == 0, so aligned 8-element chunks load as two 16-byte loads
};

struct Stage {
    float v[8];
    uint32_t code;
    float ahat;
};

typedef float f32x4a_t __attribute__((ext_vector_type(4)));

template <bool DQ>
__device__ __forceinline__ float block_scale(const Opnd& o, int64_t blk) {
    if (!DQ) return o.a2[blk];
    return __fmul_rn(__fdiv_rn(o.a2[blk >> 8], 255.0f), (float)o.q8[blk]);
}

// 8 consecutive plain values p[base .. base + 7], those with index e >= n_ok read as 0
__device__ __forceinline__ void load8(const float* p, int64_t base, int n_ok, bool vec, float (&v)[8]) {
    if (vec && n_ok >= 8) {
        const f32x4a_t a = *reinterpret_cast<const f32x4a_t*>(p + base);
        const f32x4a_t b = *reinterpret_cast<const f32x4a_t*>(p + base + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[4 + e] = b[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = e < n_ok ? p[base + e] : 0.0f;
    }
}

// global -> registers for the step whose tile starts at (i0, k0)
template <int MODE, bool DQ>
__device__ __forceinline__ void load_stage(const Opnd& o, int i0, int k0, int tid, Stage& S) {
    if constexpr (MODE == kIMaj || MODE == kQIMaj) {
        const int i = i0 + (tid >> 1), k = k0 + 8 * (tid & 1);
        if constexpr (MODE == kIMaj) {
            const int n_ok = i < o.ilen ? o.klen - k : 0;
            load8(o.p, (int64_t)i * o.ld + k, n_ok, o.vec, S.v);
        } else {
            // klen = kw is a multiple of 64 and k of 8: the 8-code chunk is wholly in range or out
            const bool ok = i < o.ilen && k < o.klen;
            const int ic = ok ? i : 0, kc = ok ? k : 0;
            S.code = *reinterpret_cast<const uint32_t*>(o.codes + ((int64_t)ic * o.kw + kc) / 2);
            const float ah = block_scale<DQ>(o, ((int64_t)ic * o.kw + kc) / kBlock);
            S.ahat = ok ? ah : 0.0f;
        }
    } else {
        const int k = k0 + (tid >> 4), i = i0 + 8 * (tid & 15);
        if constexpr (MODE == kKMaj) {
            const int n_ok = k < o.klen ? o.ilen - i : 0;
            load8(o.p, (int64_t)k * o.ld + i, n_ok, o.vec, S.v);
        } else {
            // ilen = kw is a multiple of 64
            const bool ok = k < o.klen && i < o.ilen;
            const int kc = ok ? k : 0, ic = ok ? i : 0;
            S.code = *reinterpret_cast<const uint32_t*>(o.codes + ((int64_t)kc * o.kw + ic) / 2);
            const float ah = block_scale<DQ>(o, ((int64_t)kc * o.kw + ic) / kBlock);
            S.ahat = ok ? ah : 0.0f;
        }
    }
}

// registers -> the [kFK][kFLd] LDS tile (w_hat = fl32(a_hat * c_q) for codes)
template <int MODE>
__device__ __forceinline__ void store_stage(Stage& S, float* T, const float* lvl, int tid) {
    if constexpr (MODE == kQIMaj || MODE == kQKMaj) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t nib = (S.code >> (8 * (e >> 1) + ((e & 1) ? 0 : 4))) & 0xFu;
            S.v[e] = __fmul_rn(S.ahat, lvl[nib]);
        }
    }
    if constexpr (MODE == kIMaj || MODE == kQIMaj) {
        const int ii = tid >> 1, kk = 8 * (tid & 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) T[(kk + e) * kFLd + ii] = S.v[e];
    } else {
        const int kk = tid >> 4, ii = 8 * (tid & 15);
        *reinterpret_cast<f32x4a_t*>(T + kk * kFLd + ii) = f32x4a_t{S.v[0], S.v[1], S.v[2], S.v[3]};
        *reinterpret_cast<f32x4a_t*>(T + kk * kFLd + ii + 4) = f32x4a_t{S.v[4], S.v[5], S.v[6], S.v[7]};
    }
}

// one reduction over k in [kb, ke): A tile rows i0 = m0, B tile columns i0 = n0
template <int AM, int BM, bool DQ>
__device__ __forceinline__ void run_phase(const Opnd& A, const Opnd& B, int m0, int n0, int kb, int ke, float* lds,
                                          const float* lvl, f32x16_t (&acc)[2][2], int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int kr = lane >> 5, c = lane & 31;
    constexpr int kBuf = 2 * kFK * kFLd;  // A tile + B tile
    Stage sa, sb;
    load_stage<AM, DQ>(A, m0, kb, tid, sa);
    load_stage<BM, DQ>(B, n0, kb, tid, sb);
    store_stage<AM>(sa, lds, lvl, tid);
    store_stage<BM>(sb, lds + kFK * kFLd, lvl, tid);
    __syncthreads();
    int buf = 0;
    for (int k0 = kb; k0 < ke; k0 += kFK) {
        const bool more = k0 + kFK < ke;
        if (more) {
            load_stage<AM, DQ>(A, m0, k0 + kFK, tid, sa);
            load_stage<BM, DQ>(B, n0, k0 + kFK, tid, sb);
        }
        const float* As = lds + buf * kBuf;
        const float* Bs = As + kFK * kFLd;
#pragma unroll
        for (int ks = 0; ks < kFK / 2; ++ks) {
            const int row = (2 * ks + kr) * kFLd;
            const float a0 = As[row + 64 * wm + c], a1 = As[row + 64 * wm + 32 + c];
            const float b0 = Bs[row + 64 * wn + c], b1 = Bs[row + 64 * wn + 32 + c];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (more) {
            float* An = lds + (buf ^ 1) * kBuf;
            store_stage<AM>(sa, An, lvl, tid);
            store_stage<BM>(sb, An + kFK * kFLd, lvl, tid);
        }
        __syncthreads();
        buf ^= 1;
    }
}

// C [rows, cols] (+ split * rows * cols) = scale * (sum over this split of A B, plus A2 B2 in split 0)
template <int AM, int BM, int BM2, bool DQ, int CB>
__global__ __launch_bounds__(kFT) void f32_gemm_kernel(Opnd A, Opnd B, Opnd A2, Opnd B2, float* __restrict__ C,
                                                       int rows, int cols, int kchunk, float scale) {
    __shared__ __attribute__((aligned(16))) float lds[2 * 2 * kFK * kFLd];
    __shared__ float lvl[16];
    const int tid = threadIdx.x;
    if (tid < 16) lvl[tid] = level<CB>(tid);
    const int n0 = blockIdx.x * kFTile, m0 = blockIdx.y * kFTile, split = blockIdx.z;
    const int kb = split * kchunk, ke = min(A.klen, kb + kchunk);

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

    __syncthreads();  // lvl
    if (kb < ke) run_phase<AM, BM, DQ>(A, B, m0, n0, kb, ke, lds, lvl, acc, tid);
    if constexpr (BM2 != kNone) {
        if (split == 0 && A2.klen > 0) run_phase<kIMaj, BM2, DQ>(A2, B2, m0, n0, 0, A2.klen, lds, lvl, acc, tid);
    }

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    float* out = C + (int64_t)split * rows * cols;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = n0 + 64 * wn + 32 * b + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + 64 * wm + 32 * a + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < rows && col < cols) out[(int64_t)row * cols + col] = acc[a][b][v] * scale;
            }
        }
}

// out[i] = scale * sum_{s < splits} part[s * count + i], in split order
__global__ __launch_bounds__(256) void f32_reduce_kernel(const float* __restrict__ part, int64_t count, int splits,
                                                         float scale, float* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
        float s = 0.0f;
        for (int j = 0; j < splits; ++j) s += part[(int64_t)j * count + i];
        out[i] = s * scale;
    }
}

Opnd plain(const float* p, int64_t ld, int ilen, int klen) {
    Opnd o{};
    o.p = p;
    o.ld = ld;
    o.ilen = ilen;
    o.klen = klen;
    o.vec = (ld % 4) == 0;
    return o;
}

Opnd quant(const uint8_t* codes, const uint8_t* q8, const float* a2, int ilen, int klen, int kw) {
    Opnd o{};
    o.codes = codes;
    o.q8 = q8;
    o.a2 = a2;
    o.ilen = ilen;
    o.klen = klen;
    o.kw = kw;
    return o;
}

// splits of the first reduction: enough workgroups for two per compute unit,
// at least 128 of the reduction per split, at most 32 splits
F32Plan plan(int rows, int cols, int red) {
    const int64_t tiles = (int64_t)((rows + kFTile - 1) / kFTile) * ((cols + kFTile - 1) / kFTile);
    int want = (int)std::min<int64_t>(32, (512 + tiles - 1) / tiles);
    want = std::max(1, std::min(want, red / 128));
    int kchunk = ((red + want - 1) / want + kFK - 1) / kFK * kFK;
    kchunk = std::max(kchunk, kFK);
    const int splits = std::max(1, (red + kchunk - 1) / kchunk);
    return F32Plan{splits, kchunk};
}

template <int AM, int BM, int BM2, bool DQ, int CB>
qlora_status run(const Opnd& A, const Opnd& B, const Opnd& A2, const Opnd& B2, int rows, int cols, float scale,
                 float* out, float* part, hipStream_t s) {
    const F32Plan p = plan(rows, cols, std::max(A.klen, 1));
    const dim3 grid((unsigned)((cols + kFTile - 1) / kFTile), (unsigned)((rows + kFTile - 1) / kFTile),
                    (unsigned)p.splits);
    if (p.splits == 1) {
        hipLaunchKernelGGL((f32_gemm_kernel<AM, BM, BM2, DQ, CB>), grid, dim3(kFT), 0, s, A, B, A2, B2, out, rows,
                           cols, p.kchunk, scale);
        return launch_status();
    }
    if (!part) return QLORA_ERR_WORKSPACE;
    hipLaunchKernelGGL((f32_gemm_kernel<AM, BM, BM2, DQ, CB>), grid, dim3(kFT), 0, s, A, B, A2, B2, part, rows, cols,
                       p.kchunk, 1.0f);
    const int64_t count = (int64_t)rows * cols;
    const int blocks = (int)std::min<int64_t>(2048, (count + 255) / 256);
    hipLaunchKernelGGL(f32_reduce_kernel, dim3(blocks), dim3(256), 0, s, part, count, p.splits, scale, out);
    return launch_status();
}

}  // namespace

F32Plan plan_f32(int rows, int cols, int red) { return plan(rows, cols, red); }

qlora_status launch_f32_lora(int which, const float* X, const float* Y, int M, int C, int r, float scale, float* out,
                             float* part, hipStream_t s) {
    const Opnd none{};
    switch (which) {
        case kF32LoraDown: {  // out [M, r] = scale * X [M, C] Y [C, r]
            const Opnd a = plain(X, C, M, C), b = plain(Y, r, r, C);
            return run<kIMaj, kKMaj, kNone, false, kCbNf4>(a, b, none, none, M, r, scale, out, part, s);
        }
        case kF32LoraDownT: {  // out [M, r] = scale * X [M, C] Y^T, Y [r, C]
            const Opnd a = plain(X, C, M, C), b = plain(Y, C, r, C);
            return run<kIMaj, kIMaj, kNone, false, kCbNf4>(a, b, none, none, M, r, scale, out, part, s);
        }
        case kF32Grad: {  // out [C, r] = scale * X^T S with X [M, C], S [M, r]
            const Opnd a = plain(X, C, C, M), b = plain(Y, r, r, M);
            return run<kKMaj, kKMaj, kNone, false, kCbNf4>(a, b, none, none, C, r, scale, out, part, s);
        }
        case kF32GradT: {  // out [r, C] = scale * S^T X with S [M, r] (X), X [M, C] (Y)
            const Opnd a = plain(X, r, r, M), b = plain(Y, C, C, M);
            return run<kKMaj, kKMaj, kNone, false, kCbNf4>(a, b, none, none, r, C, scale, out, part, s);
        }
        default: return QLORA_ERR_INVALID_ARG;
    }
}

qlora_status launch_f32_fwd(const float* x, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                            const float* t, const float* B, float* y, int M, int N, int K, int r, float* part,
                            hipStream_t s) {
    const Opnd a = plain(x, K, M, K), b = quant(codes, q8, a2, N, K, K);
    const Opnd a2o = plain(t, r, M, r), b2o = plain(B, N, N, r);
    qlora_status st = QLORA_OK;
    auto go = [&](auto cbc) {
        constexpr int CB = decltype(cbc)::value;
        st = q8 ? run<kIMaj, kQIMaj, kKMaj, true, CB>(a, b, a2o, b2o, M, N, 1.0f, y, part, s)
                : run<kIMaj, kQIMaj, kKMaj, false, CB>(a, b, a2o, b2o, M, N, 1.0f, y, part, s);
    };
    if (cb == kCbFp4) go(IntC<kCbFp4>{});
    else go(IntC<kCbNf4>{});
    return st;
}

qlora_status launch_f32_bwd_dx(const float* dy, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                               const float* u, const float* A, float* dx, int M, int N, int K, int r, float* part,
                               hipStream_t s) {
    const Opnd a = plain(dy, N, M, N), b = quant(codes, q8, a2, K, N, K);
    const Opnd a2o = plain(u, r, M, r), b2o = plain(A, r, K, r);
    qlora_status st = QLORA_OK;
    auto go = [&](auto cbc) {
        constexpr int CB = decltype(cbc)::value;
        st = q8 ? run<kIMaj, kQKMaj, kIMaj, true, CB>(a, b, a2o, b2o, M, K, 1.0f, dx, part, s)
                : run<kIMaj, kQKMaj, kIMaj, false, CB>(a, b, a2o, b2o, M, K, 1.0f, dx, part, s);
    };
    if (cb == kCbFp4) go(IntC<kCbFp4>{});
    else go(IntC<kCbNf4>{});
    return st;
}

}  // namespace qlora
