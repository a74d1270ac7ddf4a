// NF4 blockwise quantization with double-quantized scales, and the matching
// dequantization ("bitsandbytes deep dive", sections 5.1-5.2, 6.2, 7.2).
//
// nf4_quantize_kernel: one workgroup (256 lanes) per group of 256 blocks
// (16384 weights, 32 KB of bf16).  Every weight is read from HBM once:
//   1. each lane loads 8 bf16 (16 B) per pass, 8 passes; a wave's load covers
//      1 KB of consecutive weights (8 blocks x 8 lanes x 16 B);
//   2. block absmax: integer max of |bits| over the lane's 8 values, then a
//      3-step shuffle over the block's 8 lanes;
//   3. lane t computes block t's 15 decision thresholds
//      T_j = RD_bf16(a * m_j), m_j = (c_j + c_{j+1}) / 2, exactly (the product
//      is exact in fp64, then rounded down to the bf16 grid), the group scale
//      a2 = max a, and the 8-bit scale code;
//   4. for a bf16 weight w and any real X, w > X  <=>  w > RD_bf16(X), so the
//      code = #{j : w/a > m_j} (nearest level, ties to the lower index) needs
//      only exact compares against T_j.  A bucket index i = trunc(fma(w, 64/a,
//      64)) places 64 (w/a + 1) in [i - e, i + 1 + e] with e < 2^-16; the
//      midpoints 64 (m_j + 1) lie more than 5 buckets apart, so at most one of
//      them, j = c, is in reach of bucket i, where c = #{j : 64 (m_j + 1) <
//      i - 1/1024} comes from a 129-entry table.  Then code = c + [w > T_c]
//      (T_15 = +inf), whichever side of its bucket w fell on: one fma, one
//      table read, one threshold read and one compare per weight.  Blocks with
//      0 < a < 2^-100 (64/a could overflow) take a branchless binary search
//      over the same thresholds instead;
//   5. nibbles are packed (element 2i high) and stored as one dword per lane.
// Without double quantization (sections 7.1, 9.5) step 3 stores each block's
// absmax as its fp32 scale instead of the 8-bit code and the group scale.
// An fp32 source weight (DT = kDtF32, deep dive 8.3) takes the same steps
// with 32 B per lane per pass; for any fp32 w and real X, w > X <=>
// w > RD_f32(X), so its thresholds are those of fp16 weights.
#include "common.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int kPasses = kSuper / 32;  // 32 blocks per pass (4 waves x 8 blocks)
constexpr int kThrStride = 17;        // per block: T_0..T_14, +inf, 64/a; an odd stride spreads blocks over banks
constexpr int kBuckets = 129;         // trunc(64 (u + 1)) for u in [-1, 1]
constexpr float kTinyScale = 0x1p-100f;

// RD_bf16(x) (DT = bf16) or RD_f32(x) (fp16 and fp32 weights) of an exact product x
// whose magnitude is at least 2^-126: the double's significand cut to the target's 8
// (24) bits toward zero converts to float exactly; a negative x that lost bits in the
// cut steps one unit down (toward -inf), which may carry into the exponent.  Any
// float weight w has w > X <=> w > RD_f32(X), and a bf16 weight also w > X <=>
// w > RD_bf16(X).
template <int DT>
__device__ __forceinline__ float rd_to_grid(double x) {
    constexpr int kDrop = DT == kDtBf16 ? 52 - 7 : 52 - 23;   // double significand bits below the target's
    constexpr uint64_t kMask = (uint64_t(1) << kDrop) - 1;
    const uint64_t d = (uint64_t)__double_as_longlong(x);
    uint32_t u = __float_as_uint((float)__longlong_as_double((long long)(d & ~kMask)));
    if ((d >> 63) && (d & kMask)) u += DT == kDtBf16 ? 0x00010000u : 1u;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t absmax_bits8(u32x4_t v) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t x = v[i] & 0x7FFF7FFFu;
        m = max(m, max(x & 0xFFFFu, x >> 16));
    }
    return m;
}

// count of thresholds strictly below w; the 15 ascending thresholds come as
// four vectors (T0..T3, T4..T7, T8..T11, T12..T14 + unused).  Every select is
// on register values, so nothing is indexed dynamically.
__device__ __forceinline__ uint32_t nf4_code(float w, f32x4_t t0, f32x4_t t1, f32x4_t t2, f32x4_t t3) {
    const bool b3 = w > t1[3];                                   // T7
    const float s2 = b3 ? t2[3] : t0[3];                         // T11 : T3
    const bool b2 = w > s2;
    const float s1a = b3 ? t3[1] : t1[1];                        // T13 : T5
    const float s1b = b3 ? t2[1] : t0[1];                        // T9  : T1
    const bool b1 = w > (b2 ? s1a : s1b);
    const float e3 = b3 ? t3[2] : t1[2];                         // T14 : T6
    const float e2 = b3 ? t3[0] : t1[0];                         // T12 : T4
    const float e1 = b3 ? t2[2] : t0[2];                         // T10 : T2
    const float e0 = b3 ? t2[0] : t0[0];                         // T8  : T0
    const float s0 = b2 ? (b1 ? e3 : e2) : (b1 ? e1 : e0);
    const bool b0 = w > s0;
    return (b3 ? 8u : 0u) | (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
}

// value i (0..7) of a lane's 8 consecutive weights held as 16-bit pairs or 32-bit words
template <int DT, int NW>
__device__ __forceinline__ float elem(const u32x4_t (&v)[NW], int i) {
    if constexpr (DT == kDtF32) return __uint_as_float(v[i >> 2][i & 3]);
    else return h16_to_f32<DT>((i & 1) ? (v[0][i >> 1] >> 16) : (v[0][i >> 1] & 0xFFFFu));
}

// Group `group` (blocks 256 group .. 256 group + 255) of one weight, by one workgroup.
template <bool DQ, int CB, int DT>
__device__ __forceinline__ void quantize_group(const void* __restrict__ Wv, int64_t nblocks,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ q8,
                                               float* __restrict__ a2, int64_t group) {
    __shared__ float s_amax[kSuper];
    __shared__ float s_thr[kSuper * kThrStride];
    __shared__ float s_wmax[kThreads / 64];
    __shared__ uint8_t s_lut[kBuckets + 31];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t b0 = group * kSuper;
    const int nb_here = (int)min((int64_t)kSuper, nblocks - b0);
    const int sub = lane & 7;

    // 1. all loads in flight at once (8 weights per lane per pass: 16 B, or 32 B for fp32)
    constexpr int NW = DT == kDtF32 ? 2 : 1;
    const u32x4_t* W = static_cast<const u32x4_t*>(Wv);
    u32x4_t v[kPasses][NW];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int bl = p * 32 + wave * 8 + (lane >> 3);
#pragma unroll
        for (int h = 0; h < NW; ++h) {
            if (bl < nb_here) {
                v[p][h] = __builtin_nontemporal_load(W + ((b0 + bl) * kBlock + sub * 8) / (8 / NW) + h);
            } else {
                v[p][h] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    }

    // bucket table: c(i) = number of midpoints m_j with 64 (m_j + 1) < i - 1/1024 (fp64, exact)
    if (tid < kBuckets) {
        int c = 0;
#pragma unroll
        for (int j = 0; j + 1 < kDistinctLevels<CB>; ++j) {
            const double m = 0.5 * ((double)level<CB>(code_of_sorted<CB>(j)) +
                                    (double)level<CB>(code_of_sorted<CB>(j + 1)));
            c += (64.0 * m + 64.0 < (double)tid - 1.0 / 1024.0) ? 1 : 0;
        }
        s_lut[tid] = (uint8_t)c;
    }

    // 2. block absmax
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        uint32_t m = 0;
        if constexpr (DT == kDtF32) {
#pragma unroll
            for (int i = 0; i < 8; ++i) m = max(m, v[p][i >> 2][i & 3] & 0x7FFFFFFFu);  // |w| orders as its bits
        } else {
            m = absmax_bits8(v[p][0]);
        }
        m = max(m, (uint32_t)__shfl_xor((int)m, 1));
        m = max(m, (uint32_t)__shfl_xor((int)m, 2));
        m = max(m, (uint32_t)__shfl_xor((int)m, 4));
        const int bl = p * 32 + wave * 8 + (lane >> 3);
        if (sub == 0) {                                  // 0 for blocks past the end
            if constexpr (DT == kDtF32) s_amax[bl] = __uint_as_float(m);
            else s_amax[bl] = h16_to_f32<DT>(m);
        }
    }
    __syncthreads();

        // 3. thresholds of block `tid`, group scale, scale code
    const float a = s_amax[tid];
    {
        float T[15];
        if (a >= kTinyScale) {
            // |a m| > 2^-105: the rounding below stays in fp32's normal range
            const double ad = (double)a;
#pragma unroll
            for (int j = 0; j < 15; ++j) {
                if (j + 1 < kDistinctLevels<CB>) {
                    const double m = 0.5 * ((double)level<CB>(code_of_sorted<CB>(j)) +
                                            (double)level<CB>(code_of_sorted<CB>(j + 1)));  // exact
                    T[j] = rd_to_grid<DT>(ad * m);
                } else {
                    T[j] = __builtin_huge_valf();
                }
            }
        } else if (a > 0.0f) {
            const double ad = (double)a;
#pragma unroll
            for (int j = 0; j < 15; ++j) {
                if (j + 1 < kDistinctLevels<CB>) {
                    const double m = 0.5 * ((double)level<CB>(code_of_sorted<CB>(j)) +
                                            (double)level<CB>(code_of_sorted<CB>(j + 1)));  // exact
                    // the product is exact; any float weight w has w > X <=> w > RD_f32(X),
                    // and a bf16 weight also w > X <=> w > RD_bf16(X)
                    const float x = __double2float_rd(ad * m);
                    T[j] = DT == kDtBf16 ? f32_rd_bf16(x) : x;
                } else {
                    T[j] = __builtin_huge_valf();  // no level above the last distinct one
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 15; ++j) T[j] = (j < kZeroCode) ? -1.0f : 1.0f;  // every w = 0 -> code 7
        }
        float* dst = &s_thr[tid * kThrStride];
#pragma unroll
        for (int j = 0; j < 15; ++j) dst[j] = T[j];
        dst[15] = __builtin_huge_valf();                  // c = 15: every midpoint lies below the bucket
        dst[16] = a >= kTinyScale ? __fdiv_rn(64.0f, a) : 0.0f;  // 0 (bucket 64) for a = 0 and tiny a
    }
    if (!DQ) {
        if (tid < nb_here) a2[b0 + tid] = a;  // the exact block absmax is the fp32 scale
    }
    float gm = a;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
    if (DQ && lane == 0) s_wmax[wave] = gm;
    __syncthreads();
    const float A2 = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
    if (DQ && tid < nb_here) {
        // q8 = #{k in 1..255 : 510 a > (2k-1) A2}; all products exact in fp64
        const double x = 510.0 * (double)a;
        const double y = (double)A2;
        int k = 0;
#pragma unroll
        for (int step = 128; step >= 1; step >>= 1) {
            const int c = k + step;
            if (c <= 255 && (double)(2 * c - 1) * y < x) k = c;
        }
        q8[b0 + tid] = (uint8_t)k;
    }
    if (DQ && tid == 0) a2[group] = A2;

    // 4-5. codes against the true absmax, packed and stored
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int bl = p * 32 + wave * 8 + (lane >> 3);
        if (bl < nb_here) {
                        const float* tb = &s_thr[bl * kThrStride];
            const float sc = tb[16];
            // the block's threshold row as an LDS byte address, formed once: each weight's
            // threshold is then one shift-and-add away (c * 4 + row)
            const uint32_t trow = (uint32_t)reinterpret_cast<uintptr_t>(tb);
                        uint32_t q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float w = elem<DT, NW>(v[p], i);
                const int bucket = (int)__builtin_fmaf(w, sc, 64.0f);  // 0 .. 128 (trunc; -2^-16 -> 0)
                const uint32_t c = s_lut[bucket];
                const float tc = *reinterpret_cast<const __attribute__((address_space(3))) float*>(
                    (uintptr_t)((c << 2) + trow));
                q[i] = code_of_sorted<CB>(c + (w > tc ? 1u : 0u));
            }
            // byte j = element 2j in the high nibble, 2j + 1 in the low one
            uint32_t packed = (q[0] << 4) | q[1];
#pragma unroll
            for (int j = 1; j < 4; ++j) packed |= ((q[2 * j] << 4) | q[2 * j + 1]) << (8 * j);
            const float ab = s_amax[bl];
            if (ab > 0.0f && ab < kTinyScale) {               // rare: 64/a may not be finite
                const f32x4_t t0 = {tb[0], tb[1], tb[2], tb[3]}, t1 = {tb[4], tb[5], tb[6], tb[7]};
                const f32x4_t t2 = {tb[8], tb[9], tb[10], tb[11]}, t3 = {tb[12], tb[13], tb[14], 0.0f};
                packed = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t q = code_of_sorted<CB>(nf4_code(elem<DT, NW>(v[p], i), t0, t1, t2, t3));
                    packed |= q << (4 * (i ^ 1));
                }
            }
            *reinterpret_cast<uint32_t*>(codes + (b0 + bl) * (kBlock / 2) + sub * 4) = packed;
        }
    }
}

template <bool DQ, int CB, int DT>
__global__ __launch_bounds__(kThreads) void nf4_quantize_kernel(const void* __restrict__ Wv, int64_t nblocks,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ q8, float* __restrict__ a2) {
    quantize_group<DQ, CB, DT>(Wv, nblocks, codes, q8, a2, blockIdx.x);
}

// Several weights of one configuration in one launch: workgroup g quantizes group
// g - first[i] of weight i, first[i] <= g < first[i + 1].  One launch keeps the
// chip streaming across the weights (the workgroups of one weight all start at
// once and then compute at once), and saves a launch per weight.
struct QuantBatch {
    const void* W[kQuantBatchMax];
    uint8_t* codes[kQuantBatchMax];
    uint8_t* q8[kQuantBatchMax];
    float* a2[kQuantBatchMax];
    int64_t nblocks[kQuantBatchMax];
    int64_t first[kQuantBatchMax + 1];
    int count;
};

template <bool DQ, int CB, int DT>
__global__ __launch_bounds__(kThreads) void nf4_quantize_batch_kernel(const QuantBatch b) {
    const int64_t g = blockIdx.x;
    int i = 0;
    while (i + 1 < b.count && g >= b.first[i + 1]) ++i;   // uniform: the weight of this workgroup
    quantize_group<DQ, CB, DT>(b.W[i], b.nblocks[i], b.codes[i], b.q8[i], b.a2[i], g - b.first[i]);
}

// nf4_dequantize_kernel: 256 lanes x 8 weights = 32 blocks per workgroup.
//   a_hat = fl32(fl32(a2/255) * q8) (without double quantization: the stored
//   fp32 absmax a2[b]), w_hat = RNE_bf16(fl32(a_hat * c_code)).
// F32: write the fp32 products fl32(a_hat * c_code) themselves (out is then float*).
template <bool DQ, int CB, int DT, bool F32>
__global__ __launch_bounds__(kThreads) void nf4_dequantize_kernel(const uint8_t* __restrict__ codes,
                                                                  const uint8_t* __restrict__ q8,
                                                                  const float* __restrict__ a2,
                                                                  int64_t nblocks,
                                                                  void* __restrict__ out) {
    __shared__ float s_c[16];
    const int tid = threadIdx.x;
    if (tid < 16) s_c[tid] = level<CB>(tid);
    __syncthreads();
    const int64_t b = (int64_t)blockIdx.x * 32 + (tid >> 3);
    const int sub = tid & 7;
    if (b >= nblocks) return;
    const float ahat = DQ ? __fmul_rn(__fdiv_rn(a2[b / kSuper], 255.0f), (float)q8[b]) : a2[b];
    const uint32_t pk = *reinterpret_cast<const uint32_t*>(codes + b * (kBlock / 2) + sub * 4);
    u32x4_t o;
    float wf[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t byte = (pk >> (8 * j)) & 0xFFu;
        const float w0 = __fmul_rn(ahat, s_c[byte >> 4]);
        const float w1 = __fmul_rn(ahat, s_c[byte & 0xFu]);
        o[j] = pack2<DT>(w0, w1);
        wf[2 * j] = w0;
        wf[2 * j + 1] = w1;
    }
    if (F32) {
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + b * kBlock + sub * 8);
        dst[0] = f32x4_t{wf[0], wf[1], wf[2], wf[3]};
        dst[1] = f32x4_t{wf[4], wf[5], wf[6], wf[7]};
    } else {
        *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(out) + b * kBlock + sub * 8) = o;
    }
}

}  // namespace

qlora_status launch_quantize(const void* W, int64_t nblocks, uint8_t* codes, uint8_t* q8, float* a2, int cb,
                             int dt, hipStream_t s) {
    const int64_t groups = (nblocks + kSuper - 1) / kSuper;
    auto go = [&](auto cbc, auto dtc) {
        constexpr int CB = decltype(cbc)::value, DT = decltype(dtc)::value;
        if (q8)
            hipLaunchKernelGGL((nf4_quantize_kernel<true, CB, DT>), dim3((unsigned)groups), dim3(kThreads), 0, s, W,
                               nblocks, codes, q8, a2);
        else
            hipLaunchKernelGGL((nf4_quantize_kernel<false, CB, DT>), dim3((unsigned)groups), dim3(kThreads), 0, s, W,
                               nblocks, codes, q8, a2);
    };
    if (dt == kDtF32) {
        if (cb == kCbFp4) go(IntC<kCbFp4>{}, IntC<kDtF32>{});
        else go(IntC<kCbNf4>{}, IntC<kDtF32>{});
    } else {
        with_cb_dt(cb, dt, go);
    }
    return launch_status();
}

qlora_status launch_quantize_batch(const void* const* W, const int64_t* nblocks, uint8_t* const* codes,
                                   uint8_t* const* q8, float* const* a2, int count, int cb, int dt, hipStream_t s) {
    if (count < 1 || count > kQuantBatchMax) return QLORA_ERR_INVALID_ARG;
    QuantBatch b{};
    b.count = count;
    b.first[0] = 0;
    for (int i = 0; i < count; ++i) {
        b.W[i] = W[i];
        b.codes[i] = codes[i];
        b.q8[i] = q8[i];
        b.a2[i] = a2[i];
        b.nblocks[i] = nblocks[i];
        b.first[i + 1] = b.first[i] + (nblocks[i] + kSuper - 1) / kSuper;
    }
    const int64_t groups = b.first[count];
    if (groups >= (int64_t(1) << 31)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    const bool dq = q8[0] != nullptr;
    auto go = [&](auto cbc, auto dtc) {
        constexpr int CB = decltype(cbc)::value, DT = decltype(dtc)::value;
        if (dq)
            hipLaunchKernelGGL((nf4_quantize_batch_kernel<true, CB, DT>), dim3((unsigned)groups), dim3(kThreads), 0,
                               s, b);
        else
            hipLaunchKernelGGL((nf4_quantize_batch_kernel<false, CB, DT>), dim3((unsigned)groups), dim3(kThreads), 0,
                               s, b);
    };
    with_cb_dt(cb, dt, go);
    return launch_status();
}

qlora_status launch_dequantize(const uint8_t* codes, const uint8_t* q8, const float* a2, int cb, int dt,
                               int64_t nblocks, uint16_t* out, hipStream_t s) {
    const int64_t grid = (nblocks + 31) / 32;
    with_cb_dt(cb, dt, [&](auto cbc, auto dtc) {
        constexpr int CB = decltype(cbc)::value, DT = decltype(dtc)::value;
        if (q8)
            hipLaunchKernelGGL((nf4_dequantize_kernel<true, CB, DT, false>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                               codes, q8, a2, nblocks, static_cast<void*>(out));
        else
            hipLaunchKernelGGL((nf4_dequantize_kernel<false, CB, DT, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                               s, codes, q8, a2, nblocks, static_cast<void*>(out));
    });
    return launch_status();
}

qlora_status launch_dequantize_f32(const uint8_t* codes, const uint8_t* q8, const float* a2, int cb, int64_t nblocks,
                                   float* out, hipStream_t s) {
    const int64_t grid = (nblocks + 31) / 32;
    with_cb_dt(cb, kDtBf16, [&](auto cbc, auto) {
        constexpr int CB = decltype(cbc)::value;
        if (q8)
            hipLaunchKernelGGL((nf4_dequantize_kernel<true, CB, kDtBf16, true>), dim3((unsigned)grid), dim3(kThreads),
                               0, s, codes, q8, a2, nblocks, static_cast<void*>(out));
        else
            hipLaunchKernelGGL((nf4_dequantize_kernel<false, CB, kDtBf16, true>), dim3((unsigned)grid),
                               dim3(kThreads), 0, s, codes, q8, a2, nblocks, static_cast<void*>(out));
    });
    return launch_status();
}

}  // namespace qlora
