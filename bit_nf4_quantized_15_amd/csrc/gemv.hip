// Decode-size forward of the NF4 linear layer (M <= 16 activation rows):
//   y[M, N] = x[M, K] W_hat^T + t[M, r] B[r, N]
// ("bitsandbytes deep dive", sections 7.2-7.3: the forward dequantizes the
// frozen 4-bit base on the fly; at small batch the layer is memory-bound).
//
// The packed codes are the HBM traffic (0.5 B per weight); everything else is
// small.  The kernel streams each code byte once with as few, as wide memory
// instructions as it can, and spends about one VALU op per weight:
//  * a workgroup owns 16 weight rows (16 outputs per x row) over all of K, in
//    phases of PB blocks; wave w takes a contiguous quarter of each phase;
//  * a wave copies its codes straight from HBM into LDS (buffer_load ... lds,
//    16 B per lane), one 1 KB instruction per 8 rows x 4 blocks, and starts
//    on each 4-block group as soon as its two instructions have landed.  The
//    16-byte chunks are XOR-swizzled by row on the way in so that the
//    operand reads below hit 16 distinct bank groups;
//  * the block scales a_hat = fl32(fl32(a2 / 255) q8) of the wave's rows and
//    blocks are computed once per phase into a small LDS table;
//  * the dot products run on v_mfma_f32_16x16x32_bf16.  B operand lane
//    (n, g) holds codebook levels of row n, A operand lane (m, g) x row m;
//    within a block the two MFMAs cover k = 16 g + 8 h + [0, 8) (h = 0, 1);
//  * a code byte (two nibbles) becomes its two bf16 levels through one LDS
//    read of a 256-entry table (64 copies, one per lane, so reads never
//    conflict) at an address formed by one v_perm_b32;
//  * a block's two MFMAs start from zero and a_hat multiplies that fp32
//    partial sum into the running total:
//      y = sum_b a_hat_b * sum_{k in b} bf16(c_q) x_k.
//    The weight used, a_hat bf16(c_q), and the dequantized weight
//    RNE_bf16(a_hat c_q) are each within half a bf16 ulp (at most 2^-8
//    relative) of a_hat c_q, so they differ by at most 2^-7 relative;
//  * x is staged in LDS per phase, t and the 16 columns of B once; the LoRA
//    term t B runs on the same MFMA accumulators (r <= 128 as up to four
//    32-wide k chunks, one per wave), and the 4 waves' partial sums are added
//    through LDS before the bf16 store.
#include "common.h"

namespace qlora {

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
// direct HBM -> LDS load: lane l's `size` bytes land at lds_ptr + size * l
__device__ void gv_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) uint32_t* lds_ptr, int size,
                            int voffset, int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace {

constexpr int kGvRows = 16;                // weight rows (= outputs per x row) per workgroup
constexpr int kGvThreads = 256;            // 4 waves
constexpr int kLutBytes = 256 * 64 * 4;    // 256 byte values x 64 lane copies x 4 B
constexpr int kTBytes = 16 * 128 * 2;      // t as [16 rows][128] bf16, zero past M rows and r columns
constexpr int kBBytes = kGvRows * 128 * 2; // B^T of the 16 columns as [16][128] bf16, zero past r
constexpr int kGroupBytes = 4 * 2048;      // one 4-block code group of each of the 4 waves
constexpr int kLdsTotal = 160 * 1024;
// a phase is PB = 16 NG blocks, NG in {1, 2, 4} (4-block code groups per wave)
__host__ __device__ constexpr int scale_bytes(int NG) { return 4 * 16 * (4 * NG + 4) * 4; }
__host__ __device__ constexpr int x_bytes(int NG) {  // what is left for x
    return kLdsTotal - kLutBytes - NG * kGroupBytes - scale_bytes(NG) - kTBytes - kBBytes - 256;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ i32x4_t raw_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4_t{(int32_t)(uint32_t)a, (int32_t)(uint32_t)(a >> 32), (int32_t)bytes, 0x00020000};
}

// at most n (even, <= 14) of this wave's memory loads still in flight; n is a
// constant after unrolling, so one wait remains
__device__ __forceinline__ void wait_vm_at_most(int n) {
    switch (n) {
        case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// Workgroup barrier for data this workgroup wrote with ds_write only.  The
// compiler's own barrier also drains every pending direct HBM->LDS load, which
// would make each wave wait for all of its codes before the first group; the
// code loads are wave-private and waited for per group instead.
__device__ __forceinline__ void sync_lds_writes() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct GvPlan {
    int Kb;      // blocks per row
    int PB;      // blocks per phase (16 NG)
    int phases;
    int xs;      // LDS byte stride of an x row
    int tsh;     // log2 of the threads that stage one x row
};

// 16x16x32 MFMA on operands of the compute dtype DT (bf16 or fp16 bit patterns).
template <int DT>
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    if (DT == kDtF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int NV, int NG, bool DQ, int CB, int DT>
__global__ __launch_bounds__(kGvThreads) void nf4_gemv_kernel(const uint16_t* __restrict__ x,
                                                              const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ q8,
                                                              const float* __restrict__ a2,
                                                              const uint16_t* __restrict__ t,
                                                              const uint16_t* __restrict__ B,
                                                              uint16_t* __restrict__ y, int M, int N, int K,
                                                              int r, GvPlan P) {
    // LUT, x, scale tables, t and B share one array; each code group has an
    // array of its own, so that the compiler, which must wait for direct
    // HBM->LDS loads before LDS reads that may alias them, waits for group j's
    // loads only where group j is read
    constexpr int kX = x_bytes(NG);
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLutBytes + kX + scale_bytes(NG) + kTBytes + kBBytes];
    __shared__ __attribute__((aligned(16))) uint8_t cg0[kGroupBytes];
    __shared__ __attribute__((aligned(16))) uint8_t cg1[NG > 1 ? kGroupBytes : 16];
    __shared__ __attribute__((aligned(16))) uint8_t cg2[NG > 2 ? kGroupBytes : 16];
    __shared__ __attribute__((aligned(16))) uint8_t cg3[NG > 3 ? kGroupBytes : 16];
    uint8_t* const cgs[4] = {cg0, cg1, cg2, cg3};
    uint8_t* const lut = smem;
    uint8_t* const xl = smem + kLutBytes;
    uint8_t* const sl = smem + kLutBytes + kX;
    uint8_t* const tl = sl + scale_bytes(NG);
    uint16_t* const bl = reinterpret_cast<uint16_t*>(tl + kTBytes);

    const int tid = threadIdx.x;
    // codebook level of this thread's table entries, loaded before anything
    // that waits on HBM so that building the table never waits behind it
    const float lo_level = level<CB>(tid >> 4);
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15;  // B column (weight row) / A row (x row) of the lane
    const int lg = lane >> 4;  // k group
    const int n0 = blockIdx.x * kGvRows;
    constexpr int PBw = 4 * NG;  // blocks per wave per phase
    const int Kb = P.Kb;
    float* const aw = reinterpret_cast<float*>(sl) + w * 16 * (PBw + 4);  // this wave's scale table

    // ---- x of one phase: thread -> (row xm, 16-byte chunks xc0 + tpr * it)
    const int tpr = 1 << P.tsh;
    const int xm = tid >> P.tsh, xc0 = tid & (tpr - 1);
    u32x4_t xv[16];
    auto stage_load = [&](int p) {
        const int b0 = p * P.PB;
        const int rc = min(P.PB, Kb - b0) * 8;  // 16-byte chunks per row in this phase
        const uint16_t* src = x + (int64_t)xm * K + (int64_t)b0 * kBlock;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int c = xc0 + tpr * it;
            if (xm < M && c < rc) xv[it] = *reinterpret_cast<const u32x4_t*>(src + 8 * c);
        }
    };
    // chunks past the row end (last phase) are zero: the blocks there are
    // multiplied by a_hat = 0 and must contribute finite partial sums
    auto stage_store = [&](int p) {
        const int rc = min(P.PB, Kb - p * P.PB) * 8;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int c = xc0 + tpr * it;
            if (xm < M && c < P.PB * 8)
                *reinterpret_cast<u32x4_t*>(xl + xm * P.xs + 16 * c) = c < rc ? xv[it] : u32x4_t{0u, 0u, 0u, 0u};
        }
    };

    // ---- per phase and wave: 8-bit scales and group scales into registers, then
    // the codes straight into LDS.  Lane l computes the scales of row l % 16
    // and blocks l / 16 + 4 u of the wave's range.
    // (without double quantization: the blocks' fp32 absmax, read from a2)
    const int arow = min(n0 + (lane & 15), N - 1);
    const rsrc_t qrs = make_rsrc(q8, (uint32_t)((uint64_t)N * Kb));
    const int ngroups = (int)(((int64_t)N * Kb + kSuper - 1) / kSuper);
    const rsrc_t ars = make_rsrc(a2, DQ ? (uint32_t)ngroups * 4u : (uint32_t)((uint64_t)N * Kb * 4));
    const i32x4_t crs = raw_rsrc(codes, (uint32_t)((uint64_t)N * (uint32_t)(K >> 1)));
    // DMA lane mapping: instruction (group j, half hh) writes rows 8 hh + l / 8,
    // LDS chunk l % 8, which holds global chunk (l % 8) ^ ((row / 2) % 8)
    const int drow = lane >> 3;
    uint32_t dvoff[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int rw = 8 * hh + drow;
        const int q = (lane & 7) ^ ((rw >> 1) & 7);
        // the whole offset goes in voffset, which the buffer range check covers:
        // blocks past the end of the last row read as zero
        dvoff[hh] = (uint32_t)min(n0 + rw, N - 1) * (uint32_t)(K >> 1) + 32u * (uint32_t)(q >> 1) + 16u * (q & 1);
    }
    uint32_t qv[NG];
    float a_lo = 0.0f, a_hi = 0.0f;
    int g_lo = 0;
    auto phase_issue = [&](int p) {
        const int bw0 = p * P.PB + w * PBw;  // first block of the wave's range
        const uint32_t rkb = (uint32_t)arow * (uint32_t)Kb;
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int b = min(bw0 + (lane >> 4) + 4 * u, Kb - 1);
            qv[u] = DQ ? __builtin_amdgcn_raw_buffer_load_b8(qrs, rkb + (uint32_t)b, 0, 0)
                       : __builtin_amdgcn_raw_buffer_load_b32(ars, 4u * (rkb + (uint32_t)b), 0, 0);
        }
        if (DQ) {
            g_lo = (int)((rkb + (uint32_t)min(bw0, Kb - 1)) >> 8);
            a_lo = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ars, 4u * (uint32_t)g_lo, 0, 0));
            a_hi = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(ars, 4u * (uint32_t)min(g_lo + 1, ngroups - 1), 0, 0));
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                auto* dst = reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(
                    reinterpret_cast<uintptr_t>(cgs[j] + 2048 * w + 1024 * hh));
                gv_load_lds(crs, dst, 16, (int)(dvoff[hh] + 32u * (uint32_t)(bw0 + 4 * j)), 0, 0, 0);
            }
        }
    };
    auto phase_scales = [&](int p) {
        const int bw0 = p * P.PB + w * PBw;
        const uint32_t rkb = (uint32_t)arow * (uint32_t)Kb;
        // fl32(a2 / 255) is the fp64 product rounded, for every bf16-valued a2
        const float s_lo = (float)((double)a_lo * (1.0 / 255.0));
        const float s_hi = (float)((double)a_hi * (1.0 / 255.0));
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int jb = (lane >> 4) + 4 * u;
            const int b = bw0 + jb;
            const float step = (int)((rkb + (uint32_t)b) >> 8) == g_lo ? s_lo : s_hi;
            const float ah = DQ ? step * (float)qv[u] : __builtin_bit_cast(float, qv[u]);
            aw[(lane & 15) * (PBw + 4) + jb] = b < Kb ? ah : 0.0f;
        }
    };

    // ---- prologue: x, t, B and phase 0's scales and codes in flight, then the table
    stage_load(0);
    // t element (m, j) = i >> 7, i & 127 and B element (j, n) = i >> 4, i & 15 of
    // i = tid + 256 u; offsets past the operand read as zero
    const rsrc_t trs = make_rsrc(t, (uint32_t)(M * r * 2));
    uint16_t tv[8], bv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = tid + kGvThreads * u, m = i >> 7, j = i & 127;
        tv[u] = __builtin_amdgcn_raw_buffer_load_b16(trs, (m < M && j < r) ? 2u * (uint32_t)(m * r + j) : 0x80000000u,
                                                     0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = tid + kGvThreads * u, j = i >> 4, n = n0 + (i & 15);
        bv[u] = (j < r && n < N) ? B[(int64_t)j * N + n] : (uint16_t)0;
    }
    phase_issue(0);
    // code byte -> its two bf16 levels (element 2i, the high nibble, in the low
    // half); entry e, copy c at byte 256 e + 4 c.  16-byte chunk q = tid + 256 j
    // holds copies of entry 16 j + tid / 16, whose high nibble is j.
    {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t v = pack2<DT>(level<CB>(j), lo_level);
            *reinterpret_cast<u32x4_t*>(lut + 16 * (tid + 256 * j)) = u32x4_t{v, v, v, v};
        }
    }
    stage_store(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = tid + kGvThreads * u;
        reinterpret_cast<uint16_t*>(tl)[i] = tv[u];
        bl[(i & 15) * 128 + (i >> 4)] = bv[u];  // transposed: [n][j]
    }
    sync_lds_writes();

    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t lane4 = (uint32_t)lane << 2;
    const int xrow = ln < M ? ln : 0;  // A rows past M are don't-care
    const uint8_t* const xlane = xl + xrow * P.xs + 32 * lg;
    const int cswz = (ln >> 1) & 7;
    const int clane = 2048 * w + 128 * ln + 8 * (lg & 1);
    const float* const alane = aw + ln * (PBw + 4);

    for (int p = 0; p < P.phases; ++p) {
        if (p > 0) {
            __syncthreads();  // every wave is done with the previous phase's x
            stage_load(p);
            phase_issue(p);
            stage_store(p);
            sync_lds_writes();
        }
        phase_scales(p);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // the table is read by other lanes
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            wait_vm_at_most(2 * (NG - 1 - j));  // group j's two code loads have landed
            const f32x4_t ah = *reinterpret_cast<const f32x4_t*>(alane + 4 * j);
            const uint8_t* const xg = xlane + 128 * (w * PBw + 4 * j);
            // the group's four code words, then all 32 table reads, then the MFMAs: one
            // wave per SIMD, so the two dependent LDS round trips are paid once per group
            uint2 c[4];
#pragma unroll
            for (int h4 = 0; h4 < 4; ++h4)
                c[h4] = *reinterpret_cast<const uint2*>(cgs[j] + clane + 16 * ((2 * h4 + (lg >> 1)) ^ cswz));
            u32x4_t w0[4], w1[4];
#pragma unroll
            for (int h4 = 0; h4 < 4; ++h4)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const uint32_t sel = 0x0C0C0000u | ((4u + jj) << 8);
                    w0[h4][jj] = *reinterpret_cast<const uint32_t*>(lut + __builtin_amdgcn_perm(c[h4].x, lane4, sel));
                    w1[h4][jj] = *reinterpret_cast<const uint32_t*>(lut + __builtin_amdgcn_perm(c[h4].y, lane4, sel));
                }
#pragma unroll
            for (int h4 = 0; h4 < 4; ++h4) {
                const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xg + 128 * h4));
                const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xg + 128 * h4 + 16));
                f32x4_t part = mfma16<DT>(a0, __builtin_bit_cast(bf16x8_t, w0[h4]), f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
                part = mfma16<DT>(a1, __builtin_bit_cast(bf16x8_t, w1[h4]), part);
                // blocks past the row end have a_hat = 0; their x and codes are
                // staged values or zeros (finite), so they add exactly nothing
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[v] = __builtin_fmaf(ah[h4], part[v], acc[v]);
            }
        }
    }

    // LoRA term t B on the same accumulators: wave w takes j in [32 w, 32 w + 32)
    if (32 * w < r) {
        const bf16x8_t ta = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(tl + 2 * (xrow * 128 + 32 * w + 8 * lg)));
        const bf16x8_t tb = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(bl + ln * 128 + 32 * w + 8 * lg));
        acc = mfma16<DT>(ta, tb, acc);
    }

    // sum of the 4 waves' partial tiles and the bf16 store
    __syncthreads();
    float* red = reinterpret_cast<float*>(xl);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * lg + v;
        if (m < M) red[(w * 16 + m) * 16 + ln] = acc[v];
    }
    __syncthreads();
    if (tid < M * kGvRows) {
        const int m = tid >> 4, n = tid & 15;
        float s = red[(0 * 16 + m) * 16 + n] + red[(1 * 16 + m) * 16 + n];
        s += red[(2 * 16 + m) * 16 + n] + red[(3 * 16 + m) * 16 + n];
        if (n0 + n < N) {
            const uint32_t o = pack2<DT>(s, 0.0f);
            y[(int64_t)m * N + n0 + n] = (uint16_t)(o & 0xFFFFu);
        }
    }
}

}  // namespace

bool gemv_supported(int M, int N, int K, int r) {
    return M >= 1 && M <= kGemvMaxM && r <= 128 && (uint64_t)N * (uint64_t)K / 2 < (uint64_t(1) << 31);
}

qlora_status launch_gemv_fwd(const uint16_t* x, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                             int dt, const uint16_t* t, const uint16_t* B, uint16_t* y, int M, int N, int K, int r,
                             hipStream_t s) {
    if (!gemv_supported(M, N, K, r)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    GvPlan P;
    P.Kb = K / kBlock;
    P.tsh = 8;  // threads per staged x row: 256 / 2^ceil(log2 M)
    while ((1 << (8 - P.tsh)) < M) --P.tsh;
    // blocks per phase: a multiple of 16 such that x (rows padded by 16 B),
    // the codes (512 B per block) and the scale tables fit, and x staging
    // takes at most 16 chunks of 16 B per thread
    // blocks per phase PB = 16 NG, NG in {1, 2, 4}: the largest whose x rows
    // (padded by 16 B) fit the LDS left next to the codes, that takes at most
    // 16 chunks of 16 B per staging thread, and no larger than the row needs
    int ng = 4;
    while (ng > 1 && (M * (16 * ng * 128 + 16) > x_bytes(ng) || 16 * ng > (2 << P.tsh) || 8 * ng >= P.Kb)) ng /= 2;
    if (M * (16 * ng * 128 + 16) > x_bytes(ng)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    const int pb = 16 * ng;
    P.PB = pb;
    P.phases = (P.Kb + pb - 1) / pb;
    P.xs = pb * 128 + 16;
    const dim3 grid((unsigned)((N + kGvRows - 1) / kGvRows));
    const int nv = M == 1 ? 1 : M == 2 ? 2 : 4;
    // q8 == NULL: no double quantization, a2 holds one fp32 absmax per block
    with_cb_dt(cb, dt, [&](auto cbc, auto dtc) {
        constexpr int CB = decltype(cbc)::value, DT = decltype(dtc)::value;
#define QLORA_GEMV1(NV_, NG_, DQ_)                                                                                 \
    hipLaunchKernelGGL((nf4_gemv_kernel<NV_, NG_, DQ_, CB, DT>), grid, dim3(kGvThreads), 0, s, x, codes, q8, a2, t, B, \
                       y, M, N, K, r, P)
#define QLORA_GEMV(NV_, NG_)                                 \
    if (nv == NV_ && ng == NG_) {                            \
        if (q8) QLORA_GEMV1(NV_, NG_, true);                 \
        else QLORA_GEMV1(NV_, NG_, false);                   \
    }
        QLORA_GEMV(1, 1) QLORA_GEMV(1, 2) QLORA_GEMV(1, 4)
        QLORA_GEMV(2, 1) QLORA_GEMV(2, 2) QLORA_GEMV(2, 4)
        QLORA_GEMV(4, 1) QLORA_GEMV(4, 2) QLORA_GEMV(4, 4)
#undef QLORA_GEMV
#undef QLORA_GEMV1
    });
    return launch_status();
}

}  // namespace qlora
