// LoRA side-path kernels (MFMA v_mfma_f32_32x32x16_bf16, gfx950).
//
// The rank-r products of the layer ("bitsandbytes deep dive" 12.2:
// Y = XW + s X A B, A [Din, r], B [r, Dout], s = lora_alpha / r; the chain
// rule through the same graph for the backward, base frozen):
//   t  = s x A        [M, r]   (forward, kept for the backward)
//   u  = s dy B^T     [M, r]
//   dA = x^T u        [K, r]
//   dB = t^T dy       [r, N]
// The small operands (A, B, t, u) are read in their own layouts: a slice of
// each is staged in LDS and transposed, where needed, by the LDS reads.
// All four stream one large operand (x or dy) once and are HBM bound.  The
// reductions are split over the long dimension for parallelism; partial sums
// go to a workspace and are added in a fixed order (deterministic results).
#include "common.h"
#include "lora_plan.h"

namespace qlora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// 32x32x16 MFMA on operands of the compute dtype DT (bf16 or fp16 bit patterns).
template <int DT>
__device__ __forceinline__ f32x16_t mfma32(bf16x8 a, bf16x8 b, f32x16_t c) {
    if (DT == kDtF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
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

// Branch-free vector loads: each workgroup addresses the rows it reads through
// a buffer resource based at its first row (so offsets stay far below 2 GiB),
// and an offset is replaced by one past any buffer when the chunk lies outside
// the valid range, so the hardware returns zeros.  Straight-line loads keep
// the compiler's wait counts exact (a load under a branch makes it wait for
// everything in flight).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t buf_rsrc(const void* p, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 bload8(rsrc_t rs, bool ok, uint32_t elem) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? 2u * elem : 0x80000000u, 0, 0));
}

// Slices of a small row-major [R, r] operand (A [K, r], t or u [M, r]) live in
// LDS with rows of 32*TQ + 16 bf16: for every TQ the 16-lane groups of the
// transposed reads below then touch 16 distinct pairs of banks.
template <int TQ>
constexpr int slice_ld() { return 32 * TQ + 16; }

// Rows [row0, row0 + MAXROWS) of src (row stride r; rows at or past row_end and
// columns at or past r read as zero) into dst[row * slice_ld + col], all loads of
// a batch issued before its stores.  Every row is written, so steps padded past
// the end of a split multiply zeros.
template <int TQ, bool VEC, int MAXROWS>
__device__ __forceinline__ void stage_slice(uint16_t* __restrict__ dst, const uint16_t* __restrict__ src, int r,
                                            int row0, int row_end, int tid) {
    constexpr int kCh = 4 * TQ;  // 16-byte chunks per slice row
    constexpr int kLd = slice_ld<TQ>();
    constexpr int kPer = MAXROWS * kCh / 256;
    constexpr int kBatch = kPer < 16 ? kPer : 16;
    const rsrc_t rs = buf_rsrc(src + (int64_t)row0 * r, (uint64_t)(row_end - row0) * r * 2);
#pragma unroll
    for (int e0 = 0; e0 < kPer; e0 += kBatch) {
        bf16x8 v[kBatch];
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
            const int idx = tid + 256 * (e0 + e), row = idx / kCh, ch = idx % kCh;
            const bool ok = row0 + row < row_end;
            v[e] = VEC ? bload8(rs, ok && 8 * ch < r, (uint32_t)(row * r + 8 * ch))
                       : load8_row<false>(src, r, row0 + row, row_end, 8 * ch, r);
        }
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
            const int idx = tid + 256 * (e0 + e), row = idx / kCh, ch = idx % kCh;
            *reinterpret_cast<bf16x8*>(dst + row * kLd + 8 * ch) = v[e];
        }
    }
}

// MFMA operand of 8 consecutive slice rows row .. row+7 of column col16 + l32 % 16
// (col16 = the 16-column group of this half-wave), from two ds_read_b64_tr_b16:
// lane j of a 16-lane group receives element j of the 4-element row pieces
// addressed by lanes j%4 + 4e, which point at rows row + e, columns col16 + 4*(j%4).
__device__ __forceinline__ bf16x8 slice_col8(const uint16_t* __restrict__ slice, int ld, int row, int col16,
                                             int tj) {
    const uint16_t* p = slice + (row + (tj >> 2)) * ld + col16 + 4 * (tj & 3);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(reinterpret_cast<uintptr_t>(p)));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(reinterpret_cast<uintptr_t>(p + 4 * ld)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// part[split, m, j] = sum over c in the split's range of X[m, c] * Y[c, j]
// Y comes either as its rows' transpose Yt [r, C] (YNAT false: u = dy B^T with
// B [r, N]) or in its natural layout [C, r] (YNAT true: t = x A with A [K, r]).
// Workgroup = 4 waves = 4 tiles of 32 rows of M; TQ 32-wide tiles of j; a
// split covers `chunk` (a multiple of 64, at most kNtMaxChunk) columns of C.
// The split's slice of Y is staged in LDS once (Yt rows padded so that 16
// consecutive rows start 4 banks apart; natural rows as slice_ld, read with
// transposed loads); after that single barrier every wave streams its X rows
// through a 4-stage register ring (16 loads of 16 B per lane in flight) with
// no further synchronisation.  Lane half h takes columns c + 32h .. c + 32h +
// 31 of each 64-column step (the two halves of an MFMA's k slots may map to any
// reduction indices, as long as both operands agree).
constexpr int kNtMaxChunk = 512;  // columns of C per split
constexpr int kNtRing = 4;
static_assert(2 * kNtRing * 64 == kNtMaxChunk, "two ring passes cover a split");

template <int TQ, bool YNAT>
constexpr int nt_slice_elems() {
    return YNAT ? kNtMaxChunk * slice_ld<TQ>() : 32 * TQ * (kNtMaxChunk + 8);
}

template <int TQ, bool VEC, bool YNAT, int NST, int DT>
__global__ __launch_bounds__(256) void nt_partial_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Y,
                                                         float* __restrict__ part, int M, int C, int r, int chunk) {
    constexpr int kLdT = kNtMaxChunk + 8;  // Yt row (bf16)
    constexpr int kLdN = slice_ld<TQ>();   // natural row (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t ys[nt_slice_elems<TQ, YNAT>()];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int tj = l32 & 15, tg = l32 >> 4;
    const int m0 = blockIdx.x * 128 + wave * 32;
    const int split = blockIdx.y;
    const int c_begin = split * chunk;
    const int c_end = min(C, c_begin + chunk);

    // X ring first (the long-latency HBM stream), then the Y slice (L2).  Steps
    // past the split's end load zeros, so no load is conditional and the waits
    // for the ring are exact counts.
    const int bm0 = blockIdx.x * 128;
    const rsrc_t xrs = buf_rsrc(X + (int64_t)bm0 * C, (uint64_t)min(128, M - bm0) * C * 2);
    const int xrow = m0 + l32;
    bf16x8 xa[kNtRing][4];
    auto load_x = [&](int st, bf16x8 (&dst)[4]) {
        const int c = c_begin + 64 * st + 32 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (VEC)
                dst[i] = bload8(xrs, xrow < M && c + 8 * i < c_end, (uint32_t)((xrow - bm0) * C + c + 8 * i));
            else
                dst[i] = load8_row<false>(X, C, xrow, M, c + 8 * i, c_end);
        }
    };
#pragma unroll
    for (int st = 0; st < kNtRing; ++st) load_x(st, xa[st]);
    if (YNAT) {
        stage_slice<TQ, VEC, kNtMaxChunk>(ys, Y, r, c_begin, c_end, tid);
    } else {
        // Yt slice: 32*TQ rows x 64 chunks of 16 B (zeros past r or c_end)
        constexpr int kPer = 32 * TQ * (kNtMaxChunk / 8) / 256;
        constexpr int kBatch = kPer < 16 ? kPer : 16;
        const rsrc_t yrs = buf_rsrc(Y + c_begin, ((uint64_t)r * C - c_begin) * 2);
#pragma unroll
        for (int e0 = 0; e0 < kPer; e0 += kBatch) {
            bf16x8 yv[kBatch];
#pragma unroll
            for (int e = 0; e < kBatch; ++e) {
                const int idx = tid + 256 * (e0 + e), row = idx >> 6, ch = idx & 63;
                const int c = c_begin + 8 * ch;
                yv[e] = VEC ? bload8(yrs, row < r && c < c_end, (uint32_t)(row * C + 8 * ch))
                            : load8_row<false>(Y, C, row, r, c, c_end);
            }
#pragma unroll
            for (int e = 0; e < kBatch; ++e) {
                const int idx = tid + 256 * (e0 + e), row = idx >> 6, ch = idx & 63;
                *reinterpret_cast<bf16x8*>(&ys[row * kLdT + 8 * ch]) = yv[e];
            }
        }
    }
    __syncthreads();

    f32x16_t acc[TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][v] = 0.0f;
    // NST (4 or 8, at least the split's step count) steps, all unrolled: a
    // rolled loop copies the ring registers at its back edge, which waits for
    // the loads in flight, and an early exit lets the compiler sink the refills
    // behind it.
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        const int u = st % kNtRing;
        bf16x8 ca[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ca[i] = xa[u][i];
        if (st + kNtRing < NST) load_x(st + kNtRing, xa[u]);
        // keep the refill ahead of this step's MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < TQ; ++q) {
                const int c = 64 * st + 32 * h + 8 * i;  // slice column of the lane's k slots
                const bf16x8 yb = YNAT ? slice_col8(ys, kLdN, c, 32 * q + 16 * tg, tj)
                                       : *reinterpret_cast<const bf16x8*>(&ys[(32 * q + l32) * kLdT + c]);
                acc[q] = mfma32<DT>(ca[i], yb, acc[q]);
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

// Sum over splits of part[split * count + i] for the 64 outputs i of this
// workgroup: thread (o, g) adds splits g, g + 4, ... with 4 independent loads
// in flight, and the 4 groups' sums meet in LDS.  (A decode-size down-
// projection has up to 64 splits of a handful of outputs: a serial loop per
// output would wait for one load at a time.)
__device__ __forceinline__ float sum_splits(const float* __restrict__ part, int splits, int64_t count, int64_t i,
                                            bool ok) {
    __shared__ float red[4][64];
    const int o = threadIdx.x & 63, g = threadIdx.x >> 6;
    float acc = 0.0f;
    if (ok) {
        int p = g;
        for (; p + 12 < splits; p += 16) {
            const float v0 = part[(int64_t)p * count + i], v1 = part[(int64_t)(p + 4) * count + i];
            const float v2 = part[(int64_t)(p + 8) * count + i], v3 = part[(int64_t)(p + 12) * count + i];
            acc += (v0 + v1) + (v2 + v3);
        }
        for (; p < splits; p += 4) acc += part[(int64_t)p * count + i];
    }
    red[g][o] = acc;
    __syncthreads();
    return (red[0][o] + red[1][o]) + (red[2][o] + red[3][o]);
}

// out[m, j] = RNE_16( s * sum_split part[split, m, j] ) in the compute dtype DT;
// 256 threads per 64 outputs
template <int DT>
__global__ __launch_bounds__(256) void finalize_16_kernel(const float* __restrict__ part, int splits, int M, int r,
                                                            float s, uint16_t* __restrict__ out) {
    const int64_t count = (int64_t)M * r;
    const int64_t i = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
    const float v = sum_splits(part, splits, count, i, i < count);
    if (threadIdx.x < 64 && i < count) out[i] = (uint16_t)(pack2<DT>(s * v, 0.0f) & 0xFFFFu);
}

// part[split, d, j] = sum over m in the split's range of X[m, d] * S[m, j]
// (S [M, r] row-major: u or t).  Workgroup = 4 waves over 128 columns d of X
// (32 each); a split covers `chunk` (a multiple of 64, at most tn_max_chunk(r))
// rows m.  The split's slice of S is staged in LDS once and read with
// transposed loads as the MFMA B operand (8 consecutive m of one column j).
// The X rows stream through a 4-stage register ring into a double-buffered
// [64 m x 128 d] LDS tile, read back down its columns for the A operand (8
// consecutive m per lane), also with transposed loads.
constexpr int kTnRows = 64, kTnCols = 128, kTnLd = kTnCols + 32;  // 320-byte rows: conflict-free transposed reads
constexpr int kTnRing = 4;

template <int TQ, bool VEC, int DT>
__global__ __launch_bounds__(256) void tn_partial_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ S,
                                                         float* __restrict__ part, int M, int D, int r, int chunk) {
    constexpr int kTnMaxChunk = TQ <= 3 ? 512 : 256;  // = tn_max_chunk(r) for r in (32 (TQ-1), 32 TQ]
    constexpr int kSLd = slice_ld<TQ>();
    __shared__ __attribute__((aligned(16))) uint16_t tile[2][kTnRows * kTnLd];
    __shared__ __attribute__((aligned(16))) uint16_t ss[kTnMaxChunk * kSLd];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int tj = l32 & 15, tg = l32 >> 4;
    const int d0 = blockIdx.x * kTnCols;
    const int split = blockIdx.y;
    const int m_begin = split * chunk;
    const int m_end = min(M, m_begin + chunk);
    const int steps = (m_end - m_begin + kTnRows - 1) / kTnRows;
    // loader: row tid/4 of a 64-row step, columns 32*(tid%4) .. +31.  As in the
    // down-projection, the step loop runs a multiple of the ring depth (at most
    // kTnMaxChunk / 64 steps) and padded steps load zeros: no conditional loads.
    const int lr = tid >> 2, lc = (tid & 3) * 32;
    const rsrc_t xrs = buf_rsrc(X + (int64_t)m_begin * D, (uint64_t)(m_end - m_begin) * D * 2);
    bf16x8 xr[kTnRing][4];
    auto load_x = [&](int st, bf16x8 (&dst)[4]) {
        const int m = m_begin + kTnRows * st + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = d0 + lc + 8 * i;
            if (VEC)
                dst[i] = bload8(xrs, m < m_end && d < D, (uint32_t)((m - m_begin) * D + d));
            else
                dst[i] = load8_row<false>(X, D, m, m_end, d, D);
        }
    };
    auto store_x = [&](const bf16x8 (&src)[4], int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<bf16x8*>(&tile[buf][lr * kTnLd + lc + 8 * i]) = src[i];
    };
#pragma unroll
    for (int st = 0; st < kTnRing; ++st) load_x(st, xr[st]);
    stage_slice<TQ, VEC, kTnMaxChunk>(ss, S, r, m_begin, m_end, tid);
    store_x(xr[0], 0);
    __syncthreads();

    f32x16_t acc[TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][v] = 0.0f;
    // A operand = X^T: 8 consecutive m of column d = 32*wave + l32 of the tile
    for (int s0 = 0; s0 < steps; s0 += kTnRing) {
#pragma unroll
        for (int u = 0; u < kTnRing; ++u) {
            const int st = s0 + u;
            const int buf = u & 1;
            // next step's rows into the other buffer (read two steps ago), and
            // this ring slot's next load (its data went to LDS a step ago)
            store_x(xr[(u + 1) % kTnRing], buf ^ 1);
            load_x(st + kTnRing, xr[u]);
#pragma unroll
            for (int mc = 0; mc < kTnRows / 16; ++mc) {
                const int mr = mc * 16 + 8 * h;   // tile row of this lane's first k slot
                const bf16x8 a = slice_col8(tile[buf], kTnLd, mr, 32 * wave + 16 * tg, tj);
#pragma unroll
                for (int q = 0; q < TQ; ++q) {
                    const bf16x8 b = slice_col8(ss, kSLd, kTnRows * st + mr, 32 * q + 16 * tg, tj);
                    acc[q] = mfma32<DT>(a, b, acc[q]);
                }
            }
            __syncthreads();
        }
    }
    float* out = part + (int64_t)split * D * r;
#pragma unroll
    for (int q = 0; q < TQ; ++q) {
        const int j = 32 * q + l32;
        if (j >= r) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int d = d0 + 32 * wave + 8 * (v >> 2) + 4 * h + (v & 3);
            if (d < D) out[(int64_t)d * r + j] = acc[q][v];
        }
    }
}

// out[d * ld_d + j * ld_j] = sum_split part[split, d, j]   (fp32); 256 threads per 64 outputs
__global__ __launch_bounds__(256) void reduce_f32_kernel(const float* __restrict__ part, int splits, int D, int r,
                                                         int64_t ld_d, int64_t ld_j, float* __restrict__ out) {
    const int64_t count = (int64_t)D * r;
    const int64_t i = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
    const float v = sum_splits(part, splits, count, i, i < count);
    if (threadIdx.x < 64 && i < count) {
        const int64_t d = i / r, j = i - d * r;
        out[d * ld_d + j * ld_j] = v;
    }
}

// QA-LoRA pooled branch ("LoRA, QLoRA, QA-LoRA explained", sections 3-5):
// pool(x) A = x A~ with A~[k, j] = A[k / g, j] / g, exact in bf16 for g a power
// of two (a shift of the exponent) unless it underflows, so the plain kernels run on A~; the
// gradient of A sums each group of g rows of the gradient of A~:
// dA[i, j] = (1/g) sum_{q < g} dA~[g i + q, j], q ascending, in fp32.
template <int DT>
__global__ void expand_pooled_kernel(const uint16_t* __restrict__ A, int64_t count, int r, int g_log2,
                                     uint16_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    const int64_t k = i / r, j = i - k * r;
    const float v = h16_to_f32<DT>(A[(k >> g_log2) * r + j]) * __uint_as_float((uint32_t)(127 - g_log2) << 23);
    out[i] = (uint16_t)(pack2<DT>(v, 0.0f) & 0xFFFFu);
}

__global__ void pool_rows_kernel(const float* __restrict__ in, int64_t count, int r, int g, int g_log2,
                                 float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // output element [K/g, r]
    if (i >= count) return;
    const int64_t p = i / r, j = i - p * r;
    float acc = 0.0f;
    for (int q = 0; q < g; ++q) acc += in[(p * g + q) * r + j];
    out[i] = acc * __uint_as_float((uint32_t)(127 - g_log2) << 23);
}

__global__ void fill_f32_kernel(float* __restrict__ out, int64_t count, float v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) out[i] = v;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

qlora_status launch_nt(const uint16_t* X, const uint16_t* Y, bool y_natural, float* part, uint16_t* out,
                       float scale, int M, int C, int r, int dt, hipStream_t s) {
    const SplitPlan sp = plan_nt(M, C);
    const dim3 grid((unsigned)((M + 127) / 128), (unsigned)sp.splits);
    // vector path: 16-byte aligned rows, and one workgroup's rows (128 of X, r of
    // Yt) under 1 GiB of buffer offsets
    const bool vec = (C % 8 == 0) && (!y_natural || r % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15u) == 0) &&
                     ((reinterpret_cast<uintptr_t>(Y) & 15u) == 0) && (int64_t)C * 128 * 2 < (int64_t(1) << 30);
    const int tq = (r + 31) / 32;
    const bool short_split = sp.chunk <= 64 * kNtRing;
#define QL_NT(TQ, V, NAT)                                                                                          \
    if (short_split) hipLaunchKernelGGL((nt_partial_kernel<TQ, V, NAT, kNtRing, DT>), grid, dim3(256), 0, s, X, Y, part, \
                                        M, C, r, sp.chunk);                                                        \
    else hipLaunchKernelGGL((nt_partial_kernel<TQ, V, NAT, 2 * kNtRing, DT>), grid, dim3(256), 0, s, X, Y, part, M, C, \
                            r, sp.chunk);
#define QL_NT2(TQ)                                    \
    if (y_natural) {                                  \
        if (vec) { QL_NT(TQ, true, true) } else { QL_NT(TQ, false, true) } \
    } else {                                          \
        if (vec) { QL_NT(TQ, true, false) } else { QL_NT(TQ, false, false) } \
    }
    const int64_t count = (int64_t)M * r;
    with_dt(dt, [&](auto dtc) {
        constexpr int DT = decltype(dtc)::value;
        switch (tq) {
            case 1: QL_NT2(1) break;
            case 2: QL_NT2(2) break;
            case 3: QL_NT2(3) break;
            default: QL_NT2(4) break;
        }
        hipLaunchKernelGGL(finalize_16_kernel<DT>, dim3(blocks_for(count, 64)), dim3(256), 0, s, part, sp.splits, M, r,
                           scale, out);
    });
#undef QL_NT2
#undef QL_NT
    return launch_status();
}

qlora_status launch_tn(const uint16_t* X, const uint16_t* S, float* part, float* out, int M, int D, int r,
                       int64_t ld_d, int64_t ld_j, int dt, hipStream_t s) {
    const SplitPlan sp = plan_tn(M, D, r);
    const dim3 grid((unsigned)((D + kTnCols - 1) / kTnCols), (unsigned)sp.splits);
    // vector path: 16-byte aligned rows, and one split's rows of X under 1 GiB
    const bool vec = (D % 8 == 0) && (r % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15u) == 0) &&
                     ((reinterpret_cast<uintptr_t>(S) & 15u) == 0) && (int64_t)D * 512 * 2 < (int64_t(1) << 30);
    const int tq = (r + 31) / 32;
#define QL_TN(TQ)                                                                                                   \
    if (vec) hipLaunchKernelGGL((tn_partial_kernel<TQ, true, DT>), grid, dim3(256), 0, s, X, S, part, M, D, r, sp.chunk); \
    else hipLaunchKernelGGL((tn_partial_kernel<TQ, false, DT>), grid, dim3(256), 0, s, X, S, part, M, D, r, sp.chunk);
    with_dt(dt, [&](auto dtc) {
        constexpr int DT = decltype(dtc)::value;
        switch (tq) {
            case 1: QL_TN(1) break;
            case 2: QL_TN(2) break;
            case 3: QL_TN(3) break;
            default: QL_TN(4) break;
        }
    });
#undef QL_TN
    const int64_t count = (int64_t)D * r;
    hipLaunchKernelGGL(reduce_f32_kernel, dim3(blocks_for(count, 64)), dim3(256), 0, s, part, sp.splits, D, r, ld_d,
                       ld_j, out);
    return launch_status();
}

qlora_status launch_expand_pooled(const uint16_t* A, int K, int r, int g, int dt, uint16_t* out, hipStream_t s) {
    const int64_t count = (int64_t)K * r;
    const int g_log2 = __builtin_ctz((unsigned)g);
    with_dt(dt, [&](auto dtc) {
        constexpr int DT = decltype(dtc)::value;
        hipLaunchKernelGGL(expand_pooled_kernel<DT>, dim3(blocks_for(count, 256)), dim3(256), 0, s, A, count, r, g_log2,
                           out);
    });
    return launch_status();
}

qlora_status launch_pool_rows(const float* in, int K, int r, int g, float* out, hipStream_t s) {
    const int64_t count = (int64_t)(K / g) * r;
    const int g_log2 = __builtin_ctz((unsigned)g);
    hipLaunchKernelGGL(pool_rows_kernel, dim3(blocks_for(count, 256)), dim3(256), 0, s, in, count, r, g, g_log2, out);
    return launch_status();
}

qlora_status launch_fill(float* out, int64_t count, float v, hipStream_t s) {
    if (count > 0) hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(count, 256)), dim3(256), 0, s, out, count, v);
    return launch_status();
}

}  // namespace qlora
