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
#include "split_sync.h"

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

// ---- split sums
// Every split of a contraction but the last publishes its fp32 partial tile
// (device-coherent stores, then the launch's tag); the workgroup of the last
// split, which the grid places after all others (row y = splits - 1), adds the
// published tiles in split order, its own last, and writes the outputs.  A
// partial tile is kept in the lanes' MFMA order (wave, 32-column group q, four
// 16-byte pieces per lane), so every store and load is a 1 KB run per wave.
template <int TQ>
constexpr uint32_t part_tile_floats() { return 4u * TQ * 64u * 16u; }

// Returns true in the workgroup that writes the outputs, with the totals in acc.
template <int TQ>
__device__ __forceinline__ bool split_sum(f32x16_t (&acc)[TQ], uint64_t* __restrict__ tags, float* __restrict__ part,
                                          int tiles, int tile, int split, int splits) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr uint32_t kFloats = part_tile_floats<TQ>();
    const uint64_t tag = launch_tag();
    uint64_t* const flags = tags + (size_t)tile * splits;
    auto off = [&](int q, int v4) { return (uint32_t)((((wave * TQ + q) * 4 + v4) * 64 + lane) * 16); };
    if (split < splits - 1) {
        const rsrc_t rs = buf_rsrc(part + ((size_t)split * tiles + tile) * kFloats, kFloats * 4);
#pragma unroll
        for (int q = 0; q < TQ; ++q)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const u32x4_t v = {__float_as_uint(acc[q][4 * v4]), __float_as_uint(acc[q][4 * v4 + 1]),
                                   __float_as_uint(acc[q][4 * v4 + 2]), __float_as_uint(acc[q][4 * v4 + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(v, rs, off(q, v4), 0, kCoherent);
            }
        publish_tag(flags + split, tag);
        return false;
    }
    const int P = splits - 1;
    const bool fail = wait_tags(flags, P, tag);
    // kRound splits' pieces in flight at once (64 VGPRs of loads per round at TQ = 2;
    // a round of all 8 splits measured no faster and needs 330 VGPRs)
    constexpr int kRound = TQ == 1 ? 8 : TQ == 2 ? 4 : 2;
    f32x16_t tot[TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) tot[q][v] = 0.0f;
    for (int s0 = 0; s0 < P; s0 += kRound) {
        u32x4_t g[kRound][TQ][4];
#pragma unroll
        for (int k = 0; k < kRound; ++k) {
            const int s = min(s0 + k, P - 1);
            const bool ok = s0 + k < P;
            const rsrc_t rs = buf_rsrc(part + ((size_t)s * tiles + tile) * kFloats, kFloats * 4);
#pragma unroll
            for (int q = 0; q < TQ; ++q)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4)
                    g[k][q][v4] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off(q, v4) : 0x80000000u, 0,
                                                                        kCoherent);
        }
#pragma unroll
        for (int k = 0; k < kRound; ++k)
#pragma unroll
            for (int q = 0; q < TQ; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (s0 + k < P) tot[q][v] += __uint_as_float(g[k][q][v >> 2][v & 3]);
    }
#pragma unroll
    for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][v] = fail ? __builtin_nanf("") : tot[q][v] + acc[q][v];
    return true;
}

// out[m, j] = RNE_16( s * sum over c of X[m, c] * Y[c, j] )
// Y comes either as its rows' transpose Yt [r, C] (YNAT false: u = dy B^T with
// B [r, N]) or in its natural layout [C, r] (YNAT true: t = x A with A [K, r]).
// Workgroup = 4 waves = 4 tiles of 32 rows of M; TQ 32-wide tiles of j; a
// split covers `chunk` (a multiple of 64, at most nt_max_chunk(r)) columns of C,
// NST >= chunk / 64 steps of 64.  The split's slice of Y (from L2) is requested
// first, then every X load of the split at once (steps past its end read
// zeros), so the slice's LDS stores wait only for the slice while the X stream
// is in flight; Yt rows are padded so that 16 consecutive rows start 4 banks
// apart, natural rows are read with transposed loads.  Lane half h takes
// columns c + 32h .. c + 32h + 31 of each 64-column step (the two halves of an
// MFMA's k slots may map to any reduction indices, as long as both operands
// agree).
template <int TQ, bool VEC, bool YNAT, int NST, int DT>
__device__ __forceinline__ void nt_body(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Y,
                                        uint64_t* __restrict__ tags, float* __restrict__ part,
                                        uint16_t* __restrict__ out, float scale, int M, int C, int r, int chunk,
                                        int tile, int split, int tiles, int splits) {
    static_assert(NST * 64 <= (TQ == 4 ? 256 : 512), "steps beyond nt_max_chunk");
    constexpr int kCols = NST * 64;                   // columns of C per split (at most)
    constexpr int kLdT = kCols + 8;                   // Yt row (bf16): 16 rows start 4 banks apart
    constexpr int kLdN = slice_ld<TQ>();              // natural row (bf16)
    constexpr int kCh = YNAT ? 4 * TQ : kCols / 8;    // 16-byte chunks per slice row
    constexpr int kYPer = NST * TQ;                   // slice loads per thread
    __shared__ __attribute__((aligned(16))) uint16_t ys[YNAT ? kCols * kLdN : 32 * TQ * kLdT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int tj = l32 & 15, tg = l32 >> 4;
    const int m0 = tile * 128 + wave * 32;
    const int c_begin = split * chunk;
    const int c_end = min(C, c_begin + chunk);

    bf16x8 yv[kYPer];
    if (YNAT) {
        const rsrc_t yrs = buf_rsrc(Y + (int64_t)c_begin * r, (uint64_t)(c_end - c_begin) * r * 2);
#pragma unroll
        for (int e = 0; e < kYPer; ++e) {
            const int idx = tid + 256 * e, row = idx / kCh, ch = idx % kCh;
            yv[e] = VEC ? bload8(yrs, c_begin + row < c_end && 8 * ch < r, (uint32_t)(row * r + 8 * ch))
                        : load8_row<false>(Y, r, c_begin + row, c_end, 8 * ch, r);
        }
    } else {
        const rsrc_t yrs = buf_rsrc(Y + c_begin, ((uint64_t)r * C - c_begin) * 2);
#pragma unroll
        for (int e = 0; e < kYPer; ++e) {
            const int idx = tid + 256 * e, row = idx / kCh, ch = idx % kCh;
            const int c = c_begin + 8 * ch;
            yv[e] = VEC ? bload8(yrs, row < r && c < c_end, (uint32_t)(row * C + 8 * ch))
                        : load8_row<false>(Y, C, row, r, c, c_end);
        }
    }
    const int bm0 = tile * 128;
    const rsrc_t xrs = buf_rsrc(X + (int64_t)bm0 * C, (uint64_t)min(128, M - bm0) * C * 2);
    const int xrow = m0 + l32;
    bf16x8 xa[NST][4];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        const int c = c_begin + 64 * st + 32 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (VEC)
                xa[st][i] = bload8(xrs, xrow < M && c + 8 * i < c_end, (uint32_t)((xrow - bm0) * C + c + 8 * i));
            else
                xa[st][i] = load8_row<false>(X, C, xrow, M, c + 8 * i, c_end);
        }
    }
#pragma unroll
    for (int e = 0; e < kYPer; ++e) {
        const int idx = tid + 256 * e, row = idx / kCh, ch = idx % kCh;
        *reinterpret_cast<bf16x8*>(&ys[row * (YNAT ? kLdN : kLdT) + 8 * ch]) = yv[e];
    }
    __syncthreads();

    f32x16_t acc[TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][v] = 0.0f;
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < TQ; ++q) {
                const int c = 64 * st + 32 * h + 8 * i;  // slice column of the lane's k slots
                const bf16x8 yb = YNAT ? slice_col8(ys, kLdN, c, 32 * q + 16 * tg, tj)
                                       : *reinterpret_cast<const bf16x8*>(&ys[(32 * q + l32) * kLdT + c]);
                acc[q] = mfma32<DT>(xa[st][i], yb, acc[q]);
            }
    if (!split_sum<TQ>(acc, tags, part, tiles, tile, split, splits)) return;
#pragma unroll
    for (int q = 0; q < TQ; ++q) {
        const int j = 32 * q + l32;
        if (j >= r) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = m0 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (m < M) out[(int64_t)m * r + j] = (uint16_t)(pack2<DT>(scale * acc[q][v], 0.0f) & 0xFFFFu);
        }
    }
}

template <int TQ, bool VEC, bool YNAT, int NST, int DT>
__global__ __launch_bounds__(256) void nt_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Y,
                                                 uint64_t* __restrict__ tags, float* __restrict__ part,
                                                 uint16_t* __restrict__ out, float scale, int M, int C, int r,
                                                 int chunk) {
    nt_body<TQ, VEC, YNAT, NST, DT>(X, Y, tags, part, out, scale, M, C, r, chunk, (int)blockIdx.x, (int)blockIdx.y,
                                    (int)gridDim.x, (int)gridDim.y);
}

// Up to kNtBatch such products of one rank and one operand layout in one grid (t of
// the layers that share their input, or u of the layers whose dy arrive together):
// problem i takes workgroups [first[i], first[i + 1]), numbered split by split, so
// that every waiting workgroup waits only for workgroups with lower ids, and each
// product's split-sum tail overlaps the streaming of the ones after it.
constexpr int kNtBatch = 8;
struct NtProb {
    const uint16_t* X;
    const uint16_t* Y;
    uint64_t* tags;
    float* part;
    uint16_t* out;
    float scale;
    int M, C, chunk, tiles, splits;
};
struct NtBatch {
    NtProb p[kNtBatch];
    int first[kNtBatch + 1];
    int n, r;
};

template <int TQ, bool VEC, bool YNAT, int NST, int DT>
__global__ __launch_bounds__(256) void ntb_kernel(const NtBatch bt) {
    const int b = blockIdx.x;
    int i = 0;
    while (i + 1 < bt.n && b >= bt.first[i + 1]) ++i;
    const NtProb& p = bt.p[i];
    const int c = b - bt.first[i];
    nt_body<TQ, VEC, YNAT, NST, DT>(p.X, p.Y, p.tags, p.part, p.out, p.scale, p.M, p.C, bt.r, p.chunk, c % p.tiles,
                                    c / p.tiles, p.tiles, p.splits);
}

// out[d * ld_d + j * ld_j] = sum over m of X[m, d] * S[m, j]   (fp32; S [M, r]
// row-major: u or t).  Workgroup = 4 waves over 128 columns d of X (32 each); a
// split covers `chunk` (a multiple of 64, at most tn_max_chunk(r)) rows m, NST
// >= chunk / 64 steps of 64.  The split's slice of S is requested first, then
// every X load of the split at once; the slice is read with transposed loads as
// the MFMA B operand (8 consecutive m of one column j).  X steps go through a
// double-buffered [64 m x 128 d] LDS tile, read back down its columns for the A
// operand (8 consecutive m per lane), also with transposed loads.
constexpr int kTnRows = 64, kTnCols = 128, kTnLd = kTnCols + 32;  // 320-byte rows: conflict-free transposed reads

// One contraction out[d * ld_d + j * ld_j] = sum_m X[m, d] S[m, j]: its operands, its
// split workspace (tags, partial tiles) and its grid of tiles x splits.
struct TnProb {
    const uint16_t* X;
    const uint16_t* S;
    uint64_t* tags;
    float* part;
    float* out;
    int M, D, r, chunk, tiles, splits;
    int64_t ld_d, ld_j;
};

template <int TQ, bool VEC, int NST, int DT>
__device__ __forceinline__ void tn_body(const TnProb& pr, int ti, int split) {
    const uint16_t* __restrict__ X = pr.X;
    const uint16_t* __restrict__ S = pr.S;
    const int M = pr.M, D = pr.D, r = pr.r, chunk = pr.chunk;
    constexpr int kTnMaxChunk = TQ <= 3 ? 512 : 256;  // = tn_max_chunk(r) for r in (32 (TQ-1), 32 TQ]
    static_assert(NST * kTnRows <= kTnMaxChunk, "steps beyond the slice");
    constexpr int kSLd = slice_ld<TQ>();
        constexpr int kCh = 4 * TQ;                       // 16-byte chunks per slice row
    // An 8-step split holds its slice of S in LDS in two phases of 256 rows (the second
    // stored after step 3), so that at r <= 64 a workgroup takes 80 KB and two share a CU.
    constexpr int kSH = NST > 4 ? 2 : 1;
    constexpr int kSRows = NST * kTnRows / kSH;       // slice rows held in LDS
    constexpr int kSPer = kSRows * kCh / 256;         // slice loads per thread and phase
    __shared__ __attribute__((aligned(16))) uint16_t tile[2][kTnRows * kTnLd];
    __shared__ __attribute__((aligned(16))) uint16_t ss[kSRows * kSLd];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int tj = l32 & 15, tg = l32 >> 4;
    const int d0 = ti * kTnCols;
    const int m_begin = split * chunk;
    const int m_end = min(M, m_begin + chunk);

        bf16x8 sv[kSH][kSPer];
    {
        const rsrc_t srs = buf_rsrc(S + (int64_t)m_begin * r, (uint64_t)(m_end - m_begin) * r * 2);
#pragma unroll
        for (int ph = 0; ph < kSH; ++ph)
#pragma unroll
            for (int e = 0; e < kSPer; ++e) {
                const int idx = tid + 256 * e, row = kSRows * ph + idx / kCh, ch = idx % kCh;
                sv[ph][e] = VEC ? bload8(srs, m_begin + row < m_end && 8 * ch < r, (uint32_t)(row * r + 8 * ch))
                                : load8_row<false>(S, r, m_begin + row, m_end, 8 * ch, r);
            }
    }
    // loader: row tid/4 of a 64-row step, columns 32*(tid%4) .. +31
    const int lr = tid >> 2, lc = (tid & 3) * 32;
    const rsrc_t xrs = buf_rsrc(X + (int64_t)m_begin * D, (uint64_t)(m_end - m_begin) * D * 2);
    bf16x8 xr[NST][4];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        const int m = m_begin + kTnRows * st + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = d0 + lc + 8 * i;
            if (VEC)
                xr[st][i] = bload8(xrs, m < m_end && d < D, (uint32_t)((m - m_begin) * D + d));
            else
                xr[st][i] = load8_row<false>(X, D, m, m_end, d, D);
        }
    }
    auto store_x = [&](const bf16x8 (&src)[4], int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<bf16x8*>(&tile[buf][lr * kTnLd + lc + 8 * i]) = src[i];
    };
    auto store_s = [&](int ph) {
#pragma unroll
        for (int e = 0; e < kSPer; ++e) {
            const int idx = tid + 256 * e, row = idx / kCh, ch = idx % kCh;
            *reinterpret_cast<bf16x8*>(&ss[row * kSLd + 8 * ch]) = sv[ph][e];
        }
    };
    store_s(0);
    store_x(xr[0], 0);
    __syncthreads();

    f32x16_t acc[TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][v] = 0.0f;
    // A operand = X^T: 8 consecutive m of column d = 32*wave + l32 of the tile.  Step
    // st + 1 goes into the buffer step st - 1 was read from (closed by the barrier).
#pragma unroll
        for (int st = 0; st < NST; ++st) {
        const int buf = st & 1;
        constexpr int kHalf = NST / kSH;
        if (kSH == 2 && st == kHalf) {     // every wave is past the first phase (the barrier above)
            store_s(1);
            __syncthreads();
        }
        if (st + 1 < NST) store_x(xr[st + 1], buf ^ 1);
        const int srow = kTnRows * (st % kHalf);   // this step's rows in the slice phase
#pragma unroll
        for (int mc = 0; mc < kTnRows / 16; ++mc) {
            const int mr = mc * 16 + 8 * h;   // tile row of this lane's first k slot
            const bf16x8 a = slice_col8(tile[buf], kTnLd, mr, 32 * wave + 16 * tg, tj);
#pragma unroll
            for (int q = 0; q < TQ; ++q) {
                const bf16x8 b = slice_col8(ss, kSLd, srow + mr, 32 * q + 16 * tg, tj);
                acc[q] = mfma32<DT>(a, b, acc[q]);
            }
        }
        if (st + 1 < NST) __syncthreads();
    }
    if (!split_sum<TQ>(acc, pr.tags, pr.part, pr.tiles, ti, split, pr.splits)) return;
#pragma unroll
    for (int q = 0; q < TQ; ++q) {
        const int j = 32 * q + l32;
        if (j >= r) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int d = d0 + 32 * wave + 8 * (v >> 2) + 4 * h + (v & 3);
            if (d < D) pr.out[(int64_t)d * pr.ld_d + (int64_t)j * pr.ld_j] = acc[q][v];
        }
    }
}

// two workgroups per CU where r <= 64 on the buffer-load path (80 KB of LDS, at most 256 VGPRs)
template <int TQ, bool VEC, int NST, int DT>
__global__ __launch_bounds__(256, TQ <= 2 && VEC ? 2 : 1) void tn_kernel(const TnProb pr) {
    tn_body<TQ, VEC, NST, DT>(pr, blockIdx.x, blockIdx.y);
}

// Two independent contractions in one grid (dA and dB of a layer): workgroups
// [0, tiles0 x splits0) run the first and the rest the second, each numbered split
// by split, so that the last split of every tile is dispatched after the tile's
// other splits.  The second contraction's workgroups take the CUs that the first
// one's finished splits leave while its last splits add up their tiles.
template <int TQ, bool VEC, int NST, int DT>
__global__ __launch_bounds__(256, TQ <= 2 && VEC ? 2 : 1) void tn2_kernel(const TnProb p0, const TnProb p1) {
    const int n0 = p0.tiles * p0.splits, b = blockIdx.x;
    if (b < n0) {
        tn_body<TQ, VEC, NST, DT>(p0, b % p0.tiles, b / p0.tiles);
    } else {
        const int c = b - n0;
        tn_body<TQ, VEC, NST, DT>(p1, c % p1.tiles, c / p1.tiles);
    }
}

// Up to kTnBatch independent contractions of one rank in one grid (the weight
// gradients dA, dB of several layers, deferred to the end of a backward pass):
// problem i takes workgroups [first[i], first[i + 1]), numbered split by split as
// in tn2_kernel, so every waiting workgroup waits only for workgroups with lower
// ids.  One launch streams the x and dy of all the layers back to back, and each
// contraction's split-sum tail overlaps the streaming of the ones after it.
constexpr int kTnBatch = 16;
struct TnBatch {
    TnProb p[kTnBatch];
    int first[kTnBatch + 1];
    int n;
};

template <int TQ, bool VEC, int NST, int DT>
__global__ __launch_bounds__(256, TQ <= 2 && VEC ? 2 : 1) void tnb_kernel(const TnBatch bt) {
    const int b = blockIdx.x;
    int i = 0;
    while (i + 1 < bt.n && b >= bt.first[i + 1]) ++i;
    const int c = b - bt.first[i];
    tn_body<TQ, VEC, NST, DT>(bt.p[i], c % bt.p[i].tiles, c / bt.p[i].tiles);
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

// Smallest supported step count (2, 4 or 8 steps of 64) that covers a split.
inline int steps_template(int chunk) { return chunk <= 128 ? 2 : chunk <= 256 ? 4 : 8; }

qlora_status launch_nt(const uint16_t* X, const uint16_t* Y, bool y_natural, void* ws, uint16_t* out, float scale,
                       int M, int C, int r, int dt, hipStream_t s) {
    const SplitPlan sp = plan_nt(M, C, r);
    const int tiles = (M + 127) / 128;
    const dim3 grid((unsigned)tiles, (unsigned)sp.splits);
    uint64_t* tags = static_cast<uint64_t*>(ws);
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + split_tags_bytes(tiles, sp));
    // vector path: 16-byte aligned rows, and one workgroup's rows (128 of X, r of
    // Yt) under 1 GiB of buffer offsets
    const bool vec = (C % 8 == 0) && (!y_natural || r % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15u) == 0) &&
                     ((reinterpret_cast<uintptr_t>(Y) & 15u) == 0) && (int64_t)C * 128 * 2 < (int64_t(1) << 30);
    const int tq = (r + 31) / 32, nst = steps_template(sp.chunk);
#define QL_NT(TQ, V, NAT, NST) \
    hipLaunchKernelGGL((nt_kernel<TQ, V, NAT, NST, DT>), grid, dim3(256), 0, s, X, Y, tags, part, out, scale, M, C, r, \
                       sp.chunk);
#define QL_NT1(TQ, V, NAT)                                  \
    if (nst == 2) { QL_NT(TQ, V, NAT, 2) }                  \
    else if (nst == 4) { QL_NT(TQ, V, NAT, 4) }             \
    else { QL_NT(TQ, V, NAT, (TQ == 4 ? 4 : 8)) }
#define QL_NT2(TQ)                                                               \
    if (y_natural) {                                                             \
        if (vec) { QL_NT1(TQ, true, true) } else { QL_NT1(TQ, false, true) }    \
    } else {                                                                     \
        if (vec) { QL_NT1(TQ, true, false) } else { QL_NT1(TQ, false, false) }  \
    }
    with_dt(dt, [&](auto dtc) {
        constexpr int DT = decltype(dtc)::value;
        switch (tq) {
            case 1: QL_NT2(1) break;
            case 2: QL_NT2(2) break;
            case 3: QL_NT2(3) break;
            default: QL_NT2(4) break;
        }
    });
#undef QL_NT2
#undef QL_NT1
#undef QL_NT
    return launch_status();
}

namespace {

// The contraction out[d * ld_d + j * ld_j] = sum_m X[M, D][m, d] S[M, r][m, j] with its
// split plan and workspace; vec: the buffer-load path applies (16-byte aligned rows, and
// one split's rows of X under 1 GiB).
TnProb tn_prob(const uint16_t* X, const uint16_t* S, void* ws, float* out, int M, int D, int r, int64_t ld_d,
               int64_t ld_j, bool& vec) {
    const SplitPlan sp = plan_tn(M, D, r);
    TnProb p{};
    p.X = X;
    p.S = S;
    p.tiles = (D + kTnCols - 1) / kTnCols;
    p.splits = sp.splits;
    p.chunk = sp.chunk;
    p.tags = static_cast<uint64_t*>(ws);
    p.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + split_tags_bytes(p.tiles, sp));
    p.out = out;
    p.M = M;
    p.D = D;
    p.r = r;
    p.ld_d = ld_d;
    p.ld_j = ld_j;
    vec = (D % 8 == 0) && (r % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15u) == 0) &&
          ((reinterpret_cast<uintptr_t>(S) & 15u) == 0) && (int64_t)D * 512 * 2 < (int64_t(1) << 30);
    return p;
}

// Calls go.template operator()<TQ, VEC, NST, DT>() for the instantiation that serves rank r,
// the load path and the longest split.
template <typename Go>
void tn_dispatch(int r, bool vec, int chunk, int dt, Go&& go) {
    const int tq = (r + 31) / 32, nst = steps_template(chunk);
#define QL_TN(TQ, V, NST) go.template operator()<TQ, V, NST, DT>();
#define QL_TN1(TQ, V)                       \
    if (nst == 2) { QL_TN(TQ, V, 2) }       \
    else if (nst == 4) { QL_TN(TQ, V, 4) }  \
    else { QL_TN(TQ, V, (TQ == 4 ? 4 : 8)) }
#define QL_TN2(TQ) \
    if (vec) { QL_TN1(TQ, true) } else { QL_TN1(TQ, false) }
    with_dt(dt, [&](auto dtc) {
        constexpr int DT = decltype(dtc)::value;
        switch (tq) {
            case 1: QL_TN2(1) break;
            case 2: QL_TN2(2) break;
            case 3: QL_TN2(3) break;
            default: QL_TN2(4) break;
        }
    });
#undef QL_TN2
#undef QL_TN1
#undef QL_TN
}

struct TnLaunch1 {
    const TnProb& p;
    dim3 grid;
    hipStream_t s;
    template <int TQ, bool V, int NST, int DT>
    void operator()() const {
        hipLaunchKernelGGL((tn_kernel<TQ, V, NST, DT>), grid, dim3(256), 0, s, p);
    }
};

struct TnLaunch2 {
    const TnProb& p0;
    const TnProb& p1;
    unsigned n;
    hipStream_t s;
    template <int TQ, bool V, int NST, int DT>
    void operator()() const {
        hipLaunchKernelGGL((tn2_kernel<TQ, V, NST, DT>), dim3(n), dim3(256), 0, s, p0, p1);
    }
};

}  // namespace

qlora_status launch_tn(const uint16_t* X, const uint16_t* S, void* ws, float* out, int M, int D, int r, int64_t ld_d,
                       int64_t ld_j, int dt, hipStream_t s) {
    bool vec = false;
    const TnProb p = tn_prob(X, S, ws, out, M, D, r, ld_d, ld_j, vec);
    const dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
        const TnLaunch1 go{p, grid, s};
    tn_dispatch(r, vec, p.chunk, dt, go);
    return launch_status();
}

qlora_status launch_tn2(const uint16_t* X0, const uint16_t* S0, void* ws0, float* out0, int D0, int64_t ld_d0,
                        int64_t ld_j0, const uint16_t* X1, const uint16_t* S1, void* ws1, float* out1, int D1,
                        int64_t ld_d1, int64_t ld_j1, int M, int r, int dt, hipStream_t s) {
    bool vec0 = false, vec1 = false;
    const TnProb p0 = tn_prob(X0, S0, ws0, out0, M, D0, r, ld_d0, ld_j0, vec0);
    const TnProb p1 = tn_prob(X1, S1, ws1, out1, M, D1, r, ld_d1, ld_j1, vec1);
    const int64_t n = (int64_t)p0.tiles * p0.splits + (int64_t)p1.tiles * p1.splits;
    if (n >= (int64_t(1) << 31)) return QLORA_ERR_UNSUPPORTED_SHAPE;
        const TnLaunch2 go{p0, p1, (unsigned)n, s};
    tn_dispatch(r, vec0 && vec1, std::max(p0.chunk, p1.chunk), dt, go);
    return launch_status();
}

qlora_status launch_nt_batch(const NtDesc* d, int count, bool y_natural, int r, int dt, hipStream_t s) {
    const int tq = (r + 31) / 32;
    for (int i0 = 0; i0 < count; i0 += kNtBatch) {
        const int n = std::min(kNtBatch, count - i0);
        NtBatch b{};
        b.n = n;
        b.r = r;
        bool vec = !y_natural || r % 8 == 0;
        int chunk = 64;
        int64_t total = 0;
        for (int i = 0; i < n; ++i) {
            const NtDesc& e = d[i0 + i];
            const SplitPlan sp = plan_nt(e.M, e.C, r);
            NtProb& p = b.p[i];
            p.X = e.X;
            p.Y = e.Y;
            p.tiles = (e.M + 127) / 128;
            p.splits = sp.splits;
            p.chunk = sp.chunk;
            p.tags = static_cast<uint64_t*>(e.ws);
            p.part = reinterpret_cast<float*>(static_cast<uint8_t*>(e.ws) + split_tags_bytes(p.tiles, sp));
            p.out = e.out;
            p.scale = e.scale;
            p.M = e.M;
            p.C = e.C;
            // the conditions of launch_nt's vector path, for every product of the launch
            vec = vec && (e.C % 8 == 0) && ((reinterpret_cast<uintptr_t>(e.X) & 15u) == 0) &&
                  ((reinterpret_cast<uintptr_t>(e.Y) & 15u) == 0) && (int64_t)e.C * 128 * 2 < (int64_t(1) << 30);
            chunk = std::max(chunk, sp.chunk);
            b.first[i] = (int)total;
            total += (int64_t)p.tiles * p.splits;
            if (total >= (int64_t(1) << 31)) return QLORA_ERR_UNSUPPORTED_SHAPE;
        }
        b.first[n] = (int)total;
        const int nst = steps_template(chunk);
#define QL_NTB(TQ, V, NAT, NST) \
    hipLaunchKernelGGL((ntb_kernel<TQ, V, NAT, NST, DT>), dim3((unsigned)total), dim3(256), 0, s, b);
#define QL_NTB1(TQ, V, NAT)                                  \
    if (nst == 2) { QL_NTB(TQ, V, NAT, 2) }                  \
    else if (nst == 4) { QL_NTB(TQ, V, NAT, 4) }             \
    else { QL_NTB(TQ, V, NAT, (TQ == 4 ? 4 : 8)) }
#define QL_NTB2(TQ)                                                                \
    if (y_natural) {                                                               \
        if (vec) { QL_NTB1(TQ, true, true) } else { QL_NTB1(TQ, false, true) }    \
    } else {                                                                       \
        if (vec) { QL_NTB1(TQ, true, false) } else { QL_NTB1(TQ, false, false) }  \
    }
        with_dt(dt, [&](auto dtc) {
            constexpr int DT = decltype(dtc)::value;
            switch (tq) {
                case 1: QL_NTB2(1) break;
                case 2: QL_NTB2(2) break;
                case 3: QL_NTB2(3) break;
                default: QL_NTB2(4) break;
            }
        });
#undef QL_NTB2
#undef QL_NTB1
#undef QL_NTB
        const qlora_status st = launch_status();
        if (st != QLORA_OK) return st;
    }
    return QLORA_OK;
}

namespace {
struct TnLaunchB {
    const TnBatch& b;
    unsigned n;
    hipStream_t s;
    template <int TQ, bool V, int NST, int DT>
    void operator()() const {
        hipLaunchKernelGGL((tnb_kernel<TQ, V, NST, DT>), dim3(n), dim3(256), 0, s, b);
    }
};
}  // namespace

qlora_status launch_tn_batch(const TnDesc* d, int count, int r, int dt, hipStream_t s) {
    for (int i0 = 0; i0 < count; i0 += kTnBatch) {
        const int n = std::min(kTnBatch, count - i0);
        TnBatch b{};
        b.n = n;
        bool vec = true;
        int chunk = 64;
        int64_t total = 0;
        for (int i = 0; i < n; ++i) {
            const TnDesc& e = d[i0 + i];
            bool v = false;
            b.p[i] = tn_prob(e.X, e.S, e.ws, e.out, e.M, e.D, r, e.ld_d, e.ld_j, v);
            vec = vec && v;
            chunk = std::max(chunk, b.p[i].chunk);
            b.first[i] = (int)total;
            total += (int64_t)b.p[i].tiles * b.p[i].splits;
            if (total >= (int64_t(1) << 31)) return QLORA_ERR_UNSUPPORTED_SHAPE;
        }
        b.first[n] = (int)total;
        const TnLaunchB go{b, (unsigned)total, s};
        tn_dispatch(r, vec, chunk, dt, go);
        const qlora_status st = launch_status();
        if (st != QLORA_OK) return st;
    }
    return QLORA_OK;
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
