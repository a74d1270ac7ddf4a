// Fused NF4-dequant GEMMs on MFMA (v_mfma_f32_32x32x16_bf16), gfx950.
//
// Forward  y[m,n]  = sum_k x[m,k] w_hat[n,k] + sum_j t[m,j] B[j,n]
// Backward dx[m,k] = sum_n dy[m,n] w_hat[n,k] + sum_j u[m,j] A[k,j]
// ("bitsandbytes deep dive" 8.6 and 12.4: 4-bit storage, 16-bit compute, the
// full-precision weight is restored tile by tile and never held in memory;
// the LoRA up-projection is the same product continued over r extra
// reduction steps with operands [t | B] resp. [u | A^T]).
//
// Both kernels: output tile 256 x 256, reduction step 64 (one NF4 block); the
// forward runs 256 lanes (4 waves, one per SIMD), the backward 512 (8 waves, two
// per SIMD).  The activation tile (256 rows x 64 of x, resp. of dy) is
// copied HBM -> LDS with direct buffer loads (16 B per lane, XOR-swizzled on
// the global side), double buffered.
//  * forward: wave w owns output columns [64w, 64w+64) over all 256 rows.
//    Each lane loads the packed codes, 8-bit scale and group scale it needs
//    two steps ahead, builds the block's 16-entry bf16 table one step ahead,
//    and expands its codes with v_perm_b32 straight into MFMA B operands: the
//    dequantized weight never touches LDS or HBM.
//  * backward: the reduction runs over n, across rows of the stored codes, so
//    the weight tile is dequantized cooperatively (lane = one row x one block)
//    into LDS in its natural [n][k] layout and read transposed by the MFMA
//    operand loads (ds_read_b64_tr_b16); waves form a 2 x 4 grid of 128 x 64
//    sub-tiles, and the dequantization VALU work is interleaved with the MFMAs.
// Accumulation is fp32; outputs are rounded to bf16 (nearest even).
#include "common.h"
#include "dequant_tile.h"

namespace qlora {
namespace {

constexpr int kT = 256;             // lanes per workgroup
constexpr int kTM = 256;            // output rows per tile
constexpr int kTN = 256;            // output columns per tile
constexpr int kTK = 64;             // reduction step
constexpr int kTileBytes = kTM * kTK * 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8, v); }

// 32x32x16 MFMA on operands of the compute dtype DT (bf16 or fp16 bit patterns).
template <int DT>
__device__ __forceinline__ f32x16_t mfma32(bf16x8 a, bf16x8 b, f32x16_t c) {
    if (DT == kDtF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Map a linear workgroup id to a tile id so that the workgroups placed on one
// XCD (ids are dealt round-robin over the 8 XCDs) get a contiguous run of
// tiles, i.e. share activation rows and weight columns in that XCD's L2.
__device__ __forceinline__ int xcd_tile(int bid, int total) {
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    return xcd * per + min(xcd, rem) + idx;
}

// ---- activation tile loader: rows [row0, row0+256) x cols [col0, col0+64) of a
// row-major bf16 matrix with leading dimension ld; rows >= nrows and columns >=
// ncols read as 0.  Lane tid covers row tid/8 + 32p, chunk tid%8 (p = 0..7).
// VEC: ld % 8 == 0 and the base is 16-byte aligned, so whole chunks can be read.
template <bool VEC>
__device__ __forceinline__ void load_tile(u32x4_t (&r)[8], const uint16_t* __restrict__ src, int64_t ld,
                                          int row0, int nrows, int col0, int ncols, int tid) {
    const int lr = tid >> 3, lc = tid & 7;
    const int col = col0 + lc * 8;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int row = row0 + lr + 32 * p;
        if (VEC) {
            if (row < nrows && col < ncols) {
                r[p] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)row * ld + col);
            } else {
                r[p] = u32x4_t{0u, 0u, 0u, 0u};
            }
        } else {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c0 = col + 2 * i;
                uint32_t lo = 0, hi = 0;
                if (row < nrows && c0 < ncols) lo = src[(int64_t)row * ld + c0];
                if (row < nrows && c0 + 1 < ncols) hi = src[(int64_t)row * ld + c0 + 1];
                w[i] = lo | (hi << 16);
            }
            r[p] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
    }
}

// Branch-free variant for full-width column steps (col0 + 64 <= ld): rows past
// nrows re-read the last row; the outputs they feed are never stored.
template <bool VEC>
__device__ __forceinline__ void load_tile_clamped(u32x4_t (&r)[8], const uint16_t* __restrict__ src, int64_t ld,
                                                  int row0, int nrows, int col0, int tid) {
    if (!VEC) {
        load_tile<false>(r, src, ld, row0, nrows, col0, (int)ld, tid);
        return;
    }
    const int lr = tid >> 3, lc = tid & 7;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int row = min(row0 + lr + 32 * p, nrows - 1);
        r[p] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)row * ld + col0 + lc * 8);
    }
}

// Forward-kernel tile layout: the XOR swizzle uses only row % 32, so the
// operand reads of rows R + 32 i (i = 0..3) differ by the immediate offset
// 4096 i; 8 or 16 consecutive rows still cover distinct banks.
__device__ __forceinline__ uint32_t ftile_off(int row, int chunk) {
    return (uint32_t)row * 128u + ((uint32_t)(chunk ^ ((row ^ (row >> 3)) & 3 ^ (row & 4))) << 4);
}

__device__ __forceinline__ void store_ftile(uint8_t* lds, const u32x4_t (&r)[8], int tid) {
    const int lr = tid >> 3, lc = tid & 7;
#pragma unroll
    for (int p = 0; p < 8; ++p) *reinterpret_cast<u32x4_t*>(lds + ftile_off(lr + 32 * p, lc)) = r[p];
}

// ---- direct HBM -> LDS tile loads (buffer_load_dwordx4 ... lds).  Lane l of
// an instruction writes 16 bytes at the instruction's LDS base + 16 l, so a
// wave fills 8 consecutive tile rows (1 KB); the swizzle is applied on the
// global side by choosing which 16-byte chunk each lane fetches.  Offsets past
// the buffer's byte range read as zero (rows past M): the range check applies
// to the lane's voffset, so every row offset is kept there.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ void raw_buffer_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) uint32_t* lds_ptr, int size,
                                    int voffset, int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r[0] = (int32_t)(uint32_t)(a & 0xffffffffu);
    r[1] = (int32_t)(uint32_t)(a >> 32);   // stride 0
    r[2] = (int32_t)bytes;                 // num_records in bytes
    r[3] = 0x00020000;                     // gfx9 buffer format word
    return r;
}

// One 256 x 64 bf16 tile of a row-major matrix (row stride ld elements) whose
// row 0 is the buffer base: columns [col0, col0 + 64) into `tile` (ftile
// layout).  voff0 = this lane's byte offset of tile row 8*wave + lane/8, its
// logical chunk, column 0.
// An LDS pointer as the address_space(3) pointer the LDS builtins take.  The
// address-space cast keeps the pointer's origin, so the compiler can tell a
// direct load's destination from the tiles a step reads and waits only where
// they may overlap; a round trip through an integer would hide the origin and
// make every LDS read wait for every direct load in flight.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* as_lds(const void* p) {
    return (__attribute__((address_space(3))) T*)(p);
}

__device__ __forceinline__ void load_tile_direct(i32x4_t rs, uint8_t* tile, uint32_t voff0, int wave, int col0,
                                                 int64_t ld) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        auto* dst = as_lds<uint32_t>(tile + (32 * j + 8 * wave) * 128);
        // the row offset goes in voffset: the buffer range check covers voffset
        // (not soffset), so rows past the end of the buffer read as zero
        raw_buffer_load_lds(rs, dst, 16, (int)(voff0 + (uint32_t)(32 * j * ld * 2)), (int)(col0 * 2), 0, 0);
    }
}

__device__ __forceinline__ void wait_direct_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// In the backward's main loop a step issues the next tile's direct loads and
// then, pinned after them by a scheduling barrier, exactly N ordinary loads of
// codes and scales for two steps ahead.  Loads complete in order, so at most N loads
// in flight means the tile has landed while those N stay outstanding.
constexpr int kAllButVmem = 0x078F;  // sched_barrier mask: every class but VMEM may cross
template <int N>
__device__ __forceinline__ void wait_direct_loads_behind() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that lets the last N LDS reads of the wave stay in flight
// (every earlier LDS access, reads and writes, has completed when it passes).
template <int N>
__device__ __forceinline__ void barrier_reads_in_flight() {
    asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ void store_tile(uint8_t* lds, const u32x4_t (&r)[8], int tid) {
    const int lr = tid >> 3, lc = tid & 7;
#pragma unroll
    for (int p = 0; p < 8; ++p) *reinterpret_cast<u32x4_t*>(lds + tile_off(lr + 32 * p, lc)) = r[p];
}

__device__ __forceinline__ bf16x8 lds_operand(const uint8_t* lds, int row, int chunk) {
    return *reinterpret_cast<const bf16x8*>(lds + tile_off(row, chunk));
}

// 8 bf16 from a strided column: src[(j0 + i) * ld + col], i = 0..7, zero when
// j0 + i >= jmax or col is out of range.
__device__ __forceinline__ bf16x8 gather8(const uint16_t* __restrict__ src, int64_t ld, int j0, int jmax, int col,
                                         bool col_ok) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ja = j0 + 2 * i, jb = ja + 1;
        const uint32_t lo = (col_ok && ja < jmax) ? src[(int64_t)ja * ld + col] : 0u;
        const uint32_t hi = (col_ok && jb < jmax) ? src[(int64_t)jb * ld + col] : 0u;
        w[i] = lo | (hi << 16);
    }
    return as_bf16x8(u32x4_t{w[0], w[1], w[2], w[3]});
}

// 8 contiguous bf16 src[row * ld + j0 .. +7], zero past jmax or an invalid row.
__device__ __forceinline__ bf16x8 row8(const uint16_t* __restrict__ src, int64_t ld, int row, bool row_ok, int j0,
                                      int jmax) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ja = j0 + 2 * i, jb = ja + 1;
        const uint32_t lo = (row_ok && ja < jmax) ? src[(int64_t)row * ld + ja] : 0u;
        const uint32_t hi = (row_ok && jb < jmax) ? src[(int64_t)row * ld + jb] : 0u;
        w[i] = lo | (hi << 16);
    }
    return as_bf16x8(u32x4_t{w[0], w[1], w[2], w[3]});
}

// Store an fp32 accumulator tile (this wave: 8 x 32-row tiles times 2 x 32-col
// tiles) as bf16.  Lane l of a 32x32 tile holds column l%32 and rows
// 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
template <int DT>
__device__ __forceinline__ void store_acc(uint16_t* __restrict__ out, int64_t ld, const f32x16_t (&acc)[8][2],
                                          int m0, int M, const int (&col)[2], const bool (&col_ok)[2], int h) {
    const int l32 = threadIdx.x & 31;
    (void)l32;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (!col_ok[t]) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (m < M) out[(int64_t)m * ld + col[t]] = (uint16_t)(pack2<DT>(acc[i][t][v], 0.0f) & 0xFFFFu);
            }
        }
    }
}

// ------------------------------------------------------------------ forward
// Wave w owns output columns [64w, 64w + 64) of the 256 x 256 tile, all 256
// rows (8 x 2 MFMA tiles).  The x tile (256 x 64) arrives by direct loads one
// step ahead; every wave reads all of it (8 operand reads per 16 MFMAs).
// Codes arrive four blocks (a super-step) at a time: the tile's 256 rows of
// codes x 128 B are copied HBM -> LDS by direct loads, 8 full rows per 1 KB
// instruction, a super-step ahead (16-byte chunks XOR-swizzled by row), and
// thread t computes the block scales a_hat of tile row t for those blocks
// into a small LDS table.  The dequantized weight never touches LDS: lane
// (h, l32) reads, for its two columns, the 16 code bytes of k = 32h .. 32h +
// 31 of the block and the block's a_hat, builds each column's 16-entry bf16
// table and expands 8 codes at a time into the MFMA B operand just before use,
// interleaved with the MFMAs of the previous chunk.
constexpr int kSup = 2;                                     // blocks per super-step
constexpr int kCodeTileBytes = kTN * kSup * kBlock / 2;     // 256 rows x 64 B

template <bool Q8DW, bool DQ, int CB, int DT>
__global__ __launch_bounds__(kT, 1) void nf4_gemm_fwd_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ q8,
    const float* __restrict__ a2, const uint16_t* __restrict__ t, const uint16_t* __restrict__ Bl,
    uint16_t* __restrict__ y, int M, int N, int K, int r, int tiles_m, int tiles_n) {
    // Separate objects, so that the compiler's tracking of direct loads never
    // makes a read of one buffer wait for the loads into another.  x tiles:
    // a 3-deep ring (tile ks in xt[ks % 3]); code tiles and scale tables: one
    // per super-step, 3 deep (super-step S in cds[S % 3], ahs[S % 3]).
    __shared__ __attribute__((aligned(16))) uint8_t xt0[kTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t xt1[kTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t xt2[kTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t cds0[kCodeTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t cds1[kCodeTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t cds2[kCodeTileBytes];
    __shared__ __attribute__((aligned(16))) float ahs0[kTN * kSup];
    __shared__ __attribute__((aligned(16))) float ahs1[kTN * kSup];
    __shared__ __attribute__((aligned(16))) float ahs2[kTN * kSup];
    uint8_t* const xts[3] = {xt0, xt1, xt2};
    uint8_t* const cdss[3] = {cds0, cds1, cds2};
    float* const ahss[3] = {ahs0, ahs1, ahs2};

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    const int mt = tile / tiles_n, nt = tile - mt * tiles_n;
    const int m0 = mt * kTM, n0 = nt * kTN;
    const int KB = K / kTK;
    const int NS = (KB + kSup - 1) / kSup;
    const int wv = __builtin_amdgcn_readfirstlane(wave);

    int col[2], crl[2];  // global column; row of the code tile (column within the tile)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        crl[u] = wave * 64 + u * 32 + l32;
        col[u] = n0 + crl[u];
    }
    // A operand offsets: rows 32 i + l32, chunk 4h + c; row tiles are immediate offsets
    uint32_t offA[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) offA[c] = ftile_off(l32, 4 * h + c);

    f32x16_t acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][u][v] = 0.0f;

    // ---- code tiles: 256 rows x 64 B (2 blocks).  Instruction i of wave w fills
    // rows 16 (4w + i) .. +15: lane l takes row 16 (4w + i) + l / 4 and LDS chunk
    // l % 4, which holds that row's 16-byte chunk (l % 4) ^ ((row / 2) % 4)
    // (block chunk / 2, half chunk % 2).  Rows past N repeat row N - 1 (never
    // stored); the whole offset is in voffset, so blocks past the end of the
    // last row read as zero.
    const uint32_t half_k = (uint32_t)K >> 1;
    const i32x4_t crs = buffer_rsrc(codes, (uint32_t)((uint64_t)N * half_k));
    uint32_t cvoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * (4 * wv + i) + (lane >> 2);
        const int q = (lane & 3) ^ ((row >> 1) & 3);
        cvoff[i] = (uint32_t)min(n0 + row, N - 1) * half_k + 32u * (uint32_t)(q >> 1) + 16u * (uint32_t)(q & 1);
    }
    auto load_codes = [&](uint8_t* dst, int S) __attribute__((always_inline)) {
        const uint32_t boff = 32u * (uint32_t)(kSup * S);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            auto* d = reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(
                reinterpret_cast<uintptr_t>(dst + 1024 * (4 * wv + i)));
            raw_buffer_load_lds(crs, d, 16, (int)(cvoff[i] + boff), 0, 0, 0);
        }
    };
    // ---- block scales: thread tid, tile row tid, the 2 blocks of a super-step.
    // With an even block count per row both blocks have an even-odd flat index
    // pair, so they lie in one group of 256 blocks; with an odd count the pair
    // can straddle a group boundary and each block takes its own group's scale.
    // Without double quantization a2 holds the blocks' fp32 absmax itself.
    const int srow = min(n0 + tid, N - 1);
    const int64_t sblk = (int64_t)srow * KB;
    struct Sc {
        uint32_t q;  // 8-bit scale codes of the 2 blocks, block j in byte j (DQ off: block 0's scale bits)
        float g;     // second-level scale of block 0's group (DQ off: block 1's scale)
        float g1;    // second-level scale of block 1's group (odd block counts only)
    };
    // loads per load_scales call, all issued after the step's x tile
    constexpr int kScaleLoads = DQ ? (Q8DW ? 2 : 4) : (Q8DW ? 1 : 2);
    auto load_scales = [&](int S, Sc& sc) __attribute__((always_inline)) {
        const int b0 = kSup * S;
        if (!DQ) {
            if (Q8DW) {  // blocks per row even: the 2 scales are one aligned 8-byte pair
                const f32x2_t v = *reinterpret_cast<const f32x2_t*>(a2 + sblk + b0);
                sc.q = __builtin_bit_cast(uint32_t, v[0]);
                sc.g = v[1];
            } else {
                sc.q = __builtin_bit_cast(uint32_t, a2[sblk + b0]);
                sc.g = a2[sblk + min(b0 + 1, KB - 1)];
            }
            return;
        }
        if (Q8DW) {  // blocks per row even: the 2 codes are one aligned 16-bit word
            sc.q = *reinterpret_cast<const uint16_t*>(q8 + sblk + b0);
            sc.g = a2[(sblk + b0) >> 8];
            sc.g1 = sc.g;
        } else {
            const int64_t b1 = sblk + min(b0 + 1, KB - 1);
            sc.q = (uint32_t)q8[sblk + b0] | ((uint32_t)q8[b1] << 8);
            sc.g = a2[(sblk + b0) >> 8];
            sc.g1 = a2[b1 >> 8];
        }
    };
    auto make_scales = [&](const Sc& sc, float* dst, int S) __attribute__((always_inline)) {
        const int b0 = kSup * S;
        f32x2_t ah;
        if (DQ) {
            ah[0] = scale_step(sc.g) * (float)(sc.q & 0xFFu);
            ah[1] = b0 + 1 < KB ? scale_step(sc.g1) * (float)((sc.q >> 8) & 0xFFu) : 0.0f;
        } else {
            ah[0] = __builtin_bit_cast(float, sc.q);
            ah[1] = b0 + 1 < KB ? sc.g : 0.0f;
        }
        *reinterpret_cast<f32x2_t*>(dst + kSup * tid) = ah;
    };
    // this lane's 16 code bytes of column u at block j of a super-step
    auto read_codes = [&](const uint8_t* cd, int j, int u) __attribute__((always_inline)) {
        return *reinterpret_cast<const u32x4_t*>(cd + crl[u] * 64 + 16 * ((2 * j + h) ^ ((crl[u] >> 1) & 3)));
    };

    // x panel rows [m0, min(M, m0 + kTM)) as a buffer; lane's tile row 8*wave + lane/8, chunk
    // the panel's own rows only (at most kTM; the launcher checks kTM * K * 2 < 2^32): a range over all rows
    // to M could pass 4 GiB and wrap
    const i32x4_t xrs = buffer_rsrc(x + (int64_t)m0 * K, (uint32_t)((int64_t)min(M - m0, kTM) * K * 2));
    const int xrow = 8 * wv + (lane >> 3);
    const int xchunk = (lane & 7) ^ (((xrow ^ (xrow >> 3)) & 3) ^ (xrow & 4));
    const uint32_t xvoff = (uint32_t)(((int64_t)xrow * K + 8 * xchunk) * 2);

    // prologue: x tiles 0 and 1, super-steps 0 and 1's codes and scales, the
    // scales of super-step 2 in registers
    load_tile_direct(xrs, xt0, xvoff, wv, 0, K);
    load_tile_direct(xrs, xt1, xvoff, wv, min(1, KB - 1) * kTK, K);
    load_codes(cds0, 0);
    load_codes(cds1, min(1, NS - 1));
    Sc sc;
    load_scales(0, sc);
    make_scales(sc, ahs0, 0);
    load_scales(min(1, NS - 1), sc);
    make_scales(sc, ahs1, min(1, NS - 1));
    load_scales(min(2, NS - 1), sc);
    wait_direct_loads();
    __syncthreads();
    Nf4Tab T[2];
    u32x4_t cc[2];
    bf16x8 b[2][2];
    bf16x8 a[2][4];  // A operands by half chunk: row tiles 4 half .. 4 half + 3 of chunk c
    share_tabs(make_tab<CB, DT>(ahs0[kSup * crl[h]]), T[0], T[1]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        cc[u] = read_codes(cds0, 0, u);
        b[0][u] = as_bf16x8(deq8(T[u], cc[u][0]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) a[0][i] = *reinterpret_cast<const bf16x8*>(xt0 + offA[0] + 4096u * i);

    // One step ks = 2 S + j on x tile ks (xt[ks % 3]), in 8 half chunks: each
    // issues the next half chunk's 4 operand reads (the last one: the next
    // step's first, from tile ks + 1, which the previous barrier published),
    // then 8 MFMAs with the expansion of the next chunk's codes interleaved.
    // At its start the step requests x tile ks + 2 (into the buffer of tile
    // ks - 1, which every wave finished a barrier ago) and, at j = 0, super-step
    // S + 2's codes and the scales of S + 3; at its end tile ks + 2 must have
    // landed, and the barrier publishes it while the next step's first operand
    // reads are in flight.  At j = 0 the table of super-step S + 2 is written
    // from the scales loaded a super-step earlier.
    auto do_step = [&](int S, int j, int s) __attribute__((always_inline)) {
        const int ks = kSup * S + j;
        const int xr = (2 * s + j) % 3;  // ks % 3, as S = s (mod 3)
        const uint8_t* A = xts[xr];
        const uint8_t* A1 = xts[(xr + 1) % 3];
        uint8_t* A2 = xts[(xr + 2) % 3];
        load_tile_direct(xrs, A2, xvoff, wv, min(ks + 2, KB - 1) * kTK, K);
        if (j == 0) {
            __builtin_amdgcn_sched_barrier(kAllButVmem);  // the x tile's loads first
            load_codes(cdss[(s + 2) % 3], min(S + 2, NS - 1));
            make_scales(sc, ahss[(s + 2) % 3], min(S + 2, NS - 1));
            load_scales(min(S + 3, NS - 1), sc);
        }
        __builtin_amdgcn_sched_barrier(kAllButVmem);  // keep this step's loads in this order
        // step ks+1's codes and tables
        const uint8_t* cdN = j == 0 ? cdss[s] : cdss[(s + 1) % 3];
        const float* ahN = j == 0 ? ahss[s] : ahss[(s + 1) % 3];
        const int jn = j ^ 1;
        u32x4_t cn[2];
        Nf4Tab Tn[2], mine;
        uint32_t e[8];
#pragma unroll
        for (int u = 0; u < 2; ++u) cn[u] = read_codes(cdN, jn, u);
        const float ahn = ahN[kSup * crl[h] + jn];
#pragma unroll
        for (int hc = 0; hc < 8; ++hc) {
            const int c = hc >> 1, half = hc & 1, p = c & 1;
            if (hc < 7) {
                const int c1 = (hc + 1) >> 1, h1 = (hc + 1) & 1;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[half ^ 1][i] = *reinterpret_cast<const bf16x8*>(A + offA[c1] + 4096u * (4 * h1 + i));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) a[0][i] = *reinterpret_cast<const bf16x8*>(A1 + offA[0] + 4096u * i);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[4 * half + i][0] = mfma32<DT>(a[half][i], b[p][0], acc[4 * half + i][0]);
                acc[4 * half + i][1] = mfma32<DT>(a[half][i], b[p][1], acc[4 * half + i][1]);
            }
            if (half == 0) b[p ^ 1][0] = as_bf16x8(c < 3 ? deq8(T[0], cc[0][c + 1]) : deq8(Tn[0], cn[0][0]));
            else b[p ^ 1][1] = as_bf16x8(c < 3 ? deq8(T[1], cc[1][c + 1]) : deq8(Tn[1], cn[1][0]));
            // step ks+1's tables, spread over half chunks 2..4 (first used in 6)
            if (hc == 2 || hc == 3) {
#pragma unroll
                for (int q = 4 * (hc - 2); q < 4 * (hc - 2) + 4; ++q)
                    e[q] = pack2<DT>(ahn * level<CB>(2 * q), ahn * level<CB>(2 * q + 1));
#pragma unroll
                for (int q = 2 * (hc - 2); q < 2 * (hc - 2) + 2; ++q) {
                    mine.lo[q] = perm_b32(e[2 * q + 1], e[2 * q], 0x06040200u);
                    mine.hi[q] = perm_b32(e[2 * q + 1], e[2 * q], 0x07050301u);
                }
            }
            if (hc == 4) share_tabs(mine, Tn[0], Tn[1]);
            // 4 operand reads ahead, then each MFMA followed by up to 6 VALU;
            // nothing crosses into the next half chunk
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int m_ = 0; m_ < 8; ++m_) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // chunk 3 used b[1]; the expansion of step ks+1's chunk 0 is in b[0]
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            T[u] = Tn[u];
            cc[u] = cn[u];
        }
        // tile ks+2 must have landed (the codes and scales requested after it may
        // stay in flight); the 4 operand reads of the next step stay in flight
        // across the barrier, every earlier LDS access has completed.
        if (j == 0) wait_direct_loads_behind<4 + kScaleLoads>();
        else wait_direct_loads();
        barrier_reads_in_flight<4>();
    };
    auto do_super = [&](int S, int s) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kSup; ++j)
            if (Q8DW || kSup * S + j < KB) do_step(S, j, s);
    };
    for (int S = 0; S < NS; S += 3) {
        do_super(S, 0);
        if (S + 1 < NS) do_super(S + 1, 1);
        if (S + 2 < NS) do_super(S + 2, 2);
    }

    u32x4_t xr[8];
    // LoRA up-projection: r more reduction steps with A-operand t [M, r] and
    // B-operand B [r, N] (t already carries the alpha/r scale).  The t tile goes
    // to xt0; B's rows [j0, j0 + 64) x the tile's 256 columns are staged in LDS
    // in natural layout (rows 0-31 in xt1, 32-63 in xt2, 544-byte rows) and read
    // down their columns with ds_read_b64_tr_b16.
    const bool col_ok0 = col[0] < N, col_ok1 = col[1] < N;
    const bool tvec = (r % 8) == 0;   // t rows are whole 16-byte chunks
    const bool nvec = (N % 8) == 0;   // rows of B and y are whole 16-byte chunks
    constexpr int kBLd = 544;         // bytes per staged B row
    const int tj = l32 & 15, tg = l32 >> 4;
    for (int j0 = 0; j0 < r; j0 += kTK) {
        if (tvec) load_tile<true>(xr, t, r, m0, M, j0, r, tid);
        else load_tile<false>(xr, t, r, m0, M, j0, r, tid);
        {
            u32x4_t bv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int idx = tid + kT * e, row = idx >> 5, n = n0 + 8 * (idx & 31), j = j0 + row;
                if (nvec) {
                    bv[e] = (j < r && n < N) ? *reinterpret_cast<const u32x4_t*>(Bl + (int64_t)j * N + n)
                                             : u32x4_t{0u, 0u, 0u, 0u};
                } else {
                    uint32_t w[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t lo = (j < r && n + 2 * i < N) ? Bl[(int64_t)j * N + n + 2 * i] : 0u;
                        const uint32_t hi = (j < r && n + 2 * i + 1 < N) ? Bl[(int64_t)j * N + n + 2 * i + 1] : 0u;
                        w[i] = lo | (hi << 16);
                    }
                    bv[e] = u32x4_t{w[0], w[1], w[2], w[3]};
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int idx = tid + kT * e, row = idx >> 5;
                *reinterpret_cast<u32x4_t*>((row < 32 ? xt1 : xt2) + (row & 31) * kBLd + 16 * (idx & 31)) = bv[e];
            }
        }
        store_ftile(xt0, xr, tid);
        __syncthreads();
        const uint8_t* bhalf = h ? xt2 : xt1;   // B rows 32h .. 32h + 31 of this step
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16x8 bl[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint8_t* p = bhalf + (8 * c + (tj >> 2)) * kBLd + 2 * (wave * 64 + 32 * u + 16 * tg + 4 * (tj & 3));
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(reinterpret_cast<uintptr_t>(p)));
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(reinterpret_cast<uintptr_t>(p + 4 * kBLd)));
                bl[u] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bf16x8 av = *reinterpret_cast<const bf16x8*>(xt0 + offA[c] + 4096u * i);
                acc[i][0] = mfma32<DT>(av, bl[0], acc[i][0]);
                acc[i][1] = mfma32<DT>(av, bl[1], acc[i][1]);
            }
        }
        __syncthreads();
    }

    // y tile as bf16 through LDS, 128 rows at a time: lanes write their values
    // into a [128][256] staging area (rows 0-63 in xt0, 64-127 in xt1), then
    // each thread stores 16-byte row chunks
    if (!nvec) {
        const bool col_ok[2] = {col_ok0, col_ok1};
        store_acc<DT>(y, N, acc, m0, M, col, col_ok, h);
        return;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 4 * half + ii;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 32 * ii + 8 * (v >> 2) + 4 * h + (v & 3);
                    *reinterpret_cast<uint16_t*>((row < 64 ? xt0 : xt1) + (row & 63) * 512 + 2 * crl[u]) =
                        (uint16_t)(pack2<DT>(acc[i][u][v], 0.0f) & 0xFFFFu);
                }
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int idx = tid + kT * e, row = idx >> 5, ch = idx & 31;
            const int m = m0 + 128 * half + row, n = n0 + 8 * ch;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>((row < 64 ? xt0 : xt1) + (row & 63) * 512 + 16 * ch);
            if (m < M && n < N) *reinterpret_cast<u32x4_t*>(y + (int64_t)m * N + n) = v;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ backward dx
// dx[m, k] = sum_n dy[m, n] w_hat[n, k]: the reduction runs across rows of the
// stored codes.  Each step covers 64 rows n: lane (n = tid % 64, block =
// (tid / 64) % 4, half = tid / 256) expands 32 codes of one block of row n with
// the block's table into 4 x 16-byte stores of a natural [n][k] weight tile in
// LDS; the MFMA B operand (8
// consecutive n of one column k) is then read with ds_read_b64_tr_b16, which
// hands lane j of a 16-lane group element j of the 4-element row pieces
// addressed by 4 lanes (rows R..R+3 -> 4 consecutive n of column j).  The dy
// tile arrives by direct HBM -> LDS loads.  Waves are 2 x 4 (128 x 64 each,
// two per SIMD); the next step's codes arrive two steps ahead and are expanded
// while this step's MFMAs run.

// weight tile layout: 64 rows of 256 bf16 (512 B), 16-byte chunks XOR-swizzled
// by a 4-bit function of the row (conflict-free 16-byte row stores and
// transposed 8-byte reads)
__device__ __forceinline__ uint32_t wtile_off(int row, int col) {
    const int f = ((row & 3) << 2) | ((row >> 2) & 3);
    return (uint32_t)row * 512u + ((uint32_t)((col >> 3) ^ f) << 4) + ((uint32_t)(col & 7) << 1);
}

// Eight waves, two per SIMD: wave (wm, wk) = (wave / 4, wave % 4) owns rows
// [128 wm, 128 wm + 128) x columns [64 wk, 64 wk + 64) of the tile (4 x 2 MFMA
// tiles, 128 accumulators), so that one wave's LDS waits and barrier overlap the
// other's MFMAs (with four waves of 128 x 128, one per SIMD, the same kernel ran
// 3 % slower and its backward call 7 % slower).  Dequantization: thread (n, kb,
// half) expands 32 codes of row n, block kb of the step (both halves build the
// block's table).
constexpr int kT8 = 512;
__device__ __forceinline__ void load_tile_direct8(i32x4_t rs, uint8_t* tile, uint32_t voff0, int wave, int col0,
                                                  int64_t ld) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        auto* dst = as_lds<uint32_t>(tile + (64 * j + 8 * wave) * 128);
        raw_buffer_load_lds(rs, dst, 16, (int)(voff0 + (uint32_t)(64 * j * ld * 2)), (int)(col0 * 2), 0, 0);
    }
}

// 256 x 64 bf16 tile of a row-major matrix through registers by 512 threads (rows
// tid/8 + 64 p, 16-byte chunk tid % 8), zero outside [0, nrows) x [0, ncols).
template <bool VEC>
__device__ __forceinline__ void load_tile8(u32x4_t (&r)[4], const uint16_t* __restrict__ src, int64_t ld, int row0,
                                           int nrows, int col0, int ncols, int tid) {
    const int lr = tid >> 3, lc = tid & 7;
    const int col = col0 + lc * 8;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = row0 + lr + 64 * p;
        if (VEC) {
            r[p] = (row < nrows && col < ncols) ? *reinterpret_cast<const u32x4_t*>(src + (int64_t)row * ld + col)
                                                : u32x4_t{0u, 0u, 0u, 0u};
        } else {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c0 = col + 2 * i;
                uint32_t lo = 0, hi = 0;
                if (row < nrows && c0 < ncols) lo = src[(int64_t)row * ld + c0];
                if (row < nrows && c0 + 1 < ncols) hi = src[(int64_t)row * ld + c0 + 1];
                w[i] = lo | (hi << 16);
            }
            r[p] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
    }
}
__device__ __forceinline__ void store_ftile8(uint8_t* lds, const u32x4_t (&r)[4], int tid) {
    const int lr = tid >> 3, lc = tid & 7;
#pragma unroll
    for (int p = 0; p < 4; ++p) *reinterpret_cast<u32x4_t*>(lds + ftile_off(lr + 64 * p, lc)) = r[p];
}

template <bool DYVEC, bool DQ, int CB, int DT>
__global__ __launch_bounds__(kT8, 1) void nf4_gemm_bwd_dx_kernel(
    const uint16_t* __restrict__ dy, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ q8,
    const float* __restrict__ a2, const uint16_t* __restrict__ u_, const uint16_t* __restrict__ Al,
    uint16_t* __restrict__ dx, int M, int N, int K, int r, int tiles_m, int tiles_k) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kTileBytes];
    uint8_t* const ldsA0 = lds;                      // dy tiles (ftile layout), 2 buffers
    uint8_t* const ldsB0 = lds + 2 * kTileBytes;     // weight tiles (wtile layout), 2 buffers

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 2, wk = wave & 3;
    const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_k);
    const int mt = tile / tiles_k, kt = tile - mt * tiles_k;
    const int m0 = mt * kTM, k0 = kt * kTN;
    const int KB = K / kTK;
    const int NS = (N + kTK - 1) / kTK;

    // dequant role: row dn of the step, block dkb of the tile, half dh of the block's codes
    const int dn = tid & 63, dkb = (tid >> 6) & 3, dh = tid >> 8;
    const int dkcol = k0 + dkb * kTK;
    const bool dk_ok = dkcol < K;
    struct Step {
        u32x4_t c;
        uint32_t q;
        float g;
        bool ok;
    };
    const int dkc = dk_ok ? dkcol : K - kTK;
    auto load_step = [&](int ns, Step& S) {
        const int n = ns * kTK + dn;
        const int nc = min(n, N - 1);
        const uint8_t* p = codes + (int64_t)nc * (K / 2) + dkc / 2 + 16 * dh;
        S.c = *reinterpret_cast<const u32x4_t*>(p);
        const int64_t blk = (int64_t)nc * KB + dkc / kTK;
        S.ok = n < N && dk_ok;
        if (DQ) {
            S.q = q8[blk];
            S.g = a2[blk >> 8];
        } else {
            S.q = 0u;
            S.g = a2[blk];
        }
    };
    constexpr int kStepLoads = DQ ? 3 : 2;
    auto ahat_of = [&](const Step& S) {
        if (!DQ) {
            float g = S.g;
            asm volatile("" : "+v"(g));
            return S.ok ? g : 0.0f;
        }
        uint32_t q = S.q;
        asm volatile("" : "+v"(q));
        return scale_step(S.g) * (float)(S.ok ? q : 0u);
    };
    auto store_w = [&](uint8_t* Bt, const u32x4_t (&w)[4]) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
            *reinterpret_cast<u32x4_t*>(Bt + wtile_off(dn, dkb * kTK + 32 * dh + 8 * d)) = w[d];
    };

    uint32_t offA[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) offA[c] = ftile_off(l32, 2 * c + h);   // + 4096*(4wm + i)
    uint32_t offB[2][2];
    {
        const int j = l32 & 15, g = l32 >> 4;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                offB[u][s2] = wtile_off(8 * h + 4 * s2 + (j >> 2), 64 * wk + 32 * u + 16 * g + 4 * (j & 3));
    }
    auto read_ops = [&](const uint8_t* A, const uint8_t* Bt, int c, bf16x8 (&a)[4], bf16x8 (&b)[2]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const bf16x8*>(A + offA[c] + 4096u * (4 * wm + i));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds<s16x4_t>(Bt + offB[u][0] + 8192u * c));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds<s16x4_t>(Bt + offB[u][1] + 8192u * c));
            b[u] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][u][v] = 0.0f;

    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const i32x4_t drs = buffer_rsrc(dy + (int64_t)m0 * N, (uint32_t)((int64_t)min(M - m0, kTM) * N * 2));
    const int xrow = 8 * wv + (lane >> 3);
    const int xchunk = (lane & 7) ^ (((xrow ^ (xrow >> 3)) & 3) ^ (xrow & 4));
    const uint32_t dvoff = (uint32_t)(((int64_t)xrow * N + 8 * xchunk) * 2);
    u32x4_t ar[4];
    auto load_dy = [&](uint8_t* A, int ns) {
        if (DYVEC) {
            load_tile_direct8(drs, A, dvoff, wv, ns * kTK, N);
        } else {
            load_tile8<false>(ar, dy, N, m0, M, ns * kTK, N, tid);
            store_ftile8(A, ar, tid);
        }
    };

    Step cur, nxt;
    load_dy(ldsA0, 0);
    load_step(0, cur);
    load_step(min(1, NS - 1), nxt);
    {
        const Nf4Tab T = make_tab<CB, DT>(ahat_of(cur));
        u32x4_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) w[d] = deq8(T, cur.c[d]);
        store_w(ldsB0, w);
    }
    wait_direct_loads();
    __syncthreads();

    auto step = [&](int ns, const uint8_t* __restrict__ A, uint8_t* __restrict__ An, const uint8_t* __restrict__ Bt,
                    uint8_t* __restrict__ Bn) {
        bf16x8 a[2][4], b[2][2];
        read_ops(A, Bt, 0, a[0], b[0]);
        load_dy(An, min(ns + 1, NS - 1));
        __builtin_amdgcn_sched_barrier(kAllButVmem);
        Step nn;
        load_step(min(ns + 2, NS - 1), nn);
        u32x4_t w[4];
        const Nf4Tab T = make_tab<CB, DT>(ahat_of(nxt));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int p = c & 1;
            if (c < 3) read_ops(A, Bt, c + 1, a[p ^ 1], b[p ^ 1]);
            w[c] = deq8(T, nxt.c[c]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int u = 0; u < 2; ++u) acc[i][u] = mfma32<DT>(a[p][i], b[p][u], acc[i][u]);
            // no scheduling groups here: with two waves per SIMD the compiler's own order of
            // reads, expansion and MFMAs measured 4.5 % faster than pinned groups
        }
        store_w(Bn, w);
        cur = nxt;
        nxt = nn;
        if (DYVEC) wait_direct_loads_behind<kStepLoads>();
        __syncthreads();
    };
    for (int ns = 0; ns < NS; ++ns) {
        const int buf = ns & 1;
        step(ns, ldsA0 + buf * kTileBytes, ldsA0 + (buf ^ 1) * kTileBytes, ldsB0 + buf * kTileBytes,
             ldsB0 + (buf ^ 1) * kTileBytes);
    }

    // LoRA: r more reduction steps with A-operand u [M, r] (LDS) and B-operand A^T
    const bool rvec = (r % 8) == 0;
    for (int j0 = 0; j0 < r; j0 += kTK) {
        if (rvec) load_tile8<true>(ar, u_, r, m0, M, j0, r, tid);
        else load_tile8<false>(ar, u_, r, m0, M, j0, r, tid);
        store_ftile8(ldsA0, ar, tid);
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16x8 a[4], b[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(ldsA0 + offA[c] + 4096u * (4 * wm + i));
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int col = k0 + 64 * wk + 32 * u + l32;
                const int j = j0 + 16 * c + 8 * h;
                if (rvec) {
                    b[u] = (col < K && j < r) ? *reinterpret_cast<const bf16x8*>(Al + (int64_t)col * r + j)
                                              : as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
                } else {
                    b[u] = row8(Al, r, col, col < K, j, r);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int u = 0; u < 2; ++u) acc[i][u] = mfma32<DT>(a[i], b[u], acc[i][u]);
        }
        __syncthreads();
    }

    // dx tile as bf16 through LDS (256 x 256 x 2 B: all four tile buffers)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 128 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                *reinterpret_cast<uint16_t*>(lds + row * 512 + 2 * (64 * wk + 32 * u + l32)) =
                    (uint16_t)(pack2<DT>(acc[i][u][v], 0.0f) & 0xFFFFu);
            }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int idx = tid + kT8 * e, row = idx >> 5, ch = idx & 31;
        const int m = m0 + row, k = k0 + 8 * ch;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + row * 512 + 16 * ch);
        if (m < M && k < K) *reinterpret_cast<u32x4_t*>(dx + (int64_t)m * K + k) = v;
    }
}

}  // namespace

qlora_status launch_gemm_fwd(const uint16_t* x, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                             int dt, const uint16_t* t, const uint16_t* B, uint16_t* y, int M, int N, int K, int r,
                             hipStream_t s) {
    if (gemv_supported(M, N, K, r)) return launch_gemv_fwd(x, codes, q8, a2, cb, dt, t, B, y, M, N, K, r, s);
    const int tm = (M + kTM - 1) / kTM, tn = (N + kTN - 1) / kTN;
    // x is 16-byte aligned (checked by the caller) and K % 64 == 0, so every
    // 16-byte chunk of a row is aligned; a 256-row panel must fit a 32-bit offset
    if ((int64_t)kTM * K * 2 >= (int64_t(1) << 32)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    // code-tile offsets (including blocks past a row's end) must fit a 32-bit voffset
    if ((uint64_t)N * (uint64_t)K / 2 + 4096 >= (uint64_t(1) << 32)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    // q8 == NULL: no double quantization, a2 holds one fp32 absmax per block
    const bool even = (K / kTK) % kSup == 0;
    with_cb_dt(cb, dt, [&](auto cbc, auto dtc) {
        constexpr int CB = decltype(cbc)::value, DT = decltype(dtc)::value;
#define QL_FWD(Q8DW, DQ)                                                                                       \
    hipLaunchKernelGGL((nf4_gemm_fwd_kernel<Q8DW, DQ, CB, DT>), dim3(tm * tn), dim3(kT), 0, s, x, codes, q8, a2, t, \
                       B, y, M, N, K, r, tm, tn)
        if (q8) {
            if (even) QL_FWD(true, true); else QL_FWD(false, true);
        } else {
            if (even) QL_FWD(true, false); else QL_FWD(false, false);
        }
#undef QL_FWD
    });
    return launch_status();
}

qlora_status launch_gemm_bwd_dx(const uint16_t* dy, const uint8_t* codes, const uint8_t* q8, const float* a2,
                                int cb, int dt, const uint16_t* u, const uint16_t* A, uint16_t* dx, int M, int N, int K,
                                int r, hipStream_t s) {
    const int tm = (M + kTM - 1) / kTM, tk = (K + kTN - 1) / kTN;
    // Direct loads only when every step is 64 whole columns: a tile load puts the
    // column offset in soffset, which the buffer range check does not cover, so a
    // partial last step would read past row ends (the next row's head, or past the
    // end of dy for the panel's last row).  Other widths take the register path,
    // which zeroes every element past N.
    const bool vec = (N % kTK == 0) && ((reinterpret_cast<uintptr_t>(dy) & 15u) == 0) &&
                     ((int64_t)kTM * N * 2 < (int64_t(1) << 32));
    // q8 == NULL: no double quantization, a2 holds one fp32 absmax per block
    with_cb_dt(cb, dt, [&](auto cbc, auto dtc) {
        constexpr int CB = decltype(cbc)::value, DT = decltype(dtc)::value;
#define QL_BWD(V, DQ)                                                                                           \
    hipLaunchKernelGGL((nf4_gemm_bwd_dx_kernel<V, DQ, CB, DT>), dim3(tm * tk), dim3(kT8), 0, s, dy, codes, q8, a2, u, \
                       A, dx, M, N, K, r, tm, tk)
        if (q8) {
            if (vec) QL_BWD(true, true); else QL_BWD(false, true);
        } else {
            if (vec) QL_BWD(true, false); else QL_BWD(false, false);
        }
#undef QL_BWD
    });
    return launch_status();
}

}  // namespace qlora
