// Decode-size forward of the NF4 linear layer (M <= 16 activation rows):
//   y[M, N] = x[M, K] W_hat^T + t[M, r] B[r, N],   t = bf16(s x A)
// ("bitsandbytes deep dive" 7.2-7.3 and 8.6: the frozen 4-bit base is
// dequantized on the fly inside the product; at decode batch sizes the layer
// is bound by the bytes of the packed codes, 0.5 B per weight).
//
// Work split.  A workgroup owns 16 weight rows over all of K.  Its NW waves
// give 4 NW "slots" (wave w, lane group g = lane / 16); slot s takes the
// blocks s, s + 4 NW, s + 8 NW, ... of the 16 rows, so every block of a row
// goes to one lane: lane (n = lane % 16, g) holds the block's 32 code bytes of
// row n in registers, builds that block's 16-entry table of dequantized values
// RNE_16(fl32(a_hat c_j)) (dequant_tile.h: the same values the tiled kernels
// and qlora_dequantize produce) and expands 8 codes at a time into the B
// operand of v_mfma_f32_16x16x32_{bf16,f16}.  The 32 reduction slots of one
// MFMA may map to any k as long as both operands agree: lane group g supplies
// weights 8i .. 8i + 7 of its own block, and the A operand lane (m, g) the
// matching 8 elements of x row m.  So each lane reads each code byte once,
// with two 16-byte loads per block, and builds one table per 64 weights.
//
// Memory.  Code loads go straight to registers through a ring of two blocks
// per lane (the next block is in flight while one is expanded).  x is staged in
// LDS in phases of PB = 4 NW NI blocks (the next phase's chunk is prefetched
// into registers while the current one is used), sized to the batch rows, so a
// workgroup needs 27-41 KB of LDS and several workgroups share a CU.
//
// LoRA.  t B runs on the same accumulators (r <= 128 as up to four 32-wide
// chunks, one per wave); the waves' partial tiles are added through LDS in a
// fixed order before the single bf16 rounding of y.  With FT (the layer call),
// t = bf16(s x A) is computed in the same launch: workgroups 0 .. P-1 first
// compute partial products of x A over their own range of K, store them in
// the workspace and publish each with a per-launch tag; every workgroup sums
// the P partials in a fixed order after its main loop.  The tag identifies the
// dispatch (the queue's packet index mixed with the queue address), so stale
// tags in the workspace from earlier launches never match and no reset is
// needed.  A producer publishes before it waits for anything, and producers
// have the lowest workgroup ids, which are dispatched first; the wait is
// bounded all the same, and a workgroup that gives up writes NaN instead of
// hanging.
#include "common.h"
#include "dequant_tile.h"
#include "split_sync.h"

namespace qlora {

// 64-bit index of the dispatch packet in its queue (monotonic per queue).
namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kGvRows = 16;               // weight rows per workgroup (the MFMA's n)
constexpr int kTLd = 128;                 // t and B^T staging: [16][128] bf16, zero past M / r
constexpr int kALd = 144;                 // producer A slice rows: 128 + 16 bf16 (distinct banks for the
                                          // transposed reads of 16 lanes)
constexpr int kASliceBytes = 64 * kALd * 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// An offset chosen by a per-lane condition, hidden from the optimizer: it would
// otherwise split a load of "cond ? offset : out of range" into a branch around two
// loads, and the compiler's wait counts after the join would no longer be exact.
__device__ __forceinline__ uint32_t opq(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// 16x16x32 MFMA on operands of the compute dtype DT (bf16 or fp16 bit patterns).
template <int DT>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    if (DT == kDtF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// MFMA B operand from a row-major LDS slice S[row][col] (row stride ld bf16):
// lane (j, g) of each 16-lane group receives S[row0 + e][col16 + j], e = 0..7,
// where row0 may differ per 16-lane group.  ds_read_b64_tr_b16 hands lane j of
// a 16-lane group element j % 4 of the 4-element row piece that lane 4 e + j % 4
// addresses; each lane addresses row row0 + j / 4, columns col16 + 4 (j % 4).
__device__ __forceinline__ u32x4_t slice_col8(const uint16_t* slice, int ld, int row0, int col16, int j) {
    const uint16_t* p = slice + (row0 + (j >> 2)) * ld + col16 + 4 * (j & 3);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(reinterpret_cast<uintptr_t>(p)));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(reinterpret_cast<uintptr_t>(p + 4 * ld)));
    return __builtin_bit_cast(u32x4_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

struct GvArgs {
    const uint16_t* x;      // [M, K]
    const uint8_t* codes;   // packed codes [N * K / 2]
    const uint8_t* q8;      // 8-bit block scale codes (double quantization) or unused
    const float* a2;        // group scales, or the fp32 block absmax without double quantization
    const uint16_t* A;      // [K, r] (FT: t computed in the launch)
    const uint16_t* t;      // [M, r] (given t)
    const uint16_t* B;      // [r, N]
    uint16_t* y;            // [M, N]
    uint16_t* t_out;        // [M, r] or null (FT)
    float* part;            // [P][M][r] partial x A (FT)
    uint64_t* flags;        // [P] publication tags (FT)
    float scale;            // alpha / r (FT)
    int M, N, K, r;
    int P;                  // producer workgroups (FT)
    int kp;                 // columns of K per producer: spp slices of 64 (FT)
        int spp;                // slices loaded per group: 1, 2 or 4 (FT)
    int phases;             // phased kernel: x staging phases
    int gw;                 // streaming kernel: tile workgroups
    int rg;                 // streaming kernel: 16-row groups per tile (1 or 2)
    int nq;                 // streaming kernel: steps per tile
    int kx;                 // streaming kernel: blocks per row that the steps read (x zero past K)
    int xrs;                // streaming kernel: bytes per staged x row (16 more than kx blocks)
    uint32_t xmagic;        // streaming kernel: ceil(2^32 / (K / 8)), c / (K / 8) as a high product
};

// Every slot takes two blocks (one per ring entry) per x phase of PB = 8 NW blocks.
constexpr int kGvNI = 2;

// Producer workgroup p of the layer call: the partial product x[:, K_p] A[K_p, :] over its
// range K_p of kp columns (slices of 64, loaded G at a time), stored to part[p] with
// device-scope atomic stores and published by one store of the launch tag.
// Lane (j, g) of wave w accumulates the 16-column tiles w and w + NW of t; A slices are
// staged in LDS and read transposed as the MFMA B operand, x fragments straight from
// memory as the A operand.
template <int NW, int DT, int G, bool AVEC>
__device__ __forceinline__ void gv_produce(const GvArgs& a, uint8_t* lds, uint64_t tag) {
    constexpr int NT = NW * 64;
    constexpr int AE = 1024 / NT;                // 16-byte slice chunks per thread and slice
    const int tid = threadIdx.x, lane = tid & 63;
    const bool act = tid < NT;                   // the layer call's extra wave only keeps the barriers
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int M = a.M, K = a.K, r = a.r;
    const int xrow = min(ln, M - 1);
    const int pid = blockIdx.x;
    const int kb0 = pid * a.kp, ke = min(K, kb0 + a.kp);
    const rsrc_t Ars = make_rsrc(a.A, (uint32_t)((uint64_t)K * r * 2));
    const rsrc_t xrs = make_rsrc(a.x, (uint32_t)((uint64_t)M * K * 2));
    uint16_t* const as = reinterpret_cast<uint16_t*>(lds);
    f32x4_t pacc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    for (int kg = kb0; kg < ke; kg += 64 * G) {  // a group of G slices, all loaded up front
        u32x4_t av[G][AE], xa[G][2];
#pragma unroll
        for (int sp = 0; sp < G; ++sp) {
            const int ks = kg + 64 * sp;
            const bool in = act && ks < ke;      // slices past the range read as zero
#pragma unroll
            for (int u = 0; u < AE; ++u) {
                const int i = tid + NT * u, rr = i >> 4, ch = i & 15;
                const uint32_t e0 = (uint32_t)((ks + rr) * r + 8 * ch);
                if (AVEC) {
                    av[sp][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                Ars, opq(in && 8 * ch < r ? 2u * e0 : 0x80000000u), 0, 0));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                            Ars, opq(in && 8 * ch + 2 * e < r ? 2u * (e0 + 2 * e) : 0x80000000u), 0, 0);
                        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                            Ars, opq(in && 8 * ch + 2 * e + 1 < r ? 2u * (e0 + 2 * e + 1) : 0x80000000u), 0, 0);
                        av[sp][u][e] = lo | (hi << 16);
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
                xa[sp][h] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                 xrs, opq(in ? 2u * (uint32_t)(xrow * K + ks + 32 * h + 8 * lg) : 0x80000000u), 0, 0));
        }
#pragma unroll
        for (int sp = 0; sp < G; ++sp) {
            __syncthreads();                     // the previous slice has been read
            if (act) {
#pragma unroll
                for (int u = 0; u < AE; ++u) {
                    const int i = tid + NT * u, rr = i >> 4, ch = i & 15;
                    *reinterpret_cast<u32x4_t*>(as + rr * kALd + 8 * ch) = av[sp][u];
                }
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int jt = w + NW * u;
                if (act && 16 * jt < r) {
                    pacc[u] = mfma16<DT>(xa[sp][0], slice_col8(as, kALd, 8 * lg, 16 * jt, ln), pacc[u]);
                    pacc[u] = mfma16<DT>(xa[sp][1], slice_col8(as, kALd, 32 + 8 * lg, 16 * jt, ln), pacc[u]);
                }
            }
        }
    }
    // lane (j, g) holds rows m = 4 g + v of column j.  Device-scope atomic stores are
    // coherent across the XCDs' L2 caches; once every wave's stores have completed, one
    // store of the tag publishes them.
    float* const pp = a.part + (size_t)pid * M * r;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int j = 16 * (w + NW * u) + ln;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * lg + v;
            if (act && m < M && j < r)
                __hip_atomic_store(pp + m * r + j, pacc[u][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    publish_tag(a.flags + pid, tag);
}

// Producer dispatch (workgroups 0 .. P-1 of the layer call).
template <int NW, int DT>
__device__ __forceinline__ void gv_produce_any(const GvArgs& a, uint8_t* lds) {
    const uint64_t tag = launch_tag();
    // A rows are 16-byte loads when r % 8 == 0, 2-byte loads otherwise
    if ((a.r & 7) == 0) {
        if (a.spp == 1) gv_produce<NW, DT, 1, true>(a, lds, tag);
        else if (a.spp == 2) gv_produce<NW, DT, 2, true>(a, lds, tag);
        else gv_produce<NW, DT, 4, true>(a, lds, tag);
    } else {
        if (a.spp == 1) gv_produce<NW, DT, 1, false>(a, lds, tag);
        else if (a.spp == 2) gv_produce<NW, DT, 2, false>(a, lds, tag);
        else gv_produce<NW, DT, 4, false>(a, lds, tag);
    }
}

// The helper wave of a layer-call workgroup: waits for the P <= 16 producers' tags
// (lane p polls producer p), adds each (m, j)'s partials in producer order and writes
// t = bf16(s x A) into tl ([16][128], zero past M / r), and t_out from the first
// workgroup.  A producer that never publishes (the wait is bounded) leaves NaN in t.
template <int DT>
__device__ __forceinline__ void gv_helper_t(const GvArgs& a, uint16_t* tl, bool first) {
    const int lane = threadIdx.x & 63;
    const uint64_t tag = launch_tag();
    bool fail = false;
    if (lane < a.P) {
        int spins = 0;
        while (__hip_atomic_load(a.flags + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag) {
            if (++spins > kSpinLimit) {
                fail = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    // every lane has seen its tag before any partial is loaded (the loop above
    // reconverges first); the payload loads stay behind the polls
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    fail = __builtin_amdgcn_ballot_w64(fail) != 0;
    const int M = a.M, r = a.r, MR = M * r, P = a.P;
#pragma unroll
    for (int i = 0; i < 16 * kTLd / 64; ++i) tl[64 * i + lane] = 0;   // t past M or r is zero in the operand
    // The partials: plain loads that read device-coherent memory (the producers wrote them
    // with device-scope stores), a round of 4 values x 16 producers per lane in flight at
    // once (atomic loads would go out one at a time), added in producer order.
    const rsrc_t prs = make_rsrc(a.part, (uint32_t)((size_t)P * MR * 4));
    for (int v0 = 0; v0 < MR; v0 += 256) {
        float g[4][16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int v = v0 + 64 * k + lane;
#pragma unroll
            for (int p = 0; p < 16; ++p)
                g[k][p] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(
                               prs, opq(v < MR && p < P ? 4u * (uint32_t)(p * MR + v) : 0x80000000u), 0, kCoherent));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int v = v0 + 64 * k + lane;
            if (v < MR) {
                float sum = 0.0f;
#pragma unroll
                for (int p = 0; p < 16; ++p)
                    if (p < P) sum += g[k][p];
                uint16_t out = (uint16_t)(pack2<DT>(a.scale * sum, 0.0f) & 0xFFFFu);
                if (fail) out = 0x7FC0u;          // NaN in bf16 and in fp16 alike
                const int m = v / r, j = v - m * r;
                tl[m * kTLd + j] = out;
                if (first && a.t_out) a.t_out[v] = out;
            }
        }
    }
}

template <int NW, int MC, bool DQ, int CB, int DT, bool FT>
__global__ __launch_bounds__(NW * 64 + (FT ? 64 : 0)) void nf4_gemv_kernel(GvArgs a) {
    constexpr int NT = NW * 64;                  // compute threads (with FT, one more helper wave follows)
    constexpr int S = 4 * NW;                    // slots
    constexpr int NI = kGvNI;                    // blocks per slot per phase (one per ring entry)
    constexpr int PB = S * NI;                   // blocks per phase
    constexpr int XS = PB * 128 + 16;            // LDS bytes per staged x row (padded: rows start 4 banks apart)
    constexpr int XR = MC * XS;
    constexpr int RED = NW * 16 * 16 * 4;        // the waves' partial tiles
    constexpr int R0 = XR > kASliceBytes ? (XR > RED ? XR : RED) : (kASliceBytes > RED ? kASliceBytes : RED);
    constexpr int XCH = PB * 8;                  // 16-byte x chunks per row and phase
    constexpr int XE = (MC * XCH + NT - 1) / NT; // x chunks per thread and phase
    constexpr int SQ = 4 * PB;                   // scale quads (4 consecutive blocks of a row) per phase
    static_assert(SQ <= NT, "one scale quad per thread");
    __shared__ __attribute__((aligned(16))) uint8_t r0[R0];
    __shared__ __attribute__((aligned(16))) float ahl[16 * PB];  // a_hat of the phase's blocks, [row][block]
    __shared__ __attribute__((aligned(16))) uint16_t tl[16 * kTLd];
    __shared__ __attribute__((aligned(16))) uint16_t bl[16 * kTLd];

    // with FT, workgroups 0 .. P-1 produce the partials of x A and do nothing else;
    // they have the lowest ids, so they are dispatched first and never wait
    if (FT && (int)blockIdx.x < a.P) {
        gv_produce_any<NW, DT>(a, r0);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = a.M, N = a.N, K = a.K, r = a.r;
    const int Kb = K / kBlock;
    const int wg = blockIdx.x - (FT ? a.P : 0);
    const int n0 = wg * kGvRows;

    // ---- helper wave (FT): wait for the producers' tags, add their partials of x A in
    // producer order and leave t = bf16(s x A) in LDS, while the compute waves run.  It
    // takes part in every workgroup barrier of the compute waves (one after the
    // prologue, two per x phase change, two in the epilogue).
    if (FT && w == NW) {
        __syncthreads();                          // prologue staging done
        gv_helper_t<DT>(a, tl, n0 == 0);
        for (int p = 0; p < a.phases; ++p) {
            __syncthreads();
            __syncthreads();
        }
        __syncthreads();                          // t ready for the LoRA term
        __syncthreads();                          // the reduction
        return;
    }

    const int ln = lane & 15, lg = lane >> 4;
    const int slot = 4 * w + lg;
    const int row = min(n0 + ln, N - 1);        // rows past N read row N - 1; their outputs are not stored
    const int xrow = min(ln, M - 1);            // A operand rows past M repeat row M - 1 (outputs not stored)

    const rsrc_t crs = make_rsrc(a.codes, (uint32_t)((uint64_t)N * (uint32_t)(K >> 1)));
    const rsrc_t qrs = make_rsrc(a.q8, DQ ? (uint32_t)((uint64_t)N * Kb) : 0u);
    const uint32_t ngroups = (uint32_t)(((uint64_t)N * Kb + kSuper - 1) / kSuper);
    const rsrc_t ars = make_rsrc(a.a2, DQ ? ngroups * 4u : (uint32_t)((uint64_t)N * Kb * 4));
    const rsrc_t xrs = make_rsrc(a.x, (uint32_t)((uint64_t)M * K * 2));
    const uint32_t rowb = (uint32_t)row * (uint32_t)(K >> 1);

    // ---- code ring: block q of this lane is S q + slot (phase q / NI); past the last
    // set of slots the loads are aimed out of range (they return zero, touch nothing)
    const int nq = (Kb + S - 1) / S;
    u32x4_t c0[2], c1[2];
    auto issue = [&](int q, int k) {
        const uint32_t bc = (uint32_t)min(S * q + slot, Kb - 1);  // a slot past the row end: a valid block
        const uint32_t off = opq(q < nq ? rowb + 32u * bc : 0x80000000u);
        c0[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, off, 0, 0));
        c1[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, off + 16u, 0, 0));
    };

    // ---- per phase: x chunks (chunk c of a rotated order: workgroups start at different
    // lines of the shared x) and the scales of the 16 rows' blocks, one quad of 4
    // consecutive blocks of a row per thread: q8 codes and group scales (or the fp32
    // absmax without double quantization) -> a_hat = fl32(fl32(a2 / 255) q8)
    constexpr int XT = XE * NT;
    const int xrot = (wg * 64) % XT;
    u32x4_t xv[XE];
    uint32_t sq[4], sg[2];
    const int qt = min(tid, SQ - 1);                          // threads past the quads load a copy of the last
    const int qr = qt / (PB / 4), qq = qt % (PB / 4);        // scale quad: row, quad within the phase
    const uint32_t qrowkb = (uint32_t)min(n0 + qr, N - 1) * (uint32_t)Kb;
    auto stage_load = [&](int p) {
#pragma unroll
        for (int e = 0; e < XE; ++e) {
            const int c = (tid + NT * e + xrot) % XT, m = c / XCH, col = p * PB * 64 + 8 * (c % XCH);
            const bool ok = m < M && col < K;            // columns past K stage as zero
            xv[e] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, opq(ok ? 2u * (uint32_t)(m * K + col) : 0x80000000u), 0, 0));
        }
        const int b0 = p * PB + 4 * qq;
        // blocks past the row end (also every block of a phase past the last) load out of
        // range; their scales are set to zero when stored
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t bb = qrowkb + (uint32_t)(b0 + e);
            if (DQ) sq[e] = __builtin_amdgcn_raw_buffer_load_b8(qrs, opq(b0 + e < Kb ? bb : 0x80000000u), 0, 0);
            else sq[e] = __builtin_amdgcn_raw_buffer_load_b32(ars, opq(b0 + e < Kb ? 4u * bb : 0x80000000u), 0, 0);
        }
        if (DQ) {
            const uint32_t bl0 = qrowkb + (uint32_t)b0, bl3 = qrowkb + (uint32_t)min(b0 + 3, Kb - 1);
            sg[0] = __builtin_amdgcn_raw_buffer_load_b32(ars, opq(b0 < Kb ? 4u * (bl0 >> 8) : 0x80000000u), 0, 0);
            sg[1] = __builtin_amdgcn_raw_buffer_load_b32(ars, opq(b0 < Kb ? 4u * (bl3 >> 8) : 0x80000000u), 0, 0);
        }
    };
    auto stage_store = [&](int p) {
#pragma unroll
        for (int e = 0; e < XE; ++e) {
            const int c = (tid + NT * e + xrot) % XT, m = c / XCH;
            if (m < M) *reinterpret_cast<u32x4_t*>(r0 + m * XS + 16 * (c % XCH)) = xv[e];
        }
        if (tid < SQ) {
            const int b0 = p * PB + 4 * qq;
            const uint32_t g0 = (qrowkb + (uint32_t)b0) >> 8;
            f32x4_t ah;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (DQ) {
                    const uint32_t g = (qrowkb + (uint32_t)min(b0 + e, Kb - 1)) >> 8;
                    ah[e] = scale_step(__builtin_bit_cast(float, g == g0 ? sg[0] : sg[1])) * (float)sq[e];
                } else {
                    ah[e] = __builtin_bit_cast(float, sq[e]);
                }
                ah[e] = b0 + e < Kb ? ah[e] : 0.0f;   // past the row end: all-zero weights (x is zero there)
            }
            *reinterpret_cast<f32x4_t*>(ahl + qr * PB + 4 * qq) = ah;
        }
    };

    // ---- prologue: the first phase's x and scales and B (and t when given), then the
    // first two blocks' codes, so that staging waits for none of the code loads.  Every
    // load is a buffer load whose offset is moved past the buffer when out of range (the
    // hardware returns zero), so the code stays straight and the waits stay exact.
    stage_load(0);
    constexpr int kPer = 16 * kTLd / NT;
    uint32_t bv[kPer], tv[kPer];
    {
        const rsrc_t brs = make_rsrc(a.B, (uint32_t)((uint64_t)r * N * 2));
        const rsrc_t trs = make_rsrc(a.t, FT ? 0u : (uint32_t)(M * r * 2));
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = tid + NT * u, j = i >> 4, n = i & 15;
            bv[u] = __builtin_amdgcn_raw_buffer_load_b16(
                brs, opq((j < r && n0 + n < N) ? 2u * (uint32_t)(j * N + n0 + n) : 0x80000000u), 0, 0);
            tv[u] = 0u;
            if (!FT) {
                const int m = i >> 7, jj = i & 127;
                tv[u] = __builtin_amdgcn_raw_buffer_load_b16(trs, opq((m < M && jj < r) ? 2u * (uint32_t)(m * r + jj)
                                                                                  : 0x80000000u), 0, 0);
            }
        }
    }
    issue(0, 0);
    issue(1, 1);
    stage_store(0);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int i = tid + NT * u;
        bl[(i & 15) * kTLd + (i >> 4)] = (uint16_t)bv[u];
        if (!FT) tl[i] = (uint16_t)tv[u];
    }
    __syncthreads();

    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint8_t* const xlane = r0 + xrow * XS;
    const float* const alane = ahl + ln * PB + slot;

    // One phase: the next phase's x and scales are requested first, then the slot's two
    // blocks run from ring entries 0 and 1, each followed by the request for the block
    // two ahead.  Blocks past the row end run with zero scales, so every phase has the
    // same straight-line body and the waits for the ring are exact counts.
    for (int p = 0; p < a.phases; ++p) {
        stage_load(p + 1);                        // past the last phase: out of range, returns zero
        __builtin_amdgcn_sched_barrier(0);        // issued here, ahead of this phase's blocks
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const Nf4Tab T = make_tab<CB, DT>(alane[S * k]);
            const uint8_t* xp = xlane + 128 * (slot + S * k);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const u32x4_t wv = deq8(T, s < 4 ? c0[k][s] : c1[k][s - 4]);
                const u32x4_t xf = *reinterpret_cast<const u32x4_t*>(xp + 16 * s);
                acc = mfma16<DT>(xf, wv, acc);
            }
            issue(2 * p + k + 2, k);
        }
        __syncthreads();                          // every wave is done with this phase's x and scales
        stage_store(p + 1);
        __syncthreads();
    }
    __syncthreads();                              // t ready (FT); every wave is done with r0

    // ---- LoRA term t B on the same accumulators: wave w takes j in [32 w, 32 w + 32)
    if (32 * w < r) {
        const u32x4_t ta = *reinterpret_cast<const u32x4_t*>(tl + ln * kTLd + 32 * w + 8 * lg);
        const u32x4_t tb = *reinterpret_cast<const u32x4_t*>(bl + ln * kTLd + 32 * w + 8 * lg);
        acc = mfma16<DT>(ta, tb, acc);
    }

    // ---- the waves' partial tiles, added in wave order, and the bf16 store
    float* const red = reinterpret_cast<float*>(r0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * lg + v;
        if (m < M) red[(w * 16 + m) * 16 + ln] = acc[v];
    }
    __syncthreads();
    if (tid < M * kGvRows) {
        const int m = tid >> 4, n = tid & 15;
        float s = red[m * 16 + n];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) s += red[(ww * 16 + m) * 16 + n];
        if (n0 + n < N) a.y[(int64_t)m * N + n0 + n] = (uint16_t)(pack2<DT>(s, 0.0f) & 0xFFFFu);
    }
}

// ---------------------------------------------------------------------------
// Streaming decode kernel, used when the whole of x fits in LDS.  A workgroup of
// kSW = 8 waves stages x once, each 8 columns in the odd/even order of
// deq8_oddeven, and then runs the tiles wg, wg + G, wg + 2G, ... of 16 RG rows.
// Row group rg (WR = 8 / RG waves) owns 16 rows of a tile; its S = 4 WR slots take
// the blocks slot, slot + S, slot + 2S, ... of each row, one step per S blocks and
// nq steps per tile.  A wave whose blocks of a step all lie past the row end skips
// that step; for the others such blocks read zero scales against zero x.
//
// Each lane requests its own block's codes (two 16-byte loads, 16 rows x 4
// consecutive blocks per wave instruction) and scale bytes into a ring of D
// entries that runs across tile boundaries: the block D steps ahead is requested as
// soon as an entry has been expanded, so a workgroup pays the memory latency once,
// not once per tile.  The tile and step bookkeeping is wave-uniform (scalar).  Per
// tile: the LoRA term t B on one wave per 32 columns of r, the row group's partial
// tiles added up in LDS by the last wave to finish the tile, the bf16 store.
constexpr int kSW = 8;                       // compute waves of the streaming kernel
constexpr uint32_t kOob = 0x80000000u;       // a buffer offset past every range: loads read 0, stores drop
constexpr int kSvSlots = 2;                  // partial-tile slots in LDS (a power of two)
// static LDS of the streaming kernel: t, the partial-tile slots, their counters (with alignment)
constexpr int kSvStaticLds = 16 * kTLd * 2 + kSvSlots * kSW * 256 * 4 + 64;

template <int D>
constexpr int sv_xe() { return D == 4 ? 16 : 8; }   // 16-byte chunks of x per thread, at most

// D ring entries; TP tiles per pass of D steps (TP > 1: nq = D / TP steps per tile, so
// every tile ends at a fixed step of the pass) or, with TP = 1, nq / D passes per tile.
template <int D, int TP, bool DQ, int CB, int DT, bool FT>
__global__ __launch_bounds__(kSW * 64 + (FT ? 64 : 0)) void nf4_gemv_stream_kernel(GvArgs a) {
    constexpr int NT = kSW * 64;
    constexpr int XE = sv_xe<D>();
    constexpr int NQS = D / TP;                  // steps per tile when TP > 1
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];    // x: M rows of a.xrs bytes
    __shared__ __attribute__((aligned(16))) uint16_t tl[16 * kTLd];
    __shared__ __attribute__((aligned(16))) float red[kSvSlots * kSW * 256];
    __shared__ uint32_t arrived[kSvSlots * 2];   // waves of a row group done with a slot's tile
    __shared__ int reduced[kSvSlots * 2];        // the last tile of a slot added up, per row group
    __shared__ uint32_t tickets;                 // tile ends so far, all waves (a scheduling hint)

    if (FT && (int)blockIdx.x < a.P) {
        gv_produce_any<kSW, DT>(a, dyn);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = a.M, N = a.N, K = a.K, r = a.r;
    const int Kb = K / kBlock;
    const int RG = a.rg, WR = kSW / RG, S = 4 * WR, TR = kGvRows * RG;
    const int nq = TP > 1 ? NQS : a.nq;
    const int RS = a.xrs;
    const int wg = blockIdx.x - (FT ? a.P : 0);
    const int G = a.gw;
    const int ntiles = (N + TR - 1) / TR;
    const int mytiles = (ntiles - wg + G - 1) / G;

    if (FT && w == kSW) {                        // helper wave: t
        __syncthreads();                         // x staged
        gv_helper_t<DT>(a, tl, wg == 0);
        __syncthreads();                         // t ready
        return;
    }

    const int rg = w / WR, wq = w - rg * WR;     // row group and wave within it (uniform)
    const int ln = lane & 15, lg = lane >> 4;
    const int slot = 4 * wq + lg;
    const int xrow = min(ln, M - 1);
    const rsrc_t crs = make_rsrc(a.codes, (uint32_t)((uint64_t)N * (uint32_t)(K >> 1)));
    const rsrc_t qrs = make_rsrc(a.q8, DQ ? (uint32_t)((uint64_t)N * Kb) : 0u);
    const uint32_t ngroups = (uint32_t)(((uint64_t)N * Kb + kSuper - 1) / kSuper);
    const rsrc_t ars = make_rsrc(a.a2, DQ ? ngroups * 4u : (uint32_t)((uint64_t)N * Kb * 4));
    const rsrc_t xrs = make_rsrc(a.x, (uint32_t)((uint64_t)M * K * 2));
    const rsrc_t brs = make_rsrc(a.B, (uint32_t)((uint64_t)r * N * 2));
    const rsrc_t yrs = make_rsrc(a.y, (uint32_t)((uint64_t)M * N * 2));

    // ---- the ring: codes, q8 byte and group scale (or the fp32 absmax) of one block per entry
    u32x4_t c0[D], c1[D];
    uint32_t sq[D], sa[D];
    const uint32_t lane_code = (uint32_t)ln * (uint32_t)(K >> 1) + 32u * (uint32_t)slot;
    const uint32_t lane_blk = (uint32_t)ln * (uint32_t)Kb + (uint32_t)slot;
    auto issue = [&](int k, int ti, int si) {    // step si of local tile ti into entry k
        const int rowb = (wg + G * ti) * TR + kGvRows * rg;
        const int sb = S * si;
        const bool okr = ti < mytiles && ln < N - rowb;
        const bool ok = okr && slot < Kb - sb;
        const uint32_t co = (uint32_t)rowb * (uint32_t)(K >> 1) + 32u * (uint32_t)sb + lane_code;
        const uint32_t bo = (uint32_t)rowb * (uint32_t)Kb + (uint32_t)sb + lane_blk;
        const uint32_t cof = opq(okr ? co : kOob);
        c0[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cof, 0, 0));
        c1[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cof + 16u, 0, 0));
        if (DQ) {
            sq[k] = __builtin_amdgcn_raw_buffer_load_b8(qrs, opq(ok ? bo : kOob), 0, 0);
            sa[k] = __builtin_amdgcn_raw_buffer_load_b32(ars, opq(ok ? 4u * (bo >> 8) : kOob), 0, 0);
        } else {
            sa[k] = __builtin_amdgcn_raw_buffer_load_b32(ars, opq(ok ? 4u * bo : kOob), 0, 0);
        }
    };

    // ---- B columns of a tile for this wave's 32 columns of r (zero past r).  N is even and
    // B 4-byte aligned, so B[j][n] is the (n % 2) half of the aligned dword that holds it:
    // whole dwords are loaded, and the halves are picked where they are used (an
    // operation at the load would make the compiler wait for it there).
    uint32_t bd[8];
    const uint32_t lane_b = 2u * (((uint32_t)(32 * wq + 8 * lg) * (uint32_t)N + (uint32_t)ln) & ~1u);
    const uint32_t bsel = (ln & 1) ? 0x07060302u : 0x05040100u;
    auto load_b = [&](int tc) {
        const uint32_t n0 = (uint32_t)((wg + G * tc) * TR + kGvRows * rg);   // even
#pragma unroll
        for (int i = 0; i < 8; ++i)
            bd[i] = __builtin_amdgcn_raw_buffer_load_b32(brs, opq(lane_b + 2u * (n0 + (uint32_t)(i * N))), 0, 0);
    };

    // ---- prologue: t when given, x, the first D steps of the ring, the first tile's B
    constexpr int kPer = 16 * kTLd / NT;
    uint32_t tv[kPer];
    if (!FT) {
        const rsrc_t trs = make_rsrc(a.t, (uint32_t)(M * r * 2));
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = tid + NT * u, m = i >> 7, jj = i & 127;
            tv[u] = __builtin_amdgcn_raw_buffer_load_b16(
                trs, opq((m < M && jj < r) ? 2u * (uint32_t)(m * r + jj) : kOob), 0, 0);
        }
    }
    const int xch = K >> 3, nch = M * xch;       // 16-byte chunks of an x row, of x
    u32x4_t xv[XE];
#pragma unroll
    for (int e = 0; e < XE; ++e) {
        const int c = tid + NT * e;
        if (e == 0 || NT * e < nch)              // uniform: only the batches that hold chunks
            xv[e] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    xrs, opq(c < nch ? 16u * (uint32_t)c : kOob), 0, 0));
    }
    // x goes out first, then the ring and the first tile's B; staging x then waits for x
    // alone (loads complete in order), so the ring's first code bytes travel from HBM
    // while x is staged instead of after it
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < D; ++k) issue(k, TP > 1 ? k / NQS : 0, TP > 1 ? k % NQS : k);
    load_b(0);
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* const xl = dyn;
#pragma unroll
    for (int e = 0; e < XE; ++e) {
        const int c = tid + NT * e;
        if ((e == 0 || NT * e < nch) && c < nch) {
            const int m = (int)__umulhi((uint32_t)c, a.xmagic), ch = c - m * xch;   // c / xch, c % xch
            *reinterpret_cast<u32x4_t*>(xl + m * RS + 16 * ch) = x_order8(xv[e]);
        }
    }
    const int xz = 8 * a.kx;                     // chunks of a row that the steps read: zero past K
    for (int m = 0; m < M; ++m)
        for (int ch = xch + tid; ch < xz; ch += NT)
            *reinterpret_cast<u32x4_t*>(xl + m * RS + 16 * ch) = u32x4_t{0u, 0u, 0u, 0u};
    if (!FT) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) tl[tid + NT * u] = (uint16_t)tv[u];
    }
    if (tid < kSvSlots * 2) {
        arrived[tid] = 0u;
        reduced[tid] = (tid >> 1) - kSvSlots;    // slot s is free for tile s
    }
    if (tid == 0) tickets = 0u;
    __syncthreads();

    // ---- main loop: D steps per pass, each expanded, then its entry refilled D steps ahead
    const uint32_t xlane = (uint32_t)(xrow * RS + 128 * slot);
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](int k, int sc) {
        const uint8_t* xp = xl + xlane + 128 * S * sc;
        const float ah = DQ ? scale_step(__uint_as_float(sa[k])) * (float)sq[k] : __uint_as_float(sa[k]);
        const Nf4Tab T = make_tab<CB, DT>(ah);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4_t wv = deq8_oddeven(T, s < 4 ? c0[k][s] : c1[k][s - 4]);
            const u32x4_t xf = *reinterpret_cast<const u32x4_t*>(xp + 16 * s);
            acc = mfma16<DT>(xf, wv, acc);
        }
    };
    // The end of a tile, without a workgroup barrier: each wave leaves its partial tile in
    // LDS slot tc % kSvSlots and counts itself in; the last wave of the row group adds the
    // row group's partials in wave order (the same order for every launch) and stores
    // the bf16 tile.  A wave that comes back to a slot first waits until the slot's
    // previous tile has been added up; the slowest wave never waits, so every wait ends.
    // The y stores are issued by every wave (dropped unless it is the last), so that the
    // loads in flight are the same on both sides of the branch.
    auto epilogue = [&](int tc) {
        if (FT && tc == 0) __syncthreads();      // t from the helper wave
        if (32 * wq < r) {                       // t B: this wave's 32 columns of r
            const u32x4_t ta = *reinterpret_cast<const u32x4_t*>(tl + ln * kTLd + 32 * wq + 8 * lg);
            const u32x4_t tb = {perm_b32(bd[1], bd[0], bsel), perm_b32(bd[3], bd[2], bsel),
                                perm_b32(bd[5], bd[4], bsel), perm_b32(bd[7], bd[6], bsel)};
            acc = mfma16<DT>(ta, tb, acc);
        }
        const int sl = tc & (kSvSlots - 1), sr = 2 * sl + rg;
        if (tc >= kSvSlots) {
            int spins = 0;
            while (__hip_atomic_load(&reduced[sr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) !=
                       tc - kSvSlots &&
                   ++spins < kSpinLimit)
                __builtin_amdgcn_s_sleep(1);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
        float* const rb = red + (sl * kSW + w) * 256;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * lg + v;
            if (m < M) rb[m * 16 + ln] = acc[v];
        }
        acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        uint32_t before = 0, tk = 0;
        if (lane == 0) {
            before = __hip_atomic_fetch_add(&arrived[sr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            tk = __hip_atomic_fetch_add(&tickets, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        const bool last = __builtin_amdgcn_readfirstlane(before) == (uint32_t)(WR - 1);
        // Waves that share a SIMD drift apart (the issue arbiter favours one of them), and a
        // wave left alone on its SIMD at the end runs at a fraction of the pair's rate.  The
        // workgroup's arrival count is a hint of who is ahead: a wave that finishes this
        // tile before its fair share of arrivals (kSW per tile) lowers its issue priority
        // for the next one, a later one raises it.
        if ((int)__builtin_amdgcn_readfirstlane(tk) < kSW * tc + kSW / 2) __builtin_amdgcn_s_setprio(0);
        else __builtin_amdgcn_s_setprio(2);
        float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = lane + 64 * i;     // (m, n) = (q / 16, q % 16)
                if (q < M * 16) {
                    const float* rr = red + (sl * kSW + rg * WR) * 256 + q;
                    for (int u = 0; u < WR; ++u) sum[i] += rr[u * 256];
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            if (lane == 0) {
                arrived[sr] = 0u;
                __hip_atomic_store(&reduced[sr], tc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        const int row0 = (wg + G * tc) * TR + kGvRows * rg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = lane + 64 * i, m = q >> 4, row = row0 + (q & 15);
            const bool ok = last && q < M * 16 && row < N;
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pack2<DT>(sum[i], 0.0f) & 0xFFFFu), yrs,
                                                  opq(ok ? 2u * (uint32_t)(m * N + row) : kOob), 0, 0);
        }
        load_b(tc + 1);
    };
    // pass: TP > 1: steps 0 .. NQS - 1 of tiles tc .. tc + TP - 1; TP = 1: steps jD .. jD + D - 1 of tile tc
    const int J = TP > 1 ? 1 : nq / D;
    int tc = 0, j = 0;
    do {
#pragma unroll
        for (int k = 0; k < D; ++k) {
            const int tile = TP > 1 ? tc + k / NQS : tc;
            const int step = TP > 1 ? k % NQS : j * D + k;
            if (tile < mytiles && S * step + 4 * wq < Kb) compute(k, step);
            if (TP > 1) {
                issue(k, tile + TP, step);       // the same step of the tile TP ahead
            } else {
                const bool more = j + 1 < J;     // D steps ahead: this tile or the next
                issue(k, more ? tc : tc + 1, more ? step + D : k);
            }
            if (TP > 1 ? k % NQS == NQS - 1 : (k == D - 1 && j == J - 1)) {
                if (tile < mytiles) epilogue(tile);
            }
        }
        if (TP > 1) {
            tc += TP;
        } else if (++j == J) {
            j = 0;
            ++tc;
        }
    } while (tc < mytiles);
}

struct GvPlan {
    int nw, mc, phases;
};

GvPlan gv_plan(int M, int K) {
    GvPlan p;
    p.nw = M <= 4 ? 8 : 4;
    p.mc = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    const int pb = 4 * p.nw * kGvNI;
    const int kb = K / kBlock;
    p.phases = (kb + pb - 1) / pb;
    return p;
}

// Producers of t: at most 16 (a consumer adds up at most 16 partials per value),
// each over kp columns of K, loaded in groups of up to 4 slices of 64 (at K = 4096 a
// producer's whole range is requested at once).
struct GvProducers {
    int P, kp, spp;
};
GvProducers gv_producers(int M, int K, int r) {
    (void)M;
    (void)r;
    const int kb = K / kBlock;
    const int per = (kb + 15) / 16;               // slices per producer
    const int P = (kb + per - 1) / per;
        return GvProducers{P, per * kBlock, per >= 4 ? 4 : per >= 2 ? 2 : 1};
}

// Plan of the streaming kernel: tile height (16 or 32 rows), ring depth D, steps per
// tile, tile workgroups; ok = false when x does not fit in LDS or in the prologue's
// registers, or r exceeds the LoRA chunks of a row group (32 columns of r per wave).
struct SvPlan {
    bool ok;
    int rg, d, tp, nq, kx, xrs, gw;
    size_t lds;
};
constexpr int kLdsBytes = 160 * 1024;
constexpr int kCUs = 256;

SvPlan sv_plan(int M, int N, int K, int r, int P, const void* B) {
    SvPlan best{};
    if ((N & 1) || (reinterpret_cast<uintptr_t>(B) & 3)) return best;    // B read as aligned dword pairs
    const int kb = K / kBlock;
    double best_cost = 0.0;
    for (int rg = 1; rg <= 2; ++rg) {
        const int wr = kSW / rg, S = 4 * wr;
        if (r > 32 * wr) continue;
        const int nq0 = (kb + S - 1) / S;            // steps that hold blocks
        // ring depth and tiles per pass: a tile of up to 4 steps runs 4, 2 or 1 to a pass of
        // a 4-deep ring, longer tiles nq / 8 passes of an 8-deep one each.  A deeper ring
        // does not pay: every CU requests its whole ring at the start, and the waves wait
        // at the issue until the memory system has taken it.
        const int d = nq0 <= 4 ? 4 : 8;
        const int tp = nq0 == 1 ? 4 : nq0 == 2 ? 2 : 1;
        const int nq = tp > 1 ? d / tp : (nq0 + d - 1) / d * d;
        const int xe = d == 4 ? sv_xe<4>() : sv_xe<8>();
        if ((int64_t)M * (K / 8) > (int64_t)xe * kSW * 64) continue;
        SvPlan p{};
        p.rg = rg;
        p.d = d;
        p.tp = tp;
        p.nq = nq;
        p.kx = nq0 * S;
        p.xrs = p.kx * 128 + 16;
        const size_t xbytes = (size_t)M * p.xrs;
        p.lds = std::max(xbytes, P > 0 ? (size_t)kASliceBytes : (size_t)0);
        if (p.lds + kSvStaticLds > (size_t)kLdsBytes) continue;
        const int tiles = (N + kGvRows * rg - 1) / (kGvRows * rg);
                // With producers (the layer call), the tile workgroups leave P CUs to them: one CU
        // holds one workgroup of this kernel, so a tile workgroup beyond 256 - P would wait
        // for a producer to finish, and every tile needs t.  (Taking all 256 CUs where that
        // saves a tile per workgroup measured slower on q_proj and fused q/k/v, and no
        // faster elsewhere.)
        const int gw = std::min(tiles, kCUs - P);
        const int mk = (tiles + gw - 1) / gw;
        p.gw = gw;
        // the busiest workgroup's steps, plus about half a step of per-tile work
        const double cost = (double)mk * (nq0 + 0.5);
        p.ok = true;
        if (!best.ok || cost < best_cost) {
            best = p;
            best_cost = cost;
        }
    }
    return best;
}

template <bool FT>
qlora_status gv_launch(const GvArgs& a, int cb, int dt, hipStream_t s) {
    GvArgs g = a;
    const SvPlan sp = sv_plan(a.M, a.N, a.K, a.r, FT ? a.P : 0, a.B);
    if (sp.ok) {
        g.rg = sp.rg;
        g.nq = sp.nq;
        g.kx = sp.kx;
        g.xrs = sp.xrs;
        g.gw = sp.gw;
        const uint32_t d = (uint32_t)(a.K / 8);
        g.xmagic = (uint32_t)(((uint64_t(1) << 32) + d - 1) / d);
        const dim3 grid((unsigned)(sp.gw + (FT ? a.P : 0)));
        const dim3 blk(kSW * 64 + (FT ? 64 : 0));
        with_cb_dt(cb, dt, [&](auto cbc, auto dtc) {
            constexpr int CB = decltype(cbc)::value, DT = decltype(dtc)::value;
#define QLORA_SV(D_, TP_)                                                                                         \
    if (sp.d == D_ && sp.tp == TP_) {                                                                             \
        if (a.q8) hipLaunchKernelGGL((nf4_gemv_stream_kernel<D_, TP_, true, CB, DT, FT>), grid, blk, sp.lds, s, g); \
        else hipLaunchKernelGGL((nf4_gemv_stream_kernel<D_, TP_, false, CB, DT, FT>), grid, blk, sp.lds, s, g);     \
    }
            QLORA_SV(4, 4) QLORA_SV(4, 2) QLORA_SV(4, 1) QLORA_SV(8, 1)
#undef QLORA_SV
        });
        return launch_status();
    }
    const GvPlan P = gv_plan(a.M, a.K);
    g.phases = P.phases;
    const int ntiles = (a.N + kGvRows - 1) / kGvRows;
    const dim3 grid((unsigned)(ntiles + (FT ? a.P : 0)));
    with_cb_dt(cb, dt, [&](auto cbc, auto dtc) {
        constexpr int CB = decltype(cbc)::value, DT = decltype(dtc)::value;
#define QLORA_GV(NW_, MC_)                                                                                     \
    if (P.nw == NW_ && P.mc == MC_) {                                                                          \
        const dim3 blk(NW_ * 64 + (FT ? 64 : 0));                                                            \
        if (a.q8) hipLaunchKernelGGL((nf4_gemv_kernel<NW_, MC_, true, CB, DT, FT>), grid, blk, 0, s, g);            \
        else hipLaunchKernelGGL((nf4_gemv_kernel<NW_, MC_, false, CB, DT, FT>), grid, blk, 0, s, g);               \
    }
        QLORA_GV(8, 1) QLORA_GV(8, 2) QLORA_GV(8, 4) QLORA_GV(4, 8) QLORA_GV(4, 16)
#undef QLORA_GV
    });
    return launch_status();
}

}  // namespace

bool gemv_supported(int M, int N, int K, int r) {
    return M >= 1 && M <= kGemvMaxM && r >= 1 && r <= 128 && (uint64_t)N * (uint64_t)K / 2 < (uint64_t(1) << 31) &&
           (uint64_t)M * K * 2 < (uint64_t(1) << 31);
}

size_t gemv_linear_workspace(int M, int N, int K, int r) {
    (void)N;
    const GvProducers pr = gv_producers(M, K, r);
    return ((size_t)pr.P * M * r * 4 + 255) / 256 * 256 + ((size_t)pr.P * 8 + 255) / 256 * 256;
}

qlora_status launch_gemv_fwd(const uint16_t* x, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                             int dt, const uint16_t* t, const uint16_t* B, uint16_t* y, int M, int N, int K, int r,
                             hipStream_t s) {
    if (!gemv_supported(M, N, K, r)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    GvArgs a{};
    a.x = x; a.codes = codes; a.q8 = q8; a.a2 = a2; a.t = t; a.B = B; a.y = y;
    a.M = M; a.N = N; a.K = K; a.r = r;
    return gv_launch<false>(a, cb, dt, s);
}

qlora_status launch_gemv_linear(const uint16_t* x, const uint8_t* codes, const uint8_t* q8, const float* a2, int cb,
                                int dt, const uint16_t* A, const uint16_t* B, float scale, uint16_t* y,
                                uint16_t* t_out, void* ws, int M, int N, int K, int r, hipStream_t s) {
    if (!gemv_supported(M, N, K, r)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    const GvProducers pr = gv_producers(M, K, r);
    GvArgs a{};
    a.x = x; a.codes = codes; a.q8 = q8; a.a2 = a2; a.A = A; a.B = B; a.y = y; a.t_out = t_out;
    a.part = reinterpret_cast<float*>(ws);
    a.flags = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + ((size_t)pr.P * M * r * 4 + 255) / 256 * 256);
    a.scale = scale;
    a.M = M; a.N = N; a.K = K; a.r = r;
    a.P = pr.P; a.kp = pr.kp; a.spp = pr.spp;
    return gv_launch<true>(a, cb, dt, s);
}

}  // namespace qlora
