// C ABI of libqlora: argument validation and dispatch (declared in include/qlora.h).
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "common.h"
#include "lora_plan.h"

using namespace qlora;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// q8 == NULL selects the state without double quantization (a2 = one fp32
// absmax per block); codes and a2 are required either way.  The 16-bit entry
// points take bf16 and fp16 states, the _f32 ones fp32 states only; dtype_any
// admits all three (qlora_dequantize_f32 does not read the dtype).
enum DtypeClass { kDt16, kDt32, kDtAny };
inline qlora_status check_state(const qlora_nf4* w, DtypeClass dc = kDt16) {
    if (!w || !w->codes || !w->a2) return QLORA_ERR_INVALID_ARG;
    if (w->n < 1 || w->k < 1) return QLORA_ERR_INVALID_ARG;
    if (w->k % kBlock) return QLORA_ERR_UNSUPPORTED_SHAPE;
    if (w->n >= (int64_t(1) << 31) || w->k >= (int64_t(1) << 31)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    if (w->quant_type != QLORA_QUANT_NF4 && w->quant_type != QLORA_QUANT_FP4) return QLORA_ERR_INVALID_ARG;
    const bool is16 = w->dtype == QLORA_DTYPE_BF16 || w->dtype == QLORA_DTYPE_F16;
    const bool is32 = w->dtype == QLORA_DTYPE_F32;
    if (!(dc == kDt16 ? is16 : dc == kDt32 ? is32 : (is16 || is32))) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(w->codes) || (w->q8 && !aligned16(w->q8)) || !aligned16(w->a2)) return QLORA_ERR_MISALIGNED;
    return QLORA_OK;
}

inline int cb_of(const qlora_nf4* w) { return w->quant_type == QLORA_QUANT_FP4 ? kCbFp4 : kCbNf4; }
inline int dt_of(int dtype) { return dtype == QLORA_DTYPE_F16 ? kDtF16 : kDtBf16; }
inline int dt_of(const qlora_nf4* w) { return dt_of(w->dtype); }

inline bool bad_dims(int64_t M, int64_t N, int64_t K, int r) {
    return M < 0 || N < 1 || K < 1 || r < 1 || r > 128 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX;
}

// Workspace carve-up.  Every piece starts on a 256-byte boundary.
struct FwdWs {
    size_t part, tbuf, total;  // split sums of t; t when the caller keeps none
};
inline FwdWs fwd_ws(int64_t M, int64_t N, int64_t K, int r) {
    FwdWs w{};
    w.part = 0;
    w.tbuf = w.part + align256(nt_ws_bytes(M, K, r));
    w.total = w.tbuf + align256((size_t)M * r * 2);
    // decode sizes run as one launch whose workspace starts at offset 0
    if (gemv_supported((int)M, (int)N, (int)K, r))
        w.total = std::max(w.total, gemv_linear_workspace((int)M, (int)N, (int)K, r));
    return w;
}

struct BwdWs {
    size_t u, part, tbuf, pa, pb, total;  // u; split sums of u (and of t); t; split sums of dA, dB
};
inline BwdWs bwd_ws(int64_t M, int64_t N, int64_t K, int r) {
    BwdWs w{};
    const size_t mr2 = align256((size_t)M * r * 2);
    w.u = 0;
    w.part = w.u + mr2;
    w.tbuf = w.part + align256(std::max(nt_ws_bytes(M, N, r), nt_ws_bytes(M, K, r)));
    w.pa = w.tbuf + mr2;
    w.pb = w.pa + align256(tn_ws_bytes(M, K, r));
    w.total = w.pb + align256(tn_ws_bytes(M, N, r));
    return w;
}

inline uint8_t* at(void* ws, size_t off) { return static_cast<uint8_t*>(ws) + off; }

// Workspace of qlora_linear_fwd_noalloc: one fixed array per GPU, held until the process
// ends.  In host code `scratch` names a host-side stand-in, so kernels get the device
// address that hipGetSymbolAddress returns, taken once per device with that device
// current.  Nothing in the workspace has to start at zero: the split partial sums are
// written before they are read, and the publication tags that guard them identify
// their launch.
constexpr size_t kScratchBytes = QLORA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

qlora_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QLORA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QLORA_OK;
}

// fp32 layer: bytes of the split partial sums of one contraction (0 when it does not split)
inline size_t f32_part(int64_t rows, int64_t cols, int64_t red) {
    const F32Plan p = plan_f32((int)rows, (int)cols, (int)std::max<int64_t>(red, 1));
    return p.splits > 1 ? align256((size_t)p.splits * rows * cols * 4) : 0;
}
struct F32FwdWs {
    size_t tbuf, part, total;
};
inline F32FwdWs f32_fwd_ws(int64_t M, int64_t N, int64_t K, int r) {
    F32FwdWs w{};
    w.tbuf = 0;
    w.part = align256((size_t)M * r * 4);
    w.total = w.part + std::max(f32_part(M, r, K), f32_part(M, N, K));
    return w;
}
struct F32BwdWs {
    size_t u, tbuf, part, total;
};
inline F32BwdWs f32_bwd_ws(int64_t M, int64_t N, int64_t K, int r) {
    F32BwdWs w{};
    w.u = 0;
    w.tbuf = align256((size_t)M * r * 4);
    w.part = 2 * w.tbuf;
    const size_t p = std::max({f32_part(M, r, N), f32_part(M, r, K), f32_part(M, K, N), f32_part(K, r, M),
                               f32_part(r, N, M)});
    w.total = w.part + p;
    return w;
}

}  // namespace

extern "C" {

int qlora_version(void) { return 200; }

const char* qlora_status_string(int status) {
    switch (status) {
        case QLORA_OK: return "ok";
        case QLORA_ERR_INVALID_ARG: return "invalid argument";
        case QLORA_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (K must be a multiple of 64)";
        case QLORA_ERR_MISALIGNED: return "tensor pointer not 16-byte aligned";
        case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
        case QLORA_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

qlora_status qlora_nf4_sizes(int64_t N, int64_t K, size_t* codes_bytes, size_t* q8_bytes, size_t* a2_bytes) {
    if (N < 1 || K < 1) return QLORA_ERR_INVALID_ARG;
    if (K % kBlock) return QLORA_ERR_UNSUPPORTED_SHAPE;
    const int64_t n = N * K;
    if (codes_bytes) *codes_bytes = (size_t)(n / 2);
    if (q8_bytes) *q8_bytes = (size_t)(n / kBlock);
    if (a2_bytes) *a2_bytes = (size_t)(4 * ((n + kSuperElems - 1) / kSuperElems));
    return QLORA_OK;
}

qlora_status qlora_nf4_sizes_nodq(int64_t N, int64_t K, size_t* codes_bytes, size_t* absmax_bytes) {
    if (N < 1 || K < 1) return QLORA_ERR_INVALID_ARG;
    if (K % kBlock) return QLORA_ERR_UNSUPPORTED_SHAPE;
    const int64_t n = N * K;
    if (codes_bytes) *codes_bytes = (size_t)(n / 2);
    if (absmax_bytes) *absmax_bytes = (size_t)(4 * (n / kBlock));
    return QLORA_OK;
}

qlora_status qlora_quantize(const uint16_t* W, int64_t N, int64_t K, const qlora_nf4* out, void* stream) {
    if (!W) return QLORA_ERR_INVALID_ARG;
    qlora_status st = check_state(out);
    if (st != QLORA_OK) return st;
    if (out->n != N || out->k != K) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(W)) return QLORA_ERR_MISALIGNED;
    return launch_quantize(W, N * K / kBlock, out->codes, out->q8, out->a2, cb_of(out), dt_of(out),
                           (hipStream_t)stream);
}

qlora_status qlora_quantize_batch(const uint16_t* const* W, const qlora_nf4* out, int count, void* stream) {
    if (count < 0 || (count > 0 && (!W || !out))) return QLORA_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i) {
        if (!W[i]) return QLORA_ERR_INVALID_ARG;
        const qlora_status st = check_state(&out[i]);
        if (st != QLORA_OK) return st;
        if (!aligned16(W[i])) return QLORA_ERR_MISALIGNED;
    }
    // one launch per run of consecutive weights that share codebook, dtype and double quantization
    for (int i0 = 0; i0 < count;) {
        const qlora_nf4& f = out[i0];
        int n = 1;
        while (i0 + n < count && n < kQuantBatchMax && out[i0 + n].quant_type == f.quant_type &&
               out[i0 + n].dtype == f.dtype && (out[i0 + n].q8 == nullptr) == (f.q8 == nullptr))
            ++n;
        const void* w[kQuantBatchMax];
        int64_t nb[kQuantBatchMax];
        uint8_t* codes[kQuantBatchMax];
        uint8_t* q8[kQuantBatchMax];
        float* a2[kQuantBatchMax];
        for (int j = 0; j < n; ++j) {
            const qlora_nf4& o = out[i0 + j];
            w[j] = W[i0 + j];
            nb[j] = o.n * o.k / kBlock;
            codes[j] = o.codes;
            q8[j] = o.q8;
            a2[j] = o.a2;
        }
        const qlora_status st =
            launch_quantize_batch(w, nb, codes, q8, a2, n, cb_of(&f), dt_of(&f), (hipStream_t)stream);
        if (st != QLORA_OK) return st;
        i0 += n;
    }
    return QLORA_OK;
}

qlora_status qlora_dequantize(const qlora_nf4* w, uint16_t* out, void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    if (!out) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(out)) return QLORA_ERR_MISALIGNED;
    return launch_dequantize(w->codes, w->q8, w->a2, cb_of(w), dt_of(w), w->n * w->k / kBlock, out,
                             (hipStream_t)stream);
}

qlora_status qlora_dequantize_f32(const qlora_nf4* w, float* out, void* stream) {
    qlora_status st = check_state(w, kDtAny);
    if (st != QLORA_OK) return st;
    if (!out) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(out)) return QLORA_ERR_MISALIGNED;
    return launch_dequantize_f32(w->codes, w->q8, w->a2, cb_of(w), w->n * w->k / kBlock, out, (hipStream_t)stream);
}

qlora_status qlora_merge(const qlora_nf4* w, const uint16_t* A, const uint16_t* B, int r, float alpha,
                         uint16_t* out, void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    if (!A || !B || !out || bad_dims(0, w->n, w->k, r) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(A) || !aligned16(B) || !aligned16(out)) return QLORA_ERR_MISALIGNED;
    const float s = alpha / (float)r;
    return launch_merge(w->codes, w->q8, w->a2, cb_of(w), dt_of(w), A, B, r, s, out, (int)w->n, (int)w->k,
                        (hipStream_t)stream);
}

size_t qlora_fwd_workspace(int64_t M, int64_t N, int64_t K, int r) {
    if (bad_dims(M, N, K, r) || M == 0 || K % kBlock) return 0;
    return fwd_ws(M, N, K, r).total;
}

size_t qlora_bwd_workspace(int64_t M, int64_t N, int64_t K, int r) {
    if (bad_dims(M, N, K, r) || M == 0 || K % kBlock) return 0;
    return bwd_ws(M, N, K, r).total;
}

size_t qlora_lora_down_workspace(int64_t M, int64_t K, int r) {
    if (bad_dims(M, 1, K, r) || M == 0 || K % kBlock) return 0;
    return align256(nt_ws_bytes(M, K, r));
}

qlora_status qlora_lora_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* A, int r, float alpha,
                             int dtype, uint16_t* t_out, void* ws, size_t ws_bytes, void* stream) {
    if (bad_dims(M, 1, K, r) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (dtype != QLORA_DTYPE_BF16 && dtype != QLORA_DTYPE_F16) return QLORA_ERR_INVALID_ARG;
    if (K % kBlock) return QLORA_ERR_UNSUPPORTED_SHAPE;
    if (M == 0) return QLORA_OK;
    if (!x || !A || !t_out) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(A) || !aligned16(t_out)) return QLORA_ERR_MISALIGNED;
    const size_t need = qlora_lora_down_workspace(M, K, r);
    if (!ws || ws_bytes < need) return QLORA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QLORA_ERR_MISALIGNED;
    return launch_nt(x, A, true, ws, t_out, alpha / (float)r, (int)M, (int)K, r, dt_of(dtype), (hipStream_t)stream);
}

qlora_status qlora_fused_gemm_fwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* t,
                                  const uint16_t* B, int r, uint16_t* y, void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    const int64_t N = w->n, K = w->k;
    if (bad_dims(M, N, K, r)) return QLORA_ERR_INVALID_ARG;
    if (M == 0) return QLORA_OK;
    if (!x || !t || !B || !y) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(t) || !aligned16(B) || !aligned16(y)) return QLORA_ERR_MISALIGNED;
    return launch_gemm_fwd(x, w->codes, w->q8, w->a2, cb_of(w), dt_of(w), t, B, y, (int)M, (int)N, (int)K, r,
                           (hipStream_t)stream);
}

qlora_status qlora_fused_gemm_bwd_dx(const qlora_nf4* w, const uint16_t* dy, int64_t M, const uint16_t* u,
                                     const uint16_t* A, int r, uint16_t* dx, void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    const int64_t N = w->n, K = w->k;
    if (bad_dims(M, N, K, r)) return QLORA_ERR_INVALID_ARG;
    if (M == 0) return QLORA_OK;
    if (!dy || !u || !A || !dx) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(dy) || !aligned16(u) || !aligned16(A) || !aligned16(dx)) return QLORA_ERR_MISALIGNED;
    return launch_gemm_bwd_dx(dy, w->codes, w->q8, w->a2, cb_of(w), dt_of(w), u, A, dx, (int)M, (int)N, (int)K, r,
                              (hipStream_t)stream);
}

size_t qlora_linear_bwd_dx_workspace(int64_t M, int64_t N, int64_t K, int r) {
    if (bad_dims(M, N, K, r) || M == 0) return 0;
    return align256(nt_ws_bytes(M, N, r));
}

qlora_status qlora_linear_bwd_dx(const qlora_nf4* w, int64_t M, const uint16_t* A, const uint16_t* B, int r,
                                 float alpha, const uint16_t* dy, uint16_t* u, uint16_t* dx, void* ws,
                                 size_t ws_bytes, void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    const int64_t N = w->n, K = w->k;
    if (bad_dims(M, N, K, r) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (M == 0) return QLORA_OK;
    if (!A || !B || !dy || !u || !dx) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(A) || !aligned16(B) || !aligned16(dy) || !aligned16(u) || !aligned16(dx))
        return QLORA_ERR_MISALIGNED;
    if (!ws || ws_bytes < qlora_linear_bwd_dx_workspace(M, N, K, r)) return QLORA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QLORA_ERR_MISALIGNED;
    hipStream_t s = (hipStream_t)stream;
    // u = s dy B^T (B [r, N] is the row-major transpose of B^T), kept in the caller's buffer
    if ((st = launch_nt(dy, B, false, ws, u, alpha / (float)r, (int)M, (int)N, r, dt_of(w), s)) != QLORA_OK)
        return st;
    return launch_gemm_bwd_dx(dy, w->codes, w->q8, w->a2, cb_of(w), dt_of(w), u, A, dx, (int)M, (int)N, (int)K, r,
                              s);
}

size_t qlora_lora_prod_batch_workspace(const qlora_lora_prod* items, int count, int r) {
    if (!items || count <= 0 || r < 1 || r > 128) return 0;
    size_t total = 0;
    for (int i = 0; i < count; ++i) {
        const qlora_lora_prod& e = items[i];
        if (!bad_dims(e.M, 1, e.C, r) && e.M > 0) total += align256(nt_ws_bytes(e.M, e.C, r));
    }
    return total;
}

// t_i = s x_i A_i (y_natural) or u_i = s dy_i B_i^T for every item, in launches of up to 8.
static qlora_status lora_prod_batch(const qlora_lora_prod* items, int count, int r, float alpha, int dtype,
                                    bool y_natural, void* ws, size_t ws_bytes, void* stream) {
    if (count < 0 || r < 1 || r > 128 || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (dtype != QLORA_DTYPE_BF16 && dtype != QLORA_DTYPE_F16) return QLORA_ERR_INVALID_ARG;
    if (count == 0) return QLORA_OK;
    if (!items) return QLORA_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i) {  // every entry is checked before anything is launched
        const qlora_lora_prod& e = items[i];
        if (bad_dims(e.M, 1, e.C, r)) return QLORA_ERR_INVALID_ARG;
        if (y_natural && e.C % kBlock) return QLORA_ERR_UNSUPPORTED_SHAPE;
        if (e.M == 0) continue;
        if (!e.x || !e.w || !e.out) return QLORA_ERR_INVALID_ARG;
        if (!aligned16(e.x) || !aligned16(e.w) || !aligned16(e.out)) return QLORA_ERR_MISALIGNED;
    }
    const size_t need = qlora_lora_prod_batch_workspace(items, count, r);
    if (need && (!ws || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
    if (need && !aligned16(ws)) return QLORA_ERR_MISALIGNED;
    std::vector<NtDesc> d;
    d.reserve((size_t)count);
    size_t off = 0;
    for (int i = 0; i < count; ++i) {
        const qlora_lora_prod& e = items[i];
        if (e.M == 0) continue;
        d.push_back(NtDesc{e.x, e.w, at(ws, off), e.out, alpha / (float)r, (int)e.M, (int)e.C});
        off += align256(nt_ws_bytes(e.M, e.C, r));
    }
    if (d.empty()) return QLORA_OK;
    return launch_nt_batch(d.data(), (int)d.size(), y_natural, r, dt_of(dtype), (hipStream_t)stream);
}

qlora_status qlora_lora_down_batch(const qlora_lora_prod* items, int count, int r, float alpha, int dtype, void* ws,
                                   size_t ws_bytes, void* stream) {
    return lora_prod_batch(items, count, r, alpha, dtype, true, ws, ws_bytes, stream);
}

qlora_status qlora_lora_u_batch(const qlora_lora_prod* items, int count, int r, float alpha, int dtype, void* ws,
                                size_t ws_bytes, void* stream) {
    return lora_prod_batch(items, count, r, alpha, dtype, false, ws, ws_bytes, stream);
}

// Workspace of one layer's two gradient contractions in qlora_lora_grads_batch.
inline size_t grads_ws(const qlora_lora_grads& g, int r) {
    if (g.M == 0) return 0;
    return align256(tn_ws_bytes(g.M, g.K, r)) + align256(tn_ws_bytes(g.M, g.N, r));
}

size_t qlora_lora_grads_batch_workspace(const qlora_lora_grads* layers, int count, int r) {
    if (!layers || count <= 0 || r < 1 || r > 128) return 0;
    size_t total = 0;
    for (int i = 0; i < count; ++i)
        if (!bad_dims(layers[i].M, layers[i].N, layers[i].K, r)) total += grads_ws(layers[i], r);
    return total;
}

qlora_status qlora_lora_grads_batch(const qlora_lora_grads* layers, int count, int r, int dtype, void* ws,
                                    size_t ws_bytes, void* stream) {
    if (count < 0 || r < 1 || r > 128) return QLORA_ERR_INVALID_ARG;
    if (dtype != QLORA_DTYPE_BF16 && dtype != QLORA_DTYPE_F16) return QLORA_ERR_INVALID_ARG;
    if (count == 0) return QLORA_OK;
    if (!layers) return QLORA_ERR_INVALID_ARG;
    // every entry is checked before anything is launched
    for (int i = 0; i < count; ++i) {
        const qlora_lora_grads& g = layers[i];
        if (bad_dims(g.M, g.N, g.K, r) || !g.dA || !g.dB) return QLORA_ERR_INVALID_ARG;
        if (!aligned16(g.dA) || !aligned16(g.dB)) return QLORA_ERR_MISALIGNED;
        if (g.M == 0) continue;
        if (!g.x || !g.t || !g.u || !g.dy) return QLORA_ERR_INVALID_ARG;
        if (!aligned16(g.x) || !aligned16(g.t) || !aligned16(g.u) || !aligned16(g.dy)) return QLORA_ERR_MISALIGNED;
    }
    const size_t need = qlora_lora_grads_batch_workspace(layers, count, r);
    if (need && (!ws || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
    if (need && !aligned16(ws)) return QLORA_ERR_MISALIGNED;
    hipStream_t s = (hipStream_t)stream;
    std::vector<TnDesc> d;
    d.reserve(2 * (size_t)count);
    size_t off = 0;
    qlora_status st = QLORA_OK;
    for (int i = 0; i < count; ++i) {
        const qlora_lora_grads& g = layers[i];
        if (g.M == 0) {  // empty sums
            if ((st = launch_fill(g.dA, g.K * r, 0.0f, s)) != QLORA_OK) return st;
            if ((st = launch_fill(g.dB, (int64_t)r * g.N, 0.0f, s)) != QLORA_OK) return st;
            continue;
        }
        // dA [K, r] = x^T u ; dB [r, N] = t^T dy, stored transposed from the [N, r] reduction
        d.push_back(TnDesc{g.x, g.u, at(ws, off), g.dA, (int)g.M, (int)g.K, r, 1});
        off += align256(tn_ws_bytes(g.M, g.K, r));
        d.push_back(TnDesc{g.dy, g.t, at(ws, off), g.dB, (int)g.M, (int)g.N, 1, g.N});
        off += align256(tn_ws_bytes(g.M, g.N, r));
    }
    return launch_tn_batch(d.data(), (int)d.size(), r, dt_of(dtype), s);
}

qlora_status qlora_linear_fwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
                              int r, float alpha, uint16_t* y, uint16_t* t_out, void* ws, size_t ws_bytes,
                              void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    const int64_t N = w->n, K = w->k;
    if (bad_dims(M, N, K, r) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (M == 0) return QLORA_OK;
    if (!x || !A || !B || !y) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) || (t_out && !aligned16(t_out)))
        return QLORA_ERR_MISALIGNED;
    const FwdWs L = fwd_ws(M, N, K, r);
    if (!ws || ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QLORA_ERR_MISALIGNED;
    hipStream_t s = (hipStream_t)stream;
    const float scale = alpha / (float)r;
    if (gemv_supported((int)M, (int)N, (int)K, r))  // decode sizes: t and y in one launch
        return launch_gemv_linear(x, w->codes, w->q8, w->a2, cb_of(w), dt_of(w), A, B, scale, y, t_out, ws, (int)M,
                                  (int)N, (int)K, r, s);
    void* part = at(ws, L.part);
    uint16_t* t = t_out ? t_out : reinterpret_cast<uint16_t*>(at(ws, L.tbuf));
    if ((st = launch_nt(x, A, true, part, t, scale, (int)M, (int)K, r, dt_of(w), s)) != QLORA_OK) return st;
    return launch_gemm_fwd(x, w->codes, w->q8, w->a2, cb_of(w), dt_of(w), t, B, y, (int)M, (int)N, (int)K, r, s);
}

qlora_status qlora_linear_fwd_noalloc(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A,
                                      const uint16_t* B, int r, float alpha, uint16_t* y, uint16_t* t_out,
                                      void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    const int64_t N = w->n, K = w->k;
    if (bad_dims(M, N, K, r) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (M == 0) return QLORA_OK;
    if (fwd_ws(M, N, K, r).total > kScratchBytes) return QLORA_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != QLORA_OK) return st;
    return qlora_linear_fwd(w, x, M, A, B, r, alpha, y, t_out, ws, kScratchBytes, stream);
}

qlora_status qlora_linear_bwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
                              int r, float alpha, const uint16_t* t, const uint16_t* dy, uint16_t* dx, float* dA,
                              float* dB, void* ws, size_t ws_bytes, void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    const int64_t N = w->n, K = w->k;
    if (bad_dims(M, N, K, r) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (!dA || !dB) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(dA) || !aligned16(dB)) return QLORA_ERR_MISALIGNED;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0) {  // empty sums
        if ((st = launch_fill(dA, K * r, 0.0f, s)) != QLORA_OK) return st;
        return launch_fill(dB, (int64_t)r * N, 0.0f, s);
    }
    if (!x || !A || !B || !dy) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(dy) || (t && !aligned16(t)) ||
        (dx && !aligned16(dx)))
        return QLORA_ERR_MISALIGNED;
    const BwdWs L = bwd_ws(M, N, K, r);
    if (!ws || ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QLORA_ERR_MISALIGNED;
    const float scale = alpha / (float)r;
    uint16_t* u = reinterpret_cast<uint16_t*>(at(ws, L.u));
    void* part = at(ws, L.part);
    // u = s dy B^T  (B [r, N] is the row-major transpose of B^T)
    if ((st = launch_nt(dy, B, false, part, u, scale, (int)M, (int)N, r, dt_of(w), s)) != QLORA_OK) return st;
    if (!t) {  // recompute t = s x A
        uint16_t* tb = reinterpret_cast<uint16_t*>(at(ws, L.tbuf));
        if ((st = launch_nt(x, A, true, part, tb, scale, (int)M, (int)K, r, dt_of(w), s)) != QLORA_OK) return st;
        t = tb;
    }
    if (dx) {
        if ((st = launch_gemm_bwd_dx(dy, w->codes, w->q8, w->a2, cb_of(w), dt_of(w), u, A, dx, (int)M, (int)N, (int)K,
                                     r, s)) != QLORA_OK)
            return st;
    }
    // dA [K, r] = x^T u ; dB [r, N] = t^T dy, stored transposed from the [N, r] reduction
    // (both in one launch: the second one's workgroups fill the CUs that the first one's
    // finished splits leave while its last splits add up their tiles)
    return launch_tn2(x, u, at(ws, L.pa), dA, (int)K, r, 1, dy, t, at(ws, L.pb), dB, (int)N, 1, N, (int)M, r,
                      dt_of(w), s);
}

// ---- fp32 compute dtype (deep dive 8.3): fp32 tensors, w_hat = fl32(a_hat * c_q)
qlora_status qlora_quantize_f32(const float* W, int64_t N, int64_t K, const qlora_nf4* out, void* stream) {
    if (!W) return QLORA_ERR_INVALID_ARG;
    qlora_status st = check_state(out, kDt32);
    if (st != QLORA_OK) return st;
    if (out->n != N || out->k != K) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(W)) return QLORA_ERR_MISALIGNED;
    return launch_quantize(W, N * K / kBlock, out->codes, out->q8, out->a2, cb_of(out), kDtF32, (hipStream_t)stream);
}

size_t qlora_fwd_workspace_f32(int64_t M, int64_t N, int64_t K, int r) {
    if (bad_dims(M, N, K, r) || M == 0 || K % kBlock) return 0;
    return f32_fwd_ws(M, N, K, r).total;
}

size_t qlora_bwd_workspace_f32(int64_t M, int64_t N, int64_t K, int r) {
    if (bad_dims(M, N, K, r) || M == 0 || K % kBlock) return 0;
    return f32_bwd_ws(M, N, K, r).total;
}

qlora_status qlora_linear_fwd_f32(const qlora_nf4* w, const float* x, int64_t M, const float* A, const float* B,
                                  int r, float alpha, float* y, float* t_out, void* ws, size_t ws_bytes,
                                  void* stream) {
    qlora_status st = check_state(w, kDt32);
    if (st != QLORA_OK) return st;
    const int64_t N = w->n, K = w->k;
    if (bad_dims(M, N, K, r) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (M == 0) return QLORA_OK;
    if (!x || !A || !B || !y) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) || (t_out && !aligned16(t_out)))
        return QLORA_ERR_MISALIGNED;
    const F32FwdWs L = f32_fwd_ws(M, N, K, r);
    if (!ws || ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QLORA_ERR_MISALIGNED;
    hipStream_t s = (hipStream_t)stream;
    float* part = reinterpret_cast<float*>(at(ws, L.part));
    float* t = t_out ? t_out : reinterpret_cast<float*>(at(ws, L.tbuf));
    const float scale = alpha / (float)r;
    if ((st = launch_f32_lora(kF32LoraDown, x, A, (int)M, (int)K, r, scale, t, part, s)) != QLORA_OK) return st;
    return launch_f32_fwd(x, w->codes, w->q8, w->a2, cb_of(w), t, B, y, (int)M, (int)N, (int)K, r, part, s);
}

qlora_status qlora_linear_bwd_f32(const qlora_nf4* w, const float* x, int64_t M, const float* A, const float* B,
                                  int r, float alpha, const float* t, const float* dy, float* dx, float* dA,
                                  float* dB, void* ws, size_t ws_bytes, void* stream) {
    qlora_status st = check_state(w, kDt32);
    if (st != QLORA_OK) return st;
    const int64_t N = w->n, K = w->k;
    if (bad_dims(M, N, K, r) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (!dA || !dB) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(dA) || !aligned16(dB)) return QLORA_ERR_MISALIGNED;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0) {  // empty sums
        if ((st = launch_fill(dA, K * r, 0.0f, s)) != QLORA_OK) return st;
        return launch_fill(dB, (int64_t)r * N, 0.0f, s);
    }
    if (!x || !A || !B || !dy) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(dy) || (t && !aligned16(t)) ||
        (dx && !aligned16(dx)))
        return QLORA_ERR_MISALIGNED;
    const F32BwdWs L = f32_bwd_ws(M, N, K, r);
    if (!ws || ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QLORA_ERR_MISALIGNED;
    const float scale = alpha / (float)r;
    float* u = reinterpret_cast<float*>(at(ws, L.u));
    float* part = reinterpret_cast<float*>(at(ws, L.part));
    // u = s dy B^T
    if ((st = launch_f32_lora(kF32LoraDownT, dy, B, (int)M, (int)N, r, scale, u, part, s)) != QLORA_OK) return st;
    if (!t) {  // recompute t = s x A
        float* tb = reinterpret_cast<float*>(at(ws, L.tbuf));
        if ((st = launch_f32_lora(kF32LoraDown, x, A, (int)M, (int)K, r, scale, tb, part, s)) != QLORA_OK) return st;
        t = tb;
    }
    if (dx) {
        if ((st = launch_f32_bwd_dx(dy, w->codes, w->q8, w->a2, cb_of(w), u, A, dx, (int)M, (int)N, (int)K, r, part,
                                    s)) != QLORA_OK)
            return st;
    }
    // dA [K, r] = x^T u ; dB [r, N] = t^T dy
    if ((st = launch_f32_lora(kF32Grad, x, u, (int)M, (int)K, r, 1.0f, dA, part, s)) != QLORA_OK) return st;
    return launch_f32_lora(kF32GradT, t, dy, (int)M, (int)N, r, 1.0f, dB, part, s);
}

// ---- QA-LoRA pooled branch: A [K/g, r]; the plain path runs on A~ = expand(A) / g
static bool bad_group(int64_t K, int g) { return g < 1 || (g & (g - 1)) != 0 || K % g != 0; }

size_t qlora_pooled_fwd_workspace(int64_t M, int64_t N, int64_t K, int r, int g) {
    if (bad_dims(M, N, K, r) || M == 0 || K % kBlock || bad_group(K, g)) return 0;
    return align256((size_t)K * r * 2) + fwd_ws(M, N, K, r).total;
}

size_t qlora_pooled_bwd_workspace(int64_t M, int64_t N, int64_t K, int r, int g) {
    if (bad_dims(M, N, K, r) || K % kBlock || bad_group(K, g)) return 0;
    return align256((size_t)K * r * 2) + align256((size_t)K * r * 4) + bwd_ws(std::max<int64_t>(M, 1), N, K, r).total;
}

qlora_status qlora_pooled_fwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
                              int r, int g, float alpha, uint16_t* y, uint16_t* t_out, void* ws, size_t ws_bytes,
                              void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    if (bad_dims(M, w->n, w->k, r) || bad_group(w->k, g) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (M == 0) return QLORA_OK;
    if (!A) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(A)) return QLORA_ERR_MISALIGNED;
    const size_t head = align256((size_t)w->k * r * 2);
    if (!ws || ws_bytes < head) return QLORA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QLORA_ERR_MISALIGNED;
    uint16_t* Ax = reinterpret_cast<uint16_t*>(ws);
    if ((st = launch_expand_pooled(A, (int)w->k, r, g, dt_of(w), Ax, (hipStream_t)stream)) != QLORA_OK) return st;
    return qlora_linear_fwd(w, x, M, Ax, B, r, alpha, y, t_out, at(ws, head), ws_bytes - head, stream);
}

qlora_status qlora_pooled_bwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
                              int r, int g, float alpha, const uint16_t* t, const uint16_t* dy, uint16_t* dx, float* dA,
                              float* dB, void* ws, size_t ws_bytes, void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    if (bad_dims(M, w->n, w->k, r) || bad_group(w->k, g) || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
    if (!A || !dA) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(A) || !aligned16(dA)) return QLORA_ERR_MISALIGNED;
    const size_t ha = align256((size_t)w->k * r * 2), hd = align256((size_t)w->k * r * 4);
    if (!ws || ws_bytes < ha + hd) return QLORA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QLORA_ERR_MISALIGNED;
    hipStream_t s = (hipStream_t)stream;
    uint16_t* Ax = reinterpret_cast<uint16_t*>(ws);
    float* dAx = reinterpret_cast<float*>(at(ws, ha));
    if ((st = launch_expand_pooled(A, (int)w->k, r, g, dt_of(w), Ax, s)) != QLORA_OK) return st;
    if ((st = qlora_linear_bwd(w, x, M, Ax, B, r, alpha, t, dy, dx, dAx, dB, at(ws, ha + hd), ws_bytes - ha - hd,
                               stream)) != QLORA_OK)
        return st;
    return launch_pool_rows(dAx, (int)w->k, r, g, dA, s);
}

}  // extern "C"
