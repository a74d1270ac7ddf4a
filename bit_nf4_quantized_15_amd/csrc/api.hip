// C ABI of libqlora: argument validation and dispatch (declared in include/qlora.h).
#include <cmath>
#include <cstdint>

#include "common.h"

using namespace qlora;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline qlora_status check_state(const qlora_nf4* w) {
    if (!w || !w->codes || !w->q8 || !w->a2) return QLORA_ERR_INVALID_ARG;
    if (w->n < 1 || w->k < 1) return QLORA_ERR_INVALID_ARG;
    if (w->k % kBlock) return QLORA_ERR_UNSUPPORTED_SHAPE;
    if (w->n > (int64_t(1) << 31) || w->k > (int64_t(1) << 31)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(w->codes) || !aligned16(w->q8) || !aligned16(w->a2)) return QLORA_ERR_MISALIGNED;
    return QLORA_OK;
}

}  // namespace

extern "C" {

int qlora_version(void) { return 100; }

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

qlora_status qlora_quantize(const uint16_t* W, int64_t N, int64_t K, const qlora_nf4* out, void* stream) {
    if (!W) return QLORA_ERR_INVALID_ARG;
    qlora_status st = check_state(out);
    if (st != QLORA_OK) return st;
    if (out->n != N || out->k != K) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(W)) return QLORA_ERR_MISALIGNED;
    return launch_quantize(W, N * K / kBlock, out->codes, out->q8, out->a2, (hipStream_t)stream);
}

qlora_status qlora_dequantize(const qlora_nf4* w, uint16_t* out, void* stream) {
    qlora_status st = check_state(w);
    if (st != QLORA_OK) return st;
    if (!out) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(out)) return QLORA_ERR_MISALIGNED;
    return launch_dequantize(w->codes, w->q8, w->a2, w->n * w->k / kBlock, out, (hipStream_t)stream);
}

}  // extern "C"
