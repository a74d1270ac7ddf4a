/*
 * qlora.h -- C ABI of the NF4 frozen-base linear layer with a LoRA branch,
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * What it computes (web pages on QLoRA / NF4 / bitsandbytes):
 *  - "bitsandbytes deep dive" (aicoding.csdn.net), section 5.2: blockwise
 *    absmax 4-bit encoding, a = max|w| per block of 64, q = argmin_j |w/a - c_j|,
 *    w_hat = a * c_q, two 4-bit codes per byte;
 *  - same page, section 6.2: the 16 NF4 levels c_j (normal quantiles,
 *    normalised to [-1, 1], asymmetric, exact 0);
 *  - same page, section 7.2: double quantization -- the block absmax values
 *    are stored as 8-bit codes, with one fp32 scale per 256 blocks;
 *  - same page, sections 8.6 / 12.4, and "LoRA, QLoRA, QA-LoRA explained"
 *    (ludovicoyin.github.io), section 2: y = x dequant(W4) + (alpha/r) x A B
 *    with the dequantization fused into the matrix product, frozen base.
 *
 * Conventions shared by every entry point
 *  - Weight storage is the nn.Linear layout [N = Dout, K = Din], row-major,
 *    flattened row-major into blocks of 64 consecutive elements (K % 64 == 0,
 *    so no block straddles a row).  Block b covers flat elements
 *    [64 b, 64 b + 64); scale group S covers blocks [256 S, 256 S + 256), the
 *    last group may be short and groups may straddle rows.
 *  - Packed codes: element 2i in bits 7..4 and element 2i+1 in bits 3..0 of
 *    byte i.
 *  - bf16 tensors are passed as uint16_t bit patterns; every matrix is dense
 *    row-major with no padding; all tensor pointers are DEVICE pointers,
 *    16-byte aligned, owned by the caller.  The library allocates nothing and
 *    keeps no mutable global state.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every compute call
 *    only validates and enqueues: a return of QLORA_OK means the kernels were
 *    launched, not that they finished.  Inputs must be finite.
 *  - Errors: invalid arguments are reported before anything is launched and
 *    leave every output untouched.  No C++ exception crosses the ABI.
 *  - Reentrant; calls on different streams may run concurrently as long as
 *    they do not share output or workspace buffers.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qlora_status {
    QLORA_OK = 0,
    QLORA_ERR_INVALID_ARG = -1,       /* null pointer, negative size, r or alpha out of range */
    QLORA_ERR_UNSUPPORTED_SHAPE = -2, /* K % 64 != 0, sizes beyond the supported range */
    QLORA_ERR_MISALIGNED = -3,        /* a tensor pointer is not 16-byte aligned */
    QLORA_ERR_WORKSPACE = -4,         /* workspace missing or smaller than required */
    QLORA_ERR_HIP = -5                /* a HIP launch error was reported */
} qlora_status;

/* Quantized weight: flat device arrays plus the logical shape.  This is the
 * "quantization state" the deep dive (section 5.2) says is kept next to the
 * codes.  With double quantization (section 7.2; q8 != NULL): codes, the
 * first-level 8-bit scale codes and the second-level fp32 scales.  Without it
 * (sections 7.1 and 9.5; q8 == NULL): codes and one fp32 absmax per 64-block
 * in a2, 4.5 bits per weight.  Every entry point taking a qlora_nf4 accepts
 * both; a2 is never NULL. */
/* The 4-bit codebook: what value each code 0..15 stands for (deep dive 8.1,
 * the quant type).
 *  - NF4: the 16 normal-quantile levels of section 6.2, ascending with the code.
 *  - FP4: a floating-point-style codebook (section 6.5), whose values the page
 *    does not give.  Taken as the 4-bit float E2M1 of the OCP MX formats
 *    (bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa, subnormals at
 *    exponent 0), divided by its largest magnitude 6:
 *      c = +-{0, 1/12, 1/6, 1/4, 1/3, 1/2, 2/3, 1}, each rounded to fp32,
 *    and the code is the E2M1 bit pattern.
 * Both encode to the nearest level of w/a, ties to the lower level.  For FP4 a
 * zero weight (either sign) encodes as +0 (code 0); code 8 (-0) decodes to -0
 * but is never produced.  Everything else is the same for both. */
typedef enum qlora_quant_type { QLORA_QUANT_NF4 = 0, QLORA_QUANT_FP4 = 1 } qlora_quant_type;

/* The compute dtype (deep dive 8.3: fp32, bf16 or fp16; bf16 recommended): the
 * 16-bit float format of every 16-bit tensor exchanged with a layer -- the
 * weight given to qlora_quantize, the output of qlora_dequantize and
 * qlora_merge, and x, A, B, y, t, dy, dx of the layer calls.  bf16 (the
 * default, zero-initialised) or IEEE binary16.  Dequantized weights are
 * RNE_16(fl32(a_hat * c_q)) in that format and the products run on the MFMA
 * instruction of that type with fp32 accumulation; dA and dB stay fp32.
 * Where the text below says bf16, read "the compute dtype".
 * QLORA_DTYPE_F32: every floating-point tensor of the layer is IEEE binary32
 * and the dequantized weight is the fp32 product fl32(a_hat * c_q) itself,
 * with no 16-bit rounding.  Such a state is used through the _f32 entry points
 * below (float tensors), which take no other dtype; the 16-bit entry points
 * reject it with INVALID_ARG.  qlora_dequantize_f32 takes every dtype. */
typedef enum qlora_dtype { QLORA_DTYPE_BF16 = 0, QLORA_DTYPE_F16 = 1, QLORA_DTYPE_F32 = 2 } qlora_dtype;

typedef struct qlora_nf4 {
    uint8_t* codes;     /* [N*K/2]            packed 4-bit codes                         */
    uint8_t* q8;        /* [N*K/64]           8-bit code of each block's absmax, or NULL */
    float* a2;          /* [ceil(N*K/16384)]  fp32 absmax of each group of 256 absmaxes; */
                        /* [N*K/64] fp32 absmax of each block when q8 == NULL            */
    int64_t n;          /* N = Dout (rows of the stored weight)                          */
    int64_t k;          /* K = Din, a multiple of 64                                     */
    int32_t quant_type; /* a qlora_quant_type; 0 (zero-initialised) is NF4. Any other   */
                        /* value -> QLORA_ERR_INVALID_ARG                                */
    int32_t dtype;      /* a qlora_dtype; 0 (zero-initialised) is bf16. Any other value  */
                        /* -> QLORA_ERR_INVALID_ARG; fp32 only through the _f32 calls    */
} qlora_nf4;

/* Library version (major*10000 + minor*100 + patch). */
int qlora_version(void);

/* Static English text for a status code (never NULL). */
const char* qlora_status_string(int status);

/* Byte sizes of the three arrays of an [N, K] quantized weight:
 *   codes N*K/2, q8 N*K/64, a2 4*ceil(N*K/16384)
 * (deep dive 7.2: 4 + 8/64 + 32/(64*256) bits per weight).  Any output
 * pointer may be NULL.  Errors: N < 1 or K < 1 -> INVALID_ARG, K % 64 -> UNSUPPORTED_SHAPE. */
qlora_status qlora_nf4_sizes(int64_t N, int64_t K, size_t* codes_bytes, size_t* q8_bytes,
                             size_t* a2_bytes);

/* Byte sizes of the two arrays of an [N, K] weight quantized without double
 * quantization (deep dive 7.1: 4 + 32/64 bits per weight): codes N*K/2, fp32
 * block absmax 4*N*K/64.  Errors as qlora_nf4_sizes. */
qlora_status qlora_nf4_sizes_nodq(int64_t N, int64_t K, size_t* codes_bytes, size_t* absmax_bytes);

/* Quantize a bf16 weight W [N, K] into `out` (deep dive 5.2 and 7.2).
 *   a_b  = max |w| over block b
 *   code = argmin_j |w/a_b - c_j| in exact arithmetic, ties to the lower j;
 *          a_b = 0 gives the zero code 7
 *   a2_S = max of a_b over group S
 *   q8_b = argmin_k |a_b/a2_S - k/255| over k = 0..255, ties to the lower k
 * out->codes/q8/a2 must hold qlora_nf4_sizes() bytes; out->n/k must equal N/K.
 * Codes are computed against the true a_b, not its 8-bit reconstruction.
 * out->q8 == NULL quantizes without double quantization: a2[b] = a_b (fp32),
 * sized by qlora_nf4_sizes_nodq(); the codes are the same. */
qlora_status qlora_quantize(const uint16_t* W, int64_t N, int64_t K, const qlora_nf4* out,
                            void* stream);

/* Quantize `count` bf16/fp16 weights at once (deep dive 5.2 and 7.2, as
 * qlora_quantize): W[i] [out[i].n, out[i].k] into out[i], for i < count.
 * `out` is an array of count states (not pointers).  The results are those of
 * count calls of qlora_quantize; consecutive weights that share quant_type,
 * dtype and double quantization (all q8 set or all NULL) run as one launch of
 * up to 16 weights, so the chip streams across the weights of a training step
 * instead of ramping up and draining once per weight.  count == 0 is a no-op.
 * Errors: count < 0, null arrays or entries, a state qlora_quantize rejects
 * (checked for every entry before anything is launched), misaligned W[i]. */
qlora_status qlora_quantize_batch(const uint16_t* const* W, const qlora_nf4* out, int count, void* stream);

/* Dequantize to bf16 out [N, K] (deep dive 5.2: w_hat = a * c_q):
 *   a_hat = fl32( fl32(a2_S / 255) * q8_b ) (out->q8 == NULL: a_hat = a2_b),
 *   out = RNE_bf16( fl32(a_hat * c_code) ).
 * For tests and export only: the linear layer never materialises W. */
qlora_status qlora_dequantize(const qlora_nf4* w, uint16_t* out, void* stream);

/* Dequantize to fp32 out [N, K] (deep dive 5.2 with the fp32 compute dtype of
 * section 8.3): out = fl32(a_hat * c_code), the product itself, with no 16-bit
 * rounding (RNE_bf16 of it is what qlora_dequantize writes for a bf16 state).
 * Either scale layout and codebook; w->dtype is not used.  out 16-byte aligned;
 * NULL -> INVALID_ARG. */
qlora_status qlora_dequantize_f32(const qlora_nf4* w, float* out, void* stream);

/* LoRA merge for deployment ("LoRA, QLoRA, QA-LoRA explained", section 2:
 * W_eff = dequant(W4) + (alpha/r) A B; "bitsandbytes deep dive", section 12.10:
 * merge in higher precision, re-quantize afterwards if a 4-bit model is wanted,
 * which adds error of its own).  In the stored layout, bf16 out [N, K]:
 *   out[n, k] = RNE_bf16( fl32( w_hat[n, k] + fl32( fl32(alpha/r) * acc[n, k] ) ) ),
 *   acc[n, k] = fp32 sum over j = 0 .. r-1, in that order, of A[k, j] * B[j, n],
 * w_hat as qlora_dequantize.  w: either scale layout; A [K, r] and B [r, N] bf16.
 * Re-quantize with qlora_quantize(out, ...).  Errors: null pointer, r outside
 * 1..128 or non-finite alpha -> INVALID_ARG; unaligned pointer -> MISALIGNED. */
qlora_status qlora_merge(const qlora_nf4* w, const uint16_t* A, const uint16_t* B, int r, float alpha,
                         uint16_t* out, void* stream);

/* Workspace bytes qlora_linear_fwd needs for these sizes (0 if none). */
size_t qlora_fwd_workspace(int64_t M, int64_t N, int64_t K, int r);

/* Fused forward of the frozen NF4 linear with its LoRA branch
 * (deep dive 12.4; explained, section 2):
 *   t = s * (x A)            [M, r]  bf16, s = alpha / r
 *   y = x W_hat + t B        [M, N]  bf16, W_hat = [K, N] view of dequant(w)
 * x [M, K] bf16, A [K, r] bf16, B [r, N] bf16.  The products accumulate in
 * fp32; W_hat is dequantized inside the kernels (registers / LDS tiles) and is
 * never written to memory.  t_out (nullable) receives t for the backward.
 * 1 <= r <= 128, M >= 0 (M = 0 is a no-op), alpha finite.  ws may be NULL when
 * qlora_fwd_workspace() returns 0. */
qlora_status qlora_linear_fwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float alpha, uint16_t* y, uint16_t* t_out,
                              void* ws, size_t ws_bytes, void* stream);

/* Measurement aid, not a step of the layer: reads `bytes` of src through registers
 * with coalesced 16-byte loads and nothing else (one store to sink that never
 * happens keeps the loads alive); the bench reports the decode forward next to
 * this same-size plain read.  variant 0: 256-thread workgroups, 4 loads per lane;
 * 1: 512 threads, 8 loads.  src and sink 16-byte aligned, 0 < bytes < 2^31,
 * otherwise INVALID_ARG / MISALIGNED. */
qlora_status qlora_read_probe(const void* src, size_t bytes, uint32_t* sink, int variant, void* stream);

/* qlora_linear_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no workspace
 * argument and allocates nothing; its workspace is a fixed array of
 * QLORA_NOALLOC_SCRATCH_BYTES in the library's device memory, one per GPU, held until the
 * process ends.  Same arguments (without ws), results and errors as qlora_linear_fwd,
 * plus: sizes whose qlora_fwd_workspace() exceeds QLORA_NOALLOC_SCRATCH_BYTES ->
 * QLORA_ERR_WORKSPACE; the device address of the array not available -> QLORA_ERR_HIP.
 * Every call on one GPU uses the same array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be ordered by the caller. */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
qlora_status qlora_linear_fwd_noalloc(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A,
                                      const uint16_t* B, int r, float alpha, uint16_t* y, uint16_t* t_out,
                                      void* stream);

/* The two stages of qlora_linear_fwd, for callers that keep t across calls
 * or time the stages separately.  Above decode sizes qlora_linear_fwd is
 * exactly qlora_lora_down followed by qlora_fused_gemm_fwd, and given the t
 * that qlora_linear_fwd returns, qlora_fused_gemm_fwd reproduces its y bit for
 * bit.  At decode sizes (M <= 16, where one launch computes t and y) the layer
 * call may split the weight's rows into taller tiles than the kernel with t
 * given (it leaves CUs to the producers of t), which adds y's fp32 partial sums
 * in another order: y may then differ in the last bit.  Its t adds the fp32
 * products of x A in another order than qlora_lora_down, so t may also differ
 * from qlora_lora_down's in the last bit. */

/* Workspace bytes qlora_lora_down needs (0 for M == 0). */
size_t qlora_lora_down_workspace(int64_t M, int64_t K, int r);

/* t = s * (x A) as bf16 [M, r], s = alpha / r (the LoRA down-projection,
 * deep dive 12.2).  x [M, K] bf16 (K % 64 == 0), A [K, r] bf16, 1 <= r <= 128.
 * dtype: a qlora_dtype, the format of x, A and t (this call takes no weight
 * state to carry it); any other value -> QLORA_ERR_INVALID_ARG. */
qlora_status qlora_lora_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* A, int r, float alpha,
                             int dtype, uint16_t* t_out, void* ws, size_t ws_bytes, void* stream);

/* y = x W_hat + t B as bf16 [M, N]: the fused dequant GEMM with the LoRA
 * up-projection folded in as r extra reduction steps.  t [M, r] bf16 (already
 * scaled), B [r, N] bf16.  No workspace.  One kernel launch. */
qlora_status qlora_fused_gemm_fwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* t,
                                  const uint16_t* B, int r, uint16_t* y, void* stream);

/* Workspace bytes qlora_linear_bwd needs for these sizes. */
size_t qlora_bwd_workspace(int64_t M, int64_t N, int64_t K, int r);

/* Backward of the same layer for an upstream gradient dy [M, N] bf16.  The
 * base weight is frozen (deep dive 12.4): there is no dW.  By the chain rule:
 *   u  = s * (dy B^T)           [M, r]   (internal, workspace)
 *   dx = dy W_hat^T + u A^T     [M, K]   bf16 (skipped when dx == NULL)
 *   dA = x^T u                  [K, r]   fp32, overwritten
 *   dB = t^T dy                 [r, N]   fp32, overwritten
 * t is the forward's t_out (nullable: then it is recomputed from x and A). */
qlora_status qlora_linear_bwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float alpha, const uint16_t* t,
                              const uint16_t* dy, uint16_t* dx, float* dA, float* dB, void* ws,
                              size_t ws_bytes, void* stream);

/* The dx stage of qlora_linear_bwd alone, for a given u:
 *   dx = dy W_hat^T + u A^T    [M, K]  bf16
 * with u = s dy B^T [M, r] bf16 already scaled (s = alpha / r), A [K, r] bf16,
 * dy [M, N] bf16.  One kernel launch (the fused dequant GEMM of the backward
 * with the LoRA term folded in as r extra reduction steps), no workspace.
 * Arguments and errors as qlora_linear_bwd; M = 0 is a no-op. */
qlora_status qlora_fused_gemm_bwd_dx(const qlora_nf4* w, const uint16_t* dy, int64_t M, const uint16_t* u,
                                     const uint16_t* A, int r, uint16_t* dx, void* stream);

/* The backward split in two for callers that defer the LoRA weight gradients
 * to the end of the backward pass (deep dive 12.4: with the base frozen, dA
 * and dB are needed only by the optimizer step, while dx feeds the layer
 * below).  qlora_linear_bwd_dx computes the part of qlora_linear_bwd that the
 * layer below waits for:
 *   u  = s * (dy B^T)           [M, r]   bf16, into the caller's u (kept for
 *                                        qlora_lora_grads_batch)
 *   dx = dy W_hat^T + u A^T     [M, K]   bf16
 * and qlora_lora_grads_batch computes, for `count` layers in one launch of up
 * to 8 layers,
 *   dA = x^T u   [K, r] fp32,   dB = t^T dy   [r, N] fp32 (overwritten),
 * with t the forward's t_out.  Both give bit for bit the u, dx, dA and dB of
 * qlora_linear_bwd on the same inputs (the same kernels, split plans and
 * summation orders).  One launch streams the x and dy of all the layers back to
 * back instead of ramping up and draining once per layer.  Errors as
 * qlora_linear_bwd; M == 0: linear_bwd_dx does nothing, grads_batch writes
 * zeros.  qlora_lora_grads_batch: count < 0, r outside [1, 128], a dtype other
 * than bf16 / fp16 (the format of x, t, u and dy) or a null array ->
 * INVALID_ARG; every entry is checked before anything is launched; count == 0
 * is a no-op.  Its workspace (the split sums of each contraction) is caller
 * owned and needs no clearing. */
typedef struct qlora_lora_grads {
    const uint16_t* x;  /* [M, K] the layer's input                 */
    const uint16_t* t;  /* [M, r] the forward's t = s x A           */
    const uint16_t* u;  /* [M, r] u = s dy B^T (qlora_linear_bwd_dx) */
    const uint16_t* dy; /* [M, N] the upstream gradient              */
    float* dA;          /* [K, r] fp32 out                           */
    float* dB;          /* [r, N] fp32 out                           */
    int64_t M, N, K;
} qlora_lora_grads;

size_t qlora_linear_bwd_dx_workspace(int64_t M, int64_t N, int64_t K, int r);
qlora_status qlora_linear_bwd_dx(const qlora_nf4* w, int64_t M, const uint16_t* A, const uint16_t* B, int r,
                                 float alpha, const uint16_t* dy, uint16_t* u, uint16_t* dx, void* ws,
                                 size_t ws_bytes, void* stream);
size_t qlora_lora_grads_batch_workspace(const qlora_lora_grads* layers, int count, int r);
qlora_status qlora_lora_grads_batch(const qlora_lora_grads* layers, int count, int r, int dtype, void* ws,
                                    size_t ws_bytes, void* stream);

/* The LoRA products of several layers in one launch of up to 8 (deep dive
 * 12.2: the rank-r side path s x A B and its chain rule), for the layers whose
 * inputs are ready together: in a decoder block q, k and v share x, and gate
 * and up share theirs (and, in the backward, receive their dy together).
 *   qlora_lora_down_batch: out_i = s x_i A_i      [M_i, r] (A_i [C_i, r], the
 *                          t of qlora_lora_down; C_i % 64 == 0 else
 *                          UNSUPPORTED_SHAPE)
 *   qlora_lora_u_batch:    out_i = s dy_i B_i^T   [M_i, r] (B_i [r, C_i], the u
 *                          of qlora_linear_bwd_dx)
 * with s = alpha / r, bf16 or fp16 (dtype) in and out.  Each output is bit for
 * bit that of the single-layer call (the same kernel body, split plan and
 * summation order).  count == 0 and M_i == 0 do nothing.  Errors: count < 0, r
 * outside [1, 128], non-finite alpha, another dtype, a null array or entry ->
 * INVALID_ARG (every entry checked before anything is launched); misaligned
 * tensors; the workspace (caller owned, no clearing needed) missing or short. */
typedef struct qlora_lora_prod {
    const uint16_t* x;  /* [M, C]: x (down) or dy (u)          */
    const uint16_t* w;  /* A [C, r] (down) or B [r, C] (u)     */
    uint16_t* out;      /* [M, r]                               */
    int64_t M, C;
} qlora_lora_prod;

size_t qlora_lora_prod_batch_workspace(const qlora_lora_prod* items, int count, int r);
qlora_status qlora_lora_down_batch(const qlora_lora_prod* items, int count, int r, float alpha, int dtype, void* ws,
                                   size_t ws_bytes, void* stream);
qlora_status qlora_lora_u_batch(const qlora_lora_prod* items, int count, int r, float alpha, int dtype, void* ws,
                                size_t ws_bytes, void* stream);

/* fp32 compute dtype (deep dive 8.3 lists fp32 beside bf16 and fp16).  The
 * state's dtype must be QLORA_DTYPE_F32 (else INVALID_ARG); every tensor is
 * float, 16-byte aligned.  Definitions, arguments and errors are those of the
 * 16-bit calls with bf16 read as fp32:
 *   qlora_quantize_f32:   codes against the true absmax of fp32 W [N, K]; for
 *                         fp32 weights w > X <=> w > RD_f32(X), so the exact
 *                         thresholds are fp32 values.  Scales as qlora_quantize.
 *   qlora_linear_fwd_f32: t = s x A, y = x W_hat + t B, with W_hat =
 *                         fl32(a_hat * c_q); products on the fp32 matrix cores
 *                         with fp32 accumulation.
 *   qlora_linear_bwd_f32: u = s dy B^T, dx = dy W_hat^T + u A^T, dA = x^T u,
 *                         dB = t^T dy, all fp32.
 * Contractions with few output tiles split their reduction into fp32 partial
 * sums in the workspace, added in a fixed order: results are deterministic.
 * The decode GEMV, the merge, the pooled branch and the stage entry points are
 * offered for the 16-bit dtypes only. */
qlora_status qlora_quantize_f32(const float* W, int64_t N, int64_t K, const qlora_nf4* out, void* stream);
size_t qlora_fwd_workspace_f32(int64_t M, int64_t N, int64_t K, int r);
qlora_status qlora_linear_fwd_f32(const qlora_nf4* w, const float* x, int64_t M, const float* A, const float* B,
                                  int r, float alpha, float* y, float* t_out, void* ws, size_t ws_bytes,
                                  void* stream);
size_t qlora_bwd_workspace_f32(int64_t M, int64_t N, int64_t K, int r);
qlora_status qlora_linear_bwd_f32(const qlora_nf4* w, const float* x, int64_t M, const float* A, const float* B,
                                  int r, float alpha, const float* t, const float* dy, float* dx, float* dA,
                                  float* dB, void* ws, size_t ws_bytes, void* stream);

/* QA-LoRA pooled branch ("LoRA, QLoRA, QA-LoRA explained", sections 3-5): the
 * LoRA input is pool(x), the mean of each group of g consecutive input
 * columns, and A is [K/g, r]:
 *   y = x W_hat + s pool(x) A B,   t = s pool(x) A,   s = alpha / r.
 * Backward: u = s dy B^T, dx = dy W_hat^T + (u A^T repeated over each group) / g,
 * dA = pool(x)^T u [K/g, r] (fp32), dB = t^T dy.  g must be a power of two
 * dividing K (g = 1 is the plain layer).  Implementation: pool(x) A = x A~ with
 * A~[k, j] = A[k/g, j] / g, exact in bf16 unless it underflows, so the plain
 * kernels run on A~ (kept in the workspace); dA sums each group of g rows of
 * the gradient of A~, in fp32 in row order.  Arguments and errors as qlora_linear_fwd / _bwd, plus
 * a g that is not a power of two dividing K -> INVALID_ARG.  The workspace
 * queries return 0 for invalid sizes. */
size_t qlora_pooled_fwd_workspace(int64_t M, int64_t N, int64_t K, int r, int g);
qlora_status qlora_pooled_fwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, int g, float alpha, uint16_t* y,
                              uint16_t* t_out, void* ws, size_t ws_bytes, void* stream);
size_t qlora_pooled_bwd_workspace(int64_t M, int64_t N, int64_t K, int r, int g);
qlora_status qlora_pooled_bwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, int g, float alpha, const uint16_t* t,
                              const uint16_t* dy, uint16_t* dx, float* dA, float* dB, void* ws,
                              size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
