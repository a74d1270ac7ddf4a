"""Thin ctypes binding over libqlora.so (include/qlora.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
Importing this module loads the library and raises ImportError when it has not
been built (python -m bit_nf4_quantized_15_amd.build); there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "qlora.h")

BLOCK = 64
SUPER = 256

c_i64 = ctypes.c_int64
c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t


class NF4State(ctypes.Structure):
    """Mirror of struct qlora_nf4."""
    _fields_ = [("codes", c_vp), ("q8", c_vp), ("a2", c_vp), ("n", c_i64), ("k", c_i64), ("quant_type", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class LoraGrads(ctypes.Structure):
    """Mirror of struct qlora_lora_grads."""
    _fields_ = [("x", c_vp), ("t", c_vp), ("u", c_vp), ("dy", c_vp), ("dA", c_vp), ("dB", c_vp), ("M", c_i64),
                ("N", c_i64), ("K", c_i64)]


class LoraProd(ctypes.Structure):
    """Mirror of struct qlora_lora_prod."""
    _fields_ = [("x", c_vp), ("w", c_vp), ("out", c_vp), ("M", c_i64), ("C", c_i64)]


QUANT_TYPES = {"nf4": 0, "fp4": 1}                        # qlora_quant_type: the 4-bit codebook
DTYPES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}   # qlora_dtype: the compute dtype


def _dtype_code(dtype):
    if dtype not in DTYPES:
        raise TypeError(f"compute dtype must be torch.bfloat16, torch.float16 or torch.float32, got {dtype}")
    return DTYPES[dtype]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_nf4_quantized_15_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(NF4State)
    sig = {
        "qlora_version": (ctypes.c_int, []),
        "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "qlora_nf4_sizes": (ctypes.c_int, [c_i64, c_i64, ctypes.POINTER(c_sz), ctypes.POINTER(c_sz),
                                           ctypes.POINTER(c_sz)]),
        "qlora_nf4_sizes_nodq": (ctypes.c_int, [c_i64, c_i64, ctypes.POINTER(c_sz), ctypes.POINTER(c_sz)]),
        "qlora_quantize": (ctypes.c_int, [c_vp, c_i64, c_i64, P, c_vp]),
        "qlora_quantize_batch": (ctypes.c_int, [ctypes.POINTER(c_vp), P, ctypes.c_int, c_vp]),
        "qlora_dequantize": (ctypes.c_int, [P, c_vp, c_vp]),
        "qlora_dequantize_f32": (ctypes.c_int, [P, c_vp, c_vp]),
        "qlora_merge": (ctypes.c_int, [P, c_vp, c_vp, ctypes.c_int, ctypes.c_float, c_vp, c_vp]),
        "qlora_fwd_workspace": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int]),
        "qlora_linear_fwd": (ctypes.c_int, [P, c_vp, c_i64, c_vp, c_vp, ctypes.c_int, ctypes.c_float,
                                            c_vp, c_vp, c_vp, c_sz, c_vp]),
        "qlora_linear_fwd_noalloc": (ctypes.c_int, [P, c_vp, c_i64, c_vp, c_vp, ctypes.c_int, ctypes.c_float,
                                                    c_vp, c_vp, c_vp]),
        "qlora_read_probe": (ctypes.c_int, [c_vp, c_sz, c_vp, ctypes.c_int, c_vp]),
        "qlora_lora_down_workspace": (c_sz, [c_i64, c_i64, ctypes.c_int]),
        "qlora_lora_down": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                           c_vp, c_vp, c_sz, c_vp]),
        "qlora_fused_gemm_fwd": (ctypes.c_int, [P, c_vp, c_i64, c_vp, c_vp, ctypes.c_int, c_vp, c_vp]),
        "qlora_fused_gemm_bwd_dx": (ctypes.c_int, [P, c_vp, c_i64, c_vp, c_vp, ctypes.c_int, c_vp, c_vp]),
        "qlora_pooled_fwd_workspace": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int, ctypes.c_int]),
        "qlora_pooled_fwd": (ctypes.c_int, [P, c_vp, c_i64, c_vp, c_vp, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                            c_vp, c_vp, c_vp, c_sz, c_vp]),
        "qlora_pooled_bwd_workspace": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int, ctypes.c_int]),
        "qlora_pooled_bwd": (ctypes.c_int, [P, c_vp, c_i64, c_vp, c_vp, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                            c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
        "qlora_bwd_workspace": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int]),
        "qlora_linear_bwd": (ctypes.c_int, [P, c_vp, c_i64, c_vp, c_vp, ctypes.c_int, ctypes.c_float,
                                            c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
        "qlora_linear_bwd_dx_workspace": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int]),
        "qlora_linear_bwd_dx": (ctypes.c_int, [P, c_i64, c_vp, c_vp, ctypes.c_int, ctypes.c_float, c_vp, c_vp, c_vp,
                                               c_vp, c_sz, c_vp]),
        "qlora_lora_grads_batch_workspace": (c_sz, [ctypes.POINTER(LoraGrads), ctypes.c_int, ctypes.c_int]),
        "qlora_lora_grads_batch": (ctypes.c_int, [ctypes.POINTER(LoraGrads), ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int, c_vp, c_sz, c_vp]),
        "qlora_lora_prod_batch_workspace": (c_sz, [ctypes.POINTER(LoraProd), ctypes.c_int, ctypes.c_int]),
        "qlora_lora_down_batch": (ctypes.c_int, [ctypes.POINTER(LoraProd), ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_float, ctypes.c_int, c_vp, c_sz, c_vp]),
        "qlora_lora_u_batch": (ctypes.c_int, [ctypes.POINTER(LoraProd), ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                              ctypes.c_int, c_vp, c_sz, c_vp]),
        "qlora_quantize_f32": (ctypes.c_int, [c_vp, c_i64, c_i64, P, c_vp]),
        "qlora_fwd_workspace_f32": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int]),
        "qlora_linear_fwd_f32": (ctypes.c_int, [P, c_vp, c_i64, c_vp, c_vp, ctypes.c_int, ctypes.c_float,
                                                c_vp, c_vp, c_vp, c_sz, c_vp]),
        "qlora_bwd_workspace_f32": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int]),
        "qlora_linear_bwd_f32": (ctypes.c_int, [P, c_vp, c_i64, c_vp, c_vp, ctypes.c_int, ctypes.c_float,
                                                c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name, None)
        if fn is None:
            continue
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class QLoraError(RuntimeError):
    def __init__(self, status, where):
        msg = lib.qlora_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status


def _empty(*shape, dtype, device):
    """Every buffer this module hands to the library is allocated here (outputs, weight state and workspace).
    Uninitialised, like torch.empty; the GPU tests replace `empty_hook` to fill new buffers with a poison
    pattern, so that an element a kernel never writes cannot pass for a correct one."""
    return empty_hook(*shape, dtype=dtype, device=device)


empty_hook = torch.empty


def _check(status, where):
    if status != 0:
        raise QLoraError(status, where)


def _stream():
    return c_vp(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else c_vp(t.data_ptr())


def _dev(t, dtype, name, shape=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def sizes(N, K):
    """(codes bytes, q8 bytes, a2 bytes) of an [N, K] quantized weight."""
    cb, qb, ab = c_sz(), c_sz(), c_sz()
    _check(lib.qlora_nf4_sizes(N, K, ctypes.byref(cb), ctypes.byref(qb), ctypes.byref(ab)), "qlora_nf4_sizes")
    return cb.value, qb.value, ab.value


def sizes_nodq(N, K):
    """(codes bytes, fp32 block-absmax bytes) of an [N, K] weight quantized without double quantization."""
    cb, ab = c_sz(), c_sz()
    _check(lib.qlora_nf4_sizes_nodq(N, K, ctypes.byref(cb), ctypes.byref(ab)), "qlora_nf4_sizes_nodq")
    return cb.value, ab.value


class NF4Weight:
    """Device-resident quantized weight: codes (uint8), q8 (uint8) and a2 (float32) tensors; without
    double quantization q8 is None and a2 holds one fp32 absmax per 64-block.  quant_type names the
    4-bit codebook ("nf4" or "fp4"); dtype is the compute dtype of every float tensor used with it
    (torch.bfloat16, torch.float16, or torch.float32: then the layer calls take the _f32 entry points and the
    dequantized weight is the fp32 product itself)."""

    def __init__(self, codes, q8, a2, N, K, quant_type="nf4", dtype=torch.bfloat16):
        if quant_type not in QUANT_TYPES:
            raise ValueError(f"quant_type must be one of {sorted(QUANT_TYPES)}, got {quant_type!r}")
        _dtype_code(dtype)
        self.codes, self.q8, self.a2, self.N, self.K = codes, q8, a2, int(N), int(K)
        self.quant_type, self.dtype = quant_type, dtype

    @property
    def double_quant(self):
        return self.q8 is not None

    @classmethod
    def empty(cls, N, K, device="cuda", double_quant=True, quant_type="nf4", dtype=torch.bfloat16):
        if not double_quant:
            cb, ab = sizes_nodq(N, K)
            return cls(_empty(cb, dtype=torch.uint8, device=device), None,
                       _empty(ab // 4, dtype=torch.float32, device=device), N, K, quant_type, dtype)
        cb, qb, ab = sizes(N, K)
        return cls(_empty(cb, dtype=torch.uint8, device=device),
                   _empty(qb, dtype=torch.uint8, device=device),
                   _empty(ab // 4, dtype=torch.float32, device=device), N, K, quant_type, dtype)

    def state(self):
        q8 = None if self.q8 is None else self.q8.data_ptr()
        return NF4State(self.codes.data_ptr(), q8, self.a2.data_ptr(), self.N, self.K, QUANT_TYPES[self.quant_type],
                        _dtype_code(self.dtype))


def quantize(W, out=None, double_quant=True, quant_type="nf4"):
    """4-bit blockwise quantization of a bf16, fp16 or fp32 [N, K] device weight (qlora_quantize, or
    qlora_quantize_f32 for fp32) with the NF4 or the FP4 codebook, with or without double quantization of
    the block scales (both ignored when `out` is given: its layout and quant_type decide).  W's dtype
    becomes the weight's compute dtype."""
    N, K = W.shape
    _dtype_code(W.dtype)
    _dev(W, W.dtype, "W")
    w = NF4Weight.empty(N, K, W.device, double_quant, quant_type, W.dtype) if out is None else out
    if w.dtype != W.dtype:
        raise TypeError(f"out has compute dtype {w.dtype}, W is {W.dtype}")
    st = w.state()
    if W.dtype == torch.float32:
        _check(lib.qlora_quantize_f32(_ptr(W), N, K, ctypes.byref(st), _stream()), "qlora_quantize_f32")
    else:
        _check(lib.qlora_quantize(_ptr(W), N, K, ctypes.byref(st), _stream()), "qlora_quantize")
    return w


def quantize_batch(Ws, outs):
    """Quantize bf16/fp16 device weights Ws[i] into the existing NF4Weight outs[i] (qlora_quantize_batch:
    the results of one qlora_quantize per weight, in one launch per run of up to 16 weights that share
    their configuration)."""
    if len(Ws) != len(outs):
        raise ValueError("Ws and outs differ in length")
    for W, w in zip(Ws, outs):
        _dtype_code(W.dtype)
        _dev(W, w.dtype, "W", (w.N, w.K))
    n = len(Ws)
    ptrs = (c_vp * max(n, 1))(*[_ptr(W) for W in Ws])
    states = (NF4State * max(n, 1))(*[w.state() for w in outs])
    _check(lib.qlora_quantize_batch(ptrs, states, n, _stream()), "qlora_quantize_batch")
    return outs


def dequantize(w, out=None, fp32=False):
    """[N, K] reconstruction in the weight's compute dtype (qlora_dequantize), or with fp32=True the fp32
    products themselves (qlora_dequantize_f32, also the reconstruction of an fp32 weight); tests and export
    only."""
    fp32 = fp32 or w.dtype == torch.float32
    dt = torch.float32 if fp32 else w.dtype
    o = _empty((w.N, w.K), dtype=dt, device=w.codes.device) if out is None else out
    _dev(o, dt, "out", (w.N, w.K))
    st = w.state()
    if fp32:
        _check(lib.qlora_dequantize_f32(ctypes.byref(st), _ptr(o), _stream()), "qlora_dequantize_f32")
    else:
        _check(lib.qlora_dequantize(ctypes.byref(st), _ptr(o), _stream()), "qlora_dequantize")
    return o


def merge(w, A, B, alpha, out=None):
    """LoRA merge for deployment (qlora_merge): bf16 [N, K] = w_hat + (alpha/r) (A B)^T.
    Re-quantize with quantize(out)."""
    K, r = A.shape
    _dev(A, w.dtype, "A", (w.K, r))
    _dev(B, w.dtype, "B", (r, w.N))
    o = _empty((w.N, w.K), dtype=w.dtype, device=A.device) if out is None else out
    _dev(o, w.dtype, "out", (w.N, w.K))
    st = w.state()
    _check(lib.qlora_merge(ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha), _ptr(o), _stream()), "qlora_merge")
    return o


def fwd_workspace(M, N, K, r, dtype=torch.bfloat16):
    if dtype == torch.float32:
        return int(lib.qlora_fwd_workspace_f32(M, N, K, r))
    return int(lib.qlora_fwd_workspace(M, N, K, r))


def bwd_workspace(M, N, K, r, dtype=torch.bfloat16):
    if dtype == torch.float32:
        return int(lib.qlora_bwd_workspace_f32(M, N, K, r))
    return int(lib.qlora_bwd_workspace(M, N, K, r))


def _ws(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is not None and ws.numel() >= nbytes:
        return ws, ws.numel()
    return _empty(nbytes, dtype=torch.uint8, device=device), nbytes


def linear_fwd(w, x, A, B, alpha, y=None, t=None, want_t=True, ws=None):
    """y = x W_hat + (alpha/r)(x A) B (qlora_linear_fwd).  Returns (y, t or None)."""
    M, K = x.shape
    r = A.shape[1]
    _dev(x, w.dtype, "x", (M, w.K))
    _dev(A, w.dtype, "A", (w.K, r))
    _dev(B, w.dtype, "B", (r, w.N))
    dev = x.device
    y = _empty((M, w.N), dtype=w.dtype, device=dev) if y is None else _dev(y, w.dtype, "y", (M, w.N))
    if want_t and t is None:
        t = _empty((M, r), dtype=w.dtype, device=dev)
    if t is not None:
        _dev(t, w.dtype, "t", (M, r))
    wsb, wsn = _ws(fwd_workspace(M, w.N, w.K, r, w.dtype), dev, ws)
    st = w.state()
    fn, name = ((lib.qlora_linear_fwd_f32, "qlora_linear_fwd_f32") if w.dtype == torch.float32
                else (lib.qlora_linear_fwd, "qlora_linear_fwd"))
    _check(fn(ctypes.byref(st), _ptr(x), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(y), _ptr(t), _ptr(wsb), wsn,
              _stream()), name)
    return y, t


def linear_fwd_noalloc(w, x, A, B, alpha, y=None, t=None, want_t=True):
    """linear_fwd without a workspace argument (qlora_linear_fwd_noalloc): the library's fixed per-GPU
    array serves as workspace, so the call itself allocates nothing.  Returns (y, t or None)."""
    M, K = x.shape
    r = A.shape[1]
    _dev(x, w.dtype, "x", (M, w.K))
    _dev(A, w.dtype, "A", (w.K, r))
    _dev(B, w.dtype, "B", (r, w.N))
    dev = x.device
    y = _empty((M, w.N), dtype=w.dtype, device=dev) if y is None else _dev(y, w.dtype, "y", (M, w.N))
    if want_t and t is None:
        t = _empty((M, r), dtype=w.dtype, device=dev)
    if t is not None:
        _dev(t, w.dtype, "t", (M, r))
    st = w.state()
    _check(lib.qlora_linear_fwd_noalloc(ctypes.byref(st), _ptr(x), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(y),
                                        _ptr(t), _stream()), "qlora_linear_fwd_noalloc")
    return y, t


def read_probe(buf, sink, variant=0):
    """Plain read of a device buffer (qlora_read_probe): the same-size bandwidth ceiling of the bench."""
    _check(lib.qlora_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), variant, _stream()),
           "qlora_read_probe")


def lora_down(x, A, alpha, t=None, ws=None):
    """t = (alpha/r) x A [M, r] in x's dtype, bf16 or fp16 (qlora_lora_down)."""
    M, K = x.shape
    r = A.shape[1]
    dt = x.dtype
    code = _dtype_code(dt)
    _dev(x, dt, "x")
    _dev(A, dt, "A", (K, r))
    t = _empty((M, r), dtype=dt, device=x.device) if t is None else _dev(t, dt, "t", (M, r))
    wsb, wsn = _ws(int(lib.qlora_lora_down_workspace(M, K, r)), x.device, ws)
    _check(lib.qlora_lora_down(_ptr(x), M, K, _ptr(A), r, float(alpha), code, _ptr(t), _ptr(wsb), wsn, _stream()),
           "qlora_lora_down")
    return t


def fused_gemm_fwd(w, x, t, B, y=None):
    """y = x W_hat + t B (qlora_fused_gemm_fwd): one kernel launch."""
    M = x.shape[0]
    r = t.shape[1]
    _dev(x, w.dtype, "x", (M, w.K))
    _dev(t, w.dtype, "t", (M, r))
    _dev(B, w.dtype, "B", (r, w.N))
    y = _empty((M, w.N), dtype=w.dtype, device=x.device) if y is None else _dev(y, w.dtype, "y", (M, w.N))
    st = w.state()
    _check(lib.qlora_fused_gemm_fwd(ctypes.byref(st), _ptr(x), M, _ptr(t), _ptr(B), r, _ptr(y), _stream()),
           "qlora_fused_gemm_fwd")
    return y


def fused_gemm_bwd_dx(w, dy, u, A, dx=None):
    """dx = dy W_hat^T + u A^T (qlora_fused_gemm_bwd_dx), u = (alpha/r) dy B^T given: one kernel launch."""
    M = dy.shape[0]
    r = u.shape[1]
    _dev(dy, w.dtype, "dy", (M, w.N))
    _dev(u, w.dtype, "u", (M, r))
    _dev(A, w.dtype, "A", (w.K, r))
    dx = _empty((M, w.K), dtype=w.dtype, device=dy.device) if dx is None else _dev(dx, w.dtype, "dx", (M, w.K))
    st = w.state()
    _check(lib.qlora_fused_gemm_bwd_dx(ctypes.byref(st), _ptr(dy), M, _ptr(u), _ptr(A), r, _ptr(dx), _stream()),
           "qlora_fused_gemm_bwd_dx")
    return dx


def linear_bwd(w, x, A, B, alpha, dy, t=None, need_dx=True, dx=None, dA=None, dB=None, ws=None):
    """(dx, dA, dB) of the layer for upstream dy (qlora_linear_bwd); dx is None when not needed."""
    M, K = x.shape
    r = A.shape[1]
    _dev(x, w.dtype, "x", (M, w.K))
    _dev(A, w.dtype, "A", (w.K, r))
    _dev(B, w.dtype, "B", (r, w.N))
    _dev(dy, w.dtype, "dy", (M, w.N))
    if t is not None:
        _dev(t, w.dtype, "t", (M, r))
    dev = x.device
    if need_dx:
        dx = _empty((M, w.K), dtype=w.dtype, device=dev) if dx is None else _dev(dx, w.dtype, "dx", (M, w.K))
    dA = _empty((w.K, r), dtype=torch.float32, device=dev) if dA is None else _dev(dA, torch.float32, "dA", (w.K, r))
    dB = _empty((r, w.N), dtype=torch.float32, device=dev) if dB is None else _dev(dB, torch.float32, "dB", (r, w.N))
    wsb, wsn = _ws(bwd_workspace(M, w.N, w.K, r, w.dtype), dev, ws)
    st = w.state()
    fn, name = ((lib.qlora_linear_bwd_f32, "qlora_linear_bwd_f32") if w.dtype == torch.float32
                else (lib.qlora_linear_bwd, "qlora_linear_bwd"))
    _check(fn(ctypes.byref(st), _ptr(x), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(t), _ptr(dy),
              _ptr(dx) if need_dx else None, _ptr(dA), _ptr(dB), _ptr(wsb), wsn, _stream()), name)
    return (dx if need_dx else None), dA, dB


def linear_bwd_dx(w, A, B, alpha, dy, u=None, dx=None, ws=None):
    """(u, dx) of the layer for upstream dy (qlora_linear_bwd_dx): u = (alpha/r) dy B^T, kept for
    lora_grads_batch, and dx = dy W_hat^T + u A^T."""
    M = dy.shape[0]
    r = A.shape[1]
    _dev(A, w.dtype, "A", (w.K, r))
    _dev(B, w.dtype, "B", (r, w.N))
    _dev(dy, w.dtype, "dy", (M, w.N))
    dev = dy.device
    u = _empty((M, r), dtype=w.dtype, device=dev) if u is None else _dev(u, w.dtype, "u", (M, r))
    dx = _empty((M, w.K), dtype=w.dtype, device=dev) if dx is None else _dev(dx, w.dtype, "dx", (M, w.K))
    wsb, wsn = _ws(int(lib.qlora_linear_bwd_dx_workspace(M, w.N, w.K, r)), dev, ws)
    st = w.state()
    _check(lib.qlora_linear_bwd_dx(ctypes.byref(st), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(dy), _ptr(u),
                                   _ptr(dx), _ptr(wsb), wsn, _stream()), "qlora_linear_bwd_dx")
    return u, dx


def lora_grads_batch(layers, dA=None, dB=None, ws=None):
    """dA = x^T u and dB = t^T dy (fp32) of several layers in one launch per 8 layers
    (qlora_lora_grads_batch).  layers: a list of (x, t, u, dy), all of one rank r and one dtype (bf16 or
    fp16); dA, dB: optional lists of output tensors.  Returns the lists (dA, dB)."""
    n = len(layers)
    if n == 0:
        return [], []
    dt = layers[0][0].dtype
    code = _dtype_code(dt)
    r = layers[0][1].shape[1]
    dA = [None] * n if dA is None else list(dA)
    dB = [None] * n if dB is None else list(dB)
    descs = (LoraGrads * n)()
    for i, (x, t, u, dy) in enumerate(layers):
        M, K = x.shape
        N = dy.shape[1]
        _dev(x, dt, "x")
        _dev(t, dt, "t", (M, r))
        _dev(u, dt, "u", (M, r))
        _dev(dy, dt, "dy", (M, N))
        dev = x.device
        dA[i] = _empty((K, r), dtype=torch.float32, device=dev) if dA[i] is None else _dev(dA[i], torch.float32,
                                                                                          "dA", (K, r))
        dB[i] = _empty((r, N), dtype=torch.float32, device=dev) if dB[i] is None else _dev(dB[i], torch.float32,
                                                                                          "dB", (r, N))
        descs[i] = LoraGrads(x.data_ptr(), t.data_ptr(), u.data_ptr(), dy.data_ptr(), dA[i].data_ptr(),
                             dB[i].data_ptr(), M, N, K)
    wsb, wsn = _ws(int(lib.qlora_lora_grads_batch_workspace(descs, n, r)), layers[0][0].device, ws)
    _check(lib.qlora_lora_grads_batch(descs, n, r, code, _ptr(wsb), wsn, _stream()), "qlora_lora_grads_batch")
    return dA, dB


def _lora_prod_batch(fn, name, items, alpha, natural, outs, ws):
    n = len(items)
    if n == 0:
        return []
    dt = items[0][0].dtype
    code = _dtype_code(dt)
    r = items[0][1].shape[1] if natural else items[0][1].shape[0]
    outs = [None] * n if outs is None else list(outs)
    descs = (LoraProd * n)()
    for i, (X, Y) in enumerate(items):
        M, C = X.shape
        _dev(X, dt, "x" if natural else "dy")
        _dev(Y, dt, "A" if natural else "B", (C, r) if natural else (r, C))
        outs[i] = _empty((M, r), dtype=dt, device=X.device) if outs[i] is None else _dev(outs[i], dt, "out", (M, r))
        descs[i] = LoraProd(X.data_ptr(), Y.data_ptr(), outs[i].data_ptr(), M, C)
    wsb, wsn = _ws(int(lib.qlora_lora_prod_batch_workspace(descs, n, r)), items[0][0].device, ws)
    _check(fn(descs, n, r, float(alpha), code, _ptr(wsb), wsn, _stream()), name)
    return outs


def lora_down_batch(items, alpha, t=None, ws=None):
    """t_i = (alpha/r) x_i A_i for items [(x_i, A_i)] in one launch per 8 (qlora_lora_down_batch); each t_i is
    that of lora_down.  t: optional list of outputs.  Returns the list of t_i."""
    return _lora_prod_batch(lib.qlora_lora_down_batch, "qlora_lora_down_batch", items, alpha, True, t, ws)


def lora_u_batch(items, alpha, u=None, ws=None):
    """u_i = (alpha/r) dy_i B_i^T for items [(dy_i, B_i)], B_i [r, N_i], in one launch per 8
    (qlora_lora_u_batch); each u_i is that of linear_bwd_dx.  u: optional list of outputs."""
    return _lora_prod_batch(lib.qlora_lora_u_batch, "qlora_lora_u_batch", items, alpha, False, u, ws)


def pooled_fwd(w, x, A, B, alpha, g, y=None, t=None, ws=None):
    """QA-LoRA pooled forward (qlora_pooled_fwd): y = x W_hat + s pool(x) A B, A [K/g, r]. Returns (y, t)."""
    M, K = x.shape
    _, r = A.shape
    _dev(x, w.dtype, "x", (M, w.K))
    _dev(A, w.dtype, "A", (w.K // g, r))
    _dev(B, w.dtype, "B", (r, w.N))
    y = _empty((M, w.N), dtype=w.dtype, device=x.device) if y is None else _dev(y, w.dtype, "y", (M, w.N))
    t = _empty((M, r), dtype=w.dtype, device=x.device) if t is None else _dev(t, w.dtype, "t", (M, r))
    wsb, wsn = _ws(int(lib.qlora_pooled_fwd_workspace(M, w.N, w.K, r, g)), x.device, ws)
    st = w.state()
    _check(lib.qlora_pooled_fwd(ctypes.byref(st), _ptr(x), M, _ptr(A), _ptr(B), r, g, float(alpha), _ptr(y), _ptr(t),
                                _ptr(wsb), wsn, _stream()), "qlora_pooled_fwd")
    return y, t


def pooled_bwd(w, x, A, B, alpha, g, dy, t=None, need_dx=True, dx=None, dA=None, dB=None, ws=None):
    """QA-LoRA pooled backward (qlora_pooled_bwd). Returns (dx or None, dA [K/g, r] fp32, dB [r, N] fp32)."""
    M, K = x.shape
    _, r = A.shape
    _dev(x, w.dtype, "x", (M, w.K))
    _dev(A, w.dtype, "A", (w.K // g, r))
    _dev(B, w.dtype, "B", (r, w.N))
    _dev(dy, w.dtype, "dy", (M, w.N))
    if t is not None:
        _dev(t, w.dtype, "t", (M, r))
    if need_dx:
        dx = _empty((M, w.K), dtype=w.dtype, device=x.device) if dx is None else \
            _dev(dx, w.dtype, "dx", (M, w.K))
    else:
        dx = None
    dA = _empty((w.K // g, r), dtype=torch.float32, device=x.device) if dA is None else \
        _dev(dA, torch.float32, "dA", (w.K // g, r))
    dB = _empty((r, w.N), dtype=torch.float32, device=x.device) if dB is None else \
        _dev(dB, torch.float32, "dB", (r, w.N))
    wsb, wsn = _ws(int(lib.qlora_pooled_bwd_workspace(M, w.N, w.K, r, g)), x.device, ws)
    st = w.state()
    _check(lib.qlora_pooled_bwd(ctypes.byref(st), _ptr(x), M, _ptr(A), _ptr(B), r, g, float(alpha), _ptr(t), _ptr(dy),
                                _ptr(dx), _ptr(dA), _ptr(dB), _ptr(wsb), wsn, _stream()), "qlora_pooled_bwd")
    return dx, dA, dB


def declared_symbols():
    """Function names declared in include/qlora.h (for the export check)."""
    import re
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))
