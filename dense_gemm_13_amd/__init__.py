"""Python binding of libgemm (dense GEMM C = A*B on MI355X / gfx950).

Argument marshalling only: every step of the product runs in the HIP kernels of
libgemm.so.  torch supplies device memory and streams.  There is no fallback:
importing this package without the built library raises ImportError.

Entry points (same names as the C ABI in include/libgemm.h):
    gemm_f16(A, B, C=None, stream=None)
    gemm_bf16(A, B, C=None, stream=None)
    gemm_f32(A, B, C=None, stream=None)
    gemm_fp8_blockscaled(A, B, scale_a, scale_b, C=None, stream=None)
    gemm_quantize_fp8(X, block=64, fmt="e4m3", Q=None, scales=None, stream=None)
    gemm_f16_epilogue / gemm_bf16_epilogue / gemm_f32_epilogue(A, B, C=None, alpha=1.0,
        beta=0.0, bias=None, activation="none", stream=None)
    gemm_fp8_blockscaled_epilogue(A, B, scale_a, scale_b, C=None, alpha=1.0, beta=0.0,
        bias=None, activation="none", stream=None)
    gemm_conv2d_nhwc(X, Wt, stride=1, padding=0, dilation=1, bias=None, activation="none",
        Y=None, workspace=None, stream=None)   (NHWC input, HWIO weights: im2col + GEMM)
    gemm_conv2d_nhwc_noalloc(X, Wt, Y, stride=1, padding=0, dilation=1, bias=None,
        activation="none", stream=None)        (the same, allocating nothing)
    gemm_im2col_nhwc(X, kernel, stride=1, padding=0, dilation=1, col=None, stream=None)
    gemm_h16_ladder(rung, A, B, C=None, stream=None)      (measurement only)
    gemm_h16_mfma_ceiling(A, B, C=None, stream=None)      (measurement only)
The *_epilogue calls write act(alpha * A@B + beta * C + bias[column]) (fp32,
one rounding); C must be given when beta != 0 (its prior contents are read).
A is M x K and B is K x N (row-major: unit column stride; the row stride is the
leading dimension).  C, when given, must be M x N with unit column stride; it is
allocated when omitted.  Work is enqueued on `stream` (default: the current
torch stream of A's device) and the call returns without synchronising.

``lib`` is the raw ctypes handle for calls with plain pointers.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm.so")

GEMM_OK = 0
STATUS_NAMES = {0: "GEMM_OK", -1: "GEMM_ERR_NULL", -2: "GEMM_ERR_DIM", -3: "GEMM_ERR_LD",
                -4: "GEMM_ERR_ALIGN", -5: "GEMM_ERR_ALIAS", -6: "GEMM_ERR_DEVICE",
                -7: "GEMM_ERR_LAUNCH", -8: "GEMM_ERR_ARG", -9: "GEMM_ERR_WORKSPACE",
                -10: "GEMM_ERR_SCRATCH"}
ENTRY_POINTS = ("gemm_f16", "gemm_bf16", "gemm_f32", "gemm_fp8_blockscaled",
                "gemm_f16_epilogue", "gemm_bf16_epilogue", "gemm_f32_epilogue",
                "gemm_fp8_blockscaled_epilogue", "gemm_quantize_fp8", "gemm_h16_ladder",
                "gemm_h16_mfma_ceiling", "gemm_conv2d_nhwc", "gemm_conv2d_nhwc_noalloc",
                "gemm_conv2d_workspace_bytes", "gemm_im2col_nhwc", "gemm_status_string",
                "gemm_version")
# Bytes of the per-GPU device array gemm_conv2d_nhwc_noalloc builds its im2col
# matrix in (GEMM_CONV2D_SCRATCH_BYTES).
CONV2D_SCRATCH_BYTES = 64 << 20
DTYPES = {"f16": 0, "bf16": 1, "f32": 2}      # enum gemm_dtype


class Conv2dShape(ctypes.Structure):
    """struct gemm_conv2d_shape."""
    _fields_ = [(name, ctypes.c_int64) for name in
                ("n", "h", "w", "c_in", "c_out", "kh", "kw", "stride_h", "stride_w", "pad_h",
                 "pad_w", "dil_h", "dil_w")]
LADDER_RUNGS = {"naive": 0, "lds_tiled": 1, "register_tiled": 2, "mfma": 3,
                "mfma_double_buffer": 4, "mfma_swizzle": 5, "library": 6,
                "mfma_one_wg": 7, "mfma_double_buffer_one_wg": 8}   # enum gemm_ladder_rung
ACTIVATIONS = {"none": 0, "relu": 1}          # enum gemm_activation
FP8_FORMATS = {"e4m3": 0, "e5m2": 1}          # enum gemm_fp8_format
QUANT_INPUTS = {"f32": 0, "bf16": 1}          # enum gemm_quant_input


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libgemm is not built ({LIB_PATH} missing); run "
                          "`python dense_gemm_13_amd/build.py` or __graft_entry__.build()")
    # torch ships its own HIP runtime (soname libamdhip64.so.7, but its libraries
    # ask for "libamdhip64.so").  Loading torch first makes libgemm bind to that
    # same runtime; loading libgemm first would put a second HIP runtime in the
    # process, and device pointers / streams from torch would not belong to it.
    import torch  # noqa: F401
    h = ctypes.CDLL(LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    for name in ("gemm_f16", "gemm_bf16", "gemm_f32"):
        fn = getattr(h, name)
        fn.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
        fn.restype = ctypes.c_int
    h.gemm_fp8_blockscaled.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp, vp]
    h.gemm_fp8_blockscaled.restype = ctypes.c_int
    f32, ci = ctypes.c_float, ctypes.c_int
    for name in ("gemm_f16_epilogue", "gemm_bf16_epilogue", "gemm_f32_epilogue"):
        fn = getattr(h, name)
        fn.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32, vp, ci, vp]
        fn.restype = ctypes.c_int
    h.gemm_fp8_blockscaled_epilogue.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp,
                                                f32, f32, vp, ci, vp]
    h.gemm_fp8_blockscaled_epilogue.restype = ctypes.c_int
    h.gemm_quantize_fp8.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                    vp, i64, vp, vp]
    h.gemm_quantize_fp8.restype = ctypes.c_int
    h.gemm_h16_ladder.argtypes = [ci, ci, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
    h.gemm_h16_ladder.restype = ctypes.c_int
    h.gemm_h16_mfma_ceiling.argtypes = [ci, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
    h.gemm_h16_mfma_ceiling.restype = ctypes.c_int
    sp = ctypes.POINTER(Conv2dShape)
    h.gemm_conv2d_nhwc.argtypes = [ci, vp, vp, vp, vp, i64, sp, vp, ci, vp]
    h.gemm_conv2d_nhwc.restype = ctypes.c_int
    h.gemm_conv2d_nhwc_noalloc.argtypes = [ci, vp, vp, vp, sp, vp, ci, vp]
    h.gemm_conv2d_nhwc_noalloc.restype = ctypes.c_int
    h.gemm_conv2d_workspace_bytes.argtypes = [ci, sp]
    h.gemm_conv2d_workspace_bytes.restype = ctypes.c_int64
    h.gemm_im2col_nhwc.argtypes = [ci, vp, vp, i64, sp, vp]
    h.gemm_im2col_nhwc.restype = ctypes.c_int
    h.gemm_status_string.argtypes = [ctypes.c_int]
    h.gemm_status_string.restype = ctypes.c_char_p
    h.gemm_version.argtypes = []
    h.gemm_version.restype = ctypes.c_int
    return h


lib = _load()


def status_string(status: int) -> str:
    return lib.gemm_status_string(int(status)).decode()


def _torch():
    import torch
    return torch


def _ld(t) -> int:
    """Leading dimension of a 2-D row-major tensor (row stride in elements).

    Rows must not overlap: a row stride below the row length (a broadcast row,
    stride 0, or any other overlapping view) is rejected, since the kernels
    address row i at i * ld and would read or write past the tensor.
    """
    if t.dim() != 2:
        raise ValueError(f"expected a 2-D tensor, got {t.dim()}-D")
    if t.numel() == 0:          # no elements: strides are meaningless
        return max(t.size(1), 1)
    if t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError("tensor must have unit column stride (row-major)")
    if t.size(0) > 1 and t.stride(0) < t.size(1):
        raise ValueError(f"tensor rows overlap (row stride {t.stride(0)} < row length "
                         f"{t.size(1)}); pass a tensor with distinct rows, e.g. .contiguous()")
    return max(t.stride(0), 1) if t.size(0) > 1 else max(t.size(1), 1)


def _on_device(name, device, **tensors):
    """Every tensor handed to the library must live in GPU memory on `device`
    (the device of the first operand): the kernels dereference data_ptr() on
    that GPU, so a host tensor or one on another GPU would be read as a wild
    device address.  None entries are optional arguments that were not given."""
    for nm, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name}: {nm} must be a GPU tensor (got one on {t.device})")
        if t.device != device:
            raise ValueError(f"{name}: {nm} is on {t.device}, the operands on {device}")


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif getattr(stream, "device", device) != device:
        raise ValueError(f"stream belongs to {stream.device}, the operands to {device}")
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != GEMM_OK:
        raise GemmError(status, where)


def _epilogue_args(name, C, N, alpha, beta, bias, activation, device):
    """(alpha, beta, bias pointer, activation id) of a *_epilogue call."""
    torch = _torch()
    if activation not in ACTIVATIONS:
        raise ValueError(f"{name}: activation must be one of {sorted(ACTIVATIONS)}")
    if beta != 0.0 and C is None:
        raise ValueError(f"{name}: beta != 0 reads C, so C must be given")
    bptr = None
    if bias is not None:
        if bias.dtype != torch.float32 or tuple(bias.shape) != (N,) or not bias.is_contiguous():
            raise ValueError(f"{name}: bias must be a contiguous float32 vector of {N} values")
        _on_device(name, device, bias=bias)
        bptr = bias.data_ptr()
    return float(alpha), float(beta), bptr, ACTIVATIONS[activation]


def _h16(name, want_dtype, A, B, C, stream, epilogue=None):
    torch = _torch()
    if A.dtype != want_dtype or B.dtype != want_dtype:
        raise TypeError(f"{name}: A and B must be {want_dtype}")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"{name}: inner dimensions differ ({K} vs {K2})")
    extra = ()
    if epilogue is not None:
        extra = _epilogue_args(name, C, N, *epilogue, A.device)
    if C is None:
        C = torch.empty((M, N), dtype=want_dtype, device=A.device)
    if C.dtype != want_dtype or tuple(C.shape) != (M, N):
        raise ValueError(f"{name}: C must be {want_dtype} of shape ({M}, {N})")
    lda, ldb, ldc = _ld(A), _ld(B), _ld(C)
    _on_device(name, A.device, A=A, B=B, C=C)
    sh = _stream_handle(stream, A.device)
    _check(getattr(lib, name)(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, lda, ldb, ldc,
                              *extra, sh), name)
    return C


def gemm_f16(A, B, C=None, stream=None):
    """C = A @ B for float16 A (M x K), B (K x N); fp32 accumulation, fp16 C."""
    return _h16("gemm_f16", _torch().float16, A, B, C, stream)


def gemm_bf16(A, B, C=None, stream=None):
    """C = A @ B for bfloat16 A (M x K), B (K x N); fp32 accumulation, bf16 C."""
    return _h16("gemm_bf16", _torch().bfloat16, A, B, C, stream)


def gemm_f32(A, B, C=None, stream=None):
    """C = A @ B for float32 A (M x K), B (K x N); fp32 accumulation and C."""
    return _h16("gemm_f32", _torch().float32, A, B, C, stream)


def _fp8(name, A, B, scale_a, scale_b, C, stream, epilogue=None):
    torch = _torch()
    if A.dtype not in (torch.uint8, torch.float8_e4m3fn) or B.dtype != A.dtype:
        raise TypeError(f"{name}: A and B must be uint8 or float8_e4m3fn")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"{name}: inner dimensions differ ({K} vs {K2})")
    cdiv = lambda a, b: -(-a // b)
    for s, shape, nm in ((scale_a, (cdiv(M, 64), cdiv(K, 64)), "scale_a"),
                         (scale_b, (cdiv(K, 64), cdiv(N, 64)), "scale_b")):
        if s.dtype != torch.float32 or tuple(s.shape) != shape or not s.is_contiguous():
            raise ValueError(f"{name}: {nm} must be contiguous float32 {shape}")
    extra = ()
    if epilogue is not None:
        extra = _epilogue_args(name, C, N, *epilogue, A.device)
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if C.dtype != torch.bfloat16 or tuple(C.shape) != (M, N):
        raise ValueError(f"{name}: C must be bfloat16 of shape ({M}, {N})")
    lda, ldb, ldc = _ld(A), _ld(B), _ld(C)
    _on_device(name, A.device, A=A, B=B, C=C, scale_a=scale_a, scale_b=scale_b)
    sh = _stream_handle(stream, A.device)
    _check(getattr(lib, name)(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, lda, ldb, ldc,
                              scale_a.data_ptr(), scale_b.data_ptr(), *extra, sh), name)
    return C


def gemm_fp8_blockscaled(A, B, scale_a, scale_b, C=None, stream=None):
    """C = (A * scale_a) @ (B * scale_b) with E4M3 codes and one fp32 scale per 64 x 64 block.

    A: M x K and B: K x N, torch.uint8 or torch.float8_e4m3fn (OCP E4M3 codes).
    scale_a: ceil(M/64) x ceil(K/64) float32, scale_b: ceil(K/64) x ceil(N/64)
    float32, both contiguous.  C: M x N bfloat16.
    """
    return _fp8("gemm_fp8_blockscaled", A, B, scale_a, scale_b, C, stream)


def gemm_f16_epilogue(A, B, C=None, alpha=1.0, beta=0.0, bias=None, activation="none",
                      stream=None):
    """C = act(alpha * A@B + beta * C + bias[column]) for float16 A, B, C.

    bias: None or a float32 vector of N values; activation: "none" or "relu".
    """
    return _h16("gemm_f16_epilogue", _torch().float16, A, B, C, stream,
                (alpha, beta, bias, activation))


def gemm_bf16_epilogue(A, B, C=None, alpha=1.0, beta=0.0, bias=None, activation="none",
                       stream=None):
    """C = act(alpha * A@B + beta * C + bias[column]) for bfloat16 A, B, C."""
    return _h16("gemm_bf16_epilogue", _torch().bfloat16, A, B, C, stream,
                (alpha, beta, bias, activation))


def gemm_f32_epilogue(A, B, C=None, alpha=1.0, beta=0.0, bias=None, activation="none",
                      stream=None):
    """C = act(alpha * A@B + beta * C + bias[column]) for float32 A, B, C."""
    return _h16("gemm_f32_epilogue", _torch().float32, A, B, C, stream,
                (alpha, beta, bias, activation))


def gemm_fp8_blockscaled_epilogue(A, B, scale_a, scale_b, C=None, alpha=1.0, beta=0.0,
                                  bias=None, activation="none", stream=None):
    """C = act(alpha * (A*scale_a)@(B*scale_b) + beta * C + bias[column]), bfloat16 C."""
    return _fp8("gemm_fp8_blockscaled_epilogue", A, B, scale_a, scale_b, C, stream,
                (alpha, beta, bias, activation))


def _h16_pair(name, A, B, C):
    torch = _torch()
    if A.dtype not in (torch.float16, torch.bfloat16) or B.dtype != A.dtype:
        raise TypeError(f"{name}: A and B must both be float16 or both bfloat16")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"{name}: inner dimensions differ ({K} vs {K2})")
    if C is None:
        C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    if C.dtype != A.dtype or tuple(C.shape) != (M, N):
        raise ValueError(f"{name}: C must be {A.dtype} of shape ({M}, {N})")
    return M, N, K, int(A.dtype == torch.bfloat16), C


def gemm_h16_ladder(rung, A, B, C=None, stream=None):
    """C = A @ B by one rung of the measured optimisation ladder (a name of
    LADDER_RUNGS or its number); float16 or bfloat16 operands."""
    r = LADDER_RUNGS[rung] if isinstance(rung, str) else int(rung)
    M, N, K, bf, C = _h16_pair("gemm_h16_ladder", A, B, C)
    lda, ldb, ldc = _ld(A), _ld(B), _ld(C)
    _on_device("gemm_h16_ladder", A.device, A=A, B=B, C=C)
    sh = _stream_handle(stream, A.device)
    _check(lib.gemm_h16_ladder(r, bf, A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, lda,
                               ldb, ldc, sh), "gemm_h16_ladder")
    return C


def gemm_h16_mfma_ceiling(A, B, C=None, stream=None):
    """The large-tile kernel's MFMA sequence with register-held operands (no
    memory traffic); writes C = (K/32) * A[:, :32] @ B[:32, :]."""
    M, N, K, bf, C = _h16_pair("gemm_h16_mfma_ceiling", A, B, C)
    lda, ldb, ldc = _ld(A), _ld(B), _ld(C)
    _on_device("gemm_h16_mfma_ceiling", A.device, A=A, B=B, C=C)
    sh = _stream_handle(stream, A.device)
    _check(lib.gemm_h16_mfma_ceiling(bf, A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K,
                                     lda, ldb, ldc, sh), "gemm_h16_mfma_ceiling")
    return C


def _pair(v):
    return (int(v), int(v)) if isinstance(v, int) else (int(v[0]), int(v[1]))


def conv2d_shape(X, Wt, stride=1, padding=0, dilation=1) -> Conv2dShape:
    """struct gemm_conv2d_shape of an NHWC input and HWIO weights."""
    if X.dim() != 4 or Wt.dim() != 4:
        raise ValueError("conv2d: X must be NHWC (4-D) and Wt HWIO (4-D)")
    n, h, w, c_in = X.shape
    kh, kw, c_in2, c_out = Wt.shape
    if c_in2 != c_in:
        raise ValueError(f"conv2d: input channels differ ({c_in} vs {c_in2})")
    (sh, sw), (ph, pw), (dh, dw) = _pair(stride), _pair(padding), _pair(dilation)
    return Conv2dShape(n, h, w, c_in, c_out, kh, kw, sh, sw, ph, pw, dh, dw)


def _conv_dtype(name, *tensors):
    torch = _torch()
    names = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}
    dt = names.get(tensors[0].dtype)
    if dt is None or any(t.dtype != tensors[0].dtype for t in tensors):
        raise TypeError(f"{name}: tensors must all be float16, bfloat16 or float32")
    for t in tensors:
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensors must be contiguous")
    return dt


def conv2d_output_hw(shape: Conv2dShape):
    eh = shape.h + 2 * shape.pad_h - shape.dil_h * (shape.kh - 1) - 1
    ew = shape.w + 2 * shape.pad_w - shape.dil_w * (shape.kw - 1) - 1
    return (0 if eh < 0 else eh // shape.stride_h + 1), (0 if ew < 0 else ew // shape.stride_w + 1)


def gemm_conv2d_nhwc(X, Wt, stride=1, padding=0, dilation=1, bias=None, activation="none",
                     Y=None, workspace=None, stream=None):
    """Y = act(conv2d(X, Wt) + bias) with X NHWC, Wt HWIO (kh, kw, c_in, c_out),
    Y NHWC, through im2col + GEMM.  The im2col workspace is allocated when not
    given (a uint8 device tensor of gemm_conv2d_workspace_bytes bytes)."""
    torch = _torch()
    dt = _conv_dtype("gemm_conv2d_nhwc", X, Wt)
    shape = conv2d_shape(X, Wt, stride, padding, dilation)
    ho, wo = conv2d_output_hw(shape)
    need = lib.gemm_conv2d_workspace_bytes(DTYPES[dt], ctypes.byref(shape))
    _check(need if need < 0 else 0, "gemm_conv2d_workspace_bytes")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    if Y is None:
        Y = torch.empty((shape.n, ho, wo, shape.c_out), dtype=X.dtype, device=X.device)
    if Y.dtype != X.dtype or tuple(Y.shape) != (shape.n, ho, wo, shape.c_out) or \
            not Y.is_contiguous():
        raise ValueError(f"gemm_conv2d_nhwc: Y must be contiguous {X.dtype} "
                         f"{(shape.n, ho, wo, shape.c_out)}")
    _, _, bptr, act = _epilogue_args("gemm_conv2d_nhwc", Y, shape.c_out, 1.0, 0.0, bias,
                                     activation, X.device)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("gemm_conv2d_nhwc: workspace must be contiguous")
    _on_device("gemm_conv2d_nhwc", X.device, X=X, Wt=Wt, Y=Y, workspace=workspace)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    sh = _stream_handle(stream, X.device)
    _check(lib.gemm_conv2d_nhwc(DTYPES[dt], X.data_ptr(), Wt.data_ptr(), Y.data_ptr(), ws_ptr,
                                ws_bytes, ctypes.byref(shape), bptr, act, sh),
           "gemm_conv2d_nhwc")
    return Y


def gemm_conv2d_nhwc_noalloc(X, Wt, Y, stride=1, padding=0, dilation=1, bias=None,
                             activation="none", stream=None):
    """gemm_conv2d_nhwc for callers that cannot allocate: the im2col matrix is
    built in the library's fixed per-GPU scratch array (CONV2D_SCRATCH_BYTES)
    and Y must be given, so neither the library nor this call allocates device
    memory.  Calls whose matrix does not fit raise GemmError (GEMM_ERR_SCRATCH).
    Calls on one GPU share the array: issue them on one stream."""
    dt = _conv_dtype("gemm_conv2d_nhwc_noalloc", X, Wt, Y)
    shape = conv2d_shape(X, Wt, stride, padding, dilation)
    ho, wo = conv2d_output_hw(shape)
    if tuple(Y.shape) != (shape.n, ho, wo, shape.c_out):
        raise ValueError(f"gemm_conv2d_nhwc_noalloc: Y must be contiguous {X.dtype} "
                         f"{(shape.n, ho, wo, shape.c_out)}")
    _, _, bptr, act = _epilogue_args("gemm_conv2d_nhwc_noalloc", Y, shape.c_out, 1.0, 0.0, bias,
                                     activation, X.device)
    _on_device("gemm_conv2d_nhwc_noalloc", X.device, X=X, Wt=Wt, Y=Y)
    sh = _stream_handle(stream, X.device)
    _check(lib.gemm_conv2d_nhwc_noalloc(DTYPES[dt], X.data_ptr(), Wt.data_ptr(), Y.data_ptr(),
                                        ctypes.byref(shape), bptr, act, sh),
           "gemm_conv2d_nhwc_noalloc")
    return Y


def gemm_im2col_nhwc(X, kernel, stride=1, padding=0, dilation=1, col=None, stream=None):
    """The im2col matrix of an NHWC tensor: (n*ho*wo) x (kh*kw*c_in), row
    (n, oh, ow), column (kh, kw, ci); zeros where a tap falls in the padding."""
    torch = _torch()
    dt = _conv_dtype("gemm_im2col_nhwc", X)
    kh, kw = _pair(kernel)
    n, h, w, c_in = X.shape
    (sh, sw), (ph, pw), (dh, dw) = _pair(stride), _pair(padding), _pair(dilation)
    shape = Conv2dShape(n, h, w, c_in, 1, kh, kw, sh, sw, ph, pw, dh, dw)
    ho, wo = conv2d_output_hw(shape)
    rows, cols = n * ho * wo, kh * kw * c_in
    if col is None:
        col = torch.empty((rows, cols), dtype=X.dtype, device=X.device)
    if col.dtype != X.dtype or tuple(col.shape) != (rows, cols):
        raise ValueError(f"gemm_im2col_nhwc: col must be {X.dtype} of shape ({rows}, {cols})")
    ldcol = _ld(col)
    _on_device("gemm_im2col_nhwc", X.device, X=X, col=col)
    sh = _stream_handle(stream, X.device)
    _check(lib.gemm_im2col_nhwc(DTYPES[dt], X.data_ptr(), col.data_ptr(), ldcol,
                                ctypes.byref(shape), sh), "gemm_im2col_nhwc")
    return col


def gemm_quantize_fp8(X, block=64, fmt="e4m3", Q=None, scales=None, stream=None):
    """Block-scaled FP8 quantisation of a 2-D float32 or bfloat16 tensor.

    Returns (Q, scales): Q holds the FP8 codes (uint8, X's shape; E4M3 or E5M2),
    scales is the contiguous float32 ceil(rows/block) x ceil(cols/block) grid of
    per-block scales (block 32 or 64).  With the defaults, quantising A (M x K)
    and B (K x N) gives gemm_fp8_blockscaled's operands and scales.
    """
    torch = _torch()
    in_type = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(X.dtype)
    if in_type is None:
        raise TypeError("gemm_quantize_fp8: X must be float32 or bfloat16")
    if fmt not in FP8_FORMATS:
        raise ValueError(f"gemm_quantize_fp8: fmt must be one of {sorted(FP8_FORMATS)}")
    rows, cols = X.shape
    shape = (-(-rows // block), -(-cols // block)) if block > 0 else (0, 0)
    if Q is None:
        Q = torch.empty((rows, cols), dtype=torch.uint8, device=X.device)
    if scales is None:
        scales = torch.empty(shape, dtype=torch.float32, device=X.device)
    if Q.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2) or \
            tuple(Q.shape) != (rows, cols):
        raise ValueError(f"gemm_quantize_fp8: Q must be uint8 of shape ({rows}, {cols})")
    if scales.dtype != torch.float32 or tuple(scales.shape) != shape or \
            not scales.is_contiguous():
        raise ValueError(f"gemm_quantize_fp8: scales must be contiguous float32 {shape}")
    ldx, ldq = _ld(X), _ld(Q)
    _on_device("gemm_quantize_fp8", X.device, X=X, Q=Q, scales=scales)
    sh = _stream_handle(stream, X.device)
    _check(lib.gemm_quantize_fp8(X.data_ptr(), QUANT_INPUTS[in_type], rows, cols, ldx, block,
                                 FP8_FORMATS[fmt], Q.data_ptr(), ldq, scales.data_ptr(), sh),
           "gemm_quantize_fp8")
    return Q, scales


__all__ = ["gemm_f16", "gemm_bf16", "gemm_f32", "gemm_fp8_blockscaled", "gemm_f16_epilogue",
           "gemm_bf16_epilogue", "gemm_f32_epilogue", "gemm_fp8_blockscaled_epilogue",
           "gemm_quantize_fp8", "gemm_h16_ladder", "gemm_h16_mfma_ceiling", "gemm_conv2d_nhwc",
           "gemm_conv2d_nhwc_noalloc", "gemm_im2col_nhwc", "CONV2D_SCRATCH_BYTES", "Conv2dShape", "status_string",
           "GemmError", "lib", "LIB_PATH"]
