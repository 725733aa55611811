"""CPU oracle for the dense GEMM C = A*B -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and it
never calls the GPU library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, bit-level decoders); this
module only marshals numpy arrays into it.  What it follows:

* "[CUDA 优化实战] hgemm - 超越 cuBLAS", sections 0-1: C = A*B, A (M x K) and
  B (K x N) both row-major, fp16/bf16 inputs, fp32 accumulation;
* "CUDA GEMM 优化实践笔记", register-tiling section: the fp32 SGEMM with the
  same row-major indexing;
* "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析", section 4.3 and
  section 5.2 (third pitfall): E4M3 operands with one 32-bit scale per 64x64
  sub-block, and the quantiser that makes them (``quantize_fp8``: E4M3 or E5M2,
  32x32 or 64x64 blocks, scale = block amax / largest FP8 value, RNE);
* the same article, section 1.1 (a fully connected layer is a product plus a
  bias per output feature), and the relu epilogue of the vendor kernel in
  "[CUDA 优化实战] hgemm - 超越 cuBLAS" section 5: ``epilogue`` applies
  out = act(alpha * prod + beta * C_prior + bias[column]) to the exact product;
* the same article, section 1.1 (a convolution becomes a GEMM through im2col):
  ``conv2d_nhwc`` computes the convolution by its definition (NHWC input, HWIO
  weights, zero padding, stride, dilation), and ``im2col_nhwc`` builds the
  im2col matrix, for bit-exact checks of a packing kernel.

``gemm`` returns the exact sum (fp64, k ascending, never rounded to the
output type).  ``within_tolerance`` is the element-wise acceptance test
|gpu - ref| <= rtol*|ref| + atol, with any NaN/Inf in the candidate failing.

Parity pins: every function here is pinned by ``tests/test_oracle.py`` against
library decoders (exhaustively), closed forms and exact rational brute force.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16, F32, FP8 = 0, 1, 2, 3
DTYPES = {"f16": F16, "bf16": BF16, "f32": F32, "fp8": FP8}
SCALE_BLOCK = 64
FP8_FORMATS = {"e4m3": 0, "e5m2": 1}
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    _lib = bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def bind(lib):
    """Declare the C signatures on a loaded oracle library handle."""
    vp, i64, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p
    lib.orc_gemm.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64, dp, i64,
                             ctypes.c_int]
    lib.orc_gemm.restype = ctypes.c_int
    lib.orc_gemm_entries.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                     vp, vp, i64, dp]
    lib.orc_gemm_entries.restype = ctypes.c_int
    for name in ("orc_decode_f16", "orc_decode_bf16", "orc_decode_e4m3", "orc_decode_e5m2",
                 "orc_decode_f32"):
        getattr(lib, name).argtypes = [vp, dp, i64]
        getattr(lib, name).restype = None
    lib.orc_fp8_encode_array.argtypes = [vp, i64, ctypes.c_int, vp]
    lib.orc_fp8_encode_array.restype = None
    lib.orc_quantize_fp8.argtypes = [ctypes.c_int, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                     vp, i64, vp]
    lib.orc_quantize_fp8.restype = ctypes.c_int
    lib.orc_epilogue.argtypes = [ctypes.c_int, vp, i64, i64, ctypes.c_double, ctypes.c_double,
                                 vp, i64, vp, ctypes.c_int, vp]
    lib.orc_epilogue.restype = ctypes.c_int
    lib.orc_conv2d_output_size.argtypes = [vp, vp, vp]
    lib.orc_conv2d_output_size.restype = ctypes.c_int
    lib.orc_conv2d_nhwc.argtypes = [ctypes.c_int, vp, vp, vp, vp]
    lib.orc_conv2d_nhwc.restype = ctypes.c_int
    lib.orc_im2col_nhwc.argtypes = [ctypes.c_int, vp, vp, vp, i64]
    lib.orc_im2col_nhwc.restype = ctypes.c_int
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _raw(x: np.ndarray, dtype: str) -> np.ndarray:
    """Row-major raw bit array of an operand (uint16 / float32 / uint8)."""
    want = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32, "fp8": np.uint8}[dtype]
    if x.dtype != want:
        if dtype == "f16" and x.dtype == np.float16:
            x = x.view(np.uint16)
        elif dtype == "f32" and x.dtype == np.uint32:
            x = x.view(np.float32)
        else:
            raise TypeError(f"{dtype} operand must be {want}, got {x.dtype}")
    if x.ndim != 2 or (x.shape[1] > 1 and x.strides[1] != x.itemsize):
        raise ValueError("operand must be 2-D with unit column stride")
    return x


def _ld(x: np.ndarray) -> int:
    if x.shape[0] <= 1:
        return max(x.shape[1], 1)      # numpy may give a lone row any stride
    return x.strides[0] // x.itemsize


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of raw fp16/bf16 (uint16), e4m3 ("fp8" or "e4m3") /
    e5m2 (uint8) or fp32 bits."""
    lib = _load()
    src = np.ascontiguousarray(bits)
    out = np.empty(src.shape, dtype=np.float64)
    fn = {"f16": lib.orc_decode_f16, "bf16": lib.orc_decode_bf16,
          "fp8": lib.orc_decode_e4m3, "e4m3": lib.orc_decode_e4m3,
          "e5m2": lib.orc_decode_e5m2, "f32": lib.orc_decode_f32}[dtype]
    if dtype == "f32":
        src = src.view(np.uint32)
    fn(src.ctypes.data, out.ctypes.data, src.size)
    return out


def gemm(dtype: str, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
         scale_a: np.ndarray | None = None, scale_b: np.ndarray | None = None,
         nthreads: int | None = None) -> np.ndarray:
    """Exact (fp64) C = A[:M,:K] * B[:K,:N] of raw operands; returns M x N float64."""
    lib = _load()
    A = _raw(A, dtype)
    B = _raw(B, dtype)
    if A.shape[0] < M or A.shape[1] < K or B.shape[0] < K or B.shape[1] < N:
        raise ValueError("operand smaller than (M, N, K)")
    sa = sb = None
    if dtype == "fp8":
        sa = np.ascontiguousarray(scale_a, dtype=np.float32)
        sb = np.ascontiguousarray(scale_b, dtype=np.float32)
        if sa.shape != (-(-M // SCALE_BLOCK), -(-K // SCALE_BLOCK)) or \
           sb.shape != (-(-K // SCALE_BLOCK), -(-N // SCALE_BLOCK)):
            raise ValueError("scale grid shape does not match the 64x64 blocks")
    out = np.empty((M, N), dtype=np.float64)
    nt = nthreads or os.cpu_count() or 1
    rc = lib.orc_gemm(DTYPES[dtype], _ptr(A), _ptr(B), _ptr(sa), _ptr(sb), M, N, K,
                      _ld(A), _ld(B), out.ctypes.data, N, int(nt))
    if rc != 0:
        raise RuntimeError(f"orc_gemm failed ({rc})")
    return out


def gemm_entries(dtype: str, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
                 rows: np.ndarray, cols: np.ndarray, scale_a: np.ndarray | None = None,
                 scale_b: np.ndarray | None = None) -> np.ndarray:
    """Exact (fp64) entries C[rows[t], cols[t]] only."""
    lib = _load()
    A = _raw(A, dtype)
    B = _raw(B, dtype)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    sa = sb = None
    if dtype == "fp8":
        sa = np.ascontiguousarray(scale_a, dtype=np.float32)
        sb = np.ascontiguousarray(scale_b, dtype=np.float32)
    out = np.empty(rows.shape[0], dtype=np.float64)
    rc = lib.orc_gemm_entries(DTYPES[dtype], _ptr(A), _ptr(B), _ptr(sa), _ptr(sb), M, N, K,
                              _ld(A), _ld(B), rows.ctypes.data, cols.ctypes.data,
                              rows.shape[0], out.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"orc_gemm_entries failed ({rc})")
    return out


def within_tolerance(gpu: np.ndarray, ref: np.ndarray, rtol: float, atol: float):
    """Element-wise |gpu - ref| <= rtol*|ref| + atol; NaN/Inf in gpu fail.

    Returns (ok, n_fail, worst_ratio, worst_index) where worst_ratio is
    max |gpu-ref| / (rtol*|ref| + atol) over the finite entries.
    """
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if gpu.shape != ref.shape:
        raise ValueError(f"shape mismatch {gpu.shape} vs {ref.shape}")
    if gpu.size == 0:
        return True, 0, 0.0, None
    tol = rtol * np.abs(ref) + atol
    finite = np.isfinite(gpu)
    err = np.where(finite, np.abs(gpu - ref), np.inf)
    ratio = err / tol
    bad = ~(err <= tol)
    worst = int(np.argmax(ratio))
    idx = np.unravel_index(worst, ratio.shape)
    return (not bad.any()), int(bad.sum()), float(ratio.flat[worst]), tuple(int(i) for i in idx)


def fp8_encode(y: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest FP8 codes (ties to even) of finite float32 values within range."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib.orc_fp8_encode_array(y.ctypes.data, y.size, FP8_FORMATS[fmt], out.ctypes.data)
    return out


def quantize_fp8(X: np.ndarray, dtype: str, block: int, fmt: str):
    """Block-scaled FP8 quantisation of a 2-D fp32 (float32) or bf16 (uint16 bits)
    matrix: returns (codes uint8 of X's shape, scales float32 of
    (ceil(rows/block), ceil(cols/block)))."""
    lib = _load()
    X = _raw(X, dtype)
    rows, cols = X.shape
    Q = np.empty((rows, cols), dtype=np.uint8)
    S = np.empty((-(-rows // block), -(-cols // block)), dtype=np.float32)
    rc = lib.orc_quantize_fp8(DTYPES[dtype], X.ctypes.data, rows, cols, _ld(X), block,
                              FP8_FORMATS[fmt], Q.ctypes.data, max(cols, 1), S.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"orc_quantize_fp8 failed ({rc})")
    return Q, S


ACTIVATIONS = {"none": 0, "relu": 1}


def epilogue(out_dtype: str, prod: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
             c_prior: np.ndarray | None = None, bias: np.ndarray | None = None,
             act: str = "none") -> np.ndarray:
    """Exact (fp64) act(alpha * prod + beta * c_prior + bias[j]) of an M x N
    product.  out_dtype is C's type ("f16", "bf16", "f32"; the fp8 GEMM writes
    "bf16"); c_prior holds C's raw bits before the call (read only when beta != 0);
    bias is None or N float32 values; act is "none" or "relu".  alpha and beta
    are taken as fp32 values, as the library receives them."""
    lib = _load()
    prod = np.ascontiguousarray(prod, dtype=np.float64)
    M, N = prod.shape
    cb = None
    ldc = max(N, 1)
    if c_prior is not None:
        cb = _raw(c_prior, out_dtype)
        if cb.shape[0] < M or cb.shape[1] < N:
            raise ValueError("c_prior smaller than the product")
        ldc = _ld(cb) if M > 1 else max(cb.shape[1], 1)
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias, dtype=np.float32)
        if b.shape != (N,):
            raise ValueError("bias must hold one value per column")
    out = np.empty((M, N), dtype=np.float64)
    rc = lib.orc_epilogue(DTYPES[out_dtype], prod.ctypes.data, M, N,
                          float(np.float32(alpha)), float(np.float32(beta)), _ptr(cb), ldc,
                          _ptr(b), ACTIVATIONS[act], out.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"orc_epilogue failed ({rc})")
    return out


CONV_KEYS = ("n", "h", "w", "c_in", "c_out", "kh", "kw", "stride_h", "stride_w", "pad_h",
             "pad_w", "dil_h", "dil_w")


def conv_geom(**kw) -> np.ndarray:
    """The 13 convolution sizes in the oracle's order (stride, dilation default 1,
    padding 0)."""
    d = {"stride_h": 1, "stride_w": 1, "pad_h": 0, "pad_w": 0, "dil_h": 1, "dil_w": 1}
    d.update(kw)
    return np.array([d[k] for k in CONV_KEYS], dtype=np.int64)


def conv2d_output_size(geom: np.ndarray):
    lib = _load()
    g = np.ascontiguousarray(geom, dtype=np.int64)
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    if lib.orc_conv2d_output_size(g.ctypes.data, ctypes.addressof(ho), ctypes.addressof(wo)) != 0:
        raise ValueError("bad convolution geometry")
    return ho.value, wo.value


def conv2d_nhwc(dtype: str, X: np.ndarray, Wt: np.ndarray, geom: np.ndarray) -> np.ndarray:
    """Exact (fp64) NHWC convolution of raw X (n*h*w x c_in bits, any shape with
    that many elements) by raw HWIO weights; returns (n, Ho, Wo, c_out) float64."""
    lib = _load()
    g = np.ascontiguousarray(geom, dtype=np.int64)
    ho, wo = conv2d_output_size(g)
    n, h, w, ci, co, kh, kw = (int(v) for v in g[:7])
    X = np.ascontiguousarray(_raw(np.ascontiguousarray(X).reshape(n * h * w, ci), dtype))
    Wt = np.ascontiguousarray(_raw(np.ascontiguousarray(Wt).reshape(kh * kw * ci, co), dtype))
    out = np.empty((n, ho, wo, co), dtype=np.float64)
    if lib.orc_conv2d_nhwc(DTYPES[dtype], X.ctypes.data, Wt.ctypes.data, g.ctypes.data,
                           out.ctypes.data) != 0:
        raise RuntimeError("orc_conv2d_nhwc failed")
    return out


def im2col_nhwc(X: np.ndarray, geom: np.ndarray) -> np.ndarray:
    """The im2col matrix of an NHWC tensor (raw uint16 or float32/uint32 bits):
    (n*Ho*Wo) x (kh*kw*c_in), same element type as X."""
    lib = _load()
    g = np.ascontiguousarray(geom, dtype=np.int64)
    ho, wo = conv2d_output_size(g)
    n, kh, kw, ci = int(g[0]), int(g[5]), int(g[6]), int(g[3])
    X = np.ascontiguousarray(X)
    out = np.empty((n * ho * wo, kh * kw * ci), dtype=X.dtype)
    if lib.orc_im2col_nhwc(X.itemsize, X.ctypes.data, g.ctypes.data, out.ctypes.data,
                           max(kh * kw * ci, 1)) != 0:
        raise RuntimeError("orc_im2col_nhwc failed")
    return out
