"""Plain CPU oracle for C = alpha*op(A)*op(B) + beta*C (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's cpu_baseline leg, never by the library under dense_gemm_tiled_amd/,
and it never imports that library.  The arithmetic lives in oracle_gemm.c (a
triple loop accumulating in fp64, int64 for int8); this module only compiles it
with gcc and marshals numpy arrays.

The definition it evaluates comes from tensorcore "GEMM" (sections "Surface",
"Transposes", "Numerical guarantees"), Phobos "Matrix products" (sgemm/hgemm
epilogue, matmul_t) and tessl "Architecture" ("Integer GEMM", "Fused
Epilogue"); the C file's header states it in full.  The fused epilogue
(bias and activation after alpha/beta) is plain numpy in fp64 below.

Every function of this oracle is pinned by tests/test_oracle.py against facts
the pages and the mathematics fix (exhaustive codec round trips, ties-to-even,
exact-rational brute force, identities, alpha/beta closed forms, int8
extremes); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle_gemm.so")

# dtype names -> the oracle's own codes (see the enum in oracle_gemm.c)
DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "i32": 4}
STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16,
           "i8": np.int8, "i32": np.int32}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle_gemm.c into liboracle_gemm.so with gcc (OpenMP)."""
    if not force and os.path.exists(_LIB) and \
            os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-march=x86-64-v2",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, f64, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_gemm.restype = i32
    lib.oracle_gemm.argtypes = [i64, i64, i64, i32, i32, i32, i32, f64, f64,
                                vp, i64, vp, i64, vp, i64, vp, vp,
                                i64, i64, i64, i64, vp]
    lib.oracle_gemm_points.restype = i32
    lib.oracle_gemm_points.argtypes = [i64, i64, i64, i32, i32, i32, i32, f64, f64,
                                       vp, i64, vp, i64, vp, i64, i64, i64, i64,
                                       i64, vp, vp, vp, vp, vp, vp]
    for name in ("oracle_decode_bf16", "oracle_decode_f16"):
        getattr(lib, name).restype = f64
        getattr(lib, name).argtypes = [ctypes.c_uint16]
    for name in ("oracle_round_f32", "oracle_round_bf16", "oracle_round_f16"):
        getattr(lib, name).restype = f64
        getattr(lib, name).argtypes = [f64]
    for name in ("oracle_encode_bf16", "oracle_encode_f16"):
        getattr(lib, name).restype = ctypes.c_uint16
        getattr(lib, name).argtypes = [f64]
    lib.oracle_encode_f32.restype = ctypes.c_float
    lib.oracle_encode_f32.argtypes = [f64]
    lib.oracle_decode_array.restype = None
    lib.oracle_decode_array.argtypes = [vp, i32, i64, vp]
    lib.oracle_encode_array.restype = None
    lib.oracle_encode_array.argtypes = [vp, i32, i64, vp]
    lib.oracle_num_threads.restype = i32
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# ---------------------------------------------------------------- codecs
def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values (raw bits for f16/bf16) -> float64, elementwise."""
    if dtype not in DTYPES:
        raise ValueError(dtype)
    flat = np.ascontiguousarray(bits).ravel().view(STORAGE[dtype])
    out = np.empty(flat.size, dtype=np.float64)
    _load().oracle_decode_array(_ptr(flat), DTYPES[dtype], flat.size, _ptr(out))
    return out.reshape(np.shape(bits))


def round_to(values: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> nearest (ties to even) value of dtype, as float64."""
    lib = _load()
    fn = {"f32": lib.oracle_round_f32, "bf16": lib.oracle_round_bf16,
          "f16": lib.oracle_round_f16}[dtype]
    flat = np.asarray(values, dtype=np.float64).ravel()
    return np.array([fn(float(v)) for v in flat]).reshape(np.shape(values))


def encode(values: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> stored bit patterns of dtype (rounded to nearest even)."""
    if dtype not in ("bf16", "f16", "f32"):
        raise ValueError(dtype)
    flat = np.ascontiguousarray(np.asarray(values, dtype=np.float64).ravel())
    out = np.empty(flat.size, dtype=STORAGE[dtype])
    _load().oracle_encode_array(_ptr(flat), DTYPES[dtype], flat.size, _ptr(out))
    return out.reshape(np.shape(values))


# ---------------------------------------------------------------- GEMM
def _c_dtype_ok(a_dtype: str, c_dtype: str) -> None:
    if a_dtype not in DTYPES or c_dtype not in DTYPES:
        raise ValueError("unknown dtype %s/%s" % (a_dtype, c_dtype))


def gemm(A: np.ndarray, B: np.ndarray, C_in: Optional[np.ndarray], *,
         M: int, N: int, K: int, a_dtype: str, c_dtype: str,
         transpose_a: bool = False, transpose_b: bool = False,
         alpha: float = 1.0, beta: float = 0.0,
         lda: int = 0, ldb: int = 0, ldc: int = 0,
         batch: int = 1, stride_a: int = 0, stride_b: int = 0,
         stride_c: int = 0, C_like: Optional[np.ndarray] = None,
         want_value: bool = True, want_abs: bool = False):
    """Evaluate the whole product.

    A, B, C_in are flat-or-shaped numpy arrays of stored values (uint16 bit
    patterns for f16/bf16).  Leading dims 0 mean contiguous.  Returns
    (C_out, value) where C_out has C_in's layout (or C_like's when C_in is None)
    holding round_c(value) inside the M x N extent, and value is the unrounded
    fp64 result as a dense [batch, M, N] array (None unless want_value).
    With want_abs, returns (C_out, value, T) where T, dense [batch, M, N], is
    the sum over k of |opA(i,k) * opB(k,j)| (the magnitude that scales the
    a-priori error bound of a length-K dot product; exact for int8).
    """
    _c_dtype_ok(a_dtype, c_dtype)
    lda = lda or (M if transpose_a else K)
    ldb = ldb or (K if transpose_b else N)
    ldc = ldc or N
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if C_in is not None:
        C_in = np.ascontiguousarray(C_in)
        C_out = C_in.copy()
    else:
        if C_like is None:
            size = (batch - 1) * stride_c + (M - 1) * ldc + N
            C_like = np.zeros(size, dtype=STORAGE[c_dtype])
        C_out = np.ascontiguousarray(C_like).copy()
    value = np.empty((batch, M, N), dtype=np.float64) if want_value else None
    mag = np.empty((batch, M, N), dtype=np.float64) if want_abs else None
    rc = _load().oracle_gemm(M, N, K, DTYPES[a_dtype], DTYPES[c_dtype],
                             int(bool(transpose_a)), int(bool(transpose_b)),
                             float(alpha), float(beta), _ptr(A), lda, _ptr(B), ldb,
                             _ptr(C_in), ldc, _ptr(C_out), _ptr(value),
                             batch, stride_a, stride_b, stride_c, _ptr(mag))
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments (code %d)" % rc)
    if want_abs:
        return C_out, value, mag
    return C_out, value


def gemm_points(A: np.ndarray, B: np.ndarray, C_in: Optional[np.ndarray],
                points: Sequence[Tuple[int, int, int]], *,
                M: int, N: int, K: int, a_dtype: str, c_dtype: str,
                transpose_a: bool = False, transpose_b: bool = False,
                alpha: float = 1.0, beta: float = 0.0,
                lda: int = 0, ldb: int = 0, ldc: int = 0,
                stride_a: int = 0, stride_b: int = 0, stride_c: int = 0,
                want_abs: bool = False):
    """Evaluate the definition only at the given (z, i, j) outputs.

    Returns (rounded, value): rounded holds c_dtype stored values, value the
    unrounded fp64 results (exact sums for int8); with want_abs, (rounded,
    value, T) with T the magnitude sums at those outputs (see gemm).
    """
    _c_dtype_ok(a_dtype, c_dtype)
    lda = lda or (M if transpose_a else K)
    ldb = ldb or (K if transpose_b else N)
    ldc = ldc or N
    pts = np.asarray(points, dtype=np.int64).reshape(-1, 3)
    zs = np.ascontiguousarray(pts[:, 0])
    is_ = np.ascontiguousarray(pts[:, 1])
    js = np.ascontiguousarray(pts[:, 2])
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    C_in = None if C_in is None else np.ascontiguousarray(C_in)
    value = np.empty(len(pts), dtype=np.float64)
    rounded = np.empty(len(pts), dtype=STORAGE[c_dtype])
    mag = np.empty(len(pts), dtype=np.float64) if want_abs else None
    rc = _load().oracle_gemm_points(M, N, K, DTYPES[a_dtype], DTYPES[c_dtype],
                                    int(bool(transpose_a)), int(bool(transpose_b)),
                                    float(alpha), float(beta), _ptr(A), lda, _ptr(B),
                                    ldb, _ptr(C_in), ldc, stride_a, stride_b, stride_c,
                                    len(pts), _ptr(zs), _ptr(is_), _ptr(js),
                                    _ptr(value), _ptr(rounded), _ptr(mag))
    if rc != 0:
        raise ValueError("oracle_gemm_points rejected its arguments (code %d)" % rc)
    if want_abs:
        return rounded, value, mag
    return rounded, value


# ---------------------------------------------------------------- fused epilogue
# tessl "Architecture", section "Fused Epilogue": the fused form computes
#   C = activation(alpha * A@B + beta * C_prev + bias)
# with bias per output column (a row-stride-0 view: every row of C gets the
# same N values) and the activations none, ReLU and GELU with tanh.  Readings
# where the page is silent: bias is stored in C's element type (the view is
# C-shaped); GELU-tanh is 0.5*y*(1 + tanh(sqrt(2/pi)*(y + 0.044715*y^3))),
# the usual tanh form of GELU, whose clamp on the page only guards an
# exp-based tanh against overflow and does not change the value; ReLU is
# max(y, 0).
#
# Same page, section "Integer GEMM": gemm_i8_dequant takes the exact int32
# sum of int8 x int8 and applies a per-column dequantization in the same
# dispatch.  Reading: the dequantization is a per-column fp32 scale s[j]
# multiplying the sum, so with the epilogue above
#   C = activation(alpha * s[j] * S + beta * C_prev + bias)
# (s[j] = 1 without a scale); for int8 inputs the scale is required and C is
# fp32, fp16 or bf16.  Everything is evaluated in fp64 from the exact sums S,
# then rounded once to c_dtype (ties to even) like the plain product.
ACTIVATIONS = ("none", "relu", "gelu_tanh")


def activation(y: np.ndarray, act: str) -> np.ndarray:
    """The activation, elementwise in fp64."""
    y = np.asarray(y, dtype=np.float64)
    if act == "none":
        return y.copy()
    if act == "relu":
        return np.where(y > 0.0, y, 0.0)
    if act == "gelu_tanh":
        u = math.sqrt(2.0 / math.pi) * (y + 0.044715 * y * y * y)
        return 0.5 * y * (1.0 + np.tanh(u))
    raise ValueError("unknown activation %r" % (act,))


def _epilogue_args(kw, col_scale, act):
    a_dtype, c_dtype = kw.get("a_dtype"), kw.get("c_dtype")
    if act not in ACTIVATIONS:
        raise ValueError("unknown activation %r" % (act,))
    if a_dtype == "i8":
        if col_scale is None:
            raise ValueError("int8 takes the fused form only with a per-column dequant scale")
        if c_dtype not in ("f32", "f16", "bf16"):
            raise ValueError("dequantized int8 results are f32, f16 or bf16")


def _sum_kw(kw):
    """gemm() arguments that give the plain sums S (alpha 1, beta 0)."""
    skw = dict(kw)
    skw.update(alpha=1.0, beta=0.0)
    if kw["a_dtype"] == "i8":
        skw["c_dtype"] = "i32"
    skw.pop("ldc", None)
    skw.pop("stride_c", None)
    skw.pop("C_like", None)
    return skw


def gemm_epilogue(A: np.ndarray, B: np.ndarray, C_in: Optional[np.ndarray], *,
                  bias: Optional[np.ndarray] = None, bias_stride: int = 0,
                  col_scale: Optional[np.ndarray] = None, scale_stride: int = 0,
                  act: str = "none", want_abs: bool = False, **kw):
    """The fused form: gemm()'s arguments plus bias / bias_stride (stored
    c_dtype values, problem z's N values at z*bias_stride), col_scale /
    scale_stride (fp32 values, likewise) and act.  Returns (C_out, value) like
    gemm(), value being the fp64 result after the epilogue (before rounding
    to c_dtype), dense [batch, M, N]; with want_abs, (C_out, value, T) with
    T the magnitude sums of the product (see gemm)."""
    _epilogue_args(kw, col_scale, act)
    M, N, batch = kw["M"], kw["N"], kw.get("batch", 1)
    c_dtype, alpha, beta = kw["c_dtype"], kw.get("alpha", 1.0), kw.get("beta", 0.0)
    ldc = kw.get("ldc", 0) or N
    stride_c = kw.get("stride_c", 0)
    # the exact sums (alpha = 0 reads neither A nor B)
    if alpha != 0.0:
        _, S, T = gemm(A, B, None, want_value=True, want_abs=True, stride_c=M * N,
                       **_sum_kw(kw))
    else:
        S = np.zeros((batch, M, N))
        T = np.zeros((batch, M, N))
    if col_scale is not None:
        sc = np.asarray(col_scale, dtype=np.float32).ravel().astype(np.float64)
        for z in range(batch):
            S[z] *= sc[z * scale_stride: z * scale_stride + N][None, :]
    y = alpha * S
    if beta != 0.0:
        cin = decode(np.ascontiguousarray(C_in).ravel(), c_dtype)
        for z in range(batch):
            for i in range(M):
                o = z * stride_c + i * ldc
                y[z, i] += beta * cin[o:o + N]
    if bias is not None:
        b = decode(np.ascontiguousarray(bias).ravel(), c_dtype)
        for z in range(batch):
            y[z] += b[z * bias_stride: z * bias_stride + N][None, :]
    y = activation(y, act)
    if C_in is not None:
        C_out = np.ascontiguousarray(C_in).copy()
    else:
        C_like = kw.get("C_like")
        if C_like is None:
            C_like = np.zeros((batch - 1) * stride_c + (M - 1) * ldc + N, dtype=STORAGE[c_dtype])
        C_out = np.ascontiguousarray(C_like).copy()
    enc = encode(y, c_dtype)
    flat = C_out.ravel()
    for z in range(batch):
        for i in range(M):
            o = z * stride_c + i * ldc
            flat[o:o + N] = enc[z, i]
    if want_abs:
        return flat.reshape(C_out.shape), y, T
    return flat.reshape(C_out.shape), y


def gemm_epilogue_points(A: np.ndarray, B: np.ndarray, C_in: Optional[np.ndarray],
                         points: Sequence[Tuple[int, int, int]], *,
                         bias: Optional[np.ndarray] = None, bias_stride: int = 0,
                         col_scale: Optional[np.ndarray] = None, scale_stride: int = 0,
                         act: str = "none", want_abs: bool = False, **kw):
    """The fused form at the given (z, i, j) outputs only.  Returns (rounded,
    value) like gemm_points; with want_abs, (rounded, value, T)."""
    _epilogue_args(kw, col_scale, act)
    c_dtype, alpha, beta = kw["c_dtype"], kw.get("alpha", 1.0), kw.get("beta", 0.0)
    pts = np.asarray(points, dtype=np.int64).reshape(-1, 3)
    if alpha != 0.0:
        _, S, T = gemm_points(A, B, None, pts, want_abs=True, **_sum_kw(kw))
    else:
        S = np.zeros(len(pts))
        T = np.zeros(len(pts))
    if col_scale is not None:
        sc = np.asarray(col_scale, dtype=np.float32).ravel().astype(np.float64)
        S = S * sc[pts[:, 0] * scale_stride + pts[:, 2]]
    y = alpha * S
    if beta != 0.0:
        ldc = kw.get("ldc", 0) or kw["N"]
        cin = decode(np.ascontiguousarray(C_in).ravel(), c_dtype)
        y = y + beta * cin[pts[:, 0] * kw.get("stride_c", 0) + pts[:, 1] * ldc + pts[:, 2]]
    if bias is not None:
        b = decode(np.ascontiguousarray(bias).ravel(), c_dtype)
        y = y + b[pts[:, 0] * bias_stride + pts[:, 2]]
    y = activation(y, act)
    if want_abs:
        return encode(y, c_dtype), y, T
    return encode(y, c_dtype), y


def rel_frobenius(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_F / ||ref||_F in fp64 (the error measure of tensorcore
    "GEMM", section "Numerical guarantees", with epsilon = 0: a zero reference
    demands an exactly zero result, reported as 0 or inf)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.linalg.norm((got - ref).ravel()))
    den = float(np.linalg.norm(ref.ravel()))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
