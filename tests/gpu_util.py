"""Helpers shared by the GPU tests: move workload inputs to the device, run
the library through its C ABI binding, and compare with the oracle.

A float comparison passes two gates.  The whole result must be within the
relative Frobenius error the pages measure (tensorcore "GEMM", "Numerical
guarantees": 1e-3 for fp16/bf16 inputs, 1e-5 for fp32), and every output
must be within an a-priori bound of the exact value v (the oracle's
unrounded fp64 result):

    |C_gpu - v| <= gamma_{K+3} * |alpha * s| * T + 2u * (|beta * C_in| + |bias|)
                   + 1/2 ulp_c(max(|C_gpu|, |v|))

with u = 2^-24 (the fp32 accumulator's unit roundoff), gamma_n = n u / (1 -
n u), T = sum_k |a_ik b_kj| (from the oracle), s the per-column scale (1
without one).  gamma_K T bounds any fp32 summation order of the K products
(the standard dot-product bound; tessl "Architecture", "Reductions and
Numerical Safety", bounds its sums the same way), the three extra roundings
cover the conversion and the alpha/scale products, 2u the fma that adds
beta*C and the bias, and half an ulp of the output type the final rounding.
For exact int8 sums the gamma term has no K.  GELU multiplies the error by
its Lipschitz constant and adds its own fp32 evaluation error.  Int32
results are compared bit for bit.
"""
from __future__ import annotations

import contextlib
import dataclasses
import os
import sys
from typing import Optional

import numpy as np

import oracle
import workloads

TOL = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}

U = 2.0 ** -24                 # unit roundoff of the fp32 accumulator
GELU_LIP = 1.13                # max |d gelu_tanh / dy| = 1.1289...
_FMT = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}   # (p, emin)


def gamma(n: int) -> float:
    return n * U / (1.0 - n * U)


def ulp(x, dtype: str) -> np.ndarray:
    """Spacing of dtype's numbers in the binade of |x| (the subnormal spacing
    below the normal range and at zero)."""
    p, emin = _FMT[dtype]
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, E = np.frexp(a)
    e = np.where(a > 0, np.maximum(E.astype(np.int64) - 1, emin), emin)
    return np.ldexp(1.0, e - (p - 1))


@dataclasses.dataclass
class Ref:
    """The oracle's answer for one call.

    out: rounded result in C's padded layout (stored values); value: the
    unrounded fp64 result (after the epilogue), mag: |alpha * s| * T and
    side: |beta * C_in| + |bias|, all [batch, M, N] (None for int32 results,
    which are exact); k_terms: K for float inputs, 0 for exact int8 sums;
    act: the activation."""
    out: np.ndarray
    value: Optional[np.ndarray] = None
    mag: Optional[np.ndarray] = None
    side: Optional[np.ndarray] = None
    k_terms: int = 0
    act: str = "none"


def error_bound(ref_value, got, mag, side, k_terms: int, act: str, c_dtype: str):
    """Per-output a-priori bound on |got - value| (see the module docstring)."""
    ey = gamma(k_terms + 3) * mag + 2.0 * U * side
    if act == "gelu_tanh":
        ey = GELU_LIP * ey + 16.0 * U * (mag + side)
    big = np.maximum(np.abs(got), np.abs(ref_value))
    return ey + 0.5 * ulp(big, c_dtype)


def check_elementwise(got, ref_value, mag, side, k_terms: int, act: str, c_dtype: str,
                      label: str = "") -> float:
    """Assert every float output is within error_bound of the exact value;
    returns the largest |got - value|.  got: decoded outputs (fp64)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref_value)
    bound = error_bound(ref_value, got, mag, side, k_terms, act, c_dtype)
    bad = ~(err <= bound)                     # NaN errors count as bad
    n_bad = int(np.count_nonzero(bad))
    if n_bad:
        idx = np.unravel_index(int(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300),
                                                      -1.0))), err.shape)
        raise AssertionError(
            "%s: %d outputs outside the elementwise bound; worst at %s: got %r, exact %r, "
            "|err| %.3g > bound %.3g; max |err| over all outputs %.3g"
            % (label, n_bad, tuple(int(i) for i in idx), float(got[idx]),
               float(ref_value[idx]), float(err[idx]), float(bound[idx]), float(np.nanmax(err))))
    return float(err.max()) if err.size else 0.0


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "i8": torch.int8, "i32": torch.int32}[name]


def to_dev(arr: np.ndarray, dtype: str):
    import torch
    if dtype in ("f16", "bf16"):
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch_dtype(dtype))
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.cuda()


def from_dev(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if dtype in ("f16", "bf16"):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def logical_views(p: workloads.Problem, a_full, b_full, c_full):
    """Views of the padded device buffers with the logical column counts."""
    a_cols = p.M if p.transpose_a else p.K
    b_cols = p.K if p.transpose_b else p.N
    return a_full[..., :a_cols], b_full[..., :b_cols], c_full[..., :p.N]


def shifted(t):
    """A copy of t whose storage starts one element past a 16-byte boundary."""
    import torch
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    assert flat.data_ptr() % 16 == 0
    view = flat[1:].view(t.shape)
    view.copy_(t)
    return view


def run_library(p: workloads.Problem, A, B, C, *, sync=True, misalign=False):
    """Run the HIP path on the stored inputs; returns the whole C buffer
    (padding included) as stored values.  misalign: A and B start one element
    past a 16-byte boundary."""
    import torch
    import dense_gemm_tiled_amd as tg
    a_full, b_full, c_full = to_dev(A, p.a_dtype), to_dev(B, p.a_dtype), to_dev(C, p.c_dtype)
    if misalign:
        a_full, b_full = shifted(a_full), shifted(b_full)
    a, b, c = logical_views(p, a_full, b_full, c_full)
    tg.gemm(a, b, c, alpha=p.alpha, beta=p.beta, transpose_a=p.transpose_a,
            transpose_b=p.transpose_b)
    if sync:
        torch.cuda.synchronize()
    return from_dev(c_full, p.c_dtype)


def run_library_epilogue(p: workloads.Problem, A, B, C, bias, act, *, shared=True,
                         col_scale=None):
    """run_library with the fused epilogue: bias [nvec, N] stored values
    (None: no bias), act an activation name, col_scale [nvec, N] fp32 (None:
    no scale).  shared: one vector for every problem (1-D tensors), else one
    per problem."""
    import torch
    import dense_gemm_tiled_amd as tg
    a_full, b_full, c_full = to_dev(A, p.a_dtype), to_dev(B, p.a_dtype), to_dev(C, p.c_dtype)
    a, b, c = logical_views(p, a_full, b_full, c_full)
    bt = st = None
    if bias is not None:
        bt = to_dev(bias, p.c_dtype)
        bt = bt[0] if shared else bt
    if col_scale is not None:
        st = torch.from_numpy(np.ascontiguousarray(col_scale)).cuda()
        st = st[0] if shared else st
    tg.gemm(a, b, c, alpha=p.alpha, beta=p.beta, transpose_a=p.transpose_a,
            transpose_b=p.transpose_b, bias=bt, activation=act, col_scale=st)
    torch.cuda.synchronize()
    return from_dev(c_full, p.c_dtype)


def _side(p: workloads.Problem, C, bias=None, bias_stride=0):
    """|beta * C_in| + |bias| as [batch, M, N] (fp64)."""
    side = np.zeros((p.batch, p.M, p.N))
    if p.beta != 0.0:
        cin = oracle.decode(np.ascontiguousarray(C).ravel(), p.c_dtype)
        for z in range(p.batch):
            rows = cin[z * p.stride_c: z * p.stride_c + (p.M - 1) * p.LDC + p.N]
            side[z] = np.abs(p.beta) * np.abs(
                np.lib.stride_tricks.as_strided(rows, (p.M, p.N), (p.LDC * 8, 8)))
    if bias is not None:
        b = oracle.decode(np.ascontiguousarray(bias).ravel(), p.c_dtype)
        for z in range(p.batch):
            side[z] += np.abs(b[z * bias_stride: z * bias_stride + p.N])[None, :]
    return side


def _scale_of(p: workloads.Problem, col_scale, scale_stride):
    """|alpha * s| as a [batch, 1, N] array (s = 1 without a scale)."""
    s = np.ones((p.batch, 1, p.N))
    if col_scale is not None:
        sc = np.asarray(col_scale, dtype=np.float32).ravel().astype(np.float64)
        for z in range(p.batch):
            s[z, 0] = sc[z * scale_stride: z * scale_stride + p.N]
    return np.abs(p.alpha) * np.abs(s)


def oracle_epilogue(p: workloads.Problem, A, B, C, bias, act, *, shared=True,
                    col_scale=None) -> Ref:
    """The oracle's fused form in C's padded layout, with what the
    elementwise bound needs."""
    c_in = C if p.beta != 0.0 else None
    stride = 0 if shared else p.N
    out, value, T = oracle.gemm_epilogue(
        A, B, c_in, bias=bias, bias_stride=stride, col_scale=col_scale, scale_stride=stride,
        act=act, M=p.M, N=p.N, K=p.K, a_dtype=p.a_dtype, c_dtype=p.c_dtype,
        transpose_a=p.transpose_a, transpose_b=p.transpose_b, alpha=p.alpha, beta=p.beta,
        lda=p.LDA, ldb=p.LDB, ldc=p.LDC, batch=p.batch, stride_a=p.stride_a,
        stride_b=p.stride_b, stride_c=p.stride_c, C_like=C, want_abs=True)
    mag = _scale_of(p, col_scale, stride) * T
    return Ref(out.reshape(C.shape), value, mag, _side(p, C, bias, stride),
               0 if p.a_dtype == "i8" else p.K, act)


def oracle_full(p: workloads.Problem, A, B, C) -> Ref:
    """The whole oracle result in the same padded layout as C, with what the
    elementwise bound needs."""
    c_in = C if p.beta != 0.0 else None
    out, value, T = oracle.gemm(A, B, c_in, M=p.M, N=p.N, K=p.K, a_dtype=p.a_dtype,
                                c_dtype=p.c_dtype, transpose_a=p.transpose_a,
                                transpose_b=p.transpose_b, alpha=p.alpha, beta=p.beta,
                                lda=p.LDA, ldb=p.LDB, ldc=p.LDC, batch=p.batch,
                                stride_a=p.stride_a, stride_b=p.stride_b,
                                stride_c=p.stride_c, C_like=C, want_abs=True)
    if p.c_dtype == "i32":
        return Ref(out.reshape(C.shape))
    return Ref(out.reshape(C.shape), value, abs(p.alpha) * T, _side(p, C),
               0 if p.a_dtype == "i8" else p.K)


def logical(p: workloads.Problem, Cfull: np.ndarray) -> np.ndarray:
    return Cfull.reshape((p.batch, p.M, p.LDC))[:, :, :p.N]


def compare(p: workloads.Problem, got_full, ref: Ref, C_in=None, label=""):
    """Assert parity: bit-exact for int32 results; for floats the relative
    Frobenius error within TOL (keyed by input type) and every output within
    the elementwise bound; padding columns of C are left as they were.
    Returns the relative Frobenius error."""
    got = logical(p, got_full)
    ref_out = logical(p, ref.out)
    if C_in is not None and p.LDC > p.N:
        pad_got = got_full.reshape((p.batch, p.M, p.LDC))[:, :, p.N:]
        pad_in = C_in.reshape((p.batch, p.M, p.LDC))[:, :, p.N:]
        assert np.array_equal(pad_got.view(np.uint8), pad_in.view(np.uint8)), \
            "%s: padding of C was written" % label
    if p.c_dtype == "i32":
        bad = np.count_nonzero(got != ref_out)
        assert bad == 0, "%s: %d int32 outputs differ" % (label, bad)
        return 0.0
    g = oracle.decode(got, p.c_dtype)
    r = oracle.decode(ref_out, p.c_dtype)
    assert np.isfinite(g).all(), "%s: non-finite outputs" % label
    err = oracle.rel_frobenius(g, r)
    # keyed by the input type; int8 dequantized into floats by the output type
    tol = TOL[p.a_dtype] if p.a_dtype in TOL else TOL[p.c_dtype]
    n_diff = int(np.count_nonzero(g != r))
    assert err <= tol, "%s: relF %.3g > %.1g (%d outputs differ from the rounded oracle, " \
        "max |diff| %.3g)" % (label, err, tol, n_diff, float(np.abs(g - r).max()))
    check_elementwise(g, ref.value, ref.mag, ref.side, ref.k_terms, ref.act, p.c_dtype,
                      label)
    return err


def compare_points(p: workloads.Problem, got_vals, rounded, value, T, *, C_in=None,
                   bias=None, col_scale=None, act="none", pts=None, label=""):
    """The two float gates at sampled outputs: got_vals and rounded are
    stored values at the points, value and T the oracle's unrounded values
    and magnitude sums there (shared bias and scale vectors)."""
    g = oracle.decode(got_vals, p.c_dtype)
    r = oracle.decode(rounded, p.c_dtype)
    tol = TOL[p.a_dtype] if p.a_dtype in TOL else TOL[p.c_dtype]
    err = oracle.rel_frobenius(g, r)
    assert err <= tol, "%s: relF %.3g > %.1g at %d points" % (label, err, tol, len(g))
    s = np.ones(len(g))
    if col_scale is not None:
        s = np.abs(np.asarray(col_scale, np.float32).ravel()[pts[:, 2]].astype(np.float64))
    side = np.zeros(len(g))
    if p.beta != 0.0:
        cin = oracle.decode(np.ascontiguousarray(C_in).ravel(), p.c_dtype)
        side += abs(p.beta) * np.abs(cin[pts[:, 0] * p.stride_c + pts[:, 1] * p.LDC + pts[:, 2]])
    if bias is not None:
        side += np.abs(oracle.decode(np.ascontiguousarray(bias).ravel(), p.c_dtype)[pts[:, 2]])
    check_elementwise(g, value, abs(p.alpha) * s * T, side, 0 if p.a_dtype == "i8" else p.K,
                      act, p.c_dtype, label)
    return err


@contextlib.contextmanager
def env(**kw):
    old = {k: os.environ.get(k) for k in kw}
    for k, v in kw.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = str(v)
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def say(*args):
    """Name the case before a GPU step, flushed, so a fault points at it."""
    print(*args, flush=True)
    sys.stdout.flush()
