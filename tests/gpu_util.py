"""Helpers shared by the GPU tests: move workload inputs to the device, run
the library through its C ABI binding, and compare with the oracle."""
from __future__ import annotations

import contextlib
import os
import sys

import numpy as np

import oracle
import workloads

TOL = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}


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


def oracle_epilogue(p: workloads.Problem, A, B, C, bias, act, *, shared=True, col_scale=None):
    """The oracle's fused form in C's padded layout."""
    c_in = C if p.beta != 0.0 else None
    out, _ = oracle.gemm_epilogue(A, B, c_in, bias=bias, bias_stride=0 if shared else p.N,
                                  col_scale=col_scale, scale_stride=0 if shared else p.N,
                                  act=act, M=p.M, N=p.N, K=p.K, a_dtype=p.a_dtype,
                                  c_dtype=p.c_dtype, transpose_a=p.transpose_a,
                                  transpose_b=p.transpose_b, alpha=p.alpha, beta=p.beta,
                                  lda=p.LDA, ldb=p.LDB, ldc=p.LDC, batch=p.batch,
                                  stride_a=p.stride_a, stride_b=p.stride_b,
                                  stride_c=p.stride_c, C_like=C)
    return out.reshape(C.shape)


def oracle_full(p: workloads.Problem, A, B, C):
    """The whole oracle result in the same padded layout as C."""
    c_in = C if p.beta != 0.0 else None
    out, value = oracle.gemm(A, B, c_in, M=p.M, N=p.N, K=p.K, a_dtype=p.a_dtype,
                             c_dtype=p.c_dtype, transpose_a=p.transpose_a,
                             transpose_b=p.transpose_b, alpha=p.alpha, beta=p.beta,
                             lda=p.LDA, ldb=p.LDB, ldc=p.LDC, batch=p.batch,
                             stride_a=p.stride_a, stride_b=p.stride_b, stride_c=p.stride_c,
                             C_like=C, want_value=False)
    return out.reshape(C.shape)


def logical(p: workloads.Problem, Cfull: np.ndarray) -> np.ndarray:
    return Cfull.reshape((p.batch, p.M, p.LDC))[:, :, :p.N]


def compare(p: workloads.Problem, got_full, ref_full, C_in=None, label=""):
    """Assert parity: bit-exact for int32 results, relative Frobenius error
    within TOL (keyed by input type) for floats; padding columns of C are
    left as they were."""
    got = logical(p, got_full)
    ref = logical(p, ref_full)
    if C_in is not None and p.LDC > p.N:
        pad_got = got_full.reshape((p.batch, p.M, p.LDC))[:, :, p.N:]
        pad_in = C_in.reshape((p.batch, p.M, p.LDC))[:, :, p.N:]
        assert np.array_equal(pad_got.view(np.uint8), pad_in.view(np.uint8)), \
            "%s: padding of C was written" % label
    if p.c_dtype == "i32":
        bad = np.count_nonzero(got != ref)
        assert bad == 0, "%s: %d int32 outputs differ" % (label, bad)
        return 0.0
    g = oracle.decode(got, p.c_dtype)
    r = oracle.decode(ref, p.c_dtype)
    assert np.isfinite(g).all(), "%s: non-finite outputs" % label
    err = oracle.rel_frobenius(g, r)
    # keyed by the input type; int8 dequantized into floats by the output type
    tol = TOL[p.a_dtype] if p.a_dtype in TOL else TOL[p.c_dtype]
    assert err <= tol, "%s: relF %.3g > %.1g" % (label, err, tol)
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
