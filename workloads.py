"""Seeded synthetic inputs for the GEMM workloads.

This module holds no GEMM arithmetic.  It draws operands with numpy's PCG64
generator and converts them to their storage type; both the oracle side and
the HIP side of every test and of bench.py take their inputs from here, so the
two sides see the same bits.

Draw recipe (one generator per problem, seeded):
  * A, then B, then C (only when the workload reads C), each in its STORED
    shape, row-major: A is [K, M] when transposed else [M, K]; B is [N, K]
    when transposed else [K, N]; a leading batch dimension comes first.
  * Floats are drawn in float64 from the stated distribution and converted to
    the storage type: float32 and float16 by numpy's round-to-nearest-even
    cast, bfloat16 by rounding the float32 value to its top 16 bits (nearest,
    ties to even).
  * int8 values are numpy integers drawn uniformly from [-128, 127] inclusive.

The named workloads are the five shapes the library is measured on: fp32 SGEMM
256^3; bf16 NN 4096^3; the fp16 linear-layer backward pair (TN and NT) at
4096^3 with alpha 0.5, beta 1; the bf16 TN split-K weight-gradient shape
128 x 384 x 16384 batched x8; and the ragged int8 NN 4093 x 4099 x 4096.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

# storage numpy dtype of each element type (f16/bf16 are kept as raw bits)
STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16,
           "i8": np.int8, "i32": np.int32}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "i32": 4}


@dataclass(frozen=True)
class Problem:
    """One GEMM problem: shapes, layout, types, scalars and input recipe."""
    name: str
    M: int
    N: int
    K: int
    a_dtype: str                 # "f32" | "f16" | "bf16" | "i8" (B has the same)
    c_dtype: str                 # "f32" | "f16" | "bf16" | "i32"
    transpose_a: bool = False
    transpose_b: bool = False
    alpha: float = 1.0
    beta: float = 0.0
    batch: int = 1
    lda: int = 0                 # 0: contiguous
    ldb: int = 0
    ldc: int = 0
    dist: str = "normal"         # "normal" | "uniform" | "int8"
    scale: float = 1.0           # std of "normal", half-width of "uniform"
    c_dist: str = "zeros"        # "zeros" | "normal" | "nan"
    seed: int = 0
    extra: Dict[str, str] = field(default_factory=dict)

    # resolved leading dims and strides (elements)
    @property
    def LDA(self) -> int:
        return self.lda or (self.M if self.transpose_a else self.K)

    @property
    def LDB(self) -> int:
        return self.ldb or (self.K if self.transpose_b else self.N)

    @property
    def LDC(self) -> int:
        return self.ldc or self.N

    @property
    def a_rows(self) -> int:
        return self.K if self.transpose_a else self.M

    @property
    def b_rows(self) -> int:
        return self.N if self.transpose_b else self.K

    @property
    def stride_a(self) -> int:
        return self.a_rows * self.LDA

    @property
    def stride_b(self) -> int:
        return self.b_rows * self.LDB

    @property
    def stride_c(self) -> int:
        return self.M * self.LDC

    @property
    def layout(self) -> str:
        return ("T" if self.transpose_a else "N") + ("T" if self.transpose_b else "N")

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    @property
    def algorithmic_bytes(self) -> int:
        """A and B read once, C written once (and read once iff beta != 0)."""
        ea, ec = ELEM_BYTES[self.a_dtype], ELEM_BYTES[self.c_dtype]
        per = (self.M * self.K + self.K * self.N) * ea + self.M * self.N * ec
        if self.beta != 0.0:
            per += self.M * self.N * ec
        return per * self.batch

    def with_(self, **kw) -> "Problem":
        return replace(self, **kw)


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        bits = x.astype(np.float32).view(np.uint32).astype(np.uint64)
        rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
        return rounded.astype(np.uint16)
    raise ValueError(dtype)


def _draw(rng: np.random.Generator, shape, p: Problem) -> np.ndarray:
    if p.dist == "int8":
        return rng.integers(-128, 128, size=shape, dtype=np.int8)
    if p.dist == "normal":
        x = rng.normal(0.0, p.scale, size=shape)
    elif p.dist == "uniform":
        x = rng.uniform(-p.scale, p.scale, size=shape)
    elif p.dist == "small_int":
        # integers in [-scale, scale]: every fp32 partial sum stays exact
        x = rng.integers(-int(p.scale), int(p.scale) + 1, size=shape).astype(np.float64)
    else:
        raise ValueError(p.dist)
    return _to_storage(x, p.a_dtype)


def make_inputs(p: Problem):
    """Return (A, B, C) numpy arrays of stored values.

    A: [batch?, a_rows, LDA], B: [batch?, b_rows, LDB], C: [batch?, M, LDC]
    (the batch axis only when batch > 1).  Padding columns beyond the logical
    extent are drawn like the rest.  C holds zeros, N(0,1) values or NaNs as
    c_dist says.
    """
    rng = np.random.default_rng(p.seed)
    lead = (p.batch,) if p.batch > 1 else ()
    A = _draw(rng, lead + (p.a_rows, p.LDA), p)
    B = _draw(rng, lead + (p.b_rows, p.LDB), p)
    cshape = lead + (p.M, p.LDC)
    if p.c_dist == "zeros":
        C = np.zeros(cshape, dtype=STORAGE[p.c_dtype])
    elif p.c_dist == "normal":
        if p.c_dtype == "i32":
            C = rng.integers(-1000, 1000, size=cshape, dtype=np.int32)
        else:
            C = _to_storage(rng.normal(0.0, 1.0, size=cshape), p.c_dtype)
    elif p.c_dist == "nan":
        if p.c_dtype == "i32":
            C = np.full(cshape, -123456789, dtype=np.int32)
        elif p.c_dtype == "f32":
            C = np.full(cshape, np.nan, dtype=np.float32)
        else:
            C = np.full(cshape, 0x7FC0 if p.c_dtype == "bf16" else 0x7E00, dtype=np.uint16)
    else:
        raise ValueError(p.c_dist)
    return A, B, C


def make_bias(p: Problem, nvec: int = 1, seed_offset: int = 77) -> np.ndarray:
    """Fused-epilogue bias: nvec vectors of N values, N(0,1), stored in the
    output type (shape [nvec, N]); seeded from the problem."""
    rng = np.random.default_rng(p.seed + seed_offset)
    return _to_storage(rng.normal(0.0, 1.0, size=(nvec, p.N)), p.c_dtype)


def make_col_scale(p: Problem, nvec: int = 1, seed_offset: int = 91) -> np.ndarray:
    """Per-column dequantization scales: nvec vectors of N fp32 values drawn
    from N(0, 0.01^2) (shape [nvec, N]); seeded from the problem."""
    rng = np.random.default_rng(p.seed + seed_offset)
    return rng.normal(0.0, 0.01, size=(nvec, p.N)).astype(np.float32)


# The five measured workloads.
WORKLOADS: Dict[str, Problem] = {
    "sgemm_nn_256": Problem(
        "sgemm_nn_256", 256, 256, 256, "f32", "f32", dist="uniform", scale=1.0,
        seed=1001),
    "bf16_nn_4096": Problem(
        "bf16_nn_4096", 4096, 4096, 4096, "bf16", "bf16", dist="normal", scale=1.0,
        seed=1002),
    "f16_tn_4096": Problem(
        "f16_tn_4096", 4096, 4096, 4096, "f16", "f16", transpose_a=True,
        alpha=0.5, beta=1.0, dist="normal", scale=0.02, c_dist="normal", seed=1003),
    "f16_nt_4096": Problem(
        "f16_nt_4096", 4096, 4096, 4096, "f16", "f16", transpose_b=True,
        alpha=0.5, beta=1.0, dist="normal", scale=0.02, c_dist="normal", seed=1004),
    "bf16_tn_splitk_b8": Problem(
        "bf16_tn_splitk_b8", 128, 384, 16384, "bf16", "f32", transpose_a=True,
        batch=8, dist="uniform", scale=1.0, seed=1005),
    "i8_nn_ragged": Problem(
        "i8_nn_ragged", 4093, 4099, 4096, "i8", "i32", dist="int8", seed=1006),
    # the int8 ragged shape dequantized per column into bf16 (half the C
    # bytes of int32): not one of the five, measured against it
    "i8_nn_ragged_dequant_bf16": Problem(
        "i8_nn_ragged_dequant_bf16", 4093, 4099, 4096, "i8", "bf16", dist="int8", seed=1006,
        extra={"col_scale": "1"}),
    # a linear layer applied to 4 vectors (x @ W^T, W 16384 x 8192 bf16):
    # HBM-bound on W, the small-M route
    "bf16_gemv_nt_m4": Problem(
        "bf16_gemv_nt_m4", 4, 16384, 8192, "bf16", "bf16", transpose_b=True, dist="normal",
        scale=1.0, seed=1007, extra={"bound": "hbm"}),
    # the headline shape with the fused epilogue (a per-column bias and
    # GELU-tanh): not one of the five, measured against the plain headline
    "bf16_nn_4096_bias_gelu": Problem(
        "bf16_nn_4096_bias_gelu", 4096, 4096, 4096, "bf16", "bf16", dist="normal", scale=1.0,
        seed=1002, extra={"bias": "1", "act": "gelu_tanh"}),
}

HEADLINE = "bf16_nn_4096"


def get(name: str) -> Problem:
    return WORKLOADS[name]


def sample_points(p: Problem, n: int, seed: int = 7) -> np.ndarray:
    """(z, i, j) output coordinates: the four corners of every batch element,
    the last row and column, and n uniformly drawn ones."""
    rng = np.random.default_rng(seed)
    pts = []
    for z in range(p.batch):
        for i in (0, p.M - 1):
            for j in (0, p.N - 1):
                pts.append((z, i, j))
    for j in rng.integers(0, p.N, size=min(64, p.N)):
        pts.append((p.batch - 1, p.M - 1, int(j)))
    for i in rng.integers(0, p.M, size=min(64, p.M)):
        pts.append((p.batch - 1, int(i), p.N - 1))
    z = rng.integers(0, p.batch, size=n)
    i = rng.integers(0, p.M, size=n)
    j = rng.integers(0, p.N, size=n)
    pts.extend(zip(z.tolist(), i.tolist(), j.tolist()))
    return np.asarray(pts, dtype=np.int64)
