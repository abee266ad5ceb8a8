"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test checks the oracle against something it does not share code with:
library codecs used as a special case (numpy float16, torch bfloat16), brute
force over every value of a format, exact rational arithmetic (fractions) on
tiny problems, closed forms (identity, permutation, alpha/beta), and the
integer extremes the tessl "Architecture" page names in "Integer GEMM".
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FLOAT_TYPES = ("f32", "f16", "bf16")


# ----------------------------------------------------------------- helpers
def lib_decode(bits, dtype):
    """Decode with a library (independent of the oracle's decoders)."""
    bits = np.asarray(bits)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        t = torch.from_numpy(bits.astype(np.uint16).view(np.int16).copy())
        return t.view(torch.bfloat16).to(torch.float64).numpy()
    if dtype == "f32":
        return bits.astype(np.float32).astype(np.float64)
    return bits.astype(np.float64)


def finite_values(dtype):
    """Every finite value of a 16-bit format, sorted, with its bit pattern."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = lib_decode(bits, dtype)
    ok = np.isfinite(vals)
    vals, bits = vals[ok], bits[ok]
    order = np.lexsort((bits, vals))
    return vals[order], bits[order]


FORMAT = {  # significand bits (with hidden bit), max finite exponent
    "f16": (11, 15), "bf16": (8, 127), "f32": (24, 127)}


def nearest_by_search(x, dtype, table):
    """Round x to dtype by searching the enumerated finite values: nearest by
    exact distance, ties to the pattern whose last significand bit is 0, and
    +-inf beyond max + half an ulp (IEEE's unbounded-exponent rule)."""
    vals, bits = table
    p, emax = FORMAT[dtype]
    maxf = float(vals[-1])
    half_ulp_top = Fraction(2) ** (emax - p)        # half an ulp at the top binade
    fx = Fraction(x)
    if fx >= Fraction(maxf) + half_ulp_top:
        return math.inf
    if fx <= -Fraction(maxf) - half_ulp_top:
        return -math.inf
    k = int(np.searchsorted(vals, x))
    cands = [c for c in (k - 1, k, k + 1) if 0 <= c < len(vals)]
    best = None
    for c in cands:
        d = abs(Fraction(float(vals[c])) - fx)
        key = (d, int(bits[c]) & 1)                  # even last bit wins a tie
        if best is None or key < best[0]:
            best = (key, c)
    v = float(vals[best[1]])
    if v == 0.0:
        return math.copysign(0.0, x)
    return v


def nan_like(x, dtype):
    if dtype == "f32":
        return np.full_like(x, np.nan)
    return np.full_like(x, 0x7E00 if dtype == "f16" else 0x7FC0)


def exact_gemm(A, B, C, M, N, K, ta, tb, alpha, beta, lda, ldb, ldc):
    """The definition in exact rational arithmetic (tiny sizes only)."""
    out = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                a = A[k * lda + i] if ta else A[i * lda + k]
                b = B[j * ldb + k] if tb else B[k * ldb + j]
                s += Fraction(float(a)) * Fraction(float(b))
            v = Fraction(alpha) * s
            if beta != 0:
                v += Fraction(beta) * Fraction(float(C[i * ldc + j]))
            out[i][j] = v
    return out


def draw(rng, dtype, shape, kind="normal"):
    if dtype == "i8":
        return rng.integers(-128, 128, size=shape, dtype=np.int8)
    if kind == "small_int":
        x = rng.integers(-4, 5, size=shape).astype(np.float64)
    else:
        x = rng.normal(0, 1, size=shape)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------- codecs
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_exhaustive_matches_library(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, dtype)
    ref = lib_decode(bits, dtype)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_encode_roundtrip_exhaustive(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = lib_decode(bits, dtype)
    ok = ~np.isnan(vals)
    back = oracle.encode(vals[ok], dtype)
    assert np.array_equal(back, bits[ok])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_round_ties_to_even_at_every_midpoint(dtype):
    vals, bits = finite_values(dtype)
    pos = vals > 0
    v, b = vals[pos], bits[pos]
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2.0                    # exact in fp64 (few bits)
    even_lo = (b[:-1] & 1) == 0
    expect = np.where(even_lo, lo, hi)
    got = oracle.round_to(mid, dtype)
    assert np.array_equal(got, expect)
    assert np.array_equal(oracle.round_to(-mid, dtype), -expect)
    # just below / above a midpoint go to the nearer neighbour
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    assert np.array_equal(oracle.round_to(below, dtype), lo)
    assert np.array_equal(oracle.round_to(above, dtype), hi)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_round_matches_enumerated_nearest(dtype):
    table = finite_values(dtype)
    rng = np.random.default_rng(11)
    p, emax = FORMAT[dtype]
    xs = np.concatenate([
        rng.normal(0, 1, 400),
        rng.normal(0, 1, 300) * np.exp2(rng.integers(-30 if dtype == "f16" else -140,
                                                     emax + 2, 300)),
        rng.uniform(-1, 1, 100) * float(table[0][-1]) * 1.01,
    ])
    got = oracle.round_to(xs, dtype)
    ref = np.array([nearest_by_search(float(x), dtype, table) for x in xs])
    assert np.array_equal(got, ref)


def test_f16_round_matches_numpy_direct_cast():
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.normal(0, 1, 20000),
                         rng.normal(0, 1, 20000) * np.exp2(rng.integers(-28, 17, 20000))])
    got = oracle.encode(xs, "f16")
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f32_round_matches_hardware_cast():
    rng = np.random.default_rng(4)
    xs = rng.normal(0, 1, 50000) * np.exp2(rng.integers(-150, 129, 50000))
    got = oracle.round_to(xs, "f32")
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float32).astype(np.float64)
    assert np.array_equal(got, ref)


def test_overflow_and_specials():
    assert oracle.round_to(np.array([65520.0]), "f16")[0] == math.inf     # tie -> even -> inf
    assert oracle.round_to(np.array([65519.0]), "f16")[0] == 65504.0
    assert oracle.encode(np.array([-1e9]), "f16")[0] == 0xFC00
    assert oracle.encode(np.array([3.5e38]), "bf16")[0] == 0x7F80
    assert oracle.encode(np.array([2.0 ** -25]), "f16")[0] == 0x0000         # tie -> even zero
    assert oracle.encode(np.array([2.0 ** -25 * 1.5]), "f16")[0] == 0x0001
    assert oracle.encode(np.array([-0.0]), "bf16")[0] == 0x8000


# ----------------------------------------------------------------- GEMM vs exact rationals
LAYOUTS = [(False, False), (True, False), (False, True), (True, True)]


def _tiny_case(rng, dtype, ta, tb, M, N, K, pad, kind):
    lda = (M if ta else K) + pad
    ldb = (K if tb else N) + pad
    ldc = N + pad
    A = draw(rng, dtype, ((K if ta else M) * lda,), kind)
    B = draw(rng, dtype, ((N if tb else K) * ldb,), kind)
    return A, B, lda, ldb, ldc


@pytest.mark.parametrize("dtype", FLOAT_TYPES)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, 1.0), (-2.0, 0.25)])
def test_tiny_float_gemm_against_exact_rationals(dtype, ta, tb, alpha, beta):
    rng = np.random.default_rng(hash((dtype, ta, tb, alpha)) % 2**32)
    M, N, K, pad = 7, 5, 8, 3
    A, B, lda, ldb, ldc = _tiny_case(rng, dtype, ta, tb, M, N, K, pad, "normal")
    C_in = draw(rng, dtype, (M * ldc,), "normal")
    Ad, Bd, Cd = (lib_decode(x, dtype) for x in (A, B, C_in))
    exact = exact_gemm(Ad, Bd, Cd, M, N, K, ta, tb, alpha, beta, lda, ldb, ldc)
    C_out, value = oracle.gemm(A, B, C_in, M=M, N=N, K=K, a_dtype=dtype, c_dtype=dtype,
                               transpose_a=ta, transpose_b=tb, alpha=alpha, beta=beta,
                               lda=lda, ldb=ldb, ldc=ldc)
    table = finite_values(dtype) if dtype != "f32" else None
    got = lib_decode(C_out, dtype)
    for i in range(M):
        for j in range(N):
            ex = exact[i][j]
            # fp64 sum of K exact products: error within K*2^-53*sum|terms|
            bound = Fraction(K + 2) * Fraction(2) ** -53 * (abs(ex) + 64)
            assert abs(Fraction(value[0, i, j]) - ex) <= bound
            if dtype == "f32":
                want = float(np.float64(float(ex)).astype(np.float32))
            else:
                want = nearest_by_search(float(ex), dtype, table)
            assert got[i * ldc + j] == want, (i, j)
    # padding columns of C are untouched
    for i in range(M):
        for j in range(N, ldc):
            assert C_out[i * ldc + j] == C_in[i * ldc + j] or (
                np.isnan(got[i * ldc + j]) and np.isnan(lib_decode(C_in[i * ldc + j], dtype)))


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_tiny_int8_gemm_against_exact_integers(ta, tb):
    rng = np.random.default_rng(77)
    M, N, K, pad = 6, 9, 13, 2
    A, B, lda, ldb, ldc = _tiny_case(rng, "i8", ta, tb, M, N, K, pad, "")
    C_out, value = oracle.gemm(A, B, None, M=M, N=N, K=K, a_dtype="i8", c_dtype="i32",
                               transpose_a=ta, transpose_b=tb, lda=lda, ldb=ldb, ldc=ldc,
                               C_like=np.full(M * ldc, 99, dtype=np.int32))
    exact = exact_gemm(A.astype(np.int64), B.astype(np.int64), None, M, N, K, ta, tb,
                       1, 0, lda, ldb, ldc)
    for i in range(M):
        for j in range(N):
            assert C_out[i * ldc + j] == exact[i][j]
            assert value[0, i, j] == exact[i][j]
        for j in range(N, ldc):
            assert C_out[i * ldc + j] == 99


@pytest.mark.parametrize("dtype", FLOAT_TYPES + ("i8",))
def test_small_integer_inputs_are_exact(dtype):
    """Integer-valued inputs keep every fp64 partial sum exact, so the oracle
    value equals the exact integer sum."""
    rng = np.random.default_rng(5)
    M, N, K = 9, 11, 40
    A = draw(rng, dtype, (M * K,), "small_int")
    B = draw(rng, dtype, (K * N,), "small_int")
    c_dtype = "i32" if dtype == "i8" else dtype
    _, value = oracle.gemm(A, B, None, M=M, N=N, K=K, a_dtype=dtype, c_dtype=c_dtype)
    Ad = lib_decode(A, dtype).reshape(M, K).astype(np.int64)
    Bd = lib_decode(B, dtype).reshape(K, N).astype(np.int64)
    assert np.array_equal(value[0], (Ad @ Bd).astype(np.float64))


# ----------------------------------------------------------------- closed forms
@pytest.mark.parametrize("dtype", FLOAT_TYPES + ("i8",))
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_identity_and_permutation(dtype, ta, tb):
    rng = np.random.default_rng(9)
    n = 12
    one = {"f32": np.float32(1), "f16": np.float16(1).view(np.uint16),
           "bf16": np.uint16(0x3F80), "i8": np.int8(1)}[dtype]
    perm = rng.permutation(n)
    P = np.zeros((n, n), dtype=draw(rng, dtype, (1,)).dtype)
    P[np.arange(n), perm] = one                  # (P @ X)[i] = X[perm[i]]
    X = draw(rng, dtype, (n, n))
    c_dtype = "i32" if dtype == "i8" else dtype
    A = P.T.copy() if ta else P
    B = X.T.copy() if tb else X
    C_out, _ = oracle.gemm(A, B, None, M=n, N=n, K=n, a_dtype=dtype, c_dtype=c_dtype,
                           transpose_a=ta, transpose_b=tb)
    C_out = C_out.reshape(n, n)
    if dtype == "i8":
        assert np.array_equal(C_out, X[perm].astype(np.int32))
    else:
        assert np.array_equal(C_out, X[perm])


@pytest.mark.parametrize("dtype", FLOAT_TYPES + ("i8",))
def test_transposed_storage_equals_plain(dtype):
    rng = np.random.default_rng(10)
    M, N, K = 10, 7, 33
    A = draw(rng, dtype, (M, K))
    B = draw(rng, dtype, (K, N))
    c_dtype = "i32" if dtype == "i8" else dtype
    ref, _ = oracle.gemm(A, B, None, M=M, N=N, K=K, a_dtype=dtype, c_dtype=c_dtype)
    for ta, tb in LAYOUTS[1:]:
        As = A.T.copy() if ta else A
        Bs = B.T.copy() if tb else B
        got, _ = oracle.gemm(As, Bs, None, M=M, N=N, K=K, a_dtype=dtype, c_dtype=c_dtype,
                             transpose_a=ta, transpose_b=tb)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype", FLOAT_TYPES)
def test_alpha_beta_closed_forms(dtype):
    rng = np.random.default_rng(12)
    M, N, K = 8, 6, 16
    A = draw(rng, dtype, (M, K))
    B = draw(rng, dtype, (K, N))
    C = draw(rng, dtype, (M, N))
    Cd = lib_decode(C, dtype)
    kw = dict(M=M, N=N, K=K, a_dtype=dtype, c_dtype=dtype)
    # alpha = 0: C = round(beta*C_in) and A, B are never read (NaN operands)
    out, val = oracle.gemm(nan_like(A, dtype), nan_like(B, dtype), C,
                           alpha=0.0, beta=0.75, **kw)
    assert np.array_equal(val[0], 0.75 * Cd)
    # alpha = 0, beta = 1: C unchanged bit for bit
    out, _ = oracle.gemm(A, B, C, alpha=0.0, beta=1.0, **kw)
    assert np.array_equal(out, C)
    # alpha = 2 doubles the alpha = 1 value exactly (a power-of-two scale)
    _, v1 = oracle.gemm(A, B, None, alpha=1.0, beta=0.0, **kw)
    _, v2 = oracle.gemm(A, B, None, alpha=2.0, beta=0.0, **kw)
    assert np.array_equal(v2, 2.0 * v1)
    # beta = 0: C_in is not read, so NaNs there do not leak
    o_nan, v_nan = oracle.gemm(A, B, nan_like(C, dtype), alpha=1.0, beta=0.0, **kw)
    assert np.array_equal(v_nan, v1)
    assert not np.isnan(lib_decode(o_nan, dtype)).any()


def test_linearity_in_b():
    rng = np.random.default_rng(13)
    M, N, K = 9, 8, 64
    A = rng.normal(0, 1, (M, K)).astype(np.float32)
    # B1, B2 with few significand bits so that B1 + B2 is exact in fp32
    B1 = (np.round(rng.normal(0, 1, (K, N)) * 64) / 64).astype(np.float32)
    B2 = (np.round(rng.normal(0, 1, (K, N)) * 64) / 64).astype(np.float32)
    kw = dict(M=M, N=N, K=K, a_dtype="f32", c_dtype="f32")
    _, v12 = oracle.gemm(A, B1 + B2, None, **kw)
    _, v1 = oracle.gemm(A, B1, None, **kw)
    _, v2 = oracle.gemm(A, B2, None, **kw)
    absum = np.abs(A).astype(np.float64) @ (np.abs(B1) + np.abs(B2)).astype(np.float64)
    bound = 3 * K * 2.0 ** -53 * absum
    assert np.all(np.abs(v12[0] - v1[0] - v2[0]) <= bound)
    # a dropped or doubled term would break it by far more than the bound
    assert np.abs(v12[0] - v1[0]).max() > 1e3 * bound.max()


# ----------------------------------------------------------------- integer extremes
@pytest.mark.parametrize("K", [1, 4096, 131071])
def test_int8_extremes(K):
    """All (-128)*(-128) gives 16384*K; 127*(-128) gives -16256*K.  At
    K = 131071 the first is 2147467264, still below 2^31 - 1."""
    M, N = 2, 3
    A = np.full((M, K), -128, dtype=np.int8)
    B = np.full((K, N), -128, dtype=np.int8)
    out, val = oracle.gemm(A, B, None, M=M, N=N, K=K, a_dtype="i8", c_dtype="i32")
    assert np.all(out == 16384 * K) and np.all(val == 16384 * K)
    A[:] = 127
    out, _ = oracle.gemm(A, B, None, M=M, N=N, K=K, a_dtype="i8", c_dtype="i32")
    assert np.all(out == -16256 * K)
    if K == 131071:
        assert 16384 * K <= 2 ** 31 - 1 < 16384 * (K + 1)


# ----------------------------------------------------------------- worked example
def test_foundry_quickstart_2x2():
    with open(os.path.join(GOLDEN, "foundry_quickstart_2x2.json")) as f:
        g = json.load(f)
    A = np.array(g["A"], dtype=np.float32)
    B = np.array(g["B"], dtype=np.float32)
    C = np.array(g["C"], dtype=np.float32)
    out, _ = oracle.gemm(A, B, C, M=g["M"], N=g["N"], K=g["K"], a_dtype="f32",
                         c_dtype="f32", alpha=g["alpha"], beta=g["beta"])
    exact = exact_gemm(A, B, C, 2, 2, 2, False, False, g["alpha"], g["beta"], 2, 2, 2)
    assert out.tolist() == [float(exact[i][j]) for i in range(2) for j in range(2)]
    assert out.tolist() == [19.0, 22.0, 43.0, 50.0]


# ----------------------------------------------------------------- batched and points
@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_batched_equals_per_problem_and_points(dtype):
    rng = np.random.default_rng(14)
    b, M, N, K = 3, 5, 7, 20
    A = draw(rng, dtype, (b, K, M))      # TN
    B = draw(rng, dtype, (b, K, N))
    c_dtype = "i32" if dtype == "i8" else "f32"
    kw = dict(M=M, N=N, K=K, a_dtype=dtype, c_dtype=c_dtype, transpose_a=True)
    out, val = oracle.gemm(A, B, None, batch=b, stride_a=K * M, stride_b=K * N,
                           stride_c=M * N, **kw)
    out = out.reshape(b, M, N)
    for z in range(b):
        o1, v1 = oracle.gemm(A[z], B[z], None, **kw)
        assert np.array_equal(o1.reshape(M, N), out[z])
        assert np.array_equal(v1[0], val[z])
    pts = [(z, i, j) for z in range(b) for i in range(M) for j in range(N)]
    r, v = oracle.gemm_points(A, B, None, pts, stride_a=K * M, stride_b=K * N,
                              stride_c=M * N, **kw)
    assert np.array_equal(r.reshape(b, M, N), out)
    assert np.array_equal(v.reshape(b, M, N), val)


def test_rejects_bad_arguments():
    A = np.zeros(4, dtype=np.int8)
    with pytest.raises(ValueError):
        oracle.gemm(A, A, None, M=2, N=2, K=2, a_dtype="i8", c_dtype="i32", alpha=2.0)
    with pytest.raises(ValueError):
        oracle.gemm(A, A, None, M=0, N=2, K=2, a_dtype="i8", c_dtype="i32")
    with pytest.raises(ValueError):
        oracle.gemm(A, A, None, M=2, N=2, K=2, a_dtype="i8", c_dtype="f16")


def test_rel_frobenius():
    assert oracle.rel_frobenius(np.zeros(3), np.zeros(3)) == 0.0
    assert oracle.rel_frobenius(np.ones(3), np.zeros(3)) == math.inf
    assert oracle.rel_frobenius(np.array([3.0, 4.0]), np.array([3.0, 0.0])) == pytest.approx(4 / 3)


# ----------------------------------------------------------------- fused epilogue
def encode_lib(x, dtype):
    """Encode exactly representable values with a library (not the oracle)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def gelu_erf(x):
    """GELU by its definition x * Phi(x), with the error function."""
    return np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in np.ravel(x)])


def test_gelu_tanh_is_within_the_approximation_bound_of_erf_gelu():
    """The tanh form stays within 5e-4 of x*Phi(x) everywhere (its known
    worst case is about 4.7e-4, near |x| = 2.7); a dropped cubic term, a
    wrong constant or a sign error misses by far more."""
    x = np.linspace(-8.0, 8.0, 40001)
    g = oracle.activation(x, "gelu_tanh")
    d = np.abs(g - gelu_erf(x))
    assert d.max() < 5e-4
    assert d.max() > 1e-4          # it is the approximation, not erf itself
    no_cubic = 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * x))
    assert np.abs(no_cubic - gelu_erf(x)).max() > 1e-2


def test_gelu_tanh_identities():
    """gelu(x) - gelu(-x) = x for the tanh form (tanh is odd); gelu(0) = 0;
    gelu(x) = x once tanh has saturated to 1 in fp64; gelu(-x) -> 0."""
    x = np.linspace(-6.0, 6.0, 1201)
    g, gm = oracle.activation(x, "gelu_tanh"), oracle.activation(-x, "gelu_tanh")
    assert np.allclose(g - gm, x, rtol=0, atol=1e-12)
    assert oracle.activation(np.array([0.0]), "gelu_tanh")[0] == 0.0
    big = np.array([20.0, 50.0, 1000.0])
    assert np.array_equal(oracle.activation(big, "gelu_tanh"), big)
    assert np.all(np.abs(oracle.activation(-big, "gelu_tanh")) < 1e-30)


def test_relu_and_none():
    x = np.array([-3.5, -0.0, 0.0, 1e-30, 2.25])
    assert oracle.activation(x, "relu").tolist() == [0.0, 0.0, 0.0, 1e-30, 2.25]
    assert oracle.activation(x, "none").tolist() == x.tolist()
    with pytest.raises(ValueError):
        oracle.activation(x, "tanh")


@pytest.mark.parametrize("dtype", FLOAT_TYPES)
def test_epilogue_closed_form_bias_per_column(dtype):
    """A = B = ones gives S = K in every entry; with alpha, beta, C_in = c0
    and bias[j] = j - 5 the pre-activation value is exactly
    alpha*K + beta*c0 + j - 5, the same in every row (bias is per column)."""
    M, N, K = 7, 11, 6
    alpha, beta, c0 = 0.5, 2.0, 0.25
    A = encode_lib(np.ones((M, K)), dtype)
    B = encode_lib(np.ones((K, N)), dtype)
    C = encode_lib(np.full((M, N), c0), dtype)
    bias = encode_lib(np.arange(N) - 5.0, dtype)
    kw = dict(M=M, N=N, K=K, a_dtype=dtype, c_dtype=dtype, alpha=alpha, beta=beta)
    pre = alpha * K + beta * c0 + (np.arange(N) - 5.0)          # exact, per column
    for act, want in (("none", pre), ("relu", np.maximum(pre, 0.0))):
        out, val = oracle.gemm_epilogue(A, B, C, bias=bias, act=act, **kw)
        assert np.array_equal(val[0], np.broadcast_to(want, (M, N)))
        assert np.array_equal(lib_decode(out, dtype).reshape(M, N), np.broadcast_to(want, (M, N)))
    out, val = oracle.gemm_epilogue(A, B, C, bias=bias, act="gelu_tanh", **kw)
    assert np.allclose(val[0], np.broadcast_to(gelu_erf(pre), (M, N)), rtol=0, atol=5e-4)
    # no bias and no activation is the plain product, bit for bit
    o1, v1 = oracle.gemm_epilogue(A, B, C, **kw)
    o2, v2 = oracle.gemm(A, B, C, **kw)
    assert np.array_equal(o1, o2) and np.array_equal(v1, v2)


def test_epilogue_batched_bias_stride_and_unread_c():
    """Problem z adds its own bias vector (bias_stride = N); with stride 0
    every problem adds the first.  beta = 0 leaves a NaN C_in unread."""
    rng = np.random.default_rng(21)
    b, M, N, K = 3, 4, 5, 8
    A = draw(rng, "bf16", (b, M, K))
    B = draw(rng, "bf16", (b, K, N))
    bias = encode_lib(np.arange(b * N, dtype=np.float64) - 7.0, "f32")
    kw = dict(M=M, N=N, K=K, a_dtype="bf16", c_dtype="f32", batch=b,
              stride_a=M * K, stride_b=K * N, stride_c=M * N)
    Cnan = np.full(b * M * N, np.nan, dtype=np.float32)
    _, v0 = oracle.gemm(A, B, None, **kw)
    out, v = oracle.gemm_epilogue(A, B, Cnan, bias=bias, bias_stride=N, act="relu", **kw)
    want = np.maximum(v0 + (np.arange(b * N) - 7.0).reshape(b, 1, N), 0.0)
    assert np.array_equal(v, want)
    assert not np.isnan(out).any()
    _, v_shared = oracle.gemm_epilogue(A, B, None, bias=bias, bias_stride=0, **kw)
    assert np.array_equal(v_shared, v0 + (np.arange(N) - 7.0)[None, None, :])


def test_epilogue_rejects_int8_and_unknown_activation():
    A = np.zeros(4, dtype=np.int8)
    with pytest.raises(ValueError):      # int8 without a dequant scale
        oracle.gemm_epilogue(A, A, None, M=2, N=2, K=2, a_dtype="i8", c_dtype="i32", act="relu")
    with pytest.raises(ValueError):      # dequantized results are float
        oracle.gemm_epilogue(A, A, None, M=2, N=2, K=2, a_dtype="i8", c_dtype="i32",
                             col_scale=np.ones(2, dtype=np.float32))
    B = np.zeros(4, dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.gemm_epilogue(B, B, None, M=2, N=2, K=2, a_dtype="f32", c_dtype="f32", act="gelu")


def test_epilogue_points_equal_full():
    rng = np.random.default_rng(22)
    b, M, N, K = 2, 6, 9, 33
    A = draw(rng, "f16", (b, M, K))
    B = draw(rng, "f16", (b, N, K))
    C = draw(rng, "f16", (b, M, N))
    bias = draw(rng, "f16", (b, N))
    kw = dict(M=M, N=N, K=K, a_dtype="f16", c_dtype="f16", transpose_b=True, alpha=0.5,
              beta=1.0, batch=b, stride_a=M * K, stride_b=N * K, stride_c=M * N)
    out, val = oracle.gemm_epilogue(A, B, C, bias=bias, bias_stride=N, act="gelu_tanh", **kw)
    pts = [(z, i, j) for z in range(b) for i in range(M) for j in range(N)]
    kw.pop("batch")
    r, v = oracle.gemm_epilogue_points(A, B, C, pts, bias=bias, bias_stride=N, act="gelu_tanh", **kw)
    assert np.array_equal(v.reshape(b, M, N), val)
    assert np.array_equal(r.reshape(b, M, N), out.reshape(b, M, N))


# ----------------------------------------------------------------- int8 dequant
@pytest.mark.parametrize("c_dtype", FLOAT_TYPES)
def test_i8_dequant_against_exact_integers(c_dtype):
    """C[i][j] = round_c(s[j] * S[i][j]) with S the exact integer sum, checked
    against Python integers and fractions on a tiny ragged problem (all four
    layouts), per-column scales that differ in every column."""
    rng = np.random.default_rng(31)
    M, N, K = 5, 7, 19
    sc = np.array([0.5, 0.03125, 3.0, -1.25, 1e-3, 7.0, 2.0 ** -20], dtype=np.float32)
    for ta in (False, True):
        for tb in (False, True):
            A = rng.integers(-128, 128, size=(K, M) if ta else (M, K), dtype=np.int8)
            B = rng.integers(-128, 128, size=(N, K) if tb else (K, N), dtype=np.int8)
            out, val = oracle.gemm_epilogue(A, B, None, col_scale=sc, M=M, N=N, K=K,
                                            a_dtype="i8", c_dtype=c_dtype,
                                            transpose_a=ta, transpose_b=tb)
            got = lib_decode(out, c_dtype).reshape(M, N)
            table = finite_values(c_dtype) if c_dtype != "f32" else None
            for i in range(M):
                for j in range(N):
                    s = 0
                    for k in range(K):
                        a = int(A[k, i] if ta else A[i, k])
                        b = int(B[j, k] if tb else B[k, j])
                        s += a * b
                    exact = Fraction(s) * Fraction(float(sc[j]))
                    # |S| < 2^19 here, so s*S has at most 43 significand bits: exact in fp64
                    assert val[0, i, j] == float(exact)
                    if c_dtype == "f32":
                        assert got[i, j] == float(np.float32(float(exact)))
                    else:
                        assert got[i, j] == nearest_by_search(float(exact), c_dtype, table)


def test_i8_dequant_extremes_and_composition():
    """All (-128)*(-128): S = 16384 K exactly; scales 2^-e keep the result
    exact in fp32; with beta, a bias and ReLU the closed form is
    relu(alpha s[j] 16384 K + beta c0 + bias[j])."""
    M, N, K = 3, 4, 131071
    A = np.full((M, K), -128, dtype=np.int8)
    B = np.full((K, N), -128, dtype=np.int8)
    sc = np.array([1.0, 2.0 ** -10, 2.0 ** -20, -2.0 ** -5], dtype=np.float32)
    out, val = oracle.gemm_epilogue(A, B, None, col_scale=sc, M=M, N=N, K=K, a_dtype="i8",
                                    c_dtype="f32")
    want = 16384.0 * K * sc.astype(np.float64)
    assert np.array_equal(val[0], np.broadcast_to(want, (M, N)))
    assert np.array_equal(out.reshape(M, N), np.broadcast_to(want.astype(np.float32), (M, N)))
    C = np.full(M * N, 8.0, dtype=np.float32)
    bias = np.array([-1e9, 0.5, -3.0, 100.0], dtype=np.float32)
    _, v = oracle.gemm_epilogue(A, B, C, col_scale=sc, bias=bias, act="relu", alpha=0.5,
                                beta=2.0, M=M, N=N, K=K, a_dtype="i8", c_dtype="f32")
    pre = 0.5 * want + 16.0 + bias.astype(np.float64)
    assert np.array_equal(v[0], np.broadcast_to(np.maximum(pre, 0.0), (M, N)))


def test_float_gemm_with_column_scale():
    """A per-column scale on a float GEMM multiplies column j of alpha*A@B
    by s[j] (checked on A = B = ones: S = K)."""
    M, N, K = 4, 5, 12
    A = encode_lib(np.ones((M, K)), "bf16")
    B = encode_lib(np.ones((K, N)), "bf16")
    sc = np.array([1.0, 0.5, -2.0, 0.0, 4.0], dtype=np.float32)
    _, v = oracle.gemm_epilogue(A, B, None, col_scale=sc, alpha=0.25, M=M, N=N, K=K,
                                a_dtype="bf16", c_dtype="f32")
    assert np.array_equal(v[0], np.broadcast_to(0.25 * K * sc.astype(np.float64), (M, N)))


def test_i8_dequant_points_equal_full():
    rng = np.random.default_rng(33)
    b, M, N, K = 2, 5, 6, 40
    A = rng.integers(-128, 128, size=(b, M, K), dtype=np.int8)
    B = rng.integers(-128, 128, size=(b, K, N), dtype=np.int8)
    sc = rng.normal(0, 0.01, size=b * N).astype(np.float32)
    bias = draw(rng, "bf16", (b, N))
    kw = dict(M=M, N=N, K=K, a_dtype="i8", c_dtype="bf16", stride_a=M * K, stride_b=K * N,
              stride_c=M * N)
    out, val = oracle.gemm_epilogue(A, B, None, col_scale=sc, scale_stride=N, bias=bias,
                                    bias_stride=N, act="gelu_tanh", batch=b, **kw)
    pts = [(z, i, j) for z in range(b) for i in range(M) for j in range(N)]
    r, v = oracle.gemm_epilogue_points(A, B, None, pts, col_scale=sc, scale_stride=N, bias=bias,
                                       bias_stride=N, act="gelu_tanh", **kw)
    assert np.array_equal(v.reshape(b, M, N), val)
    assert np.array_equal(r.reshape(b, M, N), out.reshape(b, M, N))


# ----------------------------------------------------------------- magnitude sums
# T(i, j) = sum over k of |opA(i,k) * opB(k,j)|: the magnitude that scales the
# a-priori error bound of a length-K dot product (tessl "Architecture",
# "Reductions and Numerical Safety", bounds its sums by a multiple of
# eps * n * the term magnitudes); the parity tests use it for their
# elementwise gate.
@pytest.mark.parametrize("dtype", FLOAT_TYPES)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_magnitude_sum_against_exact_rationals(dtype, ta, tb):
    """Mixed-sign inputs, padded leading dims: T within the fp64 bound of the
    exact sum of |products| (Python fractions), and never below |S|."""
    rng = np.random.default_rng(hash(("mag", dtype, ta, tb)) % 2**32)
    M, N, K, pad = 7, 5, 8, 3
    A, B, lda, ldb, ldc = _tiny_case(rng, dtype, ta, tb, M, N, K, pad, "normal")
    Ad, Bd = lib_decode(A, dtype), lib_decode(B, dtype)
    _, value, T = oracle.gemm(A, B, None, M=M, N=N, K=K, a_dtype=dtype, c_dtype=dtype,
                              transpose_a=ta, transpose_b=tb, lda=lda, ldb=ldb, ldc=ldc,
                              want_abs=True)
    strictly = 0
    for i in range(M):
        for j in range(N):
            ex = Fraction(0)
            for k in range(K):
                a = Ad[k * lda + i] if ta else Ad[i * lda + k]
                b = Bd[j * ldb + k] if tb else Bd[k * ldb + j]
                ex += abs(Fraction(float(a)) * Fraction(float(b)))
            assert abs(Fraction(T[0, i, j]) - ex) <= Fraction(K) * Fraction(2) ** -53 * ex
            assert T[0, i, j] >= abs(value[0, i, j])
            strictly += T[0, i, j] > abs(value[0, i, j])
    assert strictly > 0      # mixed signs: some sums cancel


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_magnitude_sum_int8_exact(ta, tb):
    rng = np.random.default_rng(78)
    M, N, K, pad = 6, 9, 13, 2
    A, B, lda, ldb, ldc = _tiny_case(rng, "i8", ta, tb, M, N, K, pad, "")
    _, _, T = oracle.gemm(A, B, None, M=M, N=N, K=K, a_dtype="i8", c_dtype="i32",
                          transpose_a=ta, transpose_b=tb, lda=lda, ldb=ldb, ldc=ldc,
                          want_abs=True)
    for i in range(M):
        for j in range(N):
            s = 0
            for k in range(K):
                a = int(A[k * lda + i] if ta else A[i * lda + k])
                b = int(B[j * ldb + k] if tb else B[k * ldb + j])
                s += abs(a * b)
            assert T[0, i, j] == s


@pytest.mark.parametrize("dtype", FLOAT_TYPES + ("i8",))
def test_magnitude_sum_is_the_sum_for_one_signed_terms(dtype):
    """With every product non-negative T is the plain sum (same terms, same
    order: bit-equal); negating A negates the sum and leaves T; negating a
    row of A changes only that row's sums."""
    rng = np.random.default_rng(12)
    M, N, K = 9, 10, 300
    c_dtype = "i32" if dtype == "i8" else dtype
    if dtype == "i8":
        A = np.abs(rng.integers(-127, 128, size=(M, K))).astype(np.int8)
        B = np.abs(rng.integers(-127, 128, size=(K, N))).astype(np.int8)
        negA = (-A.astype(np.int16)).astype(np.int8)
    else:
        A = encode_lib(np.abs(rng.normal(0, 1, size=(M, K))), dtype)
        B = encode_lib(np.abs(rng.normal(0, 1, size=(K, N))), dtype)
        negA = encode_lib(-lib_decode(A, dtype), dtype)
    kw = dict(M=M, N=N, K=K, a_dtype=dtype, c_dtype=c_dtype, want_abs=True)
    _, v, T = oracle.gemm(A, B, None, **kw)
    assert np.array_equal(T, v)
    _, vn, Tn = oracle.gemm(negA, B, None, **kw)
    assert np.array_equal(vn, -v)
    assert np.array_equal(Tn, T)
    mixed = A.copy()
    mixed[3] = negA[3]
    _, vm, Tm = oracle.gemm(mixed, B, None, **kw)
    assert np.array_equal(Tm, T)
    assert np.array_equal(vm[0, 3], -v[0, 3])
    assert np.array_equal(np.delete(vm[0], 3, axis=0), np.delete(v[0], 3, axis=0))


def test_magnitude_sum_points_equal_full():
    rng = np.random.default_rng(23)
    b, M, N, K = 2, 6, 7, 45
    for dtype in ("bf16", "i8"):
        A = draw(rng, dtype, (b, K, M))
        B = draw(rng, dtype, (b, N, K))
        c_dtype = "i32" if dtype == "i8" else "f32"
        kw = dict(M=M, N=N, K=K, a_dtype=dtype, c_dtype=c_dtype, transpose_a=True,
                  transpose_b=True, stride_a=M * K, stride_b=N * K, stride_c=M * N)
        _, _, T = oracle.gemm(A, B, None, batch=b, want_abs=True, **kw)
        pts = [(z, i, j) for z in range(b) for i in range(M) for j in range(N)]
        _, _, Tp = oracle.gemm_points(A, B, None, pts, want_abs=True, **kw)
        assert np.array_equal(Tp.reshape(b, M, N), T)
        _, _, Te = oracle.gemm_epilogue(A, B, None, act="relu", batch=b, want_abs=True,
                                        col_scale=np.ones(N, np.float32)
                                        if dtype == "i8" else None,
                                        **dict(kw, c_dtype="f32"))
        assert np.array_equal(Te, T)
