"""The parity gates on the CPU (no GPU): the elementwise bound accepts a
result accumulated in fp32 in another order, and rejects a single wrong
output that the relative Frobenius norm alone lets through."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, compare, oracle_epilogue, oracle_full, ulp


def fp32_gemm(p, A, B, C):
    """An fp32-accumulating GEMM in another summation order (torch's CPU
    matmul in float32, then alpha, beta in fp32, then the output rounding):
    what a correct GPU kernel may return."""
    a = torch.from_numpy(oracle.decode(A, p.a_dtype).astype(np.float32))
    b = torch.from_numpy(oracle.decode(B, p.a_dtype).astype(np.float32))
    if p.transpose_a:
        a = a.T
    if p.transpose_b:
        b = b.T
    acc = (a @ b).numpy()
    v = np.float32(p.alpha) * acc
    if p.beta != 0.0:
        v = (v.astype(np.float64) + p.beta * oracle.decode(C, p.c_dtype)).astype(np.float32)
    return oracle.encode(v.astype(np.float64), p.c_dtype).reshape(C.shape)


CASES = [("bf16", "bf16", False, False, 1.0, 0.0), ("f16", "f16", True, False, 0.5, 1.0),
         ("f16", "f32", False, True, -2.0, 0.25), ("f32", "f32", False, False, 1.0, 0.0)]


@pytest.mark.parametrize("a,c,ta,tb,alpha,beta", CASES)
def test_fp32_result_in_another_order_passes(a, c, ta, tb, alpha, beta):
    p = workloads.Problem("g", 192, 160, 700, a, c, transpose_a=ta, transpose_b=tb,
                          alpha=alpha, beta=beta, c_dist="normal" if beta else "zeros",
                          seed=5)
    A, B, C = workloads.make_inputs(p)
    ref = oracle_full(p, A, B, C)
    compare(p, ref.out, ref, label="oracle itself")
    compare(p, fp32_gemm(p, A, B, C), ref, label="fp32 order")


@pytest.mark.parametrize("a,c", [("bf16", "bf16"), ("f16", "f32")])
def test_one_wrong_output_fails_the_bound_not_the_norm(a, c):
    """1024 x 1024 outputs; one of them off by a few bounds: the norm stays
    under its tolerance, the elementwise gate names the output."""
    p = workloads.Problem("g", 1024, 1024, 64, a, c, seed=6)
    A, B, C = workloads.make_inputs(p)
    ref = oracle_full(p, A, B, C)
    got = ref.out.copy()
    z, i, j = 0, 517, 33
    v = ref.value[z, i, j]
    wrong = v + 8 * (ulp(v, c) + 1e-3 * abs(v))
    got[i, j] = oracle.encode(np.array([wrong]), c)[0]
    gv = oracle.decode(got, c)
    rv = oracle.decode(ref.out, c)
    assert oracle.rel_frobenius(gv, rv) <= TOL[a]
    with pytest.raises(AssertionError, match=r"1 outputs outside the elementwise bound; "
                                             r"worst at \(0, 517, 33\)"):
        compare(p, got, ref, label="planted")


def test_one_ulp_off_bf16_output_fails():
    """bf16 output, short K: a result one ulp away from the correctly
    rounded value, where the exact value is not near a midpoint, is wrong."""
    p = workloads.Problem("g", 64, 64, 32, "bf16", "bf16", dist="small_int", scale=4.0,
                          seed=7)
    A, B, C = workloads.make_inputs(p)
    ref = oracle_full(p, A, B, C)
    got = ref.out.copy()
    got[3, 5] = np.uint16(int(got[3, 5]) ^ 1)      # flip the last significand bit
    with pytest.raises(AssertionError, match="elementwise bound"):
        compare(p, got, ref, label="ulp")


def test_fused_gelu_result_in_another_order_passes():
    p = workloads.Problem("g", 128, 96, 500, "bf16", "bf16", alpha=0.5, beta=1.0,
                          c_dist="normal", seed=8)
    A, B, C = workloads.make_inputs(p)
    bias = workloads.make_bias(p)
    ref = oracle_epilogue(p, A, B, C, bias, "gelu_tanh")
    a = torch.from_numpy(oracle.decode(A, "bf16").astype(np.float32))
    b = torch.from_numpy(oracle.decode(B, "bf16").astype(np.float32))
    y = (np.float32(0.5) * (a @ b).numpy()).astype(np.float64) + oracle.decode(C, "bf16") \
        + oracle.decode(bias, "bf16")[0][None, :]
    y = y.astype(np.float32).astype(np.float64)
    out = 0.5 * y * (1.0 + np.tanh(np.sqrt(2 / np.pi) * (y + 0.044715 * y ** 3)))
    got = oracle.encode(out.astype(np.float32).astype(np.float64), "bf16")
    compare(p, got, ref, label="fused fp32")
    v = ref.value[0, 7, 9]
    got[7, 9] = oracle.encode(np.array([v + 3 * ulp(v, "bf16")]), "bf16")[0]
    with pytest.raises(AssertionError, match="elementwise bound"):
        compare(p, got, ref, label="fused planted")
