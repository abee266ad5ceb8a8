"""The allocation-free entry point (tc_gemm_batched_async_noalloc) on the GPU,
through the C ABI: its results equal those of tc_gemm_batched_async on the
same inputs and match the oracle, on two calls in a row (the second smaller)
for plans that use scratch memory (split-K partials, a packed operand), and
a plan that needs more scratch than the static array holds is refused with
nothing launched."""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_util import compare, from_dev, oracle_full, say, to_dev

pytestmark = pytest.mark.gpu

VP = ctypes.c_void_p


def run_both(p):
    """Run p through tc_gemm_batched_async and through the allocation-free
    call (same stream, same inputs, C restored between); returns both C
    buffers as stored values, the inputs, and the kernel chain."""
    import torch
    import dense_gemm_tiled_amd as tg
    lib = tg.load_library()
    A, B, C = workloads.make_inputs(p)
    a, b = to_dev(A, p.a_dtype), to_dev(B, p.a_dtype)
    c1, c2 = to_dev(C, p.c_dtype), to_dev(C, p.c_dtype)
    av = a[..., :p.M if p.transpose_a else p.K]
    bv = b[..., :p.K if p.transpose_b else p.N]
    d = tg.make_desc(av, bv, c1[..., :p.N], alpha=p.alpha, beta=p.beta,
                     transpose_a=p.transpose_a, transpose_b=p.transpose_b)
    ctx, s = tg._torch_stream(0)
    assert tg.plan(d)["workspace_bytes"] > 0 or p.name == "plain", p.name
    say("GPU case: noalloc", p.name, p.M, p.N, p.K, p.batch, p.a_dtype, p.c_dtype, p.layout)
    st = lib.tc_gemm_batched_async(ctx, ctypes.byref(d), VP(av.data_ptr()), VP(bv.data_ptr()),
                                   VP(c1.data_ptr()), s)
    assert st == 0, lib.tc_last_error(ctx)
    chain = tg.last_kernel()
    st = lib.tc_gemm_batched_async_noalloc(ctx, ctypes.byref(d), VP(av.data_ptr()),
                                           VP(bv.data_ptr()), VP(c2.data_ptr()), s)
    assert st == 0, lib.tc_last_error(ctx)
    assert tg.last_kernel() == chain, (tg.last_kernel(), chain)
    torch.cuda.synchronize()
    return from_dev(c1, p.c_dtype), from_dev(c2, p.c_dtype), (A, B, C), chain


CASES = [
    # split-K partials: the batched weight-gradient shape, then a smaller one
    (workloads.get("bf16_tn_splitk_b8"),
     workloads.Problem("splitk_small", 128, 256, 4096, "bf16", "f32", transpose_a=True,
                       dist="uniform", seed=51)),
    # a packed A (rows of 1000 bytes) on the 256x256 tile, beta = 1, then a
    # smaller one (rows of 600 bytes) on the 128x128 tile
    (workloads.Problem("packed", 4096, 3072, 500, "f16", "f16", alpha=0.5, beta=1.0,
                       c_dist="normal", seed=52),
     workloads.Problem("packed_small", 2048, 1536, 300, "f16", "f16", alpha=0.5, beta=1.0,
                       c_dist="normal", seed=53)),
    # int8: split-K into int32, then a packed B (rows of 1602 bytes)
    (workloads.Problem("i8_splitk", 256, 128, 32768, "i8", "i32", dist="int8", seed=54),
     workloads.Problem("i8_packed", 2048, 1602, 512, "i8", "i32", ldb=1603, dist="int8",
                       seed=55)),
]


@pytest.mark.parametrize("big,small", CASES, ids=["splitk", "packed", "int8"])
def test_noalloc_matches_the_allocating_call_twice(big, small):
    for p in (big, small):
        got_alloc, got_static, (A, B, C), chain = run_both(p)
        assert np.array_equal(got_static.view(np.uint8), got_alloc.view(np.uint8)), p.name
        compare(p, got_static, oracle_full(p, A, B, C), C_in=C, label="noalloc " + p.name)
        say("noalloc", p.name, chain)


def test_noalloc_without_scratch_and_refusal():
    """A plan with no scratch runs as well; a plan needing more than the
    static array is refused before anything is enqueued."""
    import torch
    import dense_gemm_tiled_amd as tg
    lib = tg.load_library()
    p = workloads.Problem("plain", 512, 512, 512, "bf16", "bf16", seed=56)
    got_alloc, got_static, (A, B, C), chain = run_both(p)
    assert "pack" not in chain and "splitk" not in chain, chain
    assert np.array_equal(got_static, got_alloc)
    # rows of K = 8201 bf16 are not whole 16-byte chunks: A is packed into
    # 4096 rows of 16416 bytes, 67 MB > 32 MiB
    a = torch.zeros(4096, 8201, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(8201, 4096, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(4096, 4096, dtype=torch.bfloat16, device="cuda")
    d = tg.make_desc(a, b, c)
    assert tg.plan(d)["workspace_bytes"] > 32 << 20
    ctx, s = tg._torch_stream(0)
    n0 = tg.dispatch_count()
    st = lib.tc_gemm_batched_async_noalloc(ctx, ctypes.byref(d), VP(a.data_ptr()),
                                           VP(b.data_ptr()), VP(c.data_ptr()), s)
    assert st == 5, st
    assert b"scratch" in lib.tc_last_error(ctx)
    assert tg.dispatch_count() == n0
    assert lib.tc_gemm_batched_async_noalloc(ctx, ctypes.byref(d), VP(a.data_ptr()),
                                             VP(b.data_ptr()), VP(c.data_ptr()), None) == 1
