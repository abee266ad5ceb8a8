"""The C ABI's single-problem and stream calls on the GPU, through ctypes:
tc_gemm (synchronous), tc_stream_create -> tc_gemm_async -> tc_stream_sync ->
tc_stream_destroy (tensorcore "GEMM", "Async, batched, and streams"), and
split-K on an owned stream whose workspace must grow between two calls.
Every result is compared with the oracle like the parity tests."""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_util import compare, from_dev, oracle_epilogue, oracle_full, say, to_dev

pytestmark = pytest.mark.gpu

VP = ctypes.c_void_p


def lib_ctx():
    import dense_gemm_tiled_amd as tg
    return tg, tg.load_library(), tg._context(0)


def device_case(p):
    """Seeded inputs on the device (contiguous, so the logical views are the
    whole tensors) and the descriptor of the call."""
    import dense_gemm_tiled_amd as tg
    A, B, C = workloads.make_inputs(p)
    a, b, c = to_dev(A, p.a_dtype), to_dev(B, p.a_dtype), to_dev(C, p.c_dtype)
    d = tg.make_desc(a, b, c, alpha=p.alpha, beta=p.beta, transpose_a=p.transpose_a,
                     transpose_b=p.transpose_b)
    return (A, B, C), (a, b, c), d


def check_status(st, lib, ctx):
    assert st == 0, (st, lib.tc_last_error(ctx))


@pytest.mark.parametrize("a,c,ta,tb", [("bf16", "bf16", False, False), ("i8", "i32", False, True),
                                       ("f16", "f32", True, False), ("f32", "f32", False, False)])
def test_tc_gemm_sync(a, c, ta, tb):
    """tc_gemm returns with C complete (its own stream, synchronized)."""
    import torch
    tg, lib, ctx = lib_ctx()
    float_ok = a != "i8"
    p = workloads.Problem("sync", 300, 520, 264, a, c, transpose_a=ta, transpose_b=tb,
                          alpha=0.5 if float_ok else 1.0, beta=1.0 if float_ok else 0.0,
                          dist="int8" if a == "i8" else "normal",
                          c_dist="normal" if float_ok else "nan", seed=41)
    (A, B, C), (da, db, dc), d = device_case(p)
    torch.cuda.synchronize()
    say("GPU case: tc_gemm", a, c, p.layout)
    st = lib.tc_gemm(ctx, ctypes.byref(d.base), VP(da.data_ptr()), VP(db.data_ptr()),
                     VP(dc.data_ptr()))
    check_status(st, lib, ctx)
    got = from_dev(dc, c)            # no synchronization of our own: the call did it
    compare(p, got, oracle_full(p, A, B, C), C_in=C, label="tc_gemm")


def test_owned_stream_two_async_calls():
    """The pages' stream sequence: create a stream, enqueue two GEMMs into
    different C, sync, destroy; both results match the oracle."""
    import torch
    tg, lib, ctx = lib_ctx()
    p1 = workloads.Problem("s1", 512, 768, 1024, "bf16", "bf16", seed=42)
    p2 = workloads.Problem("s2", 640, 384, 200, "f16", "f16", transpose_b=True, alpha=0.5,
                           beta=1.0, c_dist="normal", seed=43)
    h1, d1, desc1 = device_case(p1)
    h2, d2, desc2 = device_case(p2)
    torch.cuda.synchronize()          # inputs written by torch's stream
    s = VP()
    check_status(lib.tc_stream_create(ctx, ctypes.byref(s)), lib, ctx)
    try:
        say("GPU case: owned stream, two async GEMMs")
        for (da, db, dc), desc in ((d1, desc1), (d2, desc2)):
            st = lib.tc_gemm_async(ctx, ctypes.byref(desc.base), VP(da.data_ptr()),
                                   VP(db.data_ptr()), VP(dc.data_ptr()), s)
            check_status(st, lib, ctx)
        check_status(lib.tc_stream_sync(s), lib, ctx)
    finally:
        lib.tc_stream_destroy(s)
    for p, (A, B, C), (_, _, dc) in ((p1, h1, d1), (p2, h2, d2)):
        compare(p, from_dev(dc, p.c_dtype), oracle_full(p, A, B, C), C_in=C, label=p.name)


def test_owned_stream_split_k_workspace_grows():
    """Split-K on an owned stream twice, the second problem larger: the
    stream's workspace is freed and allocated again between the calls (after
    the first call's work is done) and both results are right.  Then a
    smaller call reuses the larger workspace."""
    import torch
    tg, lib, ctx = lib_ctx()
    probs = [workloads.Problem("w1", 128, 384, 4096, "bf16", "f32", transpose_a=True,
                               dist="uniform", seed=44),
             workloads.Problem("w2", 128, 384, 16384, "bf16", "f32", transpose_a=True,
                               batch=4, dist="uniform", seed=45),
             workloads.Problem("w3", 64, 256, 8192, "f16", "f16", dist="uniform", seed=46)]
    cases = [device_case(p) for p in probs]
    torch.cuda.synchronize()
    s = VP()
    check_status(lib.tc_stream_create(ctx, ctypes.byref(s)), lib, ctx)
    try:
        for p, (h, (da, db, dc), desc) in zip(probs, cases):
            info = tg.plan(desc)
            assert info["splits"] > 1 and info["workspace_bytes"] > 0, info
            say("GPU case: owned-stream split-K", p.name, info["splits"], info["workspace_bytes"])
            if p.batch == 1:
                st = lib.tc_gemm_async(ctx, ctypes.byref(desc.base), VP(da.data_ptr()),
                                       VP(db.data_ptr()), VP(dc.data_ptr()), s)
            else:
                st = lib.tc_gemm_batched_async(ctx, ctypes.byref(desc), VP(da.data_ptr()),
                                               VP(db.data_ptr()), VP(dc.data_ptr()), s)
            check_status(st, lib, ctx)
            assert tg.last_kernel().endswith("+splitk_reduce"), tg.last_kernel()
        check_status(lib.tc_stream_sync(s), lib, ctx)
    finally:
        lib.tc_stream_destroy(s)
    sizes = [tg.plan(c[2])["workspace_bytes"] for c in cases]
    assert sizes[1] > sizes[0] and sizes[2] < sizes[1], sizes
    for p, (h, (_, _, dc), _) in zip(probs, cases):
        A, B, C = h
        compare(p, from_dev(dc, p.c_dtype), oracle_full(p, A, B, C), C_in=C, label=p.name)


def test_stream_calls_refuse_null():
    """NULL stream or descriptor: an error status, nothing launched."""
    tg, lib, ctx = lib_ctx()
    n0 = tg.dispatch_count()
    assert lib.tc_stream_sync(None) == 1
    assert lib.tc_stream_create(None, ctypes.byref(VP())) == 1
    assert lib.tc_gemm_async(ctx, None, VP(1), VP(1), VP(1), VP(1)) == 1
    lib.tc_stream_destroy(None)
    assert tg.dispatch_count() == n0


def _rows_of(t, rows, width):
    """Host copies of the first `width` elements of the given rows of a 2-D
    device tensor with a large leading dim."""
    return [t[r, :width].cpu() for r in rows]


def test_c_past_2gib_alpha_zero_and_split_k():
    """C spanning more than 2 GiB: the alpha = 0 kernel (beta * C, then bias
    and ReLU) and the split-K reduction address each row of C on its own, so
    rows past 2 GiB are written like the first ones and the padding after
    column N stays untouched.  Sampled rows are checked against the oracle
    run on those rows alone."""
    import torch
    import dense_gemm_tiled_amd as tg
    # alpha = 0, bf16 C of 300 rows at a pitch just under 8 MiB: 2.5 GB
    M, N, ldc = 300, 1000, (1 << 22) - 128
    store = torch.empty(M, ldc, dtype=torch.bfloat16, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    store.normal_(generator=gen)
    c = store[:, :N]
    a = torch.zeros(M, 8, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(8, N, dtype=torch.bfloat16, device="cuda")
    bias = torch.linspace(-1, 1, N, device="cuda").to(torch.bfloat16)
    rows = [0, 1, 150, 256, 257, 298, 299]          # rows from 257 on start past 2 GiB
    assert 256 * ldc * 2 < 2 ** 31 < 257 * ldc * 2
    before = _rows_of(store, rows, N + 64)
    say("GPU case: alpha = 0 on a C past 2 GiB")
    tg.gemm(a, b, c, alpha=0.0, beta=0.5, bias=bias, activation="relu")
    torch.cuda.synchronize()
    assert tg.last_kernel() == "scale_c", tg.last_kernel()
    after = _rows_of(store, rows, N + 64)
    bias_bits = bias.cpu().view(torch.int16).numpy().view(np.uint16)[None, :]
    q = workloads.Problem("row", 1, N, 8, "bf16", "bf16", alpha=0.0, beta=0.5)
    zeros_a, zeros_b = np.zeros((1, 8), np.uint16), np.zeros((8, N), np.uint16)
    for r, x0, x1 in zip(rows, before, after):
        cin = x0[:N].view(torch.int16).numpy().view(np.uint16)[None, :].copy()
        ref = oracle_epilogue(q, zeros_a, zeros_b, cin, bias_bits, "relu")
        got = x1[:N].view(torch.int16).numpy().view(np.uint16)[None, :].copy()
        compare(q, got, ref, label="alpha = 0, row %d" % r)
        assert torch.equal(x1[N:].view(torch.int16), x0[N:].view(torch.int16)), "padding %d" % r
    del store, c

    # split-K into an fp32 C of 512 rows at a pitch just under 8 MiB: 4.3 GB
    M, N, K, ldc = 512, 64, 16384, (1 << 21) - 64
    p = workloads.Problem("big_c", M, N, K, "bf16", "f32", dist="uniform", seed=47)
    A, B, _ = workloads.make_inputs(p)
    a, b = to_dev(A, "bf16"), to_dev(B, "bf16")
    store = torch.full((M, ldc), 7.0, dtype=torch.float32, device="cuda")
    c = store[:, :N]
    say("GPU case: split-K into a C past 2 GiB")
    tg.gemm(a, b, c)
    torch.cuda.synchronize()
    assert tg.last_kernel().endswith("+splitk_reduce"), tg.last_kernel()
    rows = [0, 256, 257, 300, 511]                  # rows from 257 on start past 2 GiB
    assert 256 * ldc * 4 < 2 ** 31 < 257 * ldc * 4
    q = p.with_(M=len(rows))
    sub = np.ascontiguousarray(A[rows])
    ref = oracle_full(q, sub, B, np.zeros((len(rows), N), np.float32))
    got = np.stack([x.numpy() for x in _rows_of(store, rows, N + 64)])
    compare(q, np.ascontiguousarray(got[:, :N]), ref, label="split-K big C")
    assert np.all(got[:, N:] == 7.0)
