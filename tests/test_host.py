"""Host-side tests of libtcgemm.so that need no GPU.

* the library loads and exports every function include/tcgemm.h declares;
* every invalid descriptor is refused with the documented status before any
  launch (the dispatch count stays 0), as tessl "Architecture" requires of its
  boundary ("The Kernel Library and the nn Boundary");
* the planner's choices for the measured shapes;
* the workgroup -> tile order is a bijection and keeps each XCD's tiles in a
  compact block (tessl "Architecture", "Column-Panel Grid Swizzling").
"""
import ctypes
import math
import os
import re

import pytest

import dense_gemm_tiled_amd as tg
import workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "tcgemm.h")


@pytest.fixture(scope="module")
def lib():
    return tg.load_library()


_VP = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tc_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree(lib):
    names = declared_functions()
    assert len(names) >= 17
    assert set(names) == set(tg._SIGNATURES), set(names) ^ set(tg._SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_time_next_gemm_arguments(lib, ctx):
    """The measurement hook only stores the two handles: both or neither."""
    assert lib.tc_time_next_gemm(None, _VP(16), _VP(32)) == 1
    assert lib.tc_time_next_gemm(ctx, _VP(16), None) == 1
    assert lib.tc_time_next_gemm(ctx, None, _VP(32)) == 1
    assert lib.tc_time_next_gemm(ctx, _VP(16), _VP(32)) == 0
    assert lib.tc_time_next_gemm(ctx, None, None) == 0   # disarm


def test_version_and_status_strings(lib):
    assert lib.tc_version().startswith(b"tcgemm")
    for code, name in tg._STATUS.items():
        assert lib.tc_status_string(code).decode() == name
    assert lib.tc_status_string(99) == b"TC_ERR_UNKNOWN"


def desc(M=64, N=64, K=64, a=tg.BF16, c=tg.BF16, acc=tg.F32, ta=False, tb=False, alpha=1.0,
         beta=0.0, lda=0, ldb=0, ldc=0, batch=1, sa=0, sb=0, sc=0):
    d = tg.BatchedDescT()
    b = d.base
    b.M, b.N, b.K = M, N, K
    b.a_dtype, b.b_dtype, b.c_dtype, b.accum_dtype = a, a, c, acc
    b.transpose_a, b.transpose_b = ta, tb
    b.alpha, b.beta = alpha, beta
    b.lda, b.ldb, b.ldc = lda, ldb, ldc
    d.batch, d.stride_a, d.stride_b, d.stride_c = batch, sa, sb, sc
    return d


@pytest.fixture()
def ctx(lib):
    out = ctypes.c_void_p()
    assert lib.tc_context_create(ctypes.byref(out)) == 0
    yield out.value
    lib.tc_context_destroy(out.value)


# fake, distinct, non-overlapping "device" addresses: validation must refuse
# before it ever looks at them
A_PTR, B_PTR, C_PTR = 0x10000000000, 0x20000000000, 0x30000000000

BAD = [
    ("M=0", dict(M=0), 1),
    ("N<0", dict(N=-3), 1),
    ("K=0", dict(K=0), 1),
    ("batch=0", dict(batch=0), 1),
    ("lda<K", dict(lda=63), 1),
    ("lda<M (TN)", dict(ta=True, M=100, lda=99), 1),
    ("ldb<N", dict(ldb=10), 1),
    ("ldb<K (NT)", dict(tb=True, K=70, ldb=69), 1),
    ("ldc<N", dict(ldc=63), 1),
    ("alpha=nan", dict(alpha=float("nan")), 1),
    ("beta=inf", dict(beta=float("inf")), 1),
    ("a/c dtype", dict(a=tg.BF16, c=tg.F16), 2),
    ("f32->bf16", dict(a=tg.F32, c=tg.BF16), 2),
    ("accum f16", dict(a=tg.F16, c=tg.F16, acc=tg.F16), 2),
    ("i8->f32", dict(a=tg.I8, c=tg.F32, acc=tg.I32), 2),
    ("i8 alpha", dict(a=tg.I8, c=tg.I32, acc=tg.I32, alpha=2.0), 2),
    ("i8 beta", dict(a=tg.I8, c=tg.I32, acc=tg.I32, beta=1.0), 2),
    ("i8 K wrap", dict(a=tg.I8, c=tg.I32, acc=tg.I32, K=131072), 3),
    ("A extent", dict(M=70000, K=40000), 3),
    ("C extent", dict(M=50000, N=50000, K=8), 3),
    ("ld 8MiB", dict(lda=5_000_000, M=4), 3),
    ("stride<0", dict(batch=2, sa=-1, sc=4096), 1),
    ("batch C overlap", dict(batch=2, sc=64 * 63), 4),
    ("batch C stride 0", dict(batch=2, sa=4096, sb=4096, sc=0), 4),
]


@pytest.mark.parametrize("name,kw,status", BAD, ids=[b[0] for b in BAD])
def test_invalid_descriptor_refused_before_launch(lib, ctx, name, kw, status):
    d = desc(**kw)
    st = lib.tc_gemm_batched(ctx, ctypes.byref(d), A_PTR, B_PTR, C_PTR)
    assert st == status, (tg.status_name(st), lib.tc_last_error(ctx))
    assert lib.tc_last_error(ctx) != b""
    assert lib.tc_dispatch_count(ctx) == 0
    assert lib.tc_gemm_plan(None, ctypes.byref(d), None) == status


def test_null_arguments(lib, ctx):
    d = desc()
    assert lib.tc_gemm_batched(ctx, ctypes.byref(d), None, B_PTR, C_PTR) == 1
    assert lib.tc_gemm_batched(ctx, ctypes.byref(d), A_PTR, B_PTR, None) == 1
    assert lib.tc_gemm_batched(ctx, None, A_PTR, B_PTR, C_PTR) == 1
    assert lib.tc_gemm_batched(None, ctypes.byref(d), A_PTR, B_PTR, C_PTR) == 1
    assert lib.tc_gemm(ctx, None, A_PTR, B_PTR, C_PTR) == 1
    assert lib.tc_gemm_async(ctx, ctypes.byref(d.base), A_PTR, B_PTR, C_PTR, None) == 1
    assert lib.tc_dispatch_count(ctx) == 0


def test_overlap_refused(lib, ctx):
    d = desc(M=64, N=64, K=64)                  # bf16: A spans 8192 bytes
    assert lib.tc_gemm_batched(ctx, ctypes.byref(d), A_PTR, B_PTR, A_PTR + 4096) == 4
    assert lib.tc_gemm_batched(ctx, ctypes.byref(d), A_PTR, B_PTR, B_PTR - 100) == 4
    assert lib.tc_dispatch_count(ctx) == 0


def epi(bias=None, stride=0, act=0, scale=None, sstride=0):
    e = tg.EpilogueT()
    e.bias, e.bias_stride, e.activation = bias, stride, act
    e.col_scale, e.scale_stride = scale, sstride
    return e


S_PTR = 0x50000000000      # a fake per-column scale vector


EPI_BAD = [
    # tessl "Architecture", "Fused Epilogue": refused where there is no float
    # register accumulator (int8 results are exact int32 sums)
    ("int8", dict(a=tg.I8, c=tg.I32, acc=tg.I32), {}, 2),
    ("int8 int32 with scale", dict(a=tg.I8, c=tg.I32, acc=tg.I32), dict(scale=S_PTR), 2),
    # int8 into a float C needs a per-column dequantization scale
    ("int8->f32 no scale", dict(a=tg.I8, c=tg.F32, acc=tg.I32), dict(act=1), 2),
    ("int8->bf16 accum f32", dict(a=tg.I8, c=tg.BF16, acc=tg.F32), dict(scale=S_PTR), 2),
    ("int8 dequant K wrap", dict(a=tg.I8, c=tg.F32, acc=tg.I32, K=131072), dict(scale=S_PTR), 3),
    ("scale_stride<0", dict(batch=2, sa=4096, sb=4096, sc=4096), dict(scale=S_PTR, sstride=-2), 1),
    ("scale overlaps C", {}, dict(scale=C_PTR + 4096), 4),
    ("activation 3", {}, dict(act=3), 1),
    ("activation -1", {}, dict(act=-1), 1),
    ("bias_stride<0", dict(batch=2, sa=4096, sb=4096, sc=4096), dict(bias=0x40000000000, stride=-1), 1),
    ("bias overlaps C", {}, dict(bias=C_PTR + 64), 4),
    ("batched bias overlaps C", dict(batch=3, sa=4096, sb=4096, sc=4096),
     dict(bias=C_PTR - 200, stride=64), 4),
    ("descriptor first", dict(M=0), dict(act=1), 1),
]


@pytest.mark.parametrize("name,dkw,ekw,status", EPI_BAD, ids=[b[0] for b in EPI_BAD])
def test_invalid_epilogue_refused_before_launch(lib, ctx, name, dkw, ekw, status):
    d = desc(**dkw)
    e = epi(**ekw)
    st = lib.tc_gemm_epilogue(ctx, ctypes.byref(d), ctypes.byref(e), A_PTR, B_PTR, C_PTR)
    assert st == status, (tg.status_name(st), lib.tc_last_error(ctx))
    assert lib.tc_last_error(ctx) != b""
    st = lib.tc_gemm_epilogue_async(ctx, ctypes.byref(d), ctypes.byref(e), A_PTR, B_PTR, C_PTR,
                                    _VP(0x1234))
    assert st == status
    assert lib.tc_dispatch_count(ctx) == 0


def test_epilogue_null_arguments(lib, ctx):
    d = desc()
    e = epi(act=1)
    assert lib.tc_gemm_epilogue(ctx, ctypes.byref(d), None, A_PTR, B_PTR, C_PTR) == 1
    assert lib.tc_gemm_epilogue_async(ctx, ctypes.byref(d), ctypes.byref(e), A_PTR, B_PTR,
                                      C_PTR, None) == 1
    assert lib.tc_gemm_epilogue(ctx, ctypes.byref(d), ctypes.byref(e), None, B_PTR, C_PTR) == 1
    assert lib.tc_dispatch_count(ctx) == 0


@pytest.mark.parametrize("dkw,ekw", [
    ({}, dict(bias=0x40000000000, act=2)),
    # int8 dequantized into f32 / bf16, alpha and beta free
    (dict(a=tg.I8, c=tg.F32, acc=tg.I32, alpha=0.5, beta=1.0), dict(scale=S_PTR)),
    (dict(a=tg.I8, c=tg.BF16, acc=tg.I32, K=131071), dict(scale=S_PTR, act=1)),
], ids=["bf16 bias gelu", "int8 dequant f32", "int8 dequant bf16 relu"])
def test_epilogue_valid_call_without_gpu_fails_cleanly(lib, ctx, dkw, ekw):
    """A valid epilogue passes validation and then fails at the device (no GPU
    here), launching nothing."""
    d = desc(**dkw)
    e = epi(**ekw)
    st = lib.tc_gemm_epilogue(ctx, ctypes.byref(d), ctypes.byref(e), A_PTR, B_PTR, C_PTR)
    assert st in (1, 6), (tg.status_name(st), lib.tc_last_error(ctx))
    assert lib.tc_dispatch_count(ctx) == 0


def test_python_epilogue_arguments():
    """make_epilogue's checks run before any library call (CPU tensors)."""
    import torch
    c = torch.empty(4, 8, dtype=torch.bfloat16)
    with pytest.raises(tg.TcGemmError):
        tg.make_epilogue(c, activation="gelu")
    with pytest.raises(tg.TcGemmError):
        tg.make_epilogue(c, bias=torch.zeros(8, dtype=torch.bfloat16))   # not on a GPU
    e = tg.make_epilogue(c, activation="gelu_tanh")
    assert e.activation == 2 and not e.bias


def test_autotune_switch(lib, ctx):
    assert lib.tc_set_autotune(None, 1) == 1
    assert lib.tc_autotune_entries(None) == 0
    assert lib.tc_autotune_entries(ctx) == 0
    assert lib.tc_set_autotune(ctx, 1) == 0
    assert lib.tc_set_autotune(ctx, 0) == 0
    # a refused call tunes nothing
    d = desc(M=0)
    assert lib.tc_set_autotune(ctx, 1) == 0
    assert lib.tc_gemm_batched(ctx, ctypes.byref(d), A_PTR, B_PTR, C_PTR) == 1
    assert lib.tc_autotune_entries(ctx) == 0 and lib.tc_dispatch_count(ctx) == 0


def test_int8_k_bound_accepted_at_131071(lib):
    d = desc(a=tg.I8, c=tg.I32, acc=tg.I32, K=131071, M=16, N=16)
    assert lib.tc_gemm_plan(None, ctypes.byref(d), None) == 0


def test_valid_call_without_gpu_fails_cleanly(lib, ctx):
    """With a valid descriptor but no usable device the call reports an error
    instead of launching (on a GPU host the fake pointers are refused)."""
    d = desc()
    st = lib.tc_gemm_batched(ctx, ctypes.byref(d), A_PTR, B_PTR, C_PTR)
    assert st in (1, 6)
    assert lib.tc_dispatch_count(ctx) == 0


# ------------------------------------------------------------------ planner
def plan_of(p: workloads.Problem):
    code = {"f32": tg.F32, "f16": tg.F16, "bf16": tg.BF16, "i8": tg.I8, "i32": tg.I32}
    d = desc(M=p.M, N=p.N, K=p.K, a=code[p.a_dtype], c=code[p.c_dtype],
             acc=tg.I32 if p.a_dtype == "i8" else tg.F32, ta=p.transpose_a, tb=p.transpose_b,
             alpha=p.alpha, beta=p.beta, lda=p.lda, ldb=p.ldb, ldc=p.ldc, batch=p.batch,
             sa=p.stride_a, sb=p.stride_b, sc=p.stride_c)
    return tg.plan(d)


def test_plan_headline_uses_one_256_tile_per_cu():
    pl = plan_of(workloads.get("bf16_nn_4096"))
    assert pl["kernel"] == "gemm_bf16_nn_256x256_dma"
    assert (pl["tiles_m"], pl["tiles_n"], pl["grid"], pl["splits"]) == (16, 16, 256, 1)
    assert pl["launches"] == 1 and pl["workspace_bytes"] == 0


def test_plan_splitk_shape():
    p = workloads.get("bf16_tn_splitk_b8")
    pl = plan_of(p)
    assert pl["kernel"] == "gemm_bf16_tn_128x128_dma4+splitk_reduce"
    assert pl["splits"] > 1 and pl["launches"] == 2
    assert pl["k_per_split"] % pl["tile_k"] == 0
    assert pl["splits"] * pl["k_per_split"] >= p.K > (pl["splits"] - 1) * pl["k_per_split"]
    assert pl["workspace_bytes"] == pl["splits"] * p.batch * p.M * p.N * 4
    assert 128 < pl["grid"] <= 256          # one round of one workgroup per CU


def test_plan_split_k_fits_one_round():
    """Split-K on the 4-stage 128x128 tile (one workgroup per CU) takes as
    many slices as fit one round of 256 workgroups, keeps at least 4 K-tiles
    per slice, and every slice is non-empty."""
    shapes = [(128, 384, 16384, 8, "bf16", "f32", True), (256, 256, 8192, 1, "f16", "f32", False),
              (130, 200, 1100, 2, "bf16", "bf16", True), (512, 640, 4096, 1, "i8", "i32", False),
              (64, 2000, 65536, 1, "bf16", "f32", False)]
    for M, N, K, batch, a, c, ta in shapes:
        p = workloads.Problem("s", M, N, K, a, c, transpose_a=ta, batch=batch)
        pl = plan_of(p)
        tiles = -(-M // 128) * -(-N // 128) * batch
        assert pl["kernel"].endswith("_128x128_dma4+splitk_reduce"), (M, N, K, pl["kernel"])
        assert pl["grid"] == tiles * pl["splits"] <= 256, (M, N, K, pl["grid"])
        assert pl["splits"] >= 2 and pl["k_per_split"] >= 4 * pl["tile_k"], (M, N, K, pl)
        assert (pl["splits"] - 1) * pl["k_per_split"] < K <= pl["splits"] * pl["k_per_split"]
        # one more slice would not fit the round, or the slices would get too short
        assert tiles * (pl["splits"] + 1) > 256 or -(-K // pl["tile_k"]) // (pl["splits"] + 1) < 4


def test_plan_strip_bt_from_row_packing():
    """An edge split whose main part packs B row by row and whose column
    strip runs on the thin kernel: the packing writes the strip's B^T after
    the main part's packed B (per problem when B is batched), so the strip
    has no gather pass; a B the main part need not pack keeps the gather
    (also the B of 2048 bytes at a pitch of 2051 read in place with
    TCGEMM_PACK_UNALIGNED=0)."""
    p = workloads.Problem("s", 2048, 2051, 256, "i8", "i32", batch=4)
    pl = plan_of(p)
    assert pl["kernel"] == "pack_b+gemm_i8_nn_256x256_dma|gemm_i8_nn_thin", pl["kernel"]
    assert pl["launches"] == 3
    main_b = 4 * 256 * 2048                       # 4 problems, 256 rows of 2048 packed bytes
    strip_bt = 4 * 3 * 256                        # 4 problems, 3 rows of 256 bytes
    assert pl["workspace_bytes"] == main_b + strip_bt
    os.environ["TCGEMM_PACK_UNALIGNED"] = "0"
    try:
        pl = plan_of(p)
    finally:
        del os.environ["TCGEMM_PACK_UNALIGNED"]
    assert pl["kernel"] == "gemm_i8_nn_256x256_dma|transpose_b+gemm_i8_nn_thin", pl["kernel"]
    assert pl["launches"] == 3
    assert pl["workspace_bytes"] == strip_bt
    # a B of whole 16-byte rows is read as it is: the strip gathers its B^T
    q = workloads.Problem("s", 4096, 4104, 1024, "bf16", "bf16")
    assert plan_of(q)["kernel"] == "gemm_bf16_nn_256x256_dma|transpose_b+gemm_bf16_nn_thin"


def test_plan_other_workloads():
    # ldb = 4099 bytes: B rows do not start on 16-byte boundaries, so B is
    # packed into the workspace first; N = 4099 leaves a 3-column strip past
    # 16 tile columns, which runs on the thin-output kernel of its own.  The
    # packing of B also writes the strip's columns as B^T (3 rows of 4096),
    # after the packed main columns, so the strip has no gather pass.
    pl = plan_of(workloads.get("i8_nn_ragged"))
    assert pl["kernel"] == "pack_b+gemm_i8_nn_256x256_dma|gemm_i8_nn_thin", pl["kernel"]
    assert pl["launches"] == 3
    assert pl["workspace_bytes"] == 4096 * 4096 + 3 * 4096
    assert plan_of(workloads.get("f16_tn_4096"))["kernel"] == "gemm_f16_tn_256x256_dma"
    assert plan_of(workloads.get("f16_nt_4096"))["kernel"] == "gemm_f16_nt_256x256_dma"
    # fp32 256^3: 16 tiles of 64 x 64 with 8 K-tiles each.  The 4 waves of
    # a workgroup take every 4th K-tile each, on 16 x 16 tiles (256
    # workgroups): one launch, no workspace
    pl = plan_of(workloads.get("sgemm_nn_256"))
    assert pl["kernel"] == "gemm_f32_nn_16x16_ks", pl["kernel"]
    assert pl["splits"] == 1 and pl["grid"] == 256 and pl["launches"] == 1, pl
    assert pl["workspace_bytes"] == 0, pl
    # 36 tiles of 64 x 64 give 144 of 32 x 32
    mid = plan_of(workloads.get("sgemm_nn_256").with_(M=384, N=384))
    assert mid["kernel"] == "gemm_f32_nn_32x32_ks" and mid["grid"] == 144, mid
    # the same small output with a tall K splits K across workgroups, in
    # slices of two K-tiles on up to 512 workgroups
    tall = plan_of(workloads.get("sgemm_nn_256").with_(K=8192))
    assert tall["kernel"] == "gemm_f32_nn_64x64+splitk_reduce", tall["kernel"]
    assert tall["splits"] == 32 and tall["grid"] == 512, tall
    # and a 16-bit small problem with a short K takes the K-split tile too
    small = plan_of(workloads.Problem("small", 256, 256, 512, "bf16", "bf16"))
    assert small["kernel"] == "gemm_bf16_nn_16x16_ks", small["kernel"]
    z = plan_of(workloads.get("bf16_nn_4096").with_(alpha=0.0, beta=2.0))
    assert z["kernel"] == "scale_c" and z["launches"] == 1


def test_plan_mid_size_outputs():
    """16-bit and int8 outputs of 32 to 191 tiles of 128 x 128 run on the
    128 x 128 direct-to-LDS tiles: K-sliced on the 4-stage tile to fill one
    round of workgroups when K has 32 K-tiles or more, else unsliced on the
    two-per-CU tile; fp32 keeps the register-staged tiles."""
    P = workloads.Problem
    pl = plan_of(P("m", 4096, 512, 4096, "bf16", "bf16"))
    assert pl["kernel"] == "gemm_bf16_nn_128x128_dma4+splitk_reduce", pl["kernel"]
    assert pl["splits"] == 2 and pl["grid"] == 256, pl
    pl = plan_of(P("m", 2048, 512, 4096, "bf16", "bf16"))
    assert pl["splits"] == 4 and pl["grid"] == 256, pl
    pl = plan_of(P("m", 1024, 768, 2048, "bf16", "f32"))
    assert pl["kernel"].endswith("128x128_dma4+splitk_reduce") and pl["splits"] == 5, pl
    # unsliced: the 4-stage tile with 16 K-tiles or more (one workgroup per
    # CU either way), else the 2-stage one
    for shape in [(1024, 1024, 1024, "bf16", "bf16"), (2048, 512, 2048, "i8", "i32"),
                  (3072, 512, 1024, "f16", "f16")]:
        pl = plan_of(P("m", *shape))
        assert pl["kernel"].endswith("_128x128_dma4") and pl["splits"] == 1, (shape, pl)
    for shape in [(1024, 1024, 512, "f16", "f16"), (1024, 1024, 1024, "i8", "i32")]:
        pl = plan_of(P("m", *shape))
        assert pl["kernel"].endswith("_128x128_dma") and pl["splits"] == 1, (shape, pl)
    assert plan_of(P("m", 1024, 1024, 1024, "f32", "f32"))["kernel"] == "gemm_f32_nn_64x64"


def test_plan_wide_split_on_the_256_ring():
    """129 to 191 tiles of 128 x 128 with at least 160 K-tiles: the 256 x 256
    ring with as many K slices as fit one round (at least 16 K-tiles each,
    at least 192 workgroups); 192 to 256 of them the same with at least 25
    K-tiles per slice; fewer 128 x 128 tiles keep their own split, a shorter
    K stays unsplit."""
    P = workloads.Problem
    pl = plan_of(P("w", 1536, 1536, 12288, "bf16", "bf16"))
    assert pl["kernel"] == "gemm_bf16_nn_256x256_dma+splitk_reduce", pl["kernel"]
    assert pl["splits"] == 7 and pl["grid"] == 252, pl
    assert (pl["splits"] - 1) * pl["k_per_split"] < 12288 <= pl["splits"] * pl["k_per_split"]
    assert pl["k_per_split"] >= 16 * pl["tile_k"]
    pl = plan_of(P("w", 1280, 1792, 16384, "f16", "f32", transpose_a=True))
    assert pl["kernel"] == "gemm_f16_tn_256x256_dma+splitk_reduce" and pl["grid"] == 245, pl
    # 64 tiles of 128 x 128: their own 4-stage split
    pl = plan_of(P("w", 1024, 1024, 16384, "bf16", "bf16"))
    assert pl["kernel"] == "gemm_bf16_nn_128x128_dma4+splitk_reduce", pl["kernel"]
    # too short a K
    pl = plan_of(P("w", 1536, 1536, 2048, "bf16", "bf16"))
    assert pl["kernel"] == "gemm_bf16_nn_128x128_dma4" and pl["splits"] == 1, pl
    # 192 to 256 tiles of 128 x 128: split only with at least 25 K-tiles per slice
    pl = plan_of(P("w", 2048, 2048, 16384, "bf16", "bf16"))
    assert pl["kernel"] == "gemm_bf16_nn_256x256_dma+splitk_reduce", pl
    assert pl["splits"] == 4 and pl["k_per_split"] >= 25 * pl["tile_k"], pl
    # under 160 K-tiles: the 4-stage 128 x 128 tile unsplit
    for shape in [(2048, 2048, 8192), (4096, 1024, 8192), (1664, 1544, 6144),
                  (4096, 1024, 4096), (2048, 2048, 4096), (2048, 2048, 2048)]:
        pl = plan_of(P("w", *shape, "bf16", "bf16"))
        assert pl["kernel"] == "gemm_bf16_nn_128x128_dma4" and pl["splits"] == 1, (shape, pl)


def test_plan_one_partial_round_of_256_tiles():
    """Under 192 tiles of 256 x 256 but over 512 of 128 x 128: one partly
    filled round of 256 x 256 tiles rather than two rounds of 128 x 128;
    up to 512 of them stay on 128 x 128."""
    P = workloads.Problem
    for shape in [(3072, 3072, 8192), (3328, 3072, 8192), (3072, 3072, 4096)]:
        pl = plan_of(P("r", *shape, "bf16", "bf16"))
        assert pl["kernel"] == "gemm_bf16_nn_256x256_dma" and pl["grid"] < 192, (shape, pl)
    for shape in [(2816, 2816, 8192), (2560, 2560, 8192)]:
        pl = plan_of(P("r", *shape, "bf16", "bf16"))
        assert pl["kernel"] == "gemm_bf16_nn_128x128_dma", (shape, pl)


def test_plan_tile_not_mostly_padding():
    """A class is taken only when its tile is less than half empty along M
    and N: a batch of 128 x 128 problems fills the chip with 256 x 256
    tiles by count, but each would be three quarters padding."""
    P = workloads.Problem
    pl = plan_of(P("b", 128, 128, 128, "f32", "f32", batch=256))
    assert pl["kernel"] == "gemm_f32_nn_128x128" and pl["grid"] == 256, pl
    pl = plan_of(P("b", 128, 128, 128, "bf16", "bf16", batch=256))
    assert pl["kernel"] == "gemm_bf16_nn_128x128_dma", pl
    # 200 rows: a 256-row tile is 22 % padding, still taken
    assert plan_of(P("w", 200, 65536, 256, "bf16", "bf16"))["kernel"] == "gemm_bf16_nn_256x256_dma"


def test_plan_dma_eligibility():
    """The direct-to-LDS classes take 16-bit and int8 inputs.  An operand whose
    row pitch, batch stride or row length (K for K-contiguous operands, M or N
    for M/N-contiguous ones) is not a whole number of 16-byte chunks is packed
    into the workspace first (with TCGEMM_PACK_UNALIGNED=0 only one whose row
    length is not); f32 inputs take the register-staged kernel."""
    base = workloads.get("bf16_nn_4096")
    assert plan_of(base.with_(K=4096 - 8))["kernel"] == "gemm_bf16_nn_256x256_dma"
    # K = 4092: A rows (K-contiguous) end inside a chunk; B (N-contiguous) is fine
    pl = plan_of(base.with_(K=4096 - 4))
    assert pl["kernel"] == "pack_a+gemm_bf16_nn_256x256_dma"
    assert pl["workspace_bytes"] == 4096 * 8192 and pl["launches"] == 2
    assert plan_of(base.with_(lda=4096 + 4))["kernel"] == "pack_a+gemm_bf16_nn_256x256_dma"
    assert plan_of(base.with_(lda=4096 + 8))["kernel"] == "gemm_bf16_nn_256x256_dma"
    os.environ["TCGEMM_PACK_UNALIGNED"] = "0"
    try:
        assert plan_of(base.with_(lda=4096 + 4))["kernel"] == "gemm_bf16_nn_256x256_dma"
        assert plan_of(base.with_(K=4096 - 4))["kernel"] == "pack_a+gemm_bf16_nn_256x256_dma"
    finally:
        del os.environ["TCGEMM_PACK_UNALIGNED"]
    # N = 4100: the last B row would end inside a chunk
    assert plan_of(base.with_(M=3072, N=4100, ldb=4104))["kernel"] == "pack_b+gemm_bf16_nn_256x256_dma"
    # TN: both operands M/N-contiguous, so any K is fine
    assert plan_of(base.with_(transpose_a=True, K=4093))["kernel"] == "gemm_bf16_tn_256x256_dma"
    assert plan_of(base.with_(a_dtype="f32", c_dtype="f32"))["kernel"] == "gemm_f32_nn_256x256"
    i8 = workloads.get("i8_nn_ragged")
    assert plan_of(i8.with_(N=4096 + 16))["kernel"].startswith("gemm_i8_nn_256x256_dma|")
    assert plan_of(i8.with_(N=4096))["kernel"] == "gemm_i8_nn_256x256_dma"


def test_plan_edge_split():
    """A thin ragged last tile column (or row) that would cost a second round
    of 256x256 workgroups runs as a second GEMM, and so do the tiles past the
    whole rounds when that costs fewer rounds (round split); a strip that
    saves nothing, or TCGEMM_EDGE=0, keeps one launch."""
    base = workloads.get("bf16_nn_4096")
    main = "gemm_bf16_nn_256x256_dma"
    assert plan_of(base.with_(N=4104))["kernel"] == main + "|transpose_b+gemm_bf16_nn_thin"
    assert plan_of(base.with_(M=4100))["kernel"] == main + "|gemm_bf16_nn_128x128_dma4+splitk_reduce"
    assert plan_of(base.with_(N=4096 + 128))["kernel"].startswith(main + "|")
    # a strip over half a tile, or a whole 17th tile column: the whole
    # round of 256 x 256 tiles and the rest as a second GEMM (round split)
    pl = plan_of(base.with_(N=4096 + 136))
    assert pl["kernel"] == main + "|gemm_bf16_nn_128x128_dma4+splitk_reduce", pl["kernel"]
    assert plan_of(base.with_(N=4096 + 256))["kernel"].startswith(main + "|")
    assert plan_of(base.with_(M=4096 + 2048))["kernel"] == main + "|gemm_bf16_nn_128x128_dma"
    # 400 tiles (20 x 20): 12 rows of tiles fill 240 of one round, the other
    # 8 rows still take a round of their own -- no gain, one launch
    assert plan_of(base.with_(M=4096 + 1024, N=4096 + 1024))["kernel"] == main
    # 448 tiles: one launch costs two rounds, the split two as well
    assert "|" not in plan_of(base.with_(M=7168))["kernel"]
    assert plan_of(base.with_(M=3072, N=4104))["kernel"] == main          # 204 tiles: one round
    pl = plan_of(base.with_(N=4104))
    assert pl["tiles_m"] == 16 and pl["tiles_n"] == 16 and pl["grid"] > 256
    os.environ["TCGEMM_EDGE"] = "0"
    try:
        assert plan_of(base.with_(N=4104))["kernel"] == main
        assert plan_of(base.with_(N=4096 + 136))["kernel"] == "gemm_bf16_nn_128x128_dma"
    finally:
        del os.environ["TCGEMM_EDGE"]
    # one partial tile row or column: no strip (there are no whole tiles
    # beside it)
    os.environ["TCGEMM_TILE"] = "dma"
    try:
        for shape in (dict(M=96, N=200, K=8192), dict(M=300, N=100, K=512), dict(M=40, N=40, K=64)):
            assert "|" not in plan_of(base.with_(**shape))["kernel"], shape
    finally:
        del os.environ["TCGEMM_TILE"]


def test_plan_thin_outputs():
    """At most 16 output columns with K-contiguous A rows take the vector-ALU
    thin kernel (8 rows per workgroup) once there is a workgroup per CU; a B
    stored [K, N] is gathered into B^T first.  Transposed A, too few rows or
    alpha = 0 keep the other paths."""
    p = workloads.Problem("thin", 4096, 8, 1000, "bf16", "f32")
    pl = plan_of(p)
    assert pl["kernel"] == "transpose_b+gemm_bf16_nn_thin"
    assert (pl["tile_m"], pl["grid"], pl["splits"], pl["launches"]) == (8, 512, 1, 2)
    assert pl["workspace_bytes"] == 16128          # 8 rows of 2000 bytes, 256-byte aligned
    assert plan_of(p.with_(batch=3))["workspace_bytes"] == 3 * 16000 + 128
    assert plan_of(p.with_(ldb=1000))["workspace_bytes"] == 16128
    for n in (1, 3, 16):
        pl = plan_of(p.with_(N=n, transpose_b=True))
        assert pl["kernel"] == "gemm_bf16_nt_thin" and pl["workspace_bytes"] == 0
    assert "thin" not in plan_of(p.with_(N=17))["kernel"]
    assert "thin" not in plan_of(p.with_(transpose_a=True))["kernel"]
    assert "thin" not in plan_of(p.with_(M=512))["kernel"]             # 64 workgroups
    assert plan_of(p.with_(M=512, batch=4))["grid"] == 256
    assert "thin" not in plan_of(p.with_(M=2040))["kernel"]            # 255 workgroups
    assert plan_of(p.with_(a_dtype="i8", c_dtype="i32", alpha=1.0, beta=0.0, K=4093,
                           ldb=11))["kernel"] == "transpose_b+gemm_i8_nn_thin"
    assert plan_of(p.with_(alpha=0.0))["kernel"] == "scale_c"
    os.environ["TCGEMM_TILE"] = "thin"
    try:
        assert plan_of(p.with_(M=40))["kernel"] == "transpose_b+gemm_bf16_nn_thin"
        assert "thin" not in plan_of(p.with_(M=40, N=20))["kernel"]
    finally:
        del os.environ["TCGEMM_TILE"]


def test_plan_small_m_gemv():
    """M <= 16 with B stored [N, K] runs as the transposed product on the
    thin kernel (rows = N, 8 per workgroup); A stored [K, M] is gathered
    first; B stored [K, N], M > 16, too few rows, a forced class or
    TCGEMM_GEMV=0 keep the other paths."""
    p = workloads.Problem("gemv", 1, 4096, 4096, "bf16", "bf16", transpose_b=True)
    pl = plan_of(p)
    assert pl["kernel"] == "gemv_bf16_nt_thin", pl["kernel"]
    assert (pl["tile_m"], pl["tiles_m"], pl["grid"], pl["launches"]) == (8, 512, 512, 1)
    assert plan_of(p.with_(M=16))["kernel"] == "gemv_bf16_nt_thin"
    pl = plan_of(p.with_(M=3, transpose_a=True))
    assert pl["kernel"] == "transpose_a+gemv_bf16_tt_thin" and pl["launches"] == 2
    assert plan_of(p.with_(a_dtype="i8", c_dtype="i32", M=4))["kernel"] == "gemv_i8_nt_thin"
    assert "gemv" not in plan_of(p.with_(M=17))["kernel"]
    assert "gemv" not in plan_of(p.with_(transpose_b=False))["kernel"]
    assert "gemv" not in plan_of(p.with_(N=2040))["kernel"]          # 255 row blocks
    assert plan_of(p.with_(N=1024, batch=2))["grid"] == 256
    assert plan_of(p.with_(alpha=0.0, beta=1.0))["kernel"] == "scale_c"
    for env in ({"TCGEMM_GEMV": "0"}, {"TCGEMM_TILE": "64"}):
        os.environ.update(env)
        try:
            assert "gemv" not in plan_of(p)["kernel"]
        finally:
            for k in env:
                del os.environ[k]


def test_plan_packed_batch_strides():
    """A shared operand (batch stride 0) is packed once; a batched one per
    problem, the packed copies placed after the split-K partials."""
    common = dict(M=256, N=256, K=8190, a=tg.BF16, c=tg.F32, batch=3, sb=8190 * 256, sc=256 * 256)
    pl = tg.plan(desc(sa=0, **common))
    assert pl["kernel"] == "pack_a+gemm_bf16_nn_128x128_dma4+splitk_reduce", pl["kernel"]
    part = pl["splits"] * 3 * 256 * 256 * 4
    assert part % 256 == 0
    assert pl["workspace_bytes"] == part + 256 * 16384
    pl = tg.plan(desc(sa=256 * 8190, **common))
    assert pl["workspace_bytes"] == part + 3 * 256 * 16384 and pl["launches"] == 3


def test_plan_mid_size_and_split_k_classes():
    """Outputs too small for 192 tiles of 256 x 256 take the 128 x 128 tile,
    direct-to-LDS for 16-bit and int8 inputs; tall K with few tiles splits K
    on that tile (on the 64 x 64 tile for f32)."""
    mid = workloads.Problem("mid", 1536, 2048, 1024, "bf16", "bf16")
    # 192 tiles, at most one per CU, 16 K-tiles: the 4-stage variant
    assert plan_of(mid)["kernel"] == "gemm_bf16_nn_128x128_dma4"
    assert plan_of(mid.with_(K=512))["kernel"] == "gemm_bf16_nn_128x128_dma"
    assert plan_of(mid.with_(M=3072))["kernel"] == "gemm_bf16_nn_128x128_dma"   # 384 tiles
    assert plan_of(mid.with_(a_dtype="f32", c_dtype="f32"))["kernel"] == "gemm_f32_nn_128x128"
    tall = workloads.Problem("tall", 256, 256, 8192, "f16", "f32")
    pl = plan_of(tall)
    assert pl["kernel"] == "gemm_f16_nn_128x128_dma4+splitk_reduce" and pl["splits"] > 1
    assert pl["grid"] == 4 * pl["splits"]
    pl = plan_of(tall.with_(K=8192 - 2))   # A rows (K-contiguous) not in whole chunks
    assert pl["kernel"] == "pack_a+gemm_f16_nn_128x128_dma4+splitk_reduce"
    pl = plan_of(tall.with_(a_dtype="f32"))
    assert pl["kernel"] == "gemm_f32_nn_64x64+splitk_reduce"


# ------------------------------------------------------------------ tile order
def tile_map(lib, tm_, tn_, groups, band):
    n = tm_ * tn_ * groups
    out = []
    a, b, g = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    for wg in range(n):
        assert lib.tc_tile_of_workgroup(tm_, tn_, groups, band, wg, ctypes.byref(a),
                                        ctypes.byref(b), ctypes.byref(g)) == 0
        out.append((a.value, b.value, g.value))
    return out


@pytest.mark.parametrize("tm_,tn_,groups,band", [
    (16, 16, 1, 8), (17, 33, 1, 8), (3, 5, 7, 8), (1, 1, 1, 8), (13, 4, 2, 8),
    (16, 16, 1, 0), (9, 9, 3, 4), (2, 6, 24, 8), (100, 3, 1, 8)])
def test_tile_order_is_a_bijection(lib, tm_, tn_, groups, band):
    m = tile_map(lib, tm_, tn_, groups, band)
    assert sorted(m) == [(i, j, g) for i in range(tm_) for j in range(tn_) for g in range(groups)]


def test_tile_order_out_of_range(lib):
    a, b, g = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    assert lib.tc_tile_of_workgroup(4, 4, 1, 8, 16, ctypes.byref(a), ctypes.byref(b),
                                    ctypes.byref(g)) == 1
    assert lib.tc_tile_of_workgroup(4, 4, 1, 8, -1, ctypes.byref(a), ctypes.byref(b),
                                    ctypes.byref(g)) == 1


def test_band_order_matches_the_pages_formula(lib):
    """Inside one group, logical ids follow the column-panel band order: with
    the XCD regrouping undone, id t maps to tile (band*PH + rem % h, rem / h)."""
    tm_, tn_, PH = 19, 7, 8                     # last band holds only 3 rows
    n = tm_ * tn_
    m = tile_map(lib, tm_, tn_, 1, PH)
    q, r = divmod(n, 8)
    for wg in range(n):
        xcd, j = wg % 8, wg // 8
        t = (xcd * (q + 1) if xcd < r else r * (q + 1) + (xcd - r) * q) + j
        band = t // (PH * tn_)
        rem = t - band * PH * tn_
        h = min(PH, tm_ - band * PH)
        assert m[wg][:2] == (band * PH + rem % h, rem // h)


def test_each_xcd_gets_a_compact_block(lib):
    """16x16 tiles (the 4096^3 headline with 256x256 tiles): every XCD's 32
    workgroups touch at most 8 A row panels + 4 B column panels, against 2 + 16
    for plain row-major order."""
    m = tile_map(lib, 16, 16, 1, 8)
    for xcd in range(8):
        tiles = [m[wg] for wg in range(256) if wg % 8 == xcd]
        rows = {t[0] for t in tiles}
        cols = {t[1] for t in tiles}
        assert len(tiles) == 32 and len(rows) + len(cols) <= 12
    raster = tile_map(lib, 16, 16, 1, 0)
    tiles = [raster[wg] for wg in range(256) if wg % 8 == 0]
    assert len({t[0] for t in tiles}) + len({t[1] for t in tiles}) == 18


def test_lds_budget_of_the_tile_classes():
    """The pages size their 64x64 tile against a 32 KB threadgroup budget
    (tensorcore "GEMM", "Why 64x64?": 4 KB + 4 KB + 16 KB = 24 KB).  Here each
    class double-buffers (BM + BN) rows of 128 bytes; the largest needs
    128 KiB of the 160 KiB LDS of a gfx950 CU."""
    assert 64 * 32 * 2 + 32 * 64 * 2 + 64 * 64 * 4 == 24 * 1024
    for bm, bn in ((256, 256), (128, 128), (64, 64)):
        assert 2 * (bm + bn) * 128 <= 160 * 1024
    assert 2 * (256 + 256) * 128 == 128 * 1024
