"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Every case runs the library through its C ABI (dense_gemm_tiled_amd.gemm ->
tc_gemm_batched_async) on seeded inputs from workloads.py and compares with
oracle/ on the same bits: int8 -> int32 bit-exact; float results within the
relative Frobenius error 1e-3 (fp16/bf16 inputs) or 1e-5 (fp32 inputs) of the
oracle rounded to the output type, and every float output within the
a-priori elementwise bound of the exact value (tests/gpu_util.py states it).
"""
import zlib

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (TOL, compare, compare_points, env, from_dev, logical, oracle_epilogue,
                      oracle_full, run_library, run_library_epilogue, say, to_dev)

pytestmark = pytest.mark.gpu

P = workloads.Problem

# (input, output) type pairs the library supports
PAIRS = [("f32", "f32"), ("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"),
         ("bf16", "f32"), ("i8", "i32")]
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def lay(ta, tb):
    return ("T" if ta else "N") + ("T" if tb else "N")


def problem(a, c, M, N, K, ta=False, tb=False, **kw):
    dist = "int8" if a == "i8" else kw.pop("dist", "normal")
    float_ok = a != "i8"
    alpha = kw.pop("alpha", 0.5 if float_ok else 1.0)
    beta = kw.pop("beta", 1.0 if float_ok else 0.0)
    c_dist = kw.pop("c_dist", "normal" if beta != 0.0 else "nan")
    seed = kw.pop("seed", zlib.crc32(repr((a, c, M, N, K, ta, tb)).encode()) % 2 ** 31)
    return P("case", M, N, K, a, c, transpose_a=ta, transpose_b=tb, alpha=alpha, beta=beta,
             dist=dist, c_dist=c_dist, seed=seed, **kw)


def check(p, label, **envs):
    A, B, C = workloads.make_inputs(p)
    say("GPU case:", label, p.M, p.N, p.K, p.a_dtype, p.c_dtype, p.layout, envs)
    with env(**envs):
        got = run_library(p, A, B, C)
    ref = oracle_full(p, A, B, C)
    return compare(p, got, ref, C_in=C, label=label)


# ---------------------------------------------------------------- all kernels, ragged
@pytest.mark.parametrize("tile", [256, 128, 64])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[lay(*l) for l in LAYOUTS])
@pytest.mark.parametrize("a,c", PAIRS, ids=["%s-%s" % pc for pc in PAIRS])
def test_every_kernel_ragged(a, c, ta, tb, tile):
    """M, N, K all ragged (K leaves a partial 16-byte chunk for every type),
    several tiles in M and N, alpha = 0.5 and beta = 1 for floats."""
    check(problem(a, c, 300, 270, 197, ta, tb), "ragged tile%d" % tile, TCGEMM_TILE=tile)


@pytest.mark.parametrize("tile", [256, 128, 64])
@pytest.mark.parametrize("a,c", PAIRS, ids=["%s-%s" % pc for pc in PAIRS])
def test_aligned_vector_epilogue_beta0_nan_c(a, c, tile):
    """N and ldc multiples of 4 (vector stores), beta = 0 with a NaN-filled C:
    C must not be read."""
    p = problem(a, c, 264, 520, 256, alpha=1.0, beta=0.0, c_dist="nan")
    check(p, "vec tile%d" % tile, TCGEMM_TILE=tile)


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("a,c,ta,tb", [("bf16", "f32", True, False), ("bf16", "bf16", False, False),
                                       ("f16", "f16", False, True), ("f32", "f32", False, False),
                                       ("i8", "i32", False, False), ("i8", "i32", True, True)])
def test_split_k_forced(a, c, ta, tb, splits):
    p = problem(a, c, 130, 200, 1100, ta, tb, batch=2)
    check(p, "splitk%d" % splits, TCGEMM_SPLITS=splits)


@pytest.mark.parametrize("a,c", [("bf16", "bf16"), ("f32", "f32"), ("i8", "i32")])
def test_padded_leading_dims(a, c):
    p = problem(a, c, 150, 130, 90, True, False, lda=150 + 9, ldb=130 + 3, ldc=130 + 5)
    check(p, "padded")
    p = problem(a, c, 150, 130, 90, False, True, lda=90 + 16, ldb=90 + 1, ldc=130 + 12)
    check(p, "padded2")


# ---------------------------------------------------------------- K split among the waves
KS_TILES = ["64ks", "32ks", "16ks"]
KS_NAME = {"64ks": "_64x64_ks", "32ks": "_32x32_ks", "16ks": "_16x16_ks"}


def ks_check(p, label, tile, **envs):
    """Run p with a tile whose waves split K forced, and check that it is
    the kernel that ran."""
    import dense_gemm_tiled_amd as tg
    res = check(p, label, TCGEMM_TILE=tile, **envs)
    assert tg.last_kernel().endswith(KS_NAME[tile]), tg.last_kernel()
    return res


@pytest.mark.parametrize("tile", KS_TILES)
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[lay(*l) for l in LAYOUTS])
@pytest.mark.parametrize("a,c", PAIRS, ids=["%s-%s" % pc for pc in PAIRS])
def test_ks_kernel_ragged(a, c, ta, tb, tile):
    """M, N and K ragged (K leaves a partial 16-byte chunk), several tiles,
    a K of 6..25 K-tiles so the four waves get unequal shares; alpha = 0.5
    and beta = 1 for floats."""
    check_k = {"f32": 777, "f16": 1553, "bf16": 1553, "i8": 3105}[a]
    ks_check(problem(a, c, 150, 131, check_k, ta, tb), "ks ragged", tile)
    ks_check(problem(a, c, 129, 190, 197, ta, tb), "ks ragged short", tile)


@pytest.mark.parametrize("tile", KS_TILES)
@pytest.mark.parametrize("a,c", PAIRS, ids=["%s-%s" % pc for pc in PAIRS])
def test_ks_kernel_fewer_k_tiles_than_waves(a, c, tile):
    """K of one or two K-tiles: the idle waves contribute zero partial tiles;
    beta = 0 with a NaN-filled C, which must not be read."""
    ks_check(problem(a, c, 64, 64, 5, alpha=1.0, beta=0.0, c_dist="nan"), "ks one tile", tile)
    ks_check(problem(a, c, 100, 70, 150, True, True, alpha=1.0, beta=0.0, c_dist="nan"),
             "ks two tiles", tile)


@pytest.mark.parametrize("tile", KS_TILES)
@pytest.mark.parametrize("a,c,ta,tb", [("f32", "f32", False, False), ("bf16", "f32", True, False),
                                       ("f16", "f16", False, True), ("i8", "i32", True, True)])
def test_ks_kernel_batched_padded(a, c, ta, tb, tile):
    """Batched problems with odd padded leading dims."""
    M, N, K = 130, 100, 900
    p = problem(a, c, M, N, K, ta, tb, batch=3, lda=(M if ta else K) + 3,
                ldb=(K if tb else N) + 5, ldc=N + 7)
    ks_check(p, "ks batched", tile)


@pytest.mark.parametrize("tile", KS_TILES)
@pytest.mark.parametrize("a,c", [("f32", "f32"), ("bf16", "f32"), ("f16", "f16")])
def test_ks_kernel_exact_regime_bitwise(a, c, tile):
    """Integer inputs in [-4, 4]: every partial sum and their sum in wave
    order are exact, so the result is bit-equal to the oracle."""
    p = problem(a, c, 256, 192, 1024, False, False, alpha=1.0, beta=0.0, dist="small_int",
                scale=4.0, c_dist="zeros")
    A, B, C = workloads.make_inputs(p)
    say("GPU case: ks exact", a, c, tile)
    with env(TCGEMM_TILE=tile):
        got = run_library(p, A, B, C)
    import dense_gemm_tiled_amd as tg
    assert tg.last_kernel().endswith(KS_NAME[tile]), tg.last_kernel()
    ref = oracle_full(p, A, B, C)
    assert np.array_equal(got.view(np.uint8), ref.out.view(np.uint8))


def test_ks_kernel_is_the_small_problem_plan_and_deterministic():
    """fp32 256^3 (16 tiles of 64 x 64, 8 K-tiles) plans onto the 16 x 16
    K-split tile with no workspace, and two runs give the same bits."""
    import dense_gemm_tiled_amd as tg
    p = workloads.get("sgemm_nn_256")
    A, B, C = workloads.make_inputs(p)
    say("GPU case: ks plan", p.name)
    r1 = run_library(p, A, B, C)
    assert tg.last_kernel() == "gemm_f32_nn_16x16_ks", tg.last_kernel()
    r2 = run_library(p, A, B, C)
    assert np.array_equal(r1.view(np.uint8), r2.view(np.uint8))
    compare(p, r1, oracle_full(p, A, B, C), C_in=C, label="ks plan")


# ---------------------------------------------------------------- direct-to-LDS kernel
DMA_PAIRS = [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("i8", "i32")]


DMA_TILES = ["dma", "dma8", "dma128", "dma128x4"]
DMA_NAME = {"dma": "_256x256_dma", "dma8": "_256x256_dma8", "dma128": "_128x128_dma",
            "dma128x4": "_128x128_dma4"}


def dma_check(p, label, tile, **envs):
    """Run p with a direct-to-LDS kernel (256x256 with 4 or 8 waves, or
    128x128) forced and check that it is the kernel that ran."""
    import dense_gemm_tiled_amd as tg
    res = check(p, label, TCGEMM_TILE=tile, **envs)
    want = DMA_NAME[tile] + ("+splitk_reduce" if envs.get("TCGEMM_SPLITS", 1) > 1 else "")
    assert tg.last_kernel().endswith(want), tg.last_kernel()
    return res


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[lay(*l) for l in LAYOUTS])
@pytest.mark.parametrize("a,c", DMA_PAIRS, ids=["%s-%s" % pc for pc in DMA_PAIRS])
def test_dma_kernel_ragged(a, c, ta, tb, tile):
    """2 x 2 tiles ragged in M and N, a K tail shorter than the 128-byte tile
    (whole 16-byte chunks), alpha = 0.5 and beta = 1 for floats.  M and N are
    multiples of 16 bytes so that M/N-contiguous rows stay aligned."""
    if a == "i8":
        p = problem(a, c, 304, 272, 208, ta, tb)
    else:
        p = problem(a, c, 296, 264, 200, ta, tb)
    dma_check(p, "dma ragged", tile)


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("a,c", DMA_PAIRS, ids=["%s-%s" % pc for pc in DMA_PAIRS])
def test_dma_kernel_short_k_and_nan_c(a, c, tile):
    """K below one tile (one partial tile plus an empty prefetch), and beta = 0
    with a NaN-filled C: C must not be read."""
    k = 16 if a == "i8" else 8
    p = problem(a, c, 272, 528, k, False, False, alpha=1.0, beta=0.0, c_dist="nan")
    dma_check(p, "dma shortK", tile)
    p = problem(a, c, 512, 256, 3 * k, True, False, alpha=1.0, beta=0.0, c_dist="nan")
    dma_check(p, "dma shortK TN", tile)


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("a,c,ta,tb", [("bf16", "f32", True, False), ("f16", "f16", False, True),
                                       ("i8", "i32", False, False)])
def test_dma_kernel_batched_padded(a, c, ta, tb, tile):
    """Batched problems with padded leading dims (kept 16-byte multiples)."""
    es = 1 if a == "i8" else 2
    pad = 16 // es
    M, N, K = 260, 304, 384
    lda = (M + 4 if ta else K) + pad
    ldb = (K if tb else N) + 2 * pad
    p = problem(a, c, M, N, K, ta, tb, batch=3, lda=lda, ldb=ldb, ldc=N + 3)
    dma_check(p, "dma batched", tile)


@pytest.mark.parametrize("a,c,ta,tb", [("bf16", "bf16", False, False), ("f16", "f32", True, False),
                                       ("i8", "i32", False, True)],
                         ids=["bf16-bf16-NN", "f16-f32-TN", "i8-i32-NT"])
def test_dma_ring_split_k(a, c, ta, tb):
    """Split-K on the 256x256 ring by the planner's own choice: 132 tiles of
    128 x 128 (1408 x 1544, ragged in M and N on the 256 tile) and a K of
    160 K-tiles, so 6 slices of 26 to 27 -- the partial sums and their
    reduction against the oracle."""
    import dense_gemm_tiled_amd as tg
    k = 160 * (128 if a == "i8" else 64)
    p = problem(a, c, 1408, 1544, k, ta, tb)
    check(p, "ring split-K")
    assert tg.last_kernel().endswith("_256x256_dma+splitk_reduce"), tg.last_kernel()


@pytest.mark.parametrize("k", [64, 128, 192, 320])
@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True)],
                         ids=["NN", "TN", "NT"])
@pytest.mark.parametrize("a,c", [("f16", "f16"), ("bf16", "bf16")], ids=["f16-f16", "bf16-bf16"])
def test_dma_ring_beta_c_tile(a, c, ta, tb, k):
    """beta = 1 with a 16-bit C on the 256x256 ring tile.  With at least two
    K-tiles (K = 128, 192, 320) interior tiles read C_old from an LDS image
    of the tile loaded during the loop's last two K-tiles, and store through
    LDS along rows; with one (K = 64) they read C directly.  Batch 2 with a
    padded ldc (rows stay whole 16-byte chunks), and one ragged column of
    tiles, which reads C directly."""
    p = problem(a, c, 512, 520, k, ta, tb, batch=2, ldc=520 + 8)
    dma_check(p, "dma ring beta K%d" % k, "dma")


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("a,c", [("bf16", "f32"), ("f16", "f16")])
def test_dma_kernel_exact_regime_bitwise(a, c, tile):
    """Integer inputs in [-4, 4]: exact accumulation, bit-equal to the oracle."""
    p = problem(a, c, 512, 512, 1024, False, False, alpha=1.0, beta=0.0, dist="small_int",
                scale=4.0, c_dist="zeros")
    A, B, C = workloads.make_inputs(p)
    say("GPU case: dma exact", a, c)
    with env(TCGEMM_TILE=tile):
        got = run_library(p, A, B, C)
    import dense_gemm_tiled_amd as tg
    assert tg.last_kernel().endswith(DMA_NAME[tile])
    ref = oracle_full(p, A, B, C)
    assert np.array_equal(got.view(np.uint8), ref.out.view(np.uint8))


@pytest.mark.parametrize("tile", ["dma128", "dma128x4", "dma"])
@pytest.mark.parametrize("splits", [3, 5])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[lay(*l) for l in LAYOUTS])
@pytest.mark.parametrize("a,c", DMA_PAIRS, ids=["%s-%s" % pc for pc in DMA_PAIRS])
def test_dma128_split_k(a, c, ta, tb, splits, tile):
    """Split-K on the 128x128 direct-to-LDS tiles (2 and 4 LDS stages) and
    the 256x256 ring: 2 x 2 tiles ragged in M and N (one ragged tile on the
    ring), batch 2, a K whose last slice is shorter and ends in a partial
    tile; alpha = 0.5 and beta = 1 for floats."""
    if a == "i8":
        p = problem(a, c, 144, 208, 1104, ta, tb, batch=2)
    else:
        p = problem(a, c, 136, 200, 1096, ta, tb, batch=2)
    dma_check(p, "%s splitk%d" % (tile, splits), tile, TCGEMM_SPLITS=splits)


@pytest.mark.parametrize("tile", ["dma", "dma128"])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[lay(*l) for l in LAYOUTS])
@pytest.mark.parametrize("a,c", DMA_PAIRS, ids=["%s-%s" % pc for pc in DMA_PAIRS])
def test_dma_kernel_packed_operands(a, c, ta, tb, tile):
    """M, N and K ragged with row lengths and pitches that are not whole
    16-byte chunks (odd padded leading dims): both operands are packed into
    zero-padded rows first, then the direct-to-LDS kernel runs."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, 300, 270, 197, ta, tb, lda=(300 if ta else 197) + 3,
                ldb=(197 if tb else 270) + 5)
    dma_check(p, "dma packed", tile)
    assert tg.last_kernel().startswith("pack_a+pack_b+gemm_"), tg.last_kernel()


@pytest.mark.parametrize("pack", [True, False], ids=["packed", "in_place"])
@pytest.mark.parametrize("a,c", [("bf16", "f32"), ("f16", "f16"), ("i8", "i32")])
def test_dma_kernel_misaligned_base_pointers(a, c, pack):
    """A and B one element past a 16-byte boundary (pitches aligned): the
    direct-to-LDS loads read them in place at unaligned addresses, or, with
    unaligned operands packed, the launch packs both; the split-K variant
    too."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, 512, 384, 256, True, False)
    A, B, C = workloads.make_inputs(p)
    ref = oracle_full(p, A, B, C)
    for envs, want in (({"TCGEMM_TILE": "dma128"}, "_128x128_dma"),
                       ({"TCGEMM_TILE": "dma128", "TCGEMM_SPLITS": 3}, "_128x128_dma+splitk_reduce"),
                       ({"TCGEMM_TILE": "dma"}, "_256x256_dma")):
        envs = dict(envs, TCGEMM_PACK_UNALIGNED=1 if pack else 0)
        say("GPU case: misaligned", a, c, envs)
        with env(**envs):
            got = run_library(p, A, B, C, misalign=True)
        assert tg.last_kernel().startswith("pack_a+pack_b+") == pack, tg.last_kernel()
        assert pack or "pack" not in tg.last_kernel(), tg.last_kernel()
        assert tg.last_kernel().endswith(want), tg.last_kernel()
        compare(p, got, ref, C_in=C, label="misaligned %s" % envs)


@pytest.mark.parametrize("pack", [True, False], ids=["packed", "in_place"])
def test_dma128_split_k_packed_shared_operand(pack):
    """Batched split-K with a 2-D A shared by every problem (batch stride 0)
    and an odd lda: with unaligned pitches packed, the shared A is packed
    once; by default its rows (whole 16-byte chunks) are read in place."""
    import torch
    import dense_gemm_tiled_amd as tg
    M, N, K, batch = 136, 200, 2056, 3
    p0 = problem("bf16", "f32", M, N, K, False, False, lda=K + 1, alpha=1.0, beta=0.0,
                 c_dist="zeros")
    A, _, _ = workloads.make_inputs(p0)
    bs = [workloads.make_inputs(p0.with_(seed=p0.seed + 1 + z))[1] for z in range(batch)]
    a = to_dev(A, "bf16")[:, :K]
    b = torch.stack([to_dev(x, "bf16") for x in bs])
    c = torch.zeros(batch, M, N, dtype=torch.float32, device="cuda")
    say("GPU case: shared A split-K, packed:", pack)
    with env(TCGEMM_SPLITS=4, TCGEMM_PACK_UNALIGNED=1 if pack else 0):
        tg.gemm(a, b, c)
    torch.cuda.synchronize()
    assert tg.last_kernel() == ("pack_a+" if pack else "") + \
        "gemm_bf16_nn_128x128_dma4+splitk_reduce", tg.last_kernel()
    got = from_dev(c, "f32")
    for z in range(batch):
        ref = oracle_full(p0, A, bs[z], np.zeros((M, N), np.float32))
        compare(p0, got[z], ref, label="shared A z=%d" % z)


@pytest.mark.parametrize("a,c,M,N,K,batch,ta,tb,strip,pack", [
    # column strip of 8 on the thin-output kernel
    ("bf16", "bf16", 4096, 4104, 1024, 1, False, False, "|transpose_b+gemm_bf16_nn_thin", True),
    # row strip of 4 rows, run as its transposed product (the small-M route,
    # A gathered); the main part packs A (M-contiguous rows of 4096 of 4100
    # halves: an odd pitch)
    ("f16", "f32", 4100, 4096, 192, 1, True, True, "_dma|transpose_a+gemv_f16_tt_thin", True),
    # row strip of 40 rows (too many for the small-M route)
    ("bf16", "bf16", 4136, 4096, 192, 1, True, True, "_dma|gemm_bf16_tt_64x64", True),
    # batched column strip; with B (2048 of 2051 bytes per row) read in
    # place, the strip gathers its B^T ...
    ("i8", "i32", 2048, 2051, 256, 4, False, False, "_dma|transpose_b+gemm_i8_nn_thin", False),
    # ... or, by default, the main part packs B and writes the strip's B^T
    # on the way
    ("i8", "i32", 2048, 2051, 256, 4, False, False, "pack_b+gemm_i8_nn_256x256_dma|gemm_i8_nn_thin",
     True),
    # the same with 16-bit elements: rows of 4100 halves, a 4-column strip
    ("f16", "f32", 4096, 4100, 256, 1, False, False,
     "gemm_f16_nn_256x256_dma|transpose_b+gemm_f16_nn_thin", False),
    ("f16", "f32", 4096, 4100, 256, 1, False, False,
     "pack_b+gemm_f16_nn_256x256_dma|gemm_f16_nn_thin", True),
    # strip of 40 columns: split-K on the 4-stage 128x128 tile
    ("bf16", "f32", 4096, 4136, 1024, 1, False, False, "|gemm_bf16_nn_128x128_dma4+splitk_reduce",
     True),
])
def test_edge_split(a, c, M, N, K, batch, ta, tb, strip, pack):
    """A thin ragged strip past the whole 256x256 tiles runs as a second GEMM
    after them; alpha = 0.5 and beta = 1 for floats, so both parts read C."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, M, N, K, ta, tb, batch=batch)
    check(p, "edge split", TCGEMM_PACK_UNALIGNED=1 if pack else 0)
    assert tg.last_kernel().endswith(strip), tg.last_kernel()


# ---------------------------------------------------------------- thin outputs
THIN_N = [1, 3, 8, 13, 16]


@pytest.mark.parametrize("n", THIN_N)
@pytest.mark.parametrize("tb,ldb", [(False, 0), (False, 70), (True, 0)], ids=["nn", "nn-wide", "nt"])
@pytest.mark.parametrize("a,c", PAIRS, ids=["%s-%s" % pc for pc in PAIRS])
def test_thin_kernel(a, c, tb, ldb, n):
    """The vector-ALU kernel for N <= 16: 300 rows (a ragged last block of 16),
    K = 5000 (whole 4 KiB chunks of K then a ragged one, for every type),
    batch 2, alpha = 0.5 and beta = 1 for floats; then K = 77 (one partial
    chunk) with beta = 0 and a NaN-filled C.  A B stored [K, N] (rows N or 70
    elements apart) is gathered into B^T first."""
    import dense_gemm_tiled_amd as tg
    name = "%sgemm_%s_%s_thin" % ("" if tb else "transpose_b+", a, "nt" if tb else "nn")
    p = problem(a, c, 300, n, 5000, False, tb, batch=2, ldb=ldb)
    check(p, "thin", TCGEMM_TILE="thin")
    assert tg.last_kernel() == name, tg.last_kernel()
    p = problem(a, c, 35, n, 77, False, tb, alpha=1.0, beta=0.0, c_dist="nan", ldb=ldb)
    check(p, "thin short K", TCGEMM_TILE="thin")
    assert tg.last_kernel() == name, tg.last_kernel()


@pytest.mark.parametrize("n", THIN_N)
@pytest.mark.parametrize("a,c", PAIRS, ids=["%s-%s" % pc for pc in PAIRS])
def test_thin_kernel_large_grid(a, c, n):
    """From 1024 workgroups on the thin kernel runs 512-byte chunks of K:
    8200 rows (1025 workgroups, a ragged last block), K = 1000 (whole chunks
    then a ragged one for every type), B stored [N, K] and [K, N], beta = 1
    for floats."""
    import dense_gemm_tiled_amd as tg
    for tb in (True, False):
        name = "%sgemm_%s_%s_thin" % ("" if tb else "transpose_b+", a, "nt" if tb else "nn")
        p = problem(a, c, 8200, n, 1000, False, tb)
        check(p, "thin large grid", TCGEMM_TILE="thin")
        assert tg.last_kernel() == name, tg.last_kernel()


@pytest.mark.parametrize("a,c", PAIRS, ids=["%s-%s" % pc for pc in PAIRS])
def test_thin_kernel_odd_leading_dims(a, c):
    """Odd lda, ldb and ldc (rows start off 16-byte boundaries), both B
    layouts; chosen by the planner (4096 rows: 256 workgroups)."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, 4096, 5, 1030, False, False, lda=1030 + 3, ldb=5 + 2, ldc=5 + 1)
    check(p, "thin odd ld")
    assert tg.last_kernel().endswith("_thin"), tg.last_kernel()
    p = problem(a, c, 4096, 11, 1030, False, True, lda=1030 + 1, ldb=1030 + 5, ldc=11 + 3)
    check(p, "thin odd ld nt")
    assert tg.last_kernel().endswith("_thin"), tg.last_kernel()


def test_thin_kernel_int8_extremes():
    """All (-128)*(-128) over K = 131071 (the int8 K limit) sums to
    16384 * K < 2^31 exactly; 127 * (-128) to -16256 * K."""
    import torch
    import dense_gemm_tiled_amd as tg
    K = 131071
    a = torch.full((2048, K), -128, dtype=torch.int8, device="cuda")
    b = torch.full((K, 3), -128, dtype=torch.int8, device="cuda")
    c = torch.empty(2048, 3, dtype=torch.int32, device="cuda")
    say("GPU case: thin int8 extremes")
    tg.gemm(a, b, c)
    assert tg.last_kernel() == "transpose_b+gemm_i8_nn_thin", tg.last_kernel()
    assert torch.all(c == 16384 * K)
    a.fill_(127)
    tg.gemm(a, b, c)
    assert torch.all(c == -16256 * K)


# ---------------------------------------------------------------- fused epilogue
ACTS = ["none", "relu", "gelu_tanh"]
FLOAT_PAIRS = [pc for pc in PAIRS if pc[0] != "i8"]


def epi_check(p, act, label, *, bias=True, shared=True, **envs):
    """act(alpha*op(A)op(B) + beta*C + bias) through the C ABI against the
    oracle's fused form."""
    A, B, C = workloads.make_inputs(p)
    bv = workloads.make_bias(p, 1 if shared else p.batch) if bias else None
    say("GPU case: epilogue", label, p.M, p.N, p.K, p.a_dtype, p.c_dtype, p.layout, act,
        "bias" if bias else "no bias", envs)
    with env(**envs):
        got = run_library_epilogue(p, A, B, C, bv, act, shared=shared)
    ref = oracle_epilogue(p, A, B, C, bv, act, shared=shared)
    return compare(p, got, ref, C_in=C, label=label)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("a,c", [("bf16", "bf16"), ("f16", "f32"), ("f16", "f16")])
def test_epilogue_dma_kernels(a, c, tile, act):
    """Bias + activation on the direct-to-LDS classes, ragged M/N/K tails,
    alpha = 0.5 and beta = 1."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, 296, 264, 200, False, False)
    epi_check(p, act, "epi %s" % tile, TCGEMM_TILE=tile)
    assert tg.last_kernel().endswith(DMA_NAME[tile]), tg.last_kernel()


@pytest.mark.parametrize("M,N", [(6144, 4096), (4096, 4232)], ids=["rows", "columns"])
def test_round_split(M, N):
    """Past one round of 256x256 tiles, the tiles of the whole rounds run as
    one launch and the rest as a second GEMM (rows or columns): the plain
    product with alpha = 0.5 and beta = 1, and the fused bias + GELU, whose
    bias starts at the second part's first column, against the oracle."""
    import dense_gemm_tiled_amd as tg
    p = problem("bf16", "bf16", M, N, 128)
    check(p, "round split")
    assert tg.last_kernel().startswith("gemm_bf16_nn_256x256_dma|"), tg.last_kernel()
    epi_check(p, "gelu_tanh", "round split epilogue")
    assert tg.last_kernel().startswith("gemm_bf16_nn_256x256_dma|"), tg.last_kernel()


# (input, output, epilogue) for rows past M: plain products and the fused forms
ROWS_PAST_M = [("bf16", "bf16", None), ("f16", "f32", None), ("i8", "i32", None),
               ("bf16", "bf16", "gelu_tanh"), ("f16", "f16", "relu"), ("i8", "bf16", "dequant")]


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("a,c,epi", ROWS_PAST_M, ids=["%s-%s-%s" % x for x in ROWS_PAST_M])
def test_dma_epilogue_rows_past_m(a, c, epi, tile):
    """beta = 0 with whole column tiles and M ragged (300 rows): the tiles of
    the last tile row store all of their rows and the buffer range of C drops
    those past M.  Two problems back to back (problem 0's rows past M are
    problem 1's first rows), then guard rows that must keep their bits."""
    import torch
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, 300, 512, 208 if a == "i8" else 200, beta=0.0, batch=2)
    A, B, C = workloads.make_inputs(p)
    bias = workloads.make_bias(p) if epi in ("gelu_tanh", "relu") else None
    scale = workloads.make_col_scale(p) if epi == "dequant" else None
    act = epi if epi in ("gelu_tanh", "relu") else None
    say("GPU case: rows past M", tile, p.M, p.N, p.K, a, c, epi)
    rows, guard = p.batch * p.M, 64
    guard_bits = (np.arange(guard * p.LDC) * 2654435761 % 65521).astype(np.int64)
    guard_np = guard_bits.astype(C.dtype).reshape(guard, p.LDC)
    a_dev, b_dev = to_dev(A, p.a_dtype), to_dev(B, p.a_dtype)
    big = to_dev(np.concatenate([C.reshape(rows, p.LDC), guard_np]), p.c_dtype)
    c_view = big[:rows].view(p.batch, p.M, p.LDC)[..., :p.N]
    a_v = a_dev[..., :p.K]
    b_v = b_dev[..., :p.N]
    bt = to_dev(bias, p.c_dtype)[0] if bias is not None else None
    st = torch.from_numpy(scale).cuda()[0] if scale is not None else None
    with env(TCGEMM_TILE=tile):
        tg.gemm(a_v, b_v, c_view, alpha=p.alpha, beta=p.beta, bias=bt, activation=act,
                col_scale=st)
    torch.cuda.synchronize()
    assert tg.last_kernel().endswith(DMA_NAME[tile]), tg.last_kernel()
    got_big = from_dev(big, p.c_dtype)
    assert np.array_equal(got_big[rows:].view(np.uint8), guard_np.view(np.uint8)), \
        "rows past the last problem were written"
    got = got_big[:rows].reshape(C.shape)
    if epi is None:
        ref = oracle_full(p, A, B, C)
    else:
        ref = oracle_epilogue(p, A, B, C, bias, act or "none", col_scale=scale)
    compare(p, got, ref, C_in=C, label="rows past M %s" % tile)


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[lay(*l) for l in LAYOUTS])
@pytest.mark.parametrize("tile", [256, 128, 64, "64ks", "16ks"])
def test_epilogue_register_staged_f32(tile, ta, tb):
    p = problem("f32", "f32", 300, 270, 197, ta, tb)
    epi_check(p, "gelu_tanh", "epi f32 tile%s" % tile, TCGEMM_TILE=tile)


@pytest.mark.parametrize("tile", KS_TILES)
@pytest.mark.parametrize("act", ["relu", "gelu_tanh"])
@pytest.mark.parametrize("a,c", [("bf16", "bf16"), ("f16", "f32")])
def test_epilogue_ks_kernel(a, c, act, tile):
    """The fused epilogue on the K-split small tiles, batched with one bias
    vector per problem."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, 130, 200, 1100, True, False, batch=2)
    epi_check(p, act, "epi ks", shared=False, TCGEMM_TILE=tile)
    assert tg.last_kernel().endswith(KS_NAME[tile]), tg.last_kernel()


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("a,c", FLOAT_PAIRS, ids=["%s-%s" % pc for pc in FLOAT_PAIRS])
def test_epilogue_split_k_reduce(a, c, act):
    """With split-K the reduction kernel applies the epilogue; batched, one
    bias vector per problem."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, 130, 200, 1100, True, False, batch=2)
    epi_check(p, act, "epi splitk", shared=False, TCGEMM_SPLITS=3)
    assert tg.last_kernel().endswith("+splitk_reduce"), tg.last_kernel()


@pytest.mark.parametrize("tb", [False, True], ids=["nn", "nt"])
@pytest.mark.parametrize("a,c", FLOAT_PAIRS, ids=["%s-%s" % pc for pc in FLOAT_PAIRS])
def test_epilogue_thin_kernel(a, c, tb):
    p = problem(a, c, 300, 13, 5000, False, tb, batch=2)
    epi_check(p, "gelu_tanh", "epi thin", shared=False, TCGEMM_TILE="thin")
    epi_check(p, "relu", "epi thin shared", TCGEMM_TILE="thin")


@pytest.mark.parametrize("a,c", [("bf16", "bf16"), ("f32", "f32")])
def test_epilogue_alpha_zero_and_beta_zero_nan_c(a, c):
    """alpha = 0: C = act(beta*C + bias) without reading A or B; beta = 0
    with a NaN-filled C: C is not read."""
    p = problem(a, c, 100, 90, 64, False, False, alpha=0.0, beta=0.5)
    epi_check(p, "relu", "epi alpha0")
    p = problem(a, c, 264, 520, 256, False, False, alpha=1.0, beta=0.0, c_dist="nan")
    epi_check(p, "gelu_tanh", "epi beta0 nan")
    epi_check(p, "relu", "epi activation only", bias=False)


def test_epilogue_edge_split_bias_offset():
    """The column strip of an edge split adds the bias of its own columns."""
    import dense_gemm_tiled_amd as tg
    p = problem("bf16", "bf16", 4096, 4104, 128, False, False)
    epi_check(p, "gelu_tanh", "epi edge split")
    assert tg.last_kernel().endswith("|transpose_b+gemm_bf16_nn_thin"), tg.last_kernel()


def test_epilogue_without_bias_or_activation_is_the_plain_product():
    """An epilogue of no bias and no activation gives the plain call's bits."""
    import torch
    import dense_gemm_tiled_amd as tg
    p = problem("bf16", "bf16", 300, 280, 200, False, False)
    A, B, C = workloads.make_inputs(p)
    plain = run_library(p, A, B, C)
    say("GPU case: epilogue none vs plain")
    got = run_library_epilogue(p, A, B, C, None, "none")
    assert np.array_equal(plain.view(np.uint16), got.view(np.uint16))


# ---------------------------------------------------------------- int8 dequant
DEQ_OUT = ["f32", "f16", "bf16"]


def deq_check(p, label, *, act="none", bias=False, shared=True, **envs):
    """int8 x int8 -> exact int32 sums -> per-column fp32 scale (and optionally
    alpha, beta, bias, activation) -> float C, against the oracle."""
    A, B, C = workloads.make_inputs(p)
    nvec = 1 if shared else p.batch
    sc = workloads.make_col_scale(p, nvec)
    bv = workloads.make_bias(p, nvec) if bias else None
    say("GPU case: dequant", label, p.M, p.N, p.K, p.c_dtype, p.layout, act, envs)
    with env(**envs):
        got = run_library_epilogue(p, A, B, C, bv, act, shared=shared, col_scale=sc)
    ref = oracle_epilogue(p, A, B, C, bv, act, shared=shared, col_scale=sc)
    return compare(p, got, ref, C_in=C, label=label)


def deq_problem(c, M, N, K, ta=False, tb=False, **kw):
    alpha = kw.pop("alpha", 1.0)
    beta = kw.pop("beta", 0.0)
    c_dist = kw.pop("c_dist", "normal" if beta != 0.0 else "nan")
    seed = zlib.crc32(repr(("deq", c, M, N, K, ta, tb)).encode()) % 2 ** 31
    return P("case", M, N, K, "i8", c, transpose_a=ta, transpose_b=tb, alpha=alpha, beta=beta,
             dist="int8", c_dist=c_dist, seed=seed, **kw)


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[lay(*l) for l in LAYOUTS])
@pytest.mark.parametrize("c", DEQ_OUT)
def test_i8_dequant_dma_kernels(c, ta, tb, tile):
    """The direct-to-LDS classes, every layout, ragged tiles and K tail."""
    import dense_gemm_tiled_amd as tg
    p = deq_problem(c, 304, 272, 208, ta, tb)
    deq_check(p, "dequant %s" % tile, TCGEMM_TILE=tile)
    assert tg.last_kernel().endswith(DMA_NAME[tile]), tg.last_kernel()


@pytest.mark.parametrize("tile", [256, 128, 64, "64ks", "32ks"])
@pytest.mark.parametrize("c", DEQ_OUT)
def test_i8_dequant_register_staged(c, tile):
    p = deq_problem(c, 300, 270, 197, True, False)
    deq_check(p, "dequant tile%s" % tile, TCGEMM_TILE=tile)


@pytest.mark.parametrize("c", DEQ_OUT)
def test_i8_dequant_composed_split_k(c):
    """Split-K: the reduction sums int32 slices exactly, then dequantizes and
    applies alpha, beta, a bias and GELU; one scale and bias per problem."""
    import dense_gemm_tiled_amd as tg
    p = deq_problem(c, 130, 200, 1100, False, False, alpha=0.5, beta=1.0, batch=2)
    deq_check(p, "dequant splitk", act="gelu_tanh", bias=True, shared=False, TCGEMM_SPLITS=3)
    assert tg.last_kernel().endswith("+splitk_reduce"), tg.last_kernel()


@pytest.mark.parametrize("tb", [False, True], ids=["nn", "nt"])
@pytest.mark.parametrize("c", DEQ_OUT)
def test_i8_dequant_thin(c, tb):
    p = deq_problem(c, 300, 11, 5000, False, tb, batch=2)
    deq_check(p, "dequant thin", act="relu", bias=True, shared=False, TCGEMM_TILE="thin")


def test_i8_dequant_extremes_exact():
    """All (-128)*(-128) over K = 131071 with power-of-two scales: every f32
    result is exact, 16384*K*s[j]."""
    import torch
    import dense_gemm_tiled_amd as tg
    K = 131071
    a = torch.full((2048, K), -128, dtype=torch.int8, device="cuda")
    b = torch.full((K, 20), -128, dtype=torch.int8, device="cuda")
    s = torch.tensor([2.0 ** -e for e in range(20)], dtype=torch.float32, device="cuda")
    c = torch.empty(2048, 20, dtype=torch.float32, device="cuda")
    say("GPU case: dequant extremes")
    tg.gemm(a, b, c, col_scale=s)
    torch.cuda.synchronize()
    assert torch.equal(c, (16384.0 * K * s.double()).float().expand(2048, 20))


def test_workload_i8_nn_ragged_dequant_bf16():
    """The int8 ragged shape (pack, 256x256 main part, thin strip) into bf16
    through the per-column scale, checked at sampled outputs."""
    import dense_gemm_tiled_amd as tg
    p = workloads.get("i8_nn_ragged_dequant_bf16")
    A, B, C = workloads.make_inputs(p)
    sc = workloads.make_col_scale(p)
    say("GPU case: workload", p.name)
    got = logical(p, run_library_epilogue(p, A, B, C, None, "none", col_scale=sc))
    assert tg.last_kernel() == "pack_b+gemm_i8_nn_256x256_dma|gemm_i8_nn_thin", tg.last_kernel()
    pts = workloads.sample_points(p, 4096)
    r, v, T = oracle.gemm_epilogue_points(A, B, None, pts, col_scale=sc, M=p.M, N=p.N, K=p.K,
                                          a_dtype="i8", c_dtype=p.c_dtype, ldb=p.LDB,
                                          want_abs=True)
    compare_points(p, got[pts[:, 0], pts[:, 1], pts[:, 2]], r, v, T, col_scale=sc, pts=pts,
                   label=p.name)


# ---------------------------------------------------------------- small-M GEMV
@pytest.mark.parametrize("ta", [False, True], ids=["nt", "tt"])
@pytest.mark.parametrize("m", [1, 4, 9, 16])
@pytest.mark.parametrize("a,c", PAIRS, ids=["%s-%s" % pc for pc in PAIRS])
def test_gemv_small_m(a, c, m, ta):
    """M <= 16 with B stored [N, K]: the transposed product on the thin kernel,
    C written transposed; N = 2056 (a ragged last block of 8 rows), K = 1000,
    alpha = 0.5 and beta = 1 for floats; batched with N = 1032."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, m, 2056, 1000, ta, True)
    check(p, "gemv")
    assert "gemv_%s_%s_thin" % (a, "tt" if ta else "nt") in tg.last_kernel(), tg.last_kernel()
    p = problem(a, c, m, 1032, 1000, ta, True, batch=2)
    check(p, "gemv batched")
    assert "gemv_" in tg.last_kernel(), tg.last_kernel()


@pytest.mark.parametrize("a,c", FLOAT_PAIRS, ids=["%s-%s" % pc for pc in FLOAT_PAIRS])
def test_gemv_epilogue(a, c):
    """Bias and GELU on the transposed product: the bias of C's column n
    applies to row n of the product."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, 5, 4104, 777, False, True)
    epi_check(p, "gelu_tanh", "gemv epilogue")
    assert tg.last_kernel() == "gemv_%s_nt_thin" % a, tg.last_kernel()
    p = problem(a, c, 3, 1032, 300, True, True, batch=2)
    epi_check(p, "relu", "gemv epilogue batched", shared=False)


@pytest.mark.parametrize("c", DEQ_OUT)
def test_gemv_i8_dequant(c):
    import dense_gemm_tiled_amd as tg
    p = deq_problem(c, 4, 4104, 1000, False, True)
    deq_check(p, "gemv dequant", act="relu", bias=True)
    assert tg.last_kernel() == "gemv_i8_nt_thin", tg.last_kernel()


# ---------------------------------------------------------------- autotune
def _launches(chain):
    return len([k for k in chain.replace("|", "+").split("+") if k])


@pytest.mark.parametrize("a,c,M,N,K,ta,tb", [
    ("bf16", "bf16", 1000, 1030, 512, False, False),     # mid-size: 128 or 256 tiles
    ("f16", "f32", 96, 200, 8192, True, False),          # split-K candidates
    ("i8", "i32", 600, 520, 4096, False, True),
    ("bf16", "bf16", 3, 4096, 1000, False, True),        # small-M route candidate
    ("f32", "f32", 300, 270, 197, False, False),
])
def test_autotune_first_call_then_reuse(a, c, M, N, K, ta, tb):
    """With autotuning on, the first call measures its candidates into a
    scratch C (C itself, read with beta = 1, stays correct), the second call
    of the same problem launches only the chosen plan, and both match the
    oracle."""
    import dense_gemm_tiled_amd as tg
    p = problem(a, c, M, N, K, ta, tb)
    tg.set_autotune(True)
    try:
        n_tuned = tg.autotune_entries()
        d0 = tg.dispatch_count()
        check(p, "autotune first")
        first = tg.last_kernel()
        d1 = tg.dispatch_count()
        assert tg.autotune_entries() == n_tuned + 1
        assert d1 - d0 > _launches(first)                  # the candidates ran too
        check(p, "autotune reuse")
        assert tg.last_kernel() == first
        assert tg.dispatch_count() - d1 == _launches(first)
        assert tg.autotune_entries() == n_tuned + 1
        say("autotune chose", first)
    finally:
        tg.set_autotune(False)


# ---------------------------------------------------------------- exact regime
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, 1.0)])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=[lay(*l) for l in LAYOUTS])
@pytest.mark.parametrize("a,c", [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16"), ("f32", "f32")])
def test_exact_regime_bitwise(a, c, ta, tb, alpha, beta):
    """Integer-valued inputs in [-4, 4] keep every fp32 partial sum below 2^24,
    so accumulation is exact in any order; with alpha = 0.5 (a power of two)
    and beta = 1 on an integer-valued C the epilogue is exact too, and the
    one rounding to the output type is the oracle's: the GPU must equal the
    oracle bit for bit, in every layout."""
    p = problem(a, c, 200, 190, 1000, ta, tb, alpha=alpha, beta=beta, dist="small_int",
                scale=4.0, c_dist="zeros")
    A, B, C = workloads.make_inputs(p)
    if beta != 0.0:
        ints = np.random.default_rng(3).integers(-64, 65, size=C.shape).astype(np.float64)
        C = oracle.encode(ints, c).reshape(C.shape)
    say("GPU case: exact", a, c, lay(ta, tb), alpha, beta)
    got = run_library(p, A, B, C)
    ref = oracle_full(p, A, B, C)
    assert np.array_equal(got.view(np.uint8), ref.out.view(np.uint8))


def test_ones_closed_form():
    """A = B = ones gives C = K exactly."""
    import torch
    import dense_gemm_tiled_amd as tg
    for dt, ct in ((torch.bfloat16, torch.float32), (torch.float16, torch.float16)):
        a = torch.ones(333, 2049, dtype=dt, device="cuda")
        b = torch.ones(2049, 444, dtype=dt, device="cuda")
        c = torch.empty(333, 444, dtype=ct, device="cuda")
        say("GPU case: ones", dt, ct)
        tg.gemm(a, b, c)
        want = 2049.0 if ct == torch.float32 else 2048.0   # 2049 rounds to 2048 in fp16
        assert torch.all(c.float() == want)


def test_int8_extremes():
    """All (-128)*(-128) gives 16384*K; 127*(-128) gives -16256*K (tessl
    "Architecture", "Integer GEMM": operands pinned at the extremes)."""
    import torch
    import dense_gemm_tiled_amd as tg
    K = 8192
    a = torch.full((130, K), -128, dtype=torch.int8, device="cuda")
    b = torch.full((K, 70), -128, dtype=torch.int8, device="cuda")
    c = torch.empty(130, 70, dtype=torch.int32, device="cuda")
    say("GPU case: int8 extremes")
    tg.gemm(a, b, c)
    assert torch.all(c == 16384 * K)
    a.fill_(127)
    tg.gemm(a, b, c)
    assert torch.all(c == -16256 * K)


# ---------------------------------------------------------------- edge cases
EDGE = [(1, 1, 1), (1, 300, 5), (300, 1, 77), (5, 7, 1), (17, 33, 3), (64, 64, 64),
        (65, 63, 129), (256, 256, 8)]


@pytest.mark.parametrize("M,N,K", EDGE)
@pytest.mark.parametrize("a,c,ta,tb", [("bf16", "bf16", False, False), ("f16", "f32", True, False),
                                       ("f32", "f32", False, True), ("i8", "i32", True, True)])
def test_edge_shapes(a, c, ta, tb, M, N, K):
    check(problem(a, c, M, N, K, ta, tb), "edge")


@pytest.mark.parametrize("a,c", [("bf16", "bf16"), ("f32", "f32"), ("f16", "f16")])
def test_alpha_zero(a, c):
    """alpha = 0 is C = beta * C without reading A or B (BLAS convention)."""
    p = problem(a, c, 70, 90, 40, alpha=0.0, beta=2.0)
    check(p, "alpha0")
    p = problem(a, c, 70, 90, 40, alpha=0.0, beta=0.0, c_dist="nan")
    check(p, "alpha0beta0")


def test_batched_matches_per_problem_and_broadcast():
    import torch
    import dense_gemm_tiled_amd as tg
    p = problem("bf16", "f32", 96, 80, 300, True, False, batch=3, alpha=1.0, beta=0.0,
                c_dist="zeros")
    check(p, "batched")
    A, B, C = workloads.make_inputs(p)
    a, b = to_dev(A, "bf16"), to_dev(B, "bf16")
    c = torch.zeros(3, 96, 80, dtype=torch.float32, device="cuda")
    say("GPU case: batched vs singles")
    tg.gemm(a, b, c, transpose_a=True)
    for z in range(3):
        cz = torch.zeros(96, 80, dtype=torch.float32, device="cuda")
        tg.gemm(a[z], b[z], cz, transpose_a=True)
        assert torch.equal(cz, c[z])
    # a 2-D operand is shared by every problem (stride 0)
    c2 = torch.zeros(3, 96, 80, dtype=torch.float32, device="cuda")
    tg.gemm(a[1], b, c2, transpose_a=True)
    for z in range(3):
        cz = torch.zeros(96, 80, dtype=torch.float32, device="cuda")
        tg.gemm(a[1], b[z], cz, transpose_a=True)
        assert torch.equal(cz, c2[z])


def test_deterministic_runs():
    import torch
    import dense_gemm_tiled_amd as tg
    for splits in (None, 4):
        p = problem("bf16", "f32", 128, 384, 4096, True, False, batch=2, alpha=1.0, beta=0.0,
                    c_dist="zeros", dist="uniform")
        A, B, C = workloads.make_inputs(p)
        say("GPU case: determinism", splits)
        with env(TCGEMM_SPLITS=splits):
            r1 = run_library(p, A, B, C)
            r2 = run_library(p, A, B, C)
        assert np.array_equal(r1, r2)


def test_sync_entry_point_matches_async():
    import torch
    import dense_gemm_tiled_amd as tg
    p = problem("f16", "f16", 200, 300, 150, False, True)
    A, B, C = workloads.make_inputs(p)
    a, b = to_dev(A, "f16"), to_dev(B, "f16")
    c1, c2 = to_dev(C, "f16"), to_dev(C, "f16")
    say("GPU case: sync vs async")
    tg.gemm(a, b, c1, alpha=p.alpha, beta=p.beta, transpose_b=True)
    tg.gemm_sync(a, b, c2, alpha=p.alpha, beta=p.beta, transpose_b=True)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    assert tg.last_kernel().startswith("gemm_f16_nt_")


# ---------------------------------------------------------------- refusals on a GPU
def test_refusals_launch_nothing():
    import ctypes
    import torch
    import dense_gemm_tiled_amd as tg
    a = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    tg.gemm(a, b, c)
    torch.cuda.synchronize()
    n0 = tg.dispatch_count()
    with pytest.raises(tg.TcGemmError) as e:            # shape mismatch, caught in the binding
        tg.gemm(a, b[:, :32], c)
    with pytest.raises(tg.TcGemmError) as e:            # C overlaps A
        tg.gemm(a, b, a)
    assert e.value.status == 4
    big = torch.zeros(4096, dtype=torch.bfloat16, device="cuda")
    d = tg.make_desc(a, b, c)
    d.base.M = 1 << 20                                   # A would reach far past its allocation
    d.base.ldc = 64
    lib = tg.load_library()
    ctx, s = tg._torch_stream(0)
    cbig = torch.zeros((1 << 20) * 64 + 64, dtype=torch.bfloat16, device="cuda")
    st = lib.tc_gemm_batched_async(ctx, ctypes.byref(d), ctypes.c_void_p(big.data_ptr()),
                                   ctypes.c_void_p(b.data_ptr()), ctypes.c_void_p(cbig.data_ptr()), s)
    assert st == 1 and b"allocation" in lib.tc_last_error(ctx)
    with pytest.raises(tg.TcGemmError):                 # int8 K past the wrap bound
        ai = torch.zeros(2, 131072, dtype=torch.int8, device="cuda")
        bi = torch.zeros(131072, 2, dtype=torch.int8, device="cuda")
        tg.gemm(ai, bi, torch.zeros(2, 2, dtype=torch.int32, device="cuda"))
    assert tg.dispatch_count() == n0


# ---------------------------------------------------------------- the five workloads, full size
def full_case(name, **over):
    p = workloads.get(name)
    if over:
        p = p.with_(**over)
    A, B, C = workloads.make_inputs(p)
    say("GPU case: workload", name, over)
    got = run_library(p, A, B, C)
    return p, A, B, C, got


@pytest.mark.parametrize("M,N,K,a,c,batch,want", [
    # mid-size output, long K: 2 K slices on the 4-stage 128 x 128 tile
    (4096, 512, 4096, "bf16", "bf16", 1, "gemm_bf16_nn_128x128_dma4+splitk_reduce"),
    # mid-size output, short K: the 128 x 128 tile unsliced
    (1024, 1024, 1024, "i8", "i32", 1, "gemm_i8_nn_128x128_dma"),
    # whole tiles just past one round of 256 x 256: the round of 256 x 256
    # tiles, then the last tile column as a GEMM of its own (round split)
    (4096, 4352, 1024, "bf16", "f32", 1, "gemm_bf16_nn_256x256_dma|gemm_bf16_nn_128x128_dma4"),
    # a batch of problems smaller than a 256 x 256 tile
    (128, 128, 128, "f32", "f32", 256, "gemm_f32_nn_128x128"),
])
def test_planner_choices(M, N, K, a, c, batch, want):
    """The planner's own choices for mid-size, just-past-a-round and batched
    small outputs, whole results against the oracle (alpha = 0.5 and
    beta = 1 for floats)."""
    import dense_gemm_tiled_amd as tg
    check(problem(a, c, M, N, K, batch=batch), "planner %s" % want)
    assert tg.last_kernel() == want, tg.last_kernel()


def test_workload_sgemm_nn_256():
    p, A, B, C, got = full_case("sgemm_nn_256")
    compare(p, got, oracle_full(p, A, B, C), label=p.name)


def test_workload_bf16_nn_4096():
    import dense_gemm_tiled_amd as tg
    p, A, B, C, got = full_case("bf16_nn_4096")
    say("kernel:", tg.last_kernel())
    compare(p, got, oracle_full(p, A, B, C), label=p.name)


def test_workload_bf16_nn_4096_bias_gelu():
    """The headline shape with the fused epilogue, checked at 4096 sampled
    outputs (every row block and column block, the strip edges included)."""
    import dense_gemm_tiled_amd as tg
    p = workloads.get("bf16_nn_4096_bias_gelu")
    A, B, C = workloads.make_inputs(p)
    bias = workloads.make_bias(p)
    say("GPU case: workload", p.name)
    got = logical(p, run_library_epilogue(p, A, B, C, bias, "gelu_tanh"))
    assert tg.last_kernel() == "gemm_bf16_nn_256x256_dma", tg.last_kernel()
    pts = workloads.sample_points(p, 4096)
    r, v, T = oracle.gemm_epilogue_points(A, B, None, pts, bias=bias, act="gelu_tanh",
                                          M=p.M, N=p.N, K=p.K, a_dtype=p.a_dtype,
                                          c_dtype=p.c_dtype, alpha=p.alpha, beta=p.beta,
                                          want_abs=True)
    compare_points(p, got[pts[:, 0], pts[:, 1], pts[:, 2]], r, v, T, bias=bias,
                   act="gelu_tanh", pts=pts, label=p.name)


@pytest.mark.parametrize("name", ["f16_tn_4096", "f16_nt_4096"])
def test_workload_f16_backward_pair(name):
    """Both layouts with alpha = 0.5, beta = 1; the product term is small
    against beta*C, so a beta = 0 companion run on the same A and B pins it."""
    for beta in (1.0, 0.0):
        over = {} if beta == 1.0 else dict(beta=0.0, c_dist="zeros")
        p, A, B, C, got = full_case(name, **over)
        if p.transpose_b:   # oracle on the materialized B^T: the NN form of the same sums
            q = p.with_(transpose_b=False)
            ref = oracle_full(q, A, np.ascontiguousarray(B.T), C)
        else:
            ref = oracle_full(p, A, B, C)
        compare(p, got, ref, label="%s beta=%g" % (name, beta))


def test_workload_bf16_tn_splitk_b8():
    import dense_gemm_tiled_amd as tg
    p, A, B, C, got = full_case("bf16_tn_splitk_b8")
    assert tg.last_kernel().endswith("_128x128_dma4+splitk_reduce"), tg.last_kernel()
    compare(p, got, oracle_full(p, A, B, C), label=p.name)


def test_workload_i8_nn_ragged_bit_exact():
    import dense_gemm_tiled_amd as tg
    p, A, B, C, got = full_case("i8_nn_ragged")
    assert tg.last_kernel() == "pack_b+gemm_i8_nn_256x256_dma|gemm_i8_nn_thin", tg.last_kernel()
    ref = oracle_full(p, A, B, C)
    compare(p, got, ref, label=p.name)
    # the same with B read in place at its 4099-byte pitch (the strip then
    # gathers its own B^T)
    with env(TCGEMM_PACK_UNALIGNED=0):
        got = run_library(p, A, B, C)
    assert tg.last_kernel() == "gemm_i8_nn_256x256_dma|transpose_b+gemm_i8_nn_thin", \
        tg.last_kernel()
    compare(p, got, ref, label=p.name + " in place")
