"""Throughput of the dense GEMM hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one GEMM call (all kernels it launches) over one set of synthetic
inputs already resident in HBM.  The default workload is the bf16 NN
4096 x 4096 x 4096 GEMM (fp32 accumulation, bf16 output, alpha 1, beta 0,
A and B drawn N(0,1)).  Several input/output sets (at least 512 MiB in
total) are used in rotation so that successive steps do not find their
operands in the 256 MB last-level cache.

Prints one JSON line: whole-job TFLOP/s (or GB/s for the HBM-bound split-K
workload), the roofline position of the dominant kernel (the step's main
GEMM kernel; its average duration comes from HIP events that the library
records on the launch stream right around it in every eighth timed step),
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

# MI355X published peaks
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "i8": 5033.2}
PEAK_HBM_GBS = 8000.0
KEV_EVERY = 8   # timed steps per sampled kernel duration
ROCPROF_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the default warm-up (about a quarter of a second of GEMMs) brings the
    # GPU clocks to their steady state before the timed steps
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--sets", type=int, default=0, help="input sets in rotation (0: >= 512 MiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    return ap.parse_args()


def to_dev(arr, dtype):
    import torch
    if dtype in ("f16", "bf16"):
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.cuda()


def views(p, a_full, b_full, c_full):
    a_cols = p.M if p.transpose_a else p.K
    b_cols = p.K if p.transpose_b else p.N
    return a_full[..., :a_cols], b_full[..., :b_cols], c_full[..., :p.N]


def cpu_baseline(p: workloads.Problem, A, B, C, target_s: float):
    """Time the oracle (as it is) on the first rows of the same problem,
    scaled to the workload's unit."""
    import oracle
    es = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}[p.a_dtype]

    def run(rows):
        # rows [0, rows) of batch element 0: A's first rows (or columns when
        # transposed), all of B
        if p.transpose_a:
            A0 = A[0] if p.batch > 1 else A
            a_sub, lda = A0, p.LDA
        else:
            A0 = A[0] if p.batch > 1 else A
            a_sub, lda = A0[:rows], p.LDA
        B0 = B[0] if p.batch > 1 else B
        C0 = (C[0] if p.batch > 1 else C)[:rows]
        t0 = time.perf_counter()
        if p.a_dtype == "i8" and p.c_dtype != "i32":
            # int8 dequantized: the oracle's exact sums are the work (the
            # per-column scale is one multiply per output)
            oracle.gemm(a_sub, B0, None, M=rows, N=p.N, K=p.K, a_dtype="i8", c_dtype="i32",
                        transpose_a=p.transpose_a, transpose_b=p.transpose_b, lda=lda,
                        ldb=p.LDB, want_value=False)
        else:
            oracle.gemm(a_sub, B0, C0 if p.beta != 0 else None, M=rows, N=p.N, K=p.K,
                        a_dtype=p.a_dtype, c_dtype=p.c_dtype, transpose_a=p.transpose_a,
                        transpose_b=p.transpose_b, alpha=p.alpha, beta=p.beta, lda=lda,
                        ldb=p.LDB, ldc=p.LDC, C_like=C0, want_value=False)
        return time.perf_counter() - t0

    probe = min(8, p.M)
    t_probe = max(run(probe), 1e-4)
    rows = int(max(probe, min(p.M, probe * target_s / t_probe)))
    t = run(rows)
    if t < 0.5 * target_s and rows < p.M:
        # the small probe overestimates the cost per row: size again
        rows = int(min(p.M, rows * target_s / max(t, 1e-4)))
        t = run(rows)
    # a whole problem shorter than the target runs again until the target
    reps = 1
    while rows == p.M and t < 0.67 * target_s and reps < 100000:
        t += run(rows)
        reps += 1
    flops = 2.0 * rows * p.N * p.K * reps
    bytes_ = (rows * p.K + p.K * p.N) * es * reps
    return {"rows": rows, "reps": reps, "seconds": t, "flops": flops, "bytes": bytes_,
            "cores": oracle.num_threads()}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_gemm_tiled_amd as tg

    p = workloads.get(args.workload)
    hbm_bound = p.name == "bf16_tn_splitk_b8" or p.extra.get("bound") == "hbm"
    torch.cuda.set_device(0)
    tg.load_library()

    A, B, C = workloads.make_inputs(p)
    set_bytes = A.nbytes + B.nbytes + C.nbytes
    n_sets = args.sets or max(1, int(np.ceil(512 * 2 ** 20 / set_bytes)))
    sets = []
    for i in range(n_sets):
        a_full, b_full, c_full = to_dev(A, p.a_dtype), to_dev(B, p.a_dtype), to_dev(C, p.c_dtype)
        sets.append(views(p, a_full, b_full, c_full) + (c_full,))
    # beta != 0 reads C: every step restores nothing, so C drifts; that does
    # not change the work done.

    # fused-epilogue workloads: one bias vector (C's type), an activation, a
    # per-column dequantization scale
    act = p.extra.get("act")
    bias = to_dev(workloads.make_bias(p), p.c_dtype)[0] if p.extra.get("bias") else None
    col_scale = (torch.from_numpy(workloads.make_col_scale(p)[0]).cuda()
                 if p.extra.get("col_scale") else None)

    def step(i):
        a, b, c, _ = sets[i % n_sets]
        if act is None and bias is None and col_scale is None:
            tg.gemm(a, b, c, alpha=p.alpha, beta=p.beta, transpose_a=p.transpose_a,
                    transpose_b=p.transpose_b)
        else:
            tg.gemm(a, b, c, alpha=p.alpha, beta=p.beta, transpose_a=p.transpose_a,
                    transpose_b=p.transpose_b, bias=bias, activation=act, col_scale=col_scale)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    kernel = tg.last_kernel()

    stream = torch.cuda.current_stream()
    # Every KEV_EVERY-th timed step, the library records a pair of HIP events
    # on the launch stream right around the step's main GEMM kernel.  Each
    # timestamp costs the stream a few microseconds, so only a sample of the
    # steps carries them.
    kev_steps = list(range(0, args.steps, KEV_EVERY))
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in kev_steps]
    for a_ev, b_ev in kev:   # create the HIP events before handing them over
        a_ev.record(stream)
        b_ev.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    j = 0
    for i in range(args.steps):
        if i % KEV_EVERY == 0:
            tg.time_next_gemm(kev[j][0], kev[j][1])
            j += 1
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    kdurs = np.array([s.elapsed_time(e) for s, e in kev]) * 1e-3   # seconds per main kernel
    ms_per_step = wall / args.steps * 1e3

    flops = float(p.flops)
    alg_bytes = float(p.algorithmic_bytes)
    if hbm_bound:
        value = alg_bytes * args.steps / wall / 1e9
        unit = "GB/s"
        metric = ("GEMM GB/s and % of MI355X HBM bandwidth, bf16 TN split-K 128x384x16384 x8 (1 GPU)"
                  if p.name == "bf16_tn_splitk_b8" else "GEMM GB/s, %s (1 GPU)" % p.name)
    else:
        value = flops * args.steps / wall / 1e12
        unit = "TFLOP/s" if p.a_dtype != "i8" else "TOP/s"
        metric = ("GEMM TFLOP/s and % of MI355X MFMA peak, bf16 4096^3 NN (1 GPU)"
                  if p.name == workloads.HEADLINE else "GEMM throughput, %s (1 GPU)" % p.name)

    # The dominant kernel is the main GEMM kernel of a step; its algorithmic
    # work: 2*M*N*K over the output part it computes (the whole output unless
    # a thin edge strip is split off), or for the HBM-bound split-K workload
    # the bytes of A and B it reads once (partial sums are overhead).
    pdesc = tg.make_desc(*sets[0][:3], alpha=p.alpha, beta=p.beta,
                         transpose_a=p.transpose_a, transpose_b=p.transpose_b)
    if p.a_dtype == "i8" and p.c_dtype != "i32":
        # the plan of a dequantizing call is that of its int32 form (tiles,
        # packing and split do not depend on the output type)
        pdesc.base.c_dtype, pdesc.base.alpha, pdesc.base.beta = tg.I32, 1.0, 0.0
    info = tg.plan(pdesc)
    mm = min(p.M, info["tiles_m"] * info["tile_m"])
    nm = min(p.N, info["tiles_n"] * info["tile_n"])
    kern_s = float(np.mean(kdurs))
    es = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}[p.a_dtype]
    if hbm_bound:
        kbytes = float((p.M * p.K + p.K * p.N) * es * p.batch)
        roof = {"bound": "hbm", "achieved": kbytes / kern_s / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        kflops = 2.0 * mm * nm * p.K * p.batch
        roof = {"bound": "mfma", "achieved": kflops / kern_s / 1e12,
                "peak": PEAK_TFLOPS[p.a_dtype], "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = kernel
    roof["main_part"] = [mm, nm, p.K]
    roof["kernel_us_mean"] = kern_s * 1e6
    roof["kernel_us_median"] = float(np.median(kdurs)) * 1e6
    roof["kernel_samples"] = len(kdurs)
    roof["traffic"] = None
    if os.path.exists(ROCPROF_TRAFFIC_FILE):
        with open(ROCPROF_TRAFFIC_FILE) as f:
            tr = json.load(f).get(p.name)
        if tr and tr.get("kernel") == kernel and tr.get("source_hash") == tg_source_hash():
            roof["traffic"] = tr["bytes_per_launch"]

    line = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p.a_dtype, "data": "synthetic",
        "config": {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "batch": p.batch,
                   "layout": p.layout, "a_dtype": p.a_dtype, "c_dtype": p.c_dtype,
                   "alpha": p.alpha, "beta": p.beta, "input_sets": n_sets,
                   "parallelism": "none (1 GPU)",
                   **({"epilogue": dict(p.extra)} if p.extra else {})},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(p, A, B, C, args.cpu_seconds)
        if hbm_bound:
            cv, cu = cb["bytes"] / cb["seconds"] / 1e9, "GB/s"
        else:
            cv, cu = cb["flops"] / cb["seconds"] / 1e12, unit
        line["cpu_baseline"] = {
            "value": cv, "unit": cu, "cores": cb["cores"], "kind": "oracle",
            "sample": "rows 0..%d of batch element 0 of the same problem, %d time(s) (%.1f s, "
                      "fp64 accumulation)" % (cb["rows"] - 1, cb["reps"], cb["seconds"])}
    print(json.dumps(line), flush=True)


def tg_source_hash() -> str:
    """Hash of the device sources (every csrc file but the host planner), to
    tell whether stored counters still describe the kernels that run."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_tiled_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "tcgemm.cpp":
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
