"""Throughput of the dense GEMM hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one GEMM call (all kernels it launches) over one set of synthetic
inputs already resident in HBM.  The default workload is the bf16 NN
4096 x 4096 x 4096 GEMM (fp32 accumulation, bf16 output, alpha 1, beta 0,
A and B drawn N(0,1)).  Several input/output sets (at least 512 MiB in
total) are used in rotation so that successive steps do not find their
operands in the 256 MB last-level cache.

Order of work: a clock/power sampler starts in a child process before any
GPU call; the GPU runs untimed steps for --settle seconds (the clocks of an
idle GPU take a fraction of a second to reach their loaded state), then the
W warm-up steps, then exactly K steps between two device synchronizations
(the whole-job `value` and `ms_per_step`).  A second, instrumented pass of K
steps follows: HIP events on the launch stream around every step and
around every step's main GEMM kernel give the per-step and per-kernel
p10/p50/p90 (the roofline uses the kernel median).  The CPU oracle is timed
last on a bounded sample of the same workload.

Prints one JSON line: whole-job TFLOP/s (or GB/s for the HBM-bound split-K
workload), the roofline position of the dominant kernel, the clocks, and the
CPU baseline.
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
ROCPROF_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--sets", type=int, default=0, help="input sets in rotation (0: >= 512 MiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up (clock ramp)")
    ap.add_argument("--clock-window", type=float, default=2.5,
                    help="seconds of untimed steps after the timing, while clocks are sampled")
    ap.add_argument("--table", action="store_true",
                    help="measure every workload and print a table (not the one-line contract)")
    ap.add_argument("--fused-compare", action="store_true",
                    help="fused bias+GELU against unfused passes, interleaved")
    ap.add_argument("--layout-table", action="store_true",
                    help="4096^3 over layouts, bf16/fp16 and beta 0/1, interleaved")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="bf16 NN over a spread of shapes, against torch.mm")
    ap.add_argument("--smi-sampler", type=float, default=0.0, help=argparse.SUPPRESS)
    return ap.parse_args()


def smi_sampler(interval: float) -> None:
    """Child-process mode: print one JSON line per sample of GPU 0's
    graphics clock (MHz) and socket power (W), with a wall-clock stamp, until
    terminated.  Reads the driver's metrics through amdsmi; does not touch
    HIP."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # noqa: BLE001
        print(json.dumps({"error": "amdsmi: %s" % e}), flush=True)
        return
    while True:
        rec = {"t": time.time()}
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            clk = m.get("current_gfxclks") or m.get("current_gfxclk")
            if isinstance(clk, (list, tuple)):
                clk = [c for c in clk if isinstance(c, (int, float)) and 0 < c < 65535]
                clk = sum(clk) / len(clk) if clk else None
            rec["sclk_mhz"] = clk if isinstance(clk, (int, float)) and 0 < clk < 65535 else None
            pw = m.get("current_socket_power")
            if not isinstance(pw, (int, float)) or not 0 < pw < 65535:
                pw = m.get("average_socket_power")
            rec["power_w"] = pw if isinstance(pw, (int, float)) and 0 < pw < 65535 else None
            act = m.get("average_gfx_activity")
            rec["activity"] = act if isinstance(act, (int, float)) and 0 <= act <= 100 else None
        except Exception as e:  # noqa: BLE001
            rec["error"] = str(e)
        print(json.dumps(rec), flush=True)
        time.sleep(interval)


def start_sampler():
    """Start the sampler child (before this process touches the GPU)."""
    import subprocess
    try:
        return subprocess.Popen([sys.executable, os.path.abspath(__file__), "--smi-sampler", "0.05"],
                                stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None


def stop_sampler(proc, windows):
    """Stop the sampler and summarize its samples that fall inside the
    (start, end) wall-clock windows: median, min and max of each field."""
    if proc is None:
        return None
    proc.terminate()
    try:
        out, _ = proc.communicate(timeout=10)
    except Exception:  # noqa: BLE001
        proc.kill()
        out, _ = proc.communicate()
    recs = []
    for line in out.splitlines():
        try:
            recs.append(json.loads(line))
        except ValueError:
            pass
    errs = [r["error"] for r in recs if "error" in r]
    inside = [r for r in recs if "t" in r and any(a <= r["t"] <= b for a, b in windows)]
    # the driver refreshes these metrics about once a second, so a sample
    # taken early in the window can still describe the idle time before it:
    # keep the samples whose activity reading says the GPU was busy
    busy = [r for r in inside if (r.get("activity") or 0) >= 90]
    res = {"samples": len(inside), "busy_samples": len(busy),
           "source": "amdsmi gpu metrics (refreshed about once a second), sampled every 50 ms "
                     "while steps run; clock and power of the samples with activity >= 90 %"}
    inside = busy
    for key in ("sclk_mhz", "power_w"):
        v = np.array([r[key] for r in inside if r.get(key) is not None], dtype=float)
        res[key] = ({"p50": float(np.median(v)), "min": float(v.min()), "max": float(v.max())}
                    if v.size else None)
    if errs and not inside:
        res["error"] = errs[0]
    return res


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


def is_hbm_bound(p) -> bool:
    return p.name == "bf16_tn_splitk_b8" or p.extra.get("bound") == "hbm"


def make_stepper(p, sets_arg=0, unfused=False):
    """Device input sets of workload p (at least 512 MiB in rotation unless
    sets_arg says otherwise) and step(i), one GEMM call on set i.  unfused:
    for a fused-epilogue workload, the plain GEMM followed by the same bias
    and activation as separate torch operations (the unfused baseline).
    Returns (step, sets, n_sets, host inputs)."""
    import torch
    import dense_gemm_tiled_amd as tg
    A, B, C = workloads.make_inputs(p)
    set_bytes = A.nbytes + B.nbytes + C.nbytes
    n_sets = sets_arg or max(1, int(np.ceil(512 * 2 ** 20 / set_bytes)))
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
        if unfused:
            tg.gemm(a, b, c, alpha=p.alpha, beta=p.beta, transpose_a=p.transpose_a,
                    transpose_b=p.transpose_b)
            y = c + bias if bias is not None else c
            if act == "gelu_tanh":
                y = torch.nn.functional.gelu(y, approximate="tanh")
            elif act == "relu":
                y = torch.relu(y)
            c.copy_(y)
        elif act is None and bias is None and col_scale is None:
            tg.gemm(a, b, c, alpha=p.alpha, beta=p.beta, transpose_a=p.transpose_a,
                    transpose_b=p.transpose_b)
        else:
            tg.gemm(a, b, c, alpha=p.alpha, beta=p.beta, transpose_a=p.transpose_a,
                    transpose_b=p.transpose_b, bias=bias, activation=act, col_scale=col_scale)
    return step, sets, n_sets, (A, B, C)


def settle(step, seconds):
    """Untimed steps (16 at a time) until `seconds` have passed; returns the
    number of steps and the time."""
    import torch
    n = 0
    t_s = time.perf_counter()
    while True:
        for _ in range(16):
            step(n)
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t_s >= seconds:
            return n, time.perf_counter() - t_s


def timed_steps(step, n, kernel_events=False):
    """n steps, each bracketed by HIP events on the launch stream (and, with
    kernel_events, the main GEMM kernel of each by events the library
    records); returns per-step and per-kernel microseconds."""
    import torch
    import dense_gemm_tiled_amd as tg
    stream = torch.cuda.current_stream()
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n if kernel_events else 0)]
    for a_ev, b_ev in kev:   # create the HIP events before handing them over
        a_ev.record(stream)
        b_ev.record(stream)
    torch.cuda.synchronize()
    sev[0].record(stream)
    for i in range(n):
        if kernel_events:
            tg.time_next_gemm(kev[i][0], kev[i][1])
        step(i)
        sev[i + 1].record(stream)
    torch.cuda.synchronize()
    step_us = np.array([sev[i].elapsed_time(sev[i + 1]) for i in range(n)]) * 1e3
    k_us = np.array([s.elapsed_time(e) for s, e in kev]) * 1e3
    return step_us, k_us


def block_times(step, nblocks, per, start=0):
    """nblocks blocks of `per` back-to-back steps, each block between two
    HIP events; returns the per-step microseconds of every block."""
    import torch
    blocks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(nblocks)]
    torch.cuda.synchronize()
    for bi, (s, e) in enumerate(blocks):
        s.record()
        for i in range(per):
            step(start + bi * per + i)
        e.record()
    torch.cuda.synchronize()
    return np.array([s.elapsed_time(e) * 1e3 / per for s, e in blocks])


TABLE = ["sgemm_nn_256", "bf16_nn_4096", "f16_tn_4096", "f16_nt_4096", "bf16_tn_splitk_b8",
         "i8_nn_ragged", "bf16_nn_4096_bias_gelu", "i8_nn_ragged_dequant_bf16",
         "bf16_gemv_nt_m4"]


def run_table(args):
    """Every measured workload: settle, 20 warm-up calls, then 20 blocks of
    back-to-back calls between event pairs (per-call p10/p50/p90 over the
    blocks), and 100 calls with events around each main kernel (its own
    duration).  One JSON line per workload, then a markdown table."""
    import torch
    import dense_gemm_tiled_amd as tg
    torch.cuda.set_device(0)
    tg.load_library()
    rows = []
    for name in TABLE:
        p = workloads.get(name)
        step, sets, n_sets, _ = make_stepper(p)
        settle(step, args.settle)
        for i in range(20):
            step(i)
        torch.cuda.synchronize()
        kernel = tg.last_kernel()
        # 20 blocks of 10 back-to-back calls, each block between two events
        # (sgemm 256^3: 20 blocks of 50 calls): per-call time of each block
        us = block_times(step, 20, 50 if name == "sgemm_nn_256" else 10)
        _, k_us = timed_steps(step, 100, kernel_events=True)
        med = float(np.median(us))
        rec = {"workload": name, "kernel": kernel, "call_us": pcts(us), "main_kernel_us": pcts(k_us),
               "input_sets": n_sets}
        if is_hbm_bound(p):
            rec["GB/s"] = p.algorithmic_bytes / med / 1e3
            rec["frac"] = rec["GB/s"] / PEAK_HBM_GBS
        else:
            rec["TFLOP/s"] = p.flops / med / 1e6
            rec["frac"] = rec["TFLOP/s"] / PEAK_TFLOPS[p.a_dtype]
        print(json.dumps(rec), flush=True)
        rows.append((p, rec))
        del sets, step
        torch.cuda.empty_cache()
    print("\n| workload | kernels | call us p50 (p10-p90) | main kernel us p50 (own launch) | throughput | % of peak |")
    print("|---|---|---|---|---|---|")
    for p, r in rows:
        c, k = r["call_us"], r["main_kernel_us"]
        thr = ("%.0f GB/s" % r["GB/s"]) if "GB/s" in r else (
            "%.1f %s" % (r["TFLOP/s"], "TOP/s" if p.a_dtype == "i8" else "TFLOP/s"))
        print("| %s | %s | %.1f (%.1f-%.1f) | %.1f | %s | %.1f %% |" % (
            p.name, r["kernel"], c["p50"], c["p10"], c["p90"], k["p50"], thr, 100 * r["frac"]))


def run_fused_compare(args):
    """The fused bias + GELU call against the plain GEMM followed by the same
    bias and activation as separate torch passes, and against the plain GEMM
    plus one copy of C (one read and one write of C: the least any separate
    elementwise pass moves), interleaved in one process: 10 rounds, each of
    2 blocks of 10 back-to-back calls of every variant in turn, each block
    between two events."""
    import torch
    import dense_gemm_tiled_amd as tg
    torch.cuda.set_device(0)
    tg.load_library()
    p = workloads.get("bf16_nn_4096_bias_gelu")
    fused, sets, n_sets, _ = make_stepper(p)
    unfused, sets2, _, _ = make_stepper(p, unfused=True)
    plain, sets3, _, _ = make_stepper(workloads.get("bf16_nn_4096"))
    src = torch.empty(p.M, p.N, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)

    def plain_copy(i):
        plain(i)
        dst.copy_(src)

    variants = {"fused": fused, "plain+torch_bias_gelu": unfused, "plain": plain,
                "plain+copy_of_C": plain_copy}
    for f in variants.values():
        settle(f, 0.2)
    res = {k: [] for k in variants}
    for _ in range(10):
        for k, f in variants.items():
            res[k].extend(block_times(f, 2, 10).tolist())
    out = {k: pcts(v) for k, v in res.items()}
    print(json.dumps({"fused_vs_unfused": out, "workload": p.name, "rounds": 10,
                      "blocks_per_round": 2, "calls_per_block": 10}), flush=True)


def run_layout_table(args):
    """4096^3 with alpha = 0.5 over the four layouts, bf16 and fp16 inputs
    (output in the input type) and beta 0 and 1, interleaved in one process:
    8 rounds, each a block of 20 back-to-back calls of every case in turn,
    each block between two events; four input sets in rotation (bell-shaped
    random A and B scaled by 0.02, C unscaled)."""
    import torch
    import dense_gemm_tiled_amd as tg
    torch.cuda.set_device(0)
    tg.load_library()
    n = 4096
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    types = {"bf16": torch.bfloat16, "f16": torch.float16}
    sets = {k: [tuple(torch.randn(n, n, device="cuda", generator=gen).mul_(sc).to(t)
                      for sc in (0.02, 0.02, 1.0)) for _ in range(4)]
            for k, t in types.items()}
    cases = [(dt, beta, ta, tb) for dt in types for beta in (0.0, 1.0)
             for ta in (False, True) for tb in (False, True)]

    def stepper(case):
        dt, beta, ta, tb = case

        def step(i):
            a, b, c = sets[dt][i % 4]
            tg.gemm(a, b, c, alpha=0.5, beta=beta, transpose_a=ta, transpose_b=tb)
        return step

    steps = {cs: stepper(cs) for cs in cases}
    for f in steps.values():
        settle(f, 0.1)
    res = {cs: [] for cs in cases}
    for _ in range(8):
        for cs, f in steps.items():
            res[cs].extend(block_times(f, 1, 20).tolist())
    print("| | NN | NT | TN | TT |")
    print("|---|---|---|---|---|")
    for dt in types:
        for beta in (0.0, 1.0):
            row = [np.median(res[(dt, beta, ta, tb)]) for ta in (False, True) for tb in (False, True)]
            print("| %s, beta = %g | %s |" % (dt, beta, " | ".join("%.1f" % v for v in row)), flush=True)


SWEEP = [(1024, 1024, 1024), (2048, 2048, 2048), (4096, 4096, 4096), (8192, 8192, 8192),
         (5120, 5120, 5120), (6144, 6144, 6144), (4096, 4352, 4096), (6144, 4096, 4096),
         (3072, 3072, 8192), (2048, 2048, 8192), (2048, 2048, 16384), (1536, 1536, 12288),
         (1024, 1024, 8192), (512, 512, 32768), (4096, 1024, 4096), (3072, 1024, 3072),
         (8192, 8192, 1024), (16384, 2048, 2048)]


def run_shape_sweep(args):
    """bf16 NN (alpha 1, beta 0) on each shape of SWEEP: this library and
    torch.mm on the same two input sets (bell-shaped random, unscaled), 10
    warm-up calls each, then 5 blocks of 10 calls of each between two
    events; p50 us per call and the planner's kernel chain."""
    import torch
    import dense_gemm_tiled_amd as tg
    torch.cuda.set_device(0)
    tg.load_library()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    print("| M×N×K | plan | this library | torch | ratio |")
    print("|---|---|---|---|---|")
    for M, N, K in SWEEP:
        sets = [(torch.randn(M, K, device="cuda", generator=gen).bfloat16(),
                 torch.randn(K, N, device="cuda", generator=gen).bfloat16(),
                 torch.empty(M, N, device="cuda").bfloat16()) for _ in range(2)]

        def ours(i):
            a, b, c = sets[i % 2]
            tg.gemm(a, b, c)

        def theirs(i):
            a, b, c = sets[i % 2]
            torch.mm(a, b, out=c)

        med = {}
        for name, f in (("ours", ours), ("torch", theirs)):
            for i in range(10):
                f(i)
            med[name] = float(np.median(block_times(f, 5, 10)))
            if name == "ours":
                plan = tg.last_kernel()
        print("| %dx%dx%d | %s | %.1f | %.1f | %.2f |" % (M, N, K, plan, med["ours"], med["torch"],
                                                         med["ours"] / med["torch"]), flush=True)
        del sets
        torch.cuda.empty_cache()


def pcts(x):
    x = np.asarray(x, dtype=float)
    return {"p10": float(np.percentile(x, 10)), "p50": float(np.percentile(x, 50)),
            "p90": float(np.percentile(x, 90)), "mean": float(x.mean())}


def main():
    args = parse()
    if args.smi_sampler > 0:
        smi_sampler(args.smi_sampler)
        return
    if args.table:
        run_table(args)
        return
    if args.fused_compare:
        run_fused_compare(args)
        return
    if args.layout_table:
        run_layout_table(args)
        return
    if args.shape_sweep:
        run_shape_sweep(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    sampler = start_sampler()
    windows = []
    import torch
    import dense_gemm_tiled_amd as tg

    p = workloads.get(args.workload)
    hbm_bound = is_hbm_bound(p)
    torch.cuda.set_device(0)
    tg.load_library()
    step, sets, n_sets, (A, B, C) = make_stepper(p, args.sets)

    # untimed steps until the clocks have ramped, then the W warm-up steps
    w0 = time.time()
    n_settle, settle_s = settle(step, args.settle)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    kernel = tg.last_kernel()

    # the timed region: exactly K steps between two synchronizations, with
    # one pair of HIP events on the launch stream around all of them (the
    # GPU time of the region)
    stream = torch.cuda.current_stream()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        step(i)
    r1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    ms_per_step = wall / args.steps * 1e3
    region_us = r0.elapsed_time(r1) * 1e3 / args.steps     # GPU time per step

    # instrumented pass: events around every step and (recorded by the
    # library on the launch stream) around every step's main GEMM kernel;
    # each event costs the stream a few microseconds, so these are the
    # launch's own durations with idle gaps between them
    step_us, k_us = timed_steps(step, args.steps, kernel_events=True)
    kdurs = k_us * 1e-6                 # seconds per main kernel
    # the clocks under load: sampled while steps run back to back
    w1 = time.time()
    settle(step, args.clock_window)
    windows.append((w1, time.time()))
    clocks = stop_sampler(sampler, windows)

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
    # the dominant kernel's average duration: the timed region's GPU time per
    # step when the step is that one kernel, else the median of its own
    # event-timed launches
    one_kernel = "+" not in kernel and "|" not in kernel
    kern_s = region_us * 1e-6 if one_kernel else float(np.median(kdurs))
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
    roof["kernel_us"] = kern_s * 1e6
    roof["achieved_from"] = ("timed region: HIP events around the K steps, GPU time per step "
                             "(the step is this one kernel)" if one_kernel else
                             "median of the main kernel's event-timed launches (instrumented pass)")
    roof["instrumented_launch_us"] = {k: v * 1e6 for k, v in pcts(kdurs).items()}
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
        "settle": {"steps": n_settle, "seconds": round(settle_s, 3)},
        "region_gpu_us_per_step": region_us,
        "step_us": {**pcts(step_us), "pass": "instrumented (events around every step)"},
        "clocks": clocks,
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
