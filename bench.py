"""Benchmark of the blocked GEMM C = A·B on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one call of the library's ``gemm`` (host-side plan plus the kernel)
on the workload's synthetic, seeded inputs, already resident in HBM.  Prints
one JSON line: whole-job TFLOP/s over K timed steps, the dominant kernel's
achieved TFLOP/s against the dense MFMA peak (HIP events on the stream the
kernel runs on), and the CPU oracle timed on a bounded sample of the same
workload on this host ("cpu_baseline"; "cpu_configs" adds the oracle's wall
time on every GEMM workload, a row sample of the large ones, including the
decoding of the operands to fp64, and one-thread figures for scale).  The row-softmax workloads (the second, HBM-bound
operation) are timed the same way and reported under "softmax" in GB/s of
algorithmic traffic (X read once, Y written once) against the 8 TB/s HBM
peak, back to back (operands may partly stay in the 256 MB Infinity Cache)
and cold (each call after reading 1 GiB of other data).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of MFMA peak at fp16/bf16 4096³ and 8192³ on 1 MI355X"
# MI355X dense MFMA peaks (TFLOP/s): 256 CUs x 2.4 GHz x FLOP/clk/CU
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
# host threads for the CPU baseline: the host cores one GPU's job may use on a
# shared multi-GPU host (more cores are visible than are this job's to take)
HOST_THREADS_CAP = 16
# sources of the kernels whose traffic profiles/traffic.json records (the
# pipelined and wave-K MFMA GEMMs, the fp32 MFMA GEMM, the split-K reduce, the
# row softmax)
KERNEL_SOURCES = ["dense_tiled_matrix_amd/csrc/gemm_mfma16_dma.hip",
                  "dense_tiled_matrix_amd/csrc/gemm_mfma16_wavek.hip",
                  "dense_tiled_matrix_amd/csrc/mfma16_stage.h",
                  "dense_tiled_matrix_amd/csrc/gemm_mfma32.hip",
                  "dense_tiled_matrix_amd/csrc/gemm_splitk.hip",
                  "dense_tiled_matrix_amd/csrc/softmax.hip",
                  "dense_tiled_matrix_amd/csrc/device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and blank lines are left
    out, so an edit of the prose alone keeps recorded counters valid."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    w = rec.get("workloads", {}).get(workload)
    if not w or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return w.get("hbm_bytes_per_launch")


ELEM_BYTES = {"f16": 2, "bf16": 2, "f32": 4}


def algorithmic_bytes(p) -> int:
    """Bytes a GEMM must move at the least: A and B read once, C written once."""
    return (p.M * p.K + p.K * p.N) * ELEM_BYTES[p.in_dtype] + p.M * p.N * ELEM_BYTES[p.out_dtype]


def to_device(op, torch_dtype, torch):
    import numpy as np

    store = torch.from_numpy(op.bits.view(np.int32 if op.dtype == "f32" else np.int16))
    t = store.to("cuda:0").view(torch_dtype)
    return t.as_strided((op.rows, op.cols), (op.stride_r, op.stride_c), op.offset)


def warm_up(torch, fn, calls, min_seconds=0.0):
    """`calls` untimed calls of fn, then more until `min_seconds` of wall time
    have passed (a power-management transient follows a change of load: a
    sustained bf16 8192^3 run slows by up to 35% over its first few calls and
    settles after about 50, i.e. ~45 ms)."""
    t0 = time.perf_counter()
    for _ in range(calls):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def time_gemm(dtm, torch, a, b, c, steps, warmup, min_warm_s=0.0):
    """(wall ms per step, kernel ms per launch from HIP events) over `steps`."""
    stream = torch.cuda.current_stream()
    warm_up(torch, lambda: dtm.gemm(a, b, out=c, stream=stream), warmup, min_warm_s)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        dtm.gemm(a, b, out=c, stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return wall_ms, start.elapsed_time(end) / steps


def time_gemm_per_call(dtm, torch, a, b, c, steps):
    """(median, min) ms of single calls, each bracketed by its own events."""
    stream = torch.cuda.current_stream()
    pairs = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dtm.gemm(a, b, out=c, stream=stream)
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)
    return t[len(t) // 2], t[0]


def host_us_per_call(dtm, torch, calls=500):
    """Host time to validate, plan and enqueue one call through the Python
    binding (a 256^3 bf16 problem; the calls are queued, not waited for)."""
    a = torch.zeros(256, 256, dtype=torch.bfloat16, device="cuda:0")
    b = torch.zeros(256, 256, dtype=torch.bfloat16, device="cuda:0")
    c = torch.empty(256, 256, dtype=torch.bfloat16, device="cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(20):
        dtm.gemm(a, b, out=c, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        dtm.gemm(a, b, out=c, stream=stream)
    t = time.perf_counter() - t0
    torch.cuda.synchronize()
    return t / calls * 1e6


def _first_rows(p, R, absolute=False):
    """Problem p cut to the first R rows of A (and C); with `absolute`, both
    operands replaced by their elementwise magnitudes (sign bits cleared)."""
    import numpy as np

    import workloads as W

    def mag(bits, dtype):
        if not absolute:
            return bits
        mask = 0x7FFFFFFF if dtype == "f32" else 0x7FFF
        return (np.asarray(bits).astype(np.uint64) & mask).astype(bits.dtype)

    rows = W.Operand(p.A.bits, p.A.dtype, R, p.K, p.A.offset, p.A.stride_r, p.A.stride_c)
    a = W.dense(mag(np.ascontiguousarray(rows.logical_bits()), p.in_dtype), p.in_dtype)
    b = p.B
    if absolute:
        b = W.dense(mag(np.ascontiguousarray(p.B.logical_bits()), p.in_dtype), p.in_dtype)
    return W.Problem(R, p.N, p.K, a, b, p.in_dtype, p.out_dtype)


def _oracle_rows(p, target_s: float, threads: int, keep: list | None = None):
    """Time the oracle on the first R rows of problem p (all of them when the
    whole problem fits), R sized so the timed run takes about `target_s`
    seconds.  Returns (R, seconds); with `keep`, appends the timed run's
    fp64 result (R x N) to it."""
    import oracle

    def run_rows(R, final=False):
        sub = p if R == p.M else _first_rows(p, R)
        t0 = time.perf_counter()
        c64, _ = oracle.gemm_problem(sub, threads=threads)
        t = time.perf_counter() - t0
        if final and keep is not None:
            keep.append(c64)
        return t

    # two calibration points separate the fixed cost (decoding B) from the
    # per-row cost
    r1 = min(p.M, threads)
    t1 = run_rows(r1)
    if r1 == p.M or t1 * p.M / r1 < target_s:
        return p.M, run_rows(p.M, final=True)
    r4 = min(p.M, 4 * threads)
    t4 = run_rows(r4)
    per_row = max((t4 - t1) / max(r4 - r1, 1), 1e-7)
    R = int((target_s - t1) / per_row) + r1
    R = int(min(p.M, max(r1, threads * (R // threads))))
    return R, run_rows(R, final=True)


def host_threads() -> int:
    return max(1, min(HOST_THREADS_CAP, len(os.sched_getaffinity(0))))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _half_ulp(x, dtype: str):
    """Half the spacing of `dtype` at |x|: the most the final rounding of an
    exact value to that format adds."""
    import numpy as np

    mant, emin = {"f32": (23, -126), "f16": (10, -14), "bf16": (7, -126)}[dtype]
    ax = np.abs(x)
    e = np.maximum(np.floor(np.log2(np.where(ax > 0, ax, 1.0))), emin)
    return 0.5 * np.exp2(e - mant)


HIGHAM_ROWS = 64


def result_check(p, c64, c_bits, threads: int):
    """The GPU result's first R rows (R = rows of c64) against the oracle's
    fp64 values of the same rows (Chapter 13 section 13.3, Worked Example
    13.3.1: truth in fp64 from the same rounded inputs): max |error|, the
    per-element tolerance (fp32 accumulation over K; half an output ulp for a
    rounded output), how many elements exceed it, and on the first rows the
    ratio of the error to the textbook bound gamma_K (|A||B|)_ij of K fp32
    additions (u' = 2^-23 for the matrix cores' internal adds)."""
    import numpy as np

    import oracle

    R = c64.shape[0]
    od = p.out_dtype
    got = oracle.decode(c_bits, od)
    amax = float(np.abs(oracle.decode(p.A.logical_bits(), p.in_dtype)).max())
    bmax = float(np.abs(oracle.decode(p.B.logical_bits(), p.in_dtype)).max())
    tol = oracle.tolerance(p.in_dtype, p.K, amax, bmax)
    half = _half_ulp(c64, od) if od != "f32" else 0.0
    err = np.abs(got - c64)
    over = int(np.count_nonzero(err > tol + half))
    h = min(R, HIGHAM_ROWS)
    ab64, _ = oracle.gemm_problem(_first_rows(p, h, absolute=True), threads=threads)
    u = 2.0 ** -23
    gamma = p.K * u / (1 - p.K * u)
    bound = gamma * ab64 + (_half_ulp(c64[:h], od) if od != "f32" else 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        hr = np.where(err[:h] == 0, 0.0, err[:h] / bound)
    return {"rows": R, "of_rows": p.M, "max_abs_err": float(err.max()), "tol": tol,
            "max_err_over_tol": round(float(err.max()) / tol, 4) if tol > 0 else None,
            "elements_over_tol": over, "nan": bool(np.isnan(got).any()),
            "higham_ratio": round(float(hr.max()), 4), "higham_rows": h,
            "ok": over == 0 and not np.isnan(got).any()}


def cpu_baseline(p, target_s: float, gpu_rows=None):
    """The oracle (untuned, fp64, OpenMP over rows) on the first R rows of the
    workload, R sized so the timed run takes about `target_s` seconds.  With
    `gpu_rows` (a function R -> the GPU result's first R rows as output-dtype
    bits), the oracle's rows also check the GPU result ("check")."""
    threads = host_threads()
    keep = []
    R, t = _oracle_rows(p, target_s, threads, keep)
    flops = 2.0 * R * p.N * p.K
    out = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"first {R} of {p.M} rows of A times all of B ({p.K}x{p.N}), "
                     f"{t:.1f} s wall incl. decoding the operands to fp64; {threads} threads "
                     f"(the host-core share of one GPU; "
                     f"{len(os.sched_getaffinity(0))} visible)",
           "cpu_model": cpu_model()}
    if gpu_rows is not None:
        out["check"] = result_check(p, keep[0], gpu_rows(R), threads)
    return out


def cpu_configs(target_s: float):
    """The oracle on every GEMM workload once (a row sample where the whole
    problem would take longer than `target_s`), on the host-core share and,
    for the 257 x 129 x 193 and 4096^3 workloads, on one thread for scale."""
    import workloads as W

    out = []
    threads = host_threads()
    for name, nthreads in [("int8x8x8_f32", threads), ("ragged257x129x193_f32_At", threads),
                           ("ragged257x129x193_f32_At", 1), ("f16_4096_f32out", threads),
                           ("f16_4096_f32out", 1), ("f16_skinny512x512x65536_f32out", threads)]:
        p = W.workload(name)
        R, t = _oracle_rows(p, target_s, nthreads)
        out.append({"workload": name, "threads": nthreads, "rows": R, "of_rows": p.M,
                    "seconds": round(t, 4),
                    "gflop_s": round(2.0 * R * p.N * p.K / t / 1e9, 2)})
    return out


def sustained_clocks(torch, fn, seconds=0.8, batch=20):
    """Runs fn back to back for about `seconds` (batches of `batch` calls),
    reading the GPU's own metrics table through amdsmi after each batch:
    shader clock per XCD, memory clock, socket power and activity.  The
    table refreshes only every few hundred milliseconds, hence a sustained
    run of its own rather than a reading inside the short timed region.
    Returns None when amdsmi or the device is unavailable."""
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        prop = torch.cuda.get_device_properties(0)
        want = (prop.pci_domain_id, prop.pci_bus_id, prop.pci_device_id)
        handle = None
        for h in amdsmi.amdsmi_get_processor_handles():
            dom, bus, rest = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")  # dddd:bb:dd.f
            if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                handle = h
        if handle is None:
            return None
    except Exception:
        return None

    def num(x):
        return x if isinstance(x, (int, float)) else None

    samples = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
        except Exception:
            return None
        clks = [c for c in (m.get("current_gfxclks") or []) if num(c)]
        samples.append({"sclk": sum(clks) / len(clks) if clks else None,
                        "mclk": num(m.get("current_uclk")),
                        "power": num(m.get("current_socket_power")),
                        "activity": num(m.get("average_gfx_activity"))})
    # readings taken under load (the table lags the start of the run)
    busy = [r for r in samples if (r["activity"] or 0) >= 50] or samples

    def mean(key):
        xs = [r[key] for r in busy if r[key] is not None]
        return round(sum(xs) / len(xs), 1) if xs else None

    return {"readings_under_load": len(busy), "readings": len(samples),
            "sclk_mhz_mean_over_xcds": mean("sclk"), "mclk_mhz": mean("mclk"),
            "socket_power_w": mean("power"), "gfx_activity_pct": mean("activity")}


def time_cold(torch, fn, n, flush):
    """Median ms of one call of fn, each after reading `flush` (1 GiB, four
    times the Infinity Cache), so its operands come from HBM, not from L2 or
    the Infinity Cache; only the call is inside the events."""
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(n):
        flush.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return sorted(times)[len(times) // 2]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed calls before each timed run (the chip's power management "
                         "settles about 50 calls into a sustained bf16 8192^3 run)")
    ap.add_argument("--headline-warmup-s", type=float, default=1.0,
                    help="the headline workload is warmed for at least this many seconds of "
                         "back-to-back calls as well as --warmup calls, so that its timed "
                         "steps run after the power-management transient of a new load")
    ap.add_argument("--extra-warmup-s", type=float, default=0.3,
                    help="the workloads besides the headline are warmed for at least this "
                         "many seconds of back-to-back calls as well as --warmup calls")
    ap.add_argument("--workload", default="bf16_8192_bf16out")
    ap.add_argument("--secondary",
                    default="f16_4096_f32out,f16_8192_f32out,bf16_4096_bf16out,f32_4096_f32out",
                    help="comma-separated workloads also timed (not the headline)")
    ap.add_argument("--softmax", default=",".join([
        "softmax_f32_4096x4096", "softmax_bf16_8192x8192_masked", "softmax_f16_32768x1024",
        "softmax_f32_256x65536"]),
        help="comma-separated row-softmax workloads also timed (HBM-bound; 'none' to skip)")
    ap.add_argument("--skinny", default="f16_skinny512x512x65536_f32out",
                    help="long-K workload timed warm and cold (its inputs fit the 256 MB "
                         "Infinity Cache, so cold runs read 1 GiB between calls); "
                         "'none' to skip")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-config-seconds", type=float, default=2.0,
                    help="oracle seconds per workload for the cpu_configs entry (0: skip)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run 3 plain device copies of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this GEMM library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dense_tiled_matrix_amd as dtm
    import workloads as W

    # gemm() never allocates: the split-K plans (the long-K workload) keep
    # their partials in workspace reserved here, before anything is timed
    dtm.reserve_workspace()

    TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    clocks = None

    def measure(name, sustain=False, min_warm_s=0.0):
        nonlocal clocks
        p = W.workload(name)
        a = to_device(p.A, TD[p.in_dtype], torch)
        b = to_device(p.B, TD[p.in_dtype], torch)
        c = torch.empty(p.M, p.N, dtype=TD[p.out_dtype], device="cuda:0")
        plan = dtm.gemm_plan(a, b, out=c)
        wall_ms, kern_ms = time_gemm(dtm, torch, a, b, c, args.steps, args.warmup, min_warm_s)
        med_ms, min_ms = time_gemm_per_call(dtm, torch, a, b, c, args.steps)
        if sustain:  # after the timed calls: clocks and power under this load
            clocks = sustained_clocks(torch, lambda: dtm.gemm(a, b, out=c))
        flops = 2.0 * p.M * p.N * p.K
        return p, plan, wall_ms, kern_ms, flops, (med_ms, min_ms), c

    p, plan, wall_ms, kern_ms, flops, (med_ms, min_ms), c_head = measure(
        args.workload, sustain=True, min_warm_s=args.headline_warmup_s)
    peak = PEAK_TFLOPS[p.in_dtype]
    achieved = flops / (kern_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(flops / (wall_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "host_overhead_us_per_call": round((wall_ms - kern_ms) * 1e3, 2),
        "host_us_per_call": round(host_us_per_call(dtm, torch), 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.in_dtype,
        "data": "synthetic",
        "config": {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "in_dtype": p.in_dtype,
                   "out_dtype": p.out_dtype, "kernel": plan["kernel_name"],
                   "tile": [plan["block_m"], plan["block_n"], plan["block_k"]],
                   "threads": plan["threads"],
                   "grid": [plan["grid_m"], plan["grid_n"]]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(p.name)},
        "per_call_ms": {"median": round(med_ms, 4), "min": round(min_ms, 4)},
        "clocks": clocks,
    }
    sclk = (clocks or {}).get("sclk_mhz_mean_over_xcds")
    if sclk:
        # the dense peak scaled to the shader clock the part held under this
        # load (the published peak assumes 2.4 GHz)
        at_clk = peak * sclk / 2400.0
        clocks["peak_tflops_at_sclk"] = round(at_clk, 1)
        clocks["frac_at_sclk"] = round(achieved / at_clk, 4)
    secondary = []
    for name in [s for s in args.secondary.split(",") if s and s not in (args.workload, "none")]:
        q, qplan, qwall, qkern, qflops, (qmed, qmin), _ = measure(name,
                                                                min_warm_s=args.extra_warmup_s)
        qa = qflops / (qkern * 1e-3) / 1e12
        secondary.append({"workload": q.name, "tflops_wall": round(qflops / (qwall * 1e-3) / 1e12, 2),
                          "tflops_kernel": round(qa, 2), "frac": round(qa / PEAK_TFLOPS[q.in_dtype], 4),
                          "kernel_ms": round(qkern, 4), "kernel_ms_median": round(qmed, 4),
                          "tile": [qplan["block_m"], qplan["block_n"], qplan["block_k"]],
                          "threads": qplan["threads"], "traffic": measured_traffic(q.name),
                          "algorithmic_bytes": algorithmic_bytes(q)})
    if secondary:
        line["secondary"] = secondary
    # read (not written) between cold calls, so the caches hold clean lines
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
    if args.skinny and args.skinny != "none":
        q = W.workload(args.skinny)
        a = to_device(q.A, TD[q.in_dtype], torch)
        b = to_device(q.B, TD[q.in_dtype], torch)
        c = torch.empty(q.M, q.N, dtype=TD[q.out_dtype], device="cuda:0")
        qplan = dtm.gemm_plan(a, b, out=c)
        _, warm_ms = time_gemm(dtm, torch, a, b, c, args.steps, args.warmup, args.extra_warmup_s)
        stream = torch.cuda.current_stream()
        cold_ms = time_cold(torch, lambda: dtm.gemm(a, b, out=c, stream=stream),
                            min(args.steps, 20), flush)
        alg = algorithmic_bytes(q)
        qflops = 2.0 * q.M * q.N * q.K
        line["skinny"] = {"workload": q.name, "split_k": qplan["split_k"],
                          "warm_us": round(warm_ms * 1e3, 2), "cold_us": round(cold_ms * 1e3, 2),
                          "tflops_warm": round(qflops / (warm_ms * 1e-3) / 1e12, 1),
                          "tflops_cold": round(qflops / (cold_ms * 1e-3) / 1e12, 1),
                          "bytes": alg, "hbm_roofline_us": round(alg / (PEAK_HBM_GBS * 1e3), 2),
                          "cold_frac_of_hbm_roofline": round(alg / (PEAK_HBM_GBS * 1e3) /
                                                             (cold_ms * 1e3), 4)}
        del a, b, c
    softmax = []
    for name in [s for s in args.softmax.split(",") if s and s != "none"]:
        q = W.softmax_workload(name)
        x = to_device(q.X, TD[q.in_dtype], torch)
        y = torch.empty(q.M, q.N, dtype=TD[q.out_dtype], device="cuda:0")
        splan = dtm.row_softmax_plan(x, out=y)
        stream = torch.cuda.current_stream()
        warm_up(torch, lambda: dtm.row_softmax(x, out=y, stream=stream), args.warmup,
                args.extra_warmup_s)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            dtm.row_softmax(x, out=y, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        kern_ms = e0.elapsed_time(e1) / args.steps
        cold_ms = time_cold(torch, lambda: dtm.row_softmax(x, out=y, stream=stream),
                            min(args.steps, 20), flush)
        # context: a plain device copy of the same bytes (X read, Y written),
        # cold the same way -- what this traffic pattern reaches on this part
        ysame = torch.empty_like(x)
        copy_ms = time_cold(torch, lambda: ysame.copy_(x), min(args.steps, 20), flush)
        copy_bytes = 2 * q.M * q.N * x.element_size()
        # algorithmic bytes: X read once, Y written once
        alg = q.M * q.N * (x.element_size() + y.element_size())
        gbs = alg / (kern_ms * 1e-3) / 1e9
        gbs_cold = alg / (cold_ms * 1e-3) / 1e9
        softmax.append({"workload": q.name, "form": splan["form_name"],
                        "chunks": splan["chunks"], "kernel_us": round(kern_ms * 1e3, 2),
                        "bytes": alg, "gb_s": round(gbs, 1), "peak_gb_s": PEAK_HBM_GBS,
                        "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "kernel_us_cold": round(cold_ms * 1e3, 2),
                        "gb_s_cold": round(gbs_cold, 1),
                        "frac_cold": round(gbs_cold / PEAK_HBM_GBS, 4),
                        "copy_gb_s_cold": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1)})
        del x, y, ysame
    if softmax:
        line["softmax"] = softmax
    def gpu_rows(R):
        # the headline's output after its last timed call (every call writes
        # the same values), first R rows as raw output-dtype bits
        import numpy as np

        ibits = {2: torch.int16, 4: torch.int32}[c_head.element_size()]
        ubits = {2: np.uint16, 4: np.uint32}[c_head.element_size()]
        return c_head[:R].contiguous().view(ibits).cpu().numpy().view(ubits)

    line["cpu_baseline"] = None if args.no_cpu else cpu_baseline(p, args.cpu_seconds, gpu_rows)
    if not args.no_cpu and args.cpu_config_seconds > 0:
        line["cpu_configs"] = cpu_configs(args.cpu_config_seconds)
    print(json.dumps(line), flush=True)
    check = (line["cpu_baseline"] or {}).get("check")
    if check is not None and not check["ok"]:
        print(f"bench.py: the headline result is outside the oracle's tolerance: {check}",
              file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
