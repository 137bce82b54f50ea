"""Summaries of rocprofv3 CSV output for the GEMM kernels.

    python -m dense_tiled_matrix_amd.profiling stats  <kernel_stats.csv>
    python -m dense_tiled_matrix_amd.profiling trace  <kernel_trace.csv>
    python -m dense_tiled_matrix_amd.profiling pmc    <counter_collection.csv> [...]
    python -m dense_tiled_matrix_amd.profiling traffic --fetch F.csv --write W.csv \
        --copy-mib 512 --workload NAME --kernel-substr S --source-hash H
    python -m dense_tiled_matrix_amd.profiling resources [--match S] <file.s> [...]

``stats`` prints the per-kernel table of a ``--kernel-trace --stats`` run;
``trace`` prints the same from its kernel_trace.csv per kernel and launch
shape (grid and workgroup size), splitting a group whose durations fall in
two clusters (one kernel launched on two workloads of the same shape);
``pmc`` prints per-kernel means of the counters of ``--pmc`` runs (with the
shader clock derived from GRBM_GUI_ACTIVE, which counts shader-clock cycles
per XCD, over the dispatch's own duration); ``traffic`` turns a FETCH_SIZE
run and a WRITE_SIZE run into HBM bytes per launch, each scaled by what the
same counter reads for a plain device copy of known size run in the same
command; ``resources`` tabulates, from the AMD assembly the compiler writes
for this library's own sources (``hipcc ... --cuda-device-only -S``), each
kernel's VGPR, AGPR, SGPR, LDS and scratch (spill) use and occupancy.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import sys

XCDS = 8
SIMDS = 1024


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0][:90]


def stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.1f}% |")
    return "\n".join(out)


def _clusters(durs):
    """Sorted durations, split once at the widest ratio gap if it exceeds 1.5x."""
    d = sorted(durs)
    if len(d) < 2:
        return [d]
    i = max(range(1, len(d)), key=lambda k: d[k] / max(d[k - 1], 1))
    return [d[:i], d[i:]] if d[i] / max(d[i - 1], 1) > 1.5 else [d]


def trace(path: str) -> str:
    groups = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    total = sum(sum(v) for v in groups.values())
    rows = []
    for (name, grid, wg), durs in groups.items():
        for c in _clusters(durs):
            rows.append((sum(c), name, grid // wg, wg, c))
    out = ["| kernel | workgroups x threads | calls | average (us) | median (us) | min (us) | "
           "max (us) | share |", "|---|---|---|---|---|---|---|---|"]
    for tot, name, wgs, wg, c in sorted(rows, key=lambda x: -x[0]):
        out.append(f"| `{name}` | {wgs} x {wg} | {len(c)} | {tot / len(c) / 1e3:.1f} | "
                   f"{c[len(c) // 2] / 1e3:.1f} | {c[0] / 1e3:.1f} | {c[-1] / 1e3:.1f} | "
                   f"{100 * tot / total:.1f}% |")
    return "\n".join(out)


def _dispatches(paths):
    d = collections.OrderedDict()
    for path in paths:
        for r in csv.DictReader(open(path)):
            key = (path, r["Dispatch_Id"])
            rec = d.setdefault(key, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"])})
            rec[r["Counter_Name"]] = float(r["Counter_Value"])
            rec["dur_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return list(d.values())


def pmc(paths) -> str:
    # one kernel instantiation can serve several workloads: the grid size
    # tells their dispatches apart
    per = collections.OrderedDict()
    for rec in _dispatches(paths):
        per.setdefault((_short(rec["name"]), rec["grid"]), []).append(rec)
    out = []
    for (name, grid), recs in per.items():
        out.append(f"### `{name}`, grid {grid} threads ({len(recs)} dispatch records)")
        keys = sorted({k for r in recs for k in r if k not in ("name", "dur_ns", "grid")})
        for k in keys:
            vals = [r[k] for r in recs if k in r]
            out.append(f"- {k}: mean {sum(vals) / len(vals):.6g} (n={len(vals)})")
        clk = [r["GRBM_GUI_ACTIVE"] / XCDS / r["dur_ns"] for r in recs if "GRBM_GUI_ACTIVE" in r]
        if clk:
            out.append(f"- shader clock from GRBM_GUI_ACTIVE/XCD over duration: "
                       f"{sum(clk) / len(clk):.3f} GHz")
        busy = [r["SQ_VALU_MFMA_BUSY_CYCLES"] / (r["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
                for r in recs if "SQ_VALU_MFMA_BUSY_CYCLES" in r and "GRBM_GUI_ACTIVE" in r]
        if busy:
            out.append(f"- MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x "
                       f"{SIMDS} SIMDs)): {100 * sum(busy) / len(busy):.1f}%")
        conf = [r["SQ_LDS_BANK_CONFLICT"] / r["SQ_LDS_IDX_ACTIVE"] for r in recs
                if r.get("SQ_LDS_IDX_ACTIVE")]
        if conf:
            out.append(f"- LDS bank-conflict cycles / LDS active cycles: "
                       f"{100 * sum(conf) / len(conf):.2f}%")
        wait = [r["SQ_WAIT_ANY"] / r["SQ_WAVE_CYCLES"] for r in recs if r.get("SQ_WAVE_CYCLES")]
        if wait:
            out.append(f"- SQ_WAIT_ANY / SQ_WAVE_CYCLES: {100 * sum(wait) / len(wait):.1f}%")
        hit = [r["TCC_HIT_sum"] / (r["TCC_HIT_sum"] + r["TCC_MISS_sum"]) for r in recs
               if r.get("TCC_HIT_sum", 0) + r.get("TCC_MISS_sum", 0) > 0]
        if hit:
            out.append(f"- L2 hit rate TCC_HIT / (TCC_HIT + TCC_MISS): "
                       f"{100 * sum(hit) / len(hit):.1f}%")
        lat = [r["TCP_TCC_READ_REQ_LATENCY_sum"] / r["TCP_TCC_READ_REQ_sum"] for r in recs
               if r.get("TCP_TCC_READ_REQ_sum")]
        if lat:
            out.append(f"- mean L1-to-L2 read latency TCP_TCC_READ_REQ_LATENCY / "
                       f"TCP_TCC_READ_REQ: {sum(lat) / len(lat):.0f} cycles")
        ea = [r["TCC_EA0_RDREQ_LEVEL_sum"] / r["TCC_EA0_RDREQ_sum"] for r in recs
              if r.get("TCC_EA0_RDREQ_sum")]
        if ea:
            out.append(f"- mean L2-to-fabric read latency TCC_EA0_RDREQ_LEVEL / "
                       f"TCC_EA0_RDREQ: {sum(ea) / len(ea):.0f} cycles")
    return "\n".join(out)


def _mean_kib(path, substr, largest_only=False, grid=None):
    """Mean FETCH_SIZE or WRITE_SIZE of the dispatches whose name holds
    `substr` (and, given `grid`, whose grid has that many threads: one kernel
    instantiation can serve several workloads); with largest_only, of those
    within half of the largest value (the calibration copies, not smaller
    copies the same run makes)."""
    vals = [rec for rec in _dispatches([path]) if substr in rec["name"] and
            (grid is None or rec.get("grid") == grid)]
    key = "FETCH_SIZE" if any("FETCH_SIZE" in r for r in vals) else "WRITE_SIZE"
    xs = [r[key] for r in vals if key in r]
    if largest_only:
        xs = [x for x in xs if x >= 0.5 * max(xs)]
    return sum(xs) / len(xs), key


def traffic(fetch_csv, write_csv, copy_mib, specs, source_hash):
    """Memory-fabric bytes per launch for each (workload, kernel name
    substring, grid threads or None) in `specs`, scaled by the copy
    calibration.  One kernel instantiation can serve several workloads of a
    run; the grid tells their dispatches apart."""
    copy_fetch, _ = _mean_kib(fetch_csv, "copyBuffer", largest_only=True)
    copy_write, _ = _mean_kib(write_csv, "copyBuffer", largest_only=True)
    true_kib = copy_mib * 1024.0
    f_scale = true_kib / copy_fetch
    w_scale = true_kib / copy_write
    rec = {
        "kernel_source_hash": source_hash,
        "calibration": {"copy_mib": copy_mib, "fetch_size_kib_read": copy_fetch,
                        "write_size_kib_read": copy_write, "fetch_scale": f_scale,
                        "write_scale": w_scale},
        "workloads": {},
    }
    for workload, kernel_substr, grid in specs:
        k_fetch, _ = _mean_kib(fetch_csv, kernel_substr, grid=grid)
        k_write, _ = _mean_kib(write_csv, kernel_substr, grid=grid)
        rec["workloads"][workload] = {
            "kernel": kernel_substr, "grid_threads": grid,
            "fetch_size_kib": k_fetch, "write_size_kib": k_write,
            "hbm_bytes_per_launch": round((k_fetch * f_scale + k_write * w_scale) * 1024),
        }
    return rec


def _spec(text):
    """workload=kernel-substring[@grid-threads]"""
    workload, rest = text.split("=", 1)
    kernel, _, grid = rest.rpartition("@") if "@" in rest else (rest, "", "")
    return workload, kernel, int(grid) if grid else None


def _demangled(sym: str) -> str:
    try:
        import subprocess
        return subprocess.run(["c++filt", sym], capture_output=True, text=True).stdout.strip()
    except OSError:
        return sym


def resources(paths, match=None) -> str:
    """One row per kernel of the assembly files: the register, LDS and
    scratch figures the compiler reports after each kernel body."""
    import re

    rows = []
    for path in paths:
        text = open(path).read()
        for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel(.*?)(?=\.amdhsa_kernel |\Z)",
                             text, flags=re.S):
            sym, body, tail = m.group(1), m.group(2), m.group(3)

            def num(pattern, where):
                mm = re.search(pattern, where)
                return int(mm.group(1)) if mm else None

            name = _short(_demangled(sym))
            if match and match not in name:
                continue
            rows.append((name, num(r"; NumVgprs: (\d+)", tail), num(r"; NumAgprs: (\d+)", tail),
                         num(r"; TotalNumVgprs: (\d+)", tail), num(r"; TotalNumSgprs: (\d+)", tail),
                         num(r"\.amdhsa_group_segment_fixed_size (\d+)", body),
                         num(r"; ScratchSize: (\d+)", tail), num(r"; Occupancy: (\d+)", tail)))
    out = ["| kernel | VGPR | AGPR | total VGPR | SGPR | LDS (bytes) | scratch (bytes) | "
           "waves/SIMD |", "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| `" + r[0] + "` | " + " | ".join("-" if v is None else str(v) for v in r[1:]) +
                   " |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    tr = sub.add_parser("trace")
    tr.add_argument("csv")
    p = sub.add_parser("pmc")
    p.add_argument("csv", nargs="+")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=float, required=True)
    t.add_argument("--spec", type=_spec, action="append", required=True,
                   help="workload=kernel-name-substring[@grid-threads], repeatable")
    t.add_argument("--source-hash", required=True)
    rs = sub.add_parser("resources")
    rs.add_argument("asm", nargs="+")
    rs.add_argument("--match", default=None)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats(a.csv))
    elif a.cmd == "trace":
        print(trace(a.csv))
    elif a.cmd == "pmc":
        print(pmc(a.csv))
    elif a.cmd == "resources":
        print(resources(a.asm, a.match))
    else:
        print(json.dumps(traffic(a.fetch, a.write, a.copy_mib, a.spec, a.source_hash), indent=1))


if __name__ == "__main__":
    sys.exit(main())
