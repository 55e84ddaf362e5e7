"""Short text summaries of rocprofv3 output for the bench workload.

Three subcommands, each writing one summary file:

  stats    <kernel_stats.csv>            from `rocprofv3 --kernel-trace --stats`
  traffic  <fetch_dir> <write_dir>       from two `rocprofv3 --pmc` runs, one
                                         with FETCH_SIZE, one with WRITE_SIZE
  counters <dir> [<dir> ...]             any `rocprofv3 --pmc` runs: the mean
                                         per dispatch of every counter for the
                                         kernels matching --kernel

Counter values are KiB per dispatch as the L2 reports them.  They are
calibrated on the bench's device copy of the w13 tensor (a copy kernel of
known size: every byte read once and written once), so that "calibrated
bytes" means bytes moved to or from HBM as that copy counts them.  Each
dispatch group (kernel name, read volume) is matched to the bench call it
comes from by its kernel and its calibrated read bytes, which equal the
call's algorithmic read bytes when nothing is re-read.
"""
from __future__ import annotations

import argparse
import collections
import csv
import os
import re

from . import _build, metrics, synth

COPY_KERNEL = "__amd_rocclr_copyBuffer"


def bench_calls(workload: str, experts: int):
    """(kernel pattern, label, algorithmic read bytes, algorithmic write bytes)
    for every kernel the bench launches."""
    cfg = synth.WORKLOADS[workload]
    M, N = cfg["M"], cfg["N"]
    ex = synth.EXPERT_WORKLOADS[experts]
    E, N3, K3 = ex["E"], ex["N"], ex["K"]
    one = M * N + M * N // 32  # one cast layout of an [M, N] result

    def split(total, read):
        return read, total - read

    calls = []
    for lay, name, rows_arg in ((1, "row", None), (2, "col", "false"), (3, "both", "true")):
        for op, fn, rd in (("Fwd", metrics.swiglu_fwd_bytes, 4 * M * N), ("Bwd", metrics.swiglu_bwd_bytes, 6 * M * N)):
            pat = f"k_rowwise<mx::Op{op}," if rows_arg is None else f"k_tiled<mx::Op{op}, {rows_arg}>"
            calls.append((pat, f"{op.lower()}_{name}", *split(fn(M, N, lay), rd)))
    calls += [
        ("k_rowwise<mx::OpQuant,", "quant2d_row", *split(metrics.quant_2d_bytes(M, N, 1), 2 * M * N)),
        ("k_tiled<mx::OpQuant, false>", "quant2d_col", *split(metrics.quant_2d_bytes(M, N, 2), 2 * M * N)),
        ("k_tiled<mx::OpQuant, false>", f"quant3d_E{E}", *split(metrics.quant_3d_bytes(E, N3, K3), 2 * E * N3 * K3)),
        ("k_values<mx::OpFwd,", "unfused_fwd_values", 4 * M * N, 2 * M * N),
        ("k_values<mx::OpBwd,", "unfused_bwd_values", 6 * M * N, 4 * M * N),
        ("k_tiled<mx::OpQuant, true>", "unfused_fwd_quant_both", 2 * M * N, 2 * one),
        ("k_tiled<mx::OpQuant, true>", "unfused_bwd_quant_both", 4 * M * N, 4 * one),
    ]
    copy_bytes = M * 2 * N * 2  # the w13 tensor [M, 2N] bf16
    return calls, copy_bytes


def _counter_rows(d: str):
    path = os.path.join(d, "run_counter_collection.csv")
    with open(path) as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter):
    """{dispatch id: (kernel name, value)} for one counter."""
    out = {}
    for r in rows:
        if r["Counter_Name"] == counter:
            out[r["Dispatch_Id"]] = (r["Kernel_Name"], float(r["Counter_Value"]))
    return out


def _groups(values):
    """Group (kernel, KiB) samples by kernel and by value within 1 %."""
    groups = collections.defaultdict(list)
    for kernel, v in values:
        for key in groups:
            if key[0] == kernel and abs(key[1] - v) <= 0.01 * max(key[1], 1.0):
                groups[key].append(v)
                break
        else:
            groups[(kernel, v)].append(v)
    return {(k, sum(v) / len(v)): len(v) for (k, _), v in groups.items()}


def _calibration(samples, copy_bytes):
    """Factor that turns counted bytes (KiB x 1024) into copied bytes, from the
    copy dispatches of copy_bytes."""
    vals = [v for k, v in samples if COPY_KERNEL in k]
    if not vals:
        raise SystemExit(f"no {COPY_KERNEL} dispatch in the counter output")
    top = max(vals)
    big = [v for v in vals if v >= 0.99 * top]
    kib = sum(big) / len(big)
    return copy_bytes / (kib * 1024.0), kib


def traffic(fetch_dir, write_dir, workload, experts, command, out, kernel="bwd_both"):
    calls, copy_bytes = bench_calls(workload, experts)
    fetch = _per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(write_dir), "WRITE_SIZE")
    f_fac, f_kib = _calibration(fetch.values(), copy_bytes)
    w_fac, w_kib = _calibration(write.values(), copy_bytes)
    lines = [
        f"# rocprofv3 HBM counter summary of bench.py ({workload}, 3D experts E={experts})",
        "# commands (one counter per run):",
        *[f"#   {c}" for c in command],
        f"# calibration: the bench's device copy of the w13 tensor ({COPY_KERNEL}, {copy_bytes} bytes read and written)",
        f"#   FETCH_SIZE reads {f_kib:.0f} KiB -> factor {f_fac:.4f}; WRITE_SIZE reads {w_kib:.0f} KiB -> factor {w_fac:.4f}",
        "# columns: call, kernel, dispatches, FETCH_SIZE KiB (avg), WRITE_SIZE KiB (avg),",
        "#          calibrated HBM read / write GB, algorithmic read / write GB, excess",
        "",
    ]
    fg = _groups(fetch.values())
    # WRITE samples of the dispatches in each FETCH group (same dispatch order
    # in both runs: the bench is deterministic)
    f_list = sorted(fetch.items(), key=lambda kv: int(kv[0]))
    w_list = sorted(write.items(), key=lambda kv: int(kv[0]))
    if [k for _, (k, _) in f_list] != [k for _, (k, _) in w_list]:
        raise SystemExit("the two counter runs launched different kernel sequences")
    machine = {}
    for (kname, f_avg), n in sorted(fg.items(), key=lambda kv: -kv[0][1]):
        match = [c for c in calls if c[0] in kname and abs(c[2] - f_avg * 1024 * f_fac) <= 0.01 * c[2]]
        if not match:
            continue
        pat, label, rd, wr = match[0]
        ws = [w_list[i][1][1] for i, (_, (k, v)) in enumerate(f_list)
              if k == kname and abs(v - f_avg) <= 0.01 * f_avg]
        w_avg = sum(ws) / len(ws)
        hr, hw = f_avg * 1024 * f_fac, w_avg * 1024 * w_fac
        short = re.sub(r"^void |\(.*$", "", kname)
        lines.append(f"{label:24s} {short:30s} {n:4d} {f_avg:12.0f} {w_avg:12.0f}  hbm {hr / 1e9:.4f} / {hw / 1e9:.4f}"
                     f"  alg {rd / 1e9:.4f} / {wr / 1e9:.4f}  (read {100 * (hr / rd - 1):+.2f}%, write {100 * (hw / wr - 1):+.2f}%)")
        machine[label] = (round(hr), round(hw))
    if kernel not in machine:
        raise SystemExit(f"no dispatch of the {kernel} call found")
    hr, hw = machine[kernel]
    lines += [
        "",
        "# machine-readable: calibrated HBM bytes per launch of the bench's dominant kernel,",
        "# valid for the kernel source with this hash (bench.py kernel_source_hash)",
        f"kernel_source_hash: {_build.kernel_source_hash()}",
        f"{kernel}_fetch_bytes_per_launch: {hr}",
        f"{kernel}_write_bytes_per_launch: {hw}",
        f"{kernel}_hbm_bytes_per_launch: {hr + hw}",
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def stats(csv_path, workload, experts, command, out, top=24):
    with open(csv_path) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [
        f"# rocprofv3 kernel-trace summary of bench.py ({workload}, 3D experts E={experts})",
        *[f"# command: {c}" for c in command],
        f"# kernel source hash (bench.py kernel_source_hash): {_build.kernel_source_hash()}",
        "# columns: calls, avg us, min us, max us, share of GPU time, kernel",
        "",
    ]
    for r in rows[:top]:
        lines.append("%6s %10.1f %10.1f %10.1f %6.2f%%  %s" % (
            r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["Percentage"]), r["Name"][:100]))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def counters(dirs, pattern, command, out, simds=1024, xcds=8):
    """Mean per dispatch of each counter over dispatches whose kernel name
    contains `pattern`, plus two derived figures when their counters are
    present: matrix-core utilization (MFMA busy cycles over active cycles
    times SIMDs; GRBM_GUI_ACTIVE is summed over the XCDs) and the L2 hit
    rate."""
    vals = collections.defaultdict(list)
    names = set()
    for d in dirs:
        for r in _counter_rows(d):
            if pattern in r["Kernel_Name"]:
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
                names.add(re.sub(r"^void |\(.*$", "", r["Kernel_Name"]))
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {pattern!r}")
    mean = {k: sum(v) / len(v) for k, v in vals.items()}
    lines = [
        f"# rocprofv3 counter summary: kernels matching {pattern!r} ({', '.join(sorted(names))})",
        *[f"# command: {c}" for c in command],
        f"# kernel source hash (bench.py kernel_source_hash): {_build.kernel_source_hash()}",
        "# columns: counter, mean per dispatch, dispatches",
        "",
    ]
    for k in sorted(mean):
        lines.append(f"{k:32s} {mean[k]:16.6g} {len(vals[k]):4d}")
    derived = []
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "GRBM_GUI_ACTIVE" in mean:
        util = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (mean["GRBM_GUI_ACTIVE"] / xcds * simds)
        derived.append(f"matrix-core utilization: {100 * util:.1f}% (MFMA busy cycles / (active cycles per XCD x {simds} SIMDs))")
    if "TCC_HIT_sum" in mean and "TCC_MISS_sum" in mean:
        hit = mean["TCC_HIT_sum"] / (mean["TCC_HIT_sum"] + mean["TCC_MISS_sum"])
        derived.append(f"L2 hit rate: {100 * hit:.1f}%")
    if derived:
        lines += ["", *[f"# {x}" for x in derived]]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--workload", default="swiglu_131072x8192_w13")
    p.add_argument("--experts", type=int, default=64)
    p.add_argument("--command", action="append", default=[], help="profiling command, recorded in the header")
    p.add_argument("-o", "--out", required=True)
    sub = p.add_subparsers(dest="kind", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", required=True, help="substring of the kernel name")
    a = p.parse_args(argv)
    if a.kind == "stats":
        stats(a.csv, a.workload, a.experts, a.command, a.out)
    elif a.kind == "traffic":
        traffic(a.fetch_dir, a.write_dir, a.workload, a.experts, a.command, a.out)
    else:
        counters(a.dirs, a.kernel, a.command, a.out)


if __name__ == "__main__":
    main()
