"""Short text summaries of rocprofv3 output for the bench workload.

Three subcommands, each writing one summary file:

  stats    <kernel_trace.csv>            from `rocprofv3 --kernel-trace`: the
                                         duration of every bench call, each
                                         call keyed by its kernel and grid
  traffic  <fetch_dir> <write_dir>       from two `rocprofv3 --pmc` runs, one
                                         with FETCH_SIZE, one with WRITE_SIZE
  counters <dir> [<dir> ...]             any `rocprofv3 --pmc` runs: the mean
                                         per dispatch of every counter for the
                                         kernels matching --kernel (and --grid)

The bench launches some kernels for several calls (the plain colwise cast
for the 2D cast and for the 64-expert 3D cast, the both-layout cast for each
unfused pipeline); their grids differ, so every summary keys a dispatch by
(kernel name, grid size) and labels it with the bench call of that shape.

Counter values are KiB per dispatch as the L2 reports them.  They are
calibrated on the streaming probe's copies (libmxstream.so, one input and one
output buffer of 1 GiB: every byte read once and written once, with the same
nontemporal accesses as the casts), so that "calibrated bytes" means bytes
moved to or from HBM as that copy counts them.
"""
from __future__ import annotations

import argparse
import collections
import csv
import os
import re
import statistics
from dataclasses import dataclass

from . import _build, metrics, synth

COPY_KERNEL = "k_stream<1, 1,"
COPY_BYTES = 1 << 30  # the probe's buffers (bench.py stream_ceilings)
THREADS = 256  # work-items per workgroup of every kernel the bench times
CUS = 256  # compute units of the MI355X the grids were sized for
STREAM_CONFIGS = metrics.STREAM_CONFIGS


@dataclass
class Call:
    pattern: str  # substring of the kernel name
    label: str
    read: int  # algorithmic bytes per launch
    write: int
    grid: int  # workgroups
    flops: int = 0  # matrix-core work per launch (the GEMM consumer), reported as TFLOP/s


def _tiles(M, N, E=1):
    return -(-M // 128) * -(-N // 128) * E


def bench_calls(workload: str, experts: int):
    """Every kernel call the bench times, with its algorithmic bytes and grid."""
    cfg = synth.WORKLOADS[workload]
    M, N = cfg["M"], cfg["N"]
    ex = synth.EXPERT_WORKLOADS[experts]
    E, N3, K3 = ex["E"], ex["N"], ex["K"]
    one = M * N + M * N // 32  # one cast layout of an [M, N] result
    rows = -(-M // 4)  # rowwise kernels: four rows per workgroup

    calls = []
    for lay, name in ((1, "row"), (2, "col"), (3, "both")):
        for op, fn, rd in (("Fwd", metrics.swiglu_fwd_bytes, 4 * M * N), ("Bwd", metrics.swiglu_bwd_bytes, 6 * M * N)):
            if lay == 1:
                pat, grid = f"k_rowwise<mx::Op{op},", rows
            else:
                pat, grid = f"k_tiled<mx::Op{op}, {'true' if lay == 3 else 'false'}, false>", _tiles(M, N)
            calls.append(Call(pat, f"{op.lower()}_{name}", rd, fn(M, N, lay) - rd, grid))
    for act in ("GeluTanh", "Gelu", "Relu"):
        label = {"GeluTanh": "gelu_tanh", "Gelu": "gelu", "Relu": "relu"}[act]
        for op, fn, rd in (("Fwd", metrics.swiglu_fwd_bytes, 4 * M * N), ("Bwd", metrics.swiglu_bwd_bytes, 6 * M * N)):
            calls.append(Call(f"k_tiled<mx::Gated{op}<mx::Act{act}>, true, false>", f"{label}_{op.lower()}_both", rd,
                              fn(M, N, 3) - rd, _tiles(M, N)))
    calls += [
        Call("k_rowwise<mx::OpQuant,", "quant2d_row", 2 * M * N, one, rows),
        Call("k_tiled<mx::OpQuant, false, false>", "quant2d_col", 2 * M * N, one, _tiles(M, N)),
        Call("k_tiled<mx::OpQuant, false, false>", f"quant3d_E{E}", 2 * E * N3 * K3,
             metrics.quant_3d_bytes(E, N3, K3) - 2 * E * N3 * K3, _tiles(N3, K3, E)),
        Call("k_tiled<mx::OpBwd, true, true>", "bwd_both_grouped_g8", 6 * M * N,
             metrics.swiglu_bwd_bytes(M, N, 3) - 6 * M * N, _tiles(M, N)),
        Call("k_tiled<mx::OpQuant, false, true>", "quant2d_col_grouped_g8", 2 * M * N, one, _tiles(M, N)),
        Call("k_values<mx::OpFwd,", "unfused_fwd_values", 4 * M * N, 2 * M * N, rows),
        Call("k_values<mx::OpBwd,", "unfused_bwd_values", 6 * M * N, 4 * M * N, rows),
        Call("k_tiled<mx::OpQuant, true, false>", "unfused_fwd_quant_both", 2 * M * N, 2 * one, _tiles(M, N)),
        Call("k_tiled<mx::OpQuant, true, false>", "unfused_bwd_quant_both", 4 * M * N, 4 * one, _tiles(M, 2 * N)),
    ]
    # the MX GEMM consumer (bytes: the operands and C once; it is bound by
    # the matrix cores, and the rows give its duration per call)
    for label, mode, gm, gn, gk, G in (("gemm_16384x8192x5120", 0, 16384, 8192, 5120, 0),
                                       ("grouped_gemm_16640x8192x5120_g4", 1, 16640, 8192, 5120, 4),
                                       ("dgrad_grouped_gemm_16640x5120x8192_g4", 1, 16640, 5120, 8192, 4),
                                       ("wgrad_grouped_gemm_k_8192x5120_t16640_g4", 2, 8192, 5120, 16640, 4)):
        tiles_m = -(-gm // 256) + (G if mode == 1 else 0)
        grid = tiles_m * -(-gn // 256) * (G if mode == 2 else 1)
        # the launch grid as mxfp8.hip sizes it: a short last round of T
        # tiles runs as 2 T half tiles (T <= CUS / 2) or 4 T quarter tiles
        # (T <= CUS / 4); the grouped form, whose tile count the host does
        # not know, has room for the larger of 3 (CUS / 4) and CUS / 2 extra
        tail = grid % CUS
        if mode == 1:
            grid += max(3 * (CUS // 4), CUS // 2)
        elif 0 < tail <= CUS // 4:
            grid += 3 * tail
        elif 0 < tail <= CUS // 2:
            grid += tail
        rd = gm * gk + gn * gk * (G if mode == 1 else 1)
        calls.append(Call(f"k_mx_gemm<{mode},", label, rd, 4 * gm * gn * (G if mode == 2 else 1), grid,
                          2 * gm * gn * gk))
    gib = COPY_BYTES
    for mix, (nr, nw) in (("4:1", (4, 1)), ("2:1", (2, 1)), ("3:1", (3, 1)), ("3:2", (3, 2)), ("1:1", (1, 1))):
        for u, grid in STREAM_CONFIGS:
            calls.append(Call(f"k_stream<{nr}, {nw}, {u}>", f"stream_{mix}_u{u}_g{grid}", nr * gib, nw * gib, grid))
    return calls


def _match(calls, kernel: str, grid_items: int):
    """The bench call a dispatch of `kernel` with `grid_items` work-items
    belongs to (None if it is not one of them)."""
    for c in calls:
        if c.pattern in kernel and c.grid * THREADS == grid_items:
            return c
    return None


def _short(kernel: str) -> str:
    """Kernel name without return type, parameters or spaces (one column)."""
    name = re.sub(r"^void |\(.*$", "", kernel.replace("(anonymous namespace)::", ""))
    return name.replace(", ", ",")


def _counter_rows(d: str):
    path = os.path.join(d, "run_counter_collection.csv")
    with open(path) as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter):
    """{dispatch id: (kernel name, grid work-items, value)} for one counter."""
    out = {}
    for r in rows:
        if r["Counter_Name"] == counter:
            out[int(r["Dispatch_Id"])] = (r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]))
    return out


def _calibration(samples):
    """Factor that turns counted bytes (KiB x 1024) into bytes moved, from
    the probe's copies of COPY_BYTES (every byte read once, written once)."""
    vals = [v for k, _, v in samples if COPY_KERNEL in k]
    if not vals:
        raise SystemExit(f"no {COPY_KERNEL} dispatch (the probe's copy) in the counter output")
    kib = statistics.median(vals)
    return COPY_BYTES / (kib * 1024.0), kib


def traffic(fetch_dir, write_dir, workload, experts, command, out, kernel="bwd_both"):
    calls = bench_calls(workload, experts)
    fetch = _per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(write_dir), "WRITE_SIZE")
    f_fac, f_kib = _calibration(fetch.values())
    w_fac, w_kib = _calibration(write.values())
    lines = [
        f"# rocprofv3 HBM counter summary of bench.py ({workload}, 3D experts E={experts})",
        "# commands (one counter per run):",
        *[f"#   {c}" for c in command],
        f"# calibration: the streaming probe's copies ({COPY_KERNEL}...>, {COPY_BYTES} bytes read and written)",
        f"#   FETCH_SIZE reads {f_kib:.0f} KiB -> factor {f_fac:.4f}; WRITE_SIZE reads {w_kib:.0f} KiB -> factor {w_fac:.4f}",
        "# columns: call, kernel, grid (workgroups), dispatches, FETCH_SIZE KiB (avg), WRITE_SIZE KiB (avg),",
        "#          calibrated HBM read / write GB, algorithmic read / write GB, excess",
        "",
    ]
    groups = collections.defaultdict(lambda: ([], []))
    for did, (k, grid, v) in fetch.items():
        c = _match(calls, k, grid)
        if c is not None and not c.label.startswith("stream_"):
            groups[c.label][0].append(v)
    for did, (k, grid, v) in write.items():
        c = _match(calls, k, grid)
        if c is not None and not c.label.startswith("stream_"):
            groups[c.label][1].append(v)
    machine = {}
    by_label = {c.label: c for c in calls}
    for label, (fv, wv) in sorted(groups.items(), key=lambda kv: -(by_label[kv[0]].read + by_label[kv[0]].write)):
        if not fv or not wv:
            continue
        c = by_label[label]
        f_avg, w_avg = sum(fv) / len(fv), sum(wv) / len(wv)
        hr, hw = f_avg * 1024 * f_fac, w_avg * 1024 * w_fac
        lines.append(f"{label:24s} {_short(c.pattern):34s} {c.grid:7d} {len(fv):4d} {f_avg:12.0f} {w_avg:12.0f}"
                     f"  hbm {hr / 1e9:.4f} / {hw / 1e9:.4f}  alg {c.read / 1e9:.4f} / {c.write / 1e9:.4f}"
                     f"  (read {100 * (hr / c.read - 1):+.2f}%, write {100 * (hw / c.write - 1):+.2f}%)")
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


def stats(csv_path, workload, experts, command, out, top_other=6):
    """Per-call kernel durations from a kernel_trace.csv: every dispatch is
    keyed by (kernel, grid) and labelled with its bench call; the algorithmic
    GB/s of the call follows from its average duration."""
    calls = bench_calls(workload, experts)
    with open(csv_path) as f:
        rows = list(csv.DictReader(f))
    durs = collections.defaultdict(list)
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
        durs[(r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1))].append(d)
    lines = [
        f"# rocprofv3 kernel-trace summary of bench.py ({workload}, 3D experts E={experts}), one row per bench call",
        *[f"# command: {c}" for c in command],
        f"# kernel source hash (bench.py kernel_source_hash): {_build.kernel_source_hash()}",
        "# columns: call, kernel, grid (workgroups), dispatches, avg / median / min / max us,",
        "#          algorithmic GB/s at the average and % of 8 TB/s (the GEMM consumer: TFLOP/s and %",
        "#          of the 5.0 PFLOP/s dense fp8 peak)",
        "",
    ]
    other = []
    labelled = []
    for (kernel, grid), d in durs.items():
        c = _match(calls, kernel, grid)
        if c is None:
            other.append((sum(d), kernel, grid, d))
            continue
        avg = sum(d) / len(d)
        if c.flops:
            rate, peak, unit = c.flops / (avg * 1e-6) / 1e12, metrics.MFMA_FP8_PEAK_TFLOPS, "TFLOP/s"
        else:
            rate, peak, unit = metrics.gbps(c.read + c.write, avg * 1e-6), metrics.HBM_PEAK_GBPS, "GB/s"
        labelled.append((c.label, _short(kernel), grid // THREADS, len(d), avg, statistics.median(d), min(d), max(d),
                         rate, 100 * rate / peak, unit))
    order = {c.label: i for i, c in enumerate(calls)}
    for row in sorted(labelled, key=lambda r: order[r[0]]):
        lines.append("%-24s %-34s %7d %4d %9.1f %9.1f %9.1f %9.1f %8.1f %6.2f%% %s" % row)
    if other:
        lines += ["", "# other kernels (not a bench call), by total time: dispatches, avg us, kernel"]
        for tot, kernel, grid, d in sorted(other, reverse=True)[:top_other]:
            lines.append("# %5d %9.1f  %s" % (len(d), tot / len(d), _short(kernel)[:90]))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def counters(dirs, pattern, command, out, simds=1024, xcds=8, grid=None):
    """Mean per dispatch of each counter over dispatches whose kernel name
    contains `pattern`, plus two derived figures when their counters are
    present: matrix-core utilization (MFMA busy cycles over active cycles
    times SIMDs; GRBM_GUI_ACTIVE is summed over the XCDs) and the L2 hit
    rate."""
    vals = collections.defaultdict(list)
    names = set()
    for d in dirs:
        for r in _counter_rows(d):
            if pattern in r["Kernel_Name"] and (grid is None or int(r["Grid_Size"]) == grid * THREADS):
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
                names.add(re.sub(r"^void |\(.*$", "", r["Kernel_Name"]))
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {pattern!r}")
    mean = {k: sum(v) / len(v) for k, v in vals.items()}
    lines = [
        f"# rocprofv3 counter summary: kernels matching {pattern!r} ({', '.join(sorted(names))})"
        + (f", grid {grid} workgroups" if grid else ""),
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
    if "TCC_EA0_WRREQ_sum" in mean and "TCC_EA0_WRREQ_64B_sum" in mean:
        n, n64 = mean["TCC_EA0_WRREQ_sum"], mean["TCC_EA0_WRREQ_64B_sum"]
        derived.append(f"L2->memory writes: {n64:.4g} 64-byte and {n - n64:.4g} 32-byte requests, "
                       f"{(64 * n64 + 32 * (n - n64)) / 1e9:.4f} GB")
    if "TCC_EA0_RDREQ_sum" in mean:
        derived.append(f"L2->memory reads: {mean['TCC_EA0_RDREQ_sum']:.4g} requests")
    cycles = mean.get("GRBM_GUI_ACTIVE", 0.0) / xcds  # per XCD (the counter is summed over XCDs)
    if cycles:
        derived.append(f"active cycles per XCD: {cycles:.4g}")
        for c, what in (("TCC_EA0_RDREQ_LEVEL_sum", "read"), ("TCC_EA0_WRREQ_LEVEL_sum", "write")):
            if c in mean:
                derived.append(f"L2->memory {what} requests in flight (mean over active cycles): {mean[c] / cycles:.0f}")
        if "SQ_ACTIVE_INST_VALU" in mean:
            derived.append(f"VALUBusy (rocprof's formula, SQ_ACTIVE_INST_VALU / CUs / active cycles): "
                           f"{100 * mean['SQ_ACTIVE_INST_VALU'] / (simds // 4) / cycles:.1f}%")
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
    c.add_argument("--grid", type=int, default=None, help="only dispatches of this many workgroups")
    a = p.parse_args(argv)
    if a.kind == "stats":
        stats(a.csv, a.workload, a.experts, a.command, a.out)
    elif a.kind == "traffic":
        traffic(a.fetch_dir, a.write_dir, a.workload, a.experts, a.command, a.out)
    else:
        counters(a.dirs, a.kernel, a.command, a.out, grid=a.grid)


if __name__ == "__main__":
    main()
