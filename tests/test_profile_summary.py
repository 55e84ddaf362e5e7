"""Host logic of the rocprofv3 summarizer, on synthetic counter and trace files.

The values are invented: the streaming probe's 1 GiB copies, which
FETCH_SIZE counts at half their bytes and WRITE_SIZE at full; a bwd
both-layout dispatch with 8 % excess writes; and the plain 2D and 3D colwise
casts, which share one kernel name and differ only in their grids.
"""
import csv
import os

import pytest

from swiglu_activation_cast_amd import _build, profile_summary as ps

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
W = "swiglu_131072x8192_w13"


def _write(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (k, grid, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Grid_Size": grid * ps.THREADS,
                        "Counter_Name": counter, "Counter_Value": v})


def _calls():
    return {c.label: c for c in ps.bench_calls(W, 64)}


def _fake(tmp_path):
    c = _calls()
    kib = 1024.0
    bwd, q2, q3 = c["bwd_both"], c["quant2d_col"], c["quant3d_E64"]
    copy = "void (anonymous namespace)::k_stream<1, 1, 8>((anonymous namespace)::StreamArgs)"
    seq = [
        ("void mx::k_tiled<mx::OpBwd, true, false>(mx::Args)", bwd.grid, bwd.read / 2 / kib, bwd.write * 1.08 / kib),
        ("void mx::k_tiled<mx::OpBwd, true, false>(mx::Args)", bwd.grid, bwd.read / 2 / kib, bwd.write * 1.08 / kib),
        ("void mx::k_tiled<mx::OpQuant, false, false>(mx::Args)", q2.grid, q2.read / 2 / kib, q2.write / kib),
        ("void mx::k_tiled<mx::OpQuant, false, false>(mx::Args)", q3.grid, q3.read / 2 / kib, q3.write * 1.01 / kib),
        (copy, 4096, ps.COPY_BYTES / 2 / kib, ps.COPY_BYTES / kib),
        (copy, 2048, ps.COPY_BYTES / 2 / kib, ps.COPY_BYTES / kib),
        (copy, 8192, ps.COPY_BYTES / 2 / kib, ps.COPY_BYTES / kib),
    ]
    _write(str(tmp_path / "f"), "FETCH_SIZE", [(k, g, f) for k, g, f, _ in seq])
    _write(str(tmp_path / "w"), "WRITE_SIZE", [(k, g, w) for k, g, _, w in seq])
    return c


def test_calls_have_distinct_keys():
    """No two bench calls share a (kernel, grid) key, so every dispatch has
    one label."""
    keys = {}
    for c in ps.bench_calls(W, 64):
        key = (c.pattern, c.grid)
        assert key not in keys, (c.label, keys.get(key))
        keys[key] = c.label
    assert ps._match(ps.bench_calls(W, 64), "void mx::k_tiled<mx::OpQuant, false, false>(mx::Args)",
                     _calls()["quant3d_E64"].grid * ps.THREADS).label == "quant3d_E64"


def test_traffic_summary(tmp_path):
    c = _fake(tmp_path)
    out = str(tmp_path / "t.txt")
    ps.traffic(str(tmp_path / "f"), str(tmp_path / "w"), W, 64, ["cmd"], out)
    text = open(out).read()
    fields = dict(l.split(":", 1) for l in text.splitlines() if l and not l.startswith("#") and ":" in l
                  and not l.startswith(("bwd_both ", "quant")))
    assert fields["kernel_source_hash"].strip() == _build.kernel_source_hash()
    assert int(fields["bwd_both_fetch_bytes_per_launch"]) == pytest.approx(c["bwd_both"].read, rel=1e-6)
    assert int(fields["bwd_both_write_bytes_per_launch"]) == pytest.approx(c["bwd_both"].write * 1.08, rel=1e-6)
    lines = {l.split()[0]: l for l in text.splitlines() if l and not l.startswith("#") and ":" not in l.split()[0]}
    assert "write +8.00%" in lines["bwd_both"]
    assert "write +0.00%" in lines["quant2d_col"] and "write +1.00%" in lines["quant3d_E64"]


def test_traffic_needs_the_copy(tmp_path):
    _write(str(tmp_path / "f"), "FETCH_SIZE", [("void mx::k_tiled<mx::OpBwd, true, false>(mx::Args)", 65536, 1.0)])
    _write(str(tmp_path / "w"), "WRITE_SIZE", [("void mx::k_tiled<mx::OpBwd, true, false>(mx::Args)", 65536, 1.0)])
    with pytest.raises(SystemExit):
        ps.traffic(str(tmp_path / "f"), str(tmp_path / "w"), W, 64, [], str(tmp_path / "o"))


def test_stats_per_call(tmp_path):
    """The same kernel at two grids gives two rows with their own averages."""
    c = _calls()
    rows = []
    t = 1000
    for grid, dur in ((c["quant2d_col"].grid, 500_000), (c["quant3d_E64"].grid, 1_400_000),
                      (c["quant2d_col"].grid, 520_000), (c["quant3d_E64"].grid, 1_420_000), (77, 5_000)):
        rows.append({"Kernel_Name": "void mx::k_tiled<mx::OpQuant, false, false>(mx::Args)", "Grid_Size_X": grid * 256,
                     "Grid_Size_Y": 1, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 10
    p = tmp_path / "k.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    out = tmp_path / "s.txt"
    ps.stats(str(p), W, 64, ["cmd"], str(out))
    lines = {l.split()[0]: l.split() for l in out.read_text().splitlines() if l and not l.startswith("#")}
    assert float(lines["quant2d_col"][4]) == pytest.approx(510.0)
    assert float(lines["quant3d_E64"][4]) == pytest.approx(1410.0)
    gbps = (c["quant3d_E64"].read + c["quant3d_E64"].write) / 1410e-6 / 1e9
    assert float(lines["quant3d_E64"][8]) == pytest.approx(gbps, abs=0.1) and lines["quant3d_E64"][10] == "GB/s"
    assert "other kernels" in out.read_text()


def test_counters_mean_and_derived_figures(tmp_path):
    """Per-dispatch means for the matching kernel (and grid) only, and the
    derived matrix-core utilization and L2 hit rate (invented values: 8 XCDs
    of 1000 active cycles each, 1024 SIMDs busy 250 cycles each -> 25 %; 90
    hits, 10 misses -> 90 %)."""
    k = "void mx::k_mx_gemm<0, true>(mx::GemmArgs)"
    other = "void mx::k_tiled<mx::OpBwd, true, false>(mx::Args)"
    rows = []
    for name, grid, counter, vals in ((k, 2048, "SQ_VALU_MFMA_BUSY_CYCLES", (256000.0, 256000.0)),
                                      (k, 2048, "GRBM_GUI_ACTIVE", (8000.0, 8000.0)),
                                      (k, 2048, "TCC_HIT_sum", (80.0, 100.0)), (k, 2048, "TCC_MISS_sum", (10.0, 10.0)),
                                      (k, 99, "TCC_HIT_sum", (5.0,)),
                                      (other, 65536, "TCC_HIT_sum", (1.0, 1.0))):
        rows += [(name, grid, counter, v) for v in vals]
    d = tmp_path / "c"
    os.makedirs(d)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, counter, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": grid * 256, "Counter_Name": counter,
                        "Counter_Value": v})
    out = tmp_path / "o.txt"
    ps.counters([str(d)], "k_mx_gemm<0,", ["cmd"], str(out), grid=2048)
    text = out.read_text()
    assert "matrix-core utilization: 25.0%" in text
    assert "L2 hit rate: 90.0%" in text
    assert "TCC_HIT_sum                                    90    2" in text
    with pytest.raises(SystemExit):
        ps.counters([str(d)], "no_such_kernel", [], str(out))
