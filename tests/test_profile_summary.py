"""Host logic of the rocprofv3 summarizer, on synthetic counter files.

The counter values are invented: a copy of the w13 tensor that FETCH_SIZE
counts at half its bytes (as the L2 counter does on MI355X) and WRITE_SIZE at
full, a bwd both-layout dispatch with 8 % excess writes, and the plain 2D and
3D colwise casts, which share one kernel name and differ only in volume.
"""
import csv
import os

import pytest

from swiglu_activation_cast_amd import _build, profile_summary as ps

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def _fake(tmp_path):
    calls, copy_bytes = ps.bench_calls("swiglu_131072x8192_w13", 64)
    alg = {label: (rd, wr) for _, label, rd, wr in calls}
    kib = 1024.0
    seq = [
        ("void mx::k_tiled<mx::OpBwd, true>(mx::Args)", alg["bwd_both"][0] / 2 / kib, alg["bwd_both"][1] * 1.08 / kib),
        ("void mx::k_tiled<mx::OpBwd, true>(mx::Args)", alg["bwd_both"][0] / 2 / kib, alg["bwd_both"][1] * 1.08 / kib),
        ("void mx::k_tiled<mx::OpQuant, false>(mx::Args)", alg["quant2d_col"][0] / 2 / kib, alg["quant2d_col"][1] / kib),
        ("void mx::k_tiled<mx::OpQuant, false>(mx::Args)", alg["quant3d_E64"][0] / 2 / kib, alg["quant3d_E64"][1] / kib),
        ("__amd_rocclr_copyBuffer", copy_bytes / 2 / kib, copy_bytes / kib),
        ("__amd_rocclr_copyBuffer", 64.0 / 2, 64.0),  # a small copy, ignored by the calibration
    ]
    _write(str(tmp_path / "f"), "FETCH_SIZE", [(k, f) for k, f, _ in seq])
    _write(str(tmp_path / "w"), "WRITE_SIZE", [(k, w) for k, _, w in seq])
    return alg


def test_traffic_summary(tmp_path):
    alg = _fake(tmp_path)
    out = str(tmp_path / "t.txt")
    ps.traffic(str(tmp_path / "f"), str(tmp_path / "w"), "swiglu_131072x8192_w13", 64, ["cmd"], out)
    text = open(out).read()
    fields = dict(l.split(":", 1) for l in text.splitlines() if l and not l.startswith("#") and ":" in l
                  and not l.startswith(("bwd_both ", "quant")))
    assert fields["kernel_source_hash"].strip() == _build.kernel_source_hash()
    rd, wr = alg["bwd_both"]
    assert int(fields["bwd_both_fetch_bytes_per_launch"]) == pytest.approx(rd, rel=1e-6)
    assert int(fields["bwd_both_write_bytes_per_launch"]) == pytest.approx(wr * 1.08, rel=1e-6)
    # both colwise-cast volumes are told apart and matched to their calls
    assert "quant2d_col" in text and "quant3d_E64" in text
    assert "write +8.00%" in text


def test_traffic_needs_the_copy(tmp_path):
    _write(str(tmp_path / "f"), "FETCH_SIZE", [("void mx::k_tiled<mx::OpBwd, true>(mx::Args)", 1.0)])
    _write(str(tmp_path / "w"), "WRITE_SIZE", [("void mx::k_tiled<mx::OpBwd, true>(mx::Args)", 1.0)])
    with pytest.raises(SystemExit):
        ps.traffic(str(tmp_path / "f"), str(tmp_path / "w"), "swiglu_131072x8192_w13", 64, [], str(tmp_path / "o"))


def test_counters_mean_and_derived_figures(tmp_path):
    """Per-dispatch means for the matching kernel only, and the derived
    matrix-core utilization and L2 hit rate (invented values: 8 XCDs of 1000
    active cycles each, 1024 SIMDs busy 250 cycles each -> 25 %; 90 hits, 10
    misses -> 90 %)."""
    k = "void mx::k_mx_gemm<false>(mx::GemmArgs)"
    other = "void mx::k_tiled<mx::OpBwd, true>(mx::Args)"
    rows = []
    for name, counter, vals in ((k, "SQ_VALU_MFMA_BUSY_CYCLES", (256000.0, 256000.0)), (k, "GRBM_GUI_ACTIVE", (8000.0, 8000.0)),
                                (k, "TCC_HIT_sum", (80.0, 100.0)), (k, "TCC_MISS_sum", (10.0, 10.0)),
                                (other, "TCC_HIT_sum", (1.0, 1.0))):
        rows += [(name, counter, v) for v in vals]
    d = tmp_path / "c"
    os.makedirs(d)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, counter, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})
    out = tmp_path / "o.txt"
    ps.counters([str(d)], "k_mx_gemm<false>", ["cmd"], str(out))
    text = out.read_text()
    assert "matrix-core utilization: 25.0%" in text
    assert "L2 hit rate: 90.0%" in text
    assert "TCC_HIT_sum                                    90    2" in text
    with pytest.raises(SystemExit):
        ps.counters([str(d)], "no_such_kernel", [], str(out))
