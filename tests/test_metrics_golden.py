"""The byte model behind the roofline, pinned to the pages' own tables.

"Add swiglu + MXFP8 fused CuTe DSL kernel" (Performance) and "[mxfp8 moe
training] update 3d quant colwise scaling kernel ..." (Performance) quote
achieved bandwidth next to kernel time.  Their product must equal the
algorithmic bytes (inputs read once, E4M3 data plus E8M0 scales written once
per emitted layout): that ties swiglu_activation_cast_amd.metrics to the
pages' accounting.  The pages print GB/s to 4-5 significant digits; rows
with tiny shapes (1.3 GB/s) are checked to their 2 digits.
"""
import os

import pytest

from swiglu_activation_cast_amd import metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUT = {"rowwise": 1, "colwise": 2, "both": 3}


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def test_fused_table_matches_byte_model():
    rows = _rows("p1_fused_perf.txt")
    assert len(rows) == 30
    for M, K, direction, scales, us, gbps in rows:
        M, K, us, gbps = int(M), int(K), float(us), float(gbps)
        fn = metrics.swiglu_fwd_bytes if direction == "forward" else metrics.swiglu_bwd_bytes
        nbytes = fn(M, K, LAYOUT[scales])
        implied = gbps * 1e9 * us * 1e-6
        tol = 0.05 if M < 4096 else 2e-3
        assert implied == pytest.approx(nbytes, rel=tol), (M, K, direction, scales)


def test_3d_table_matches_byte_model():
    rows = _rows("p3_3d_perf.txt")
    assert len(rows) == 6
    for E, N, K, us, gbps in rows:
        nbytes = metrics.quant_3d_bytes(int(E), int(N), int(K))
        assert float(gbps) * 1e9 * float(us) * 1e-6 == pytest.approx(nbytes, rel=2e-3), E


def test_layout_counts():
    M, N = 64, 128
    assert metrics.swiglu_fwd_bytes(M, N, 3) - metrics.swiglu_fwd_bytes(M, N, 1) == M * N + M * N // 32
    assert metrics.swiglu_bwd_bytes(M, N, 2) == 6 * M * N + 2 * M * N + 2 * M * N // 32
    assert metrics.quant_2d_bytes(M, N, 1) == 2 * M * N + M * N + M * N // 32
