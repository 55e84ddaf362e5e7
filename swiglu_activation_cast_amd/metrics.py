"""Algorithmic byte counts of the casts (the roofline's numerator).

The pages quote achieved bandwidth as algorithmic bytes over kernel time:
inputs read once, E4M3 data (1 byte per element) and E8M0 scales (1 byte
per 32 elements) written once per emitted layout.  Their tables ("Add
swiglu + MXFP8 fused CuTe DSL kernel", Performance; "[mxfp8 moe training]
update 3d quant colwise scaling kernel ...", Performance) satisfy
GB/s x us = these bytes for every row, which the tests check.
"""
from __future__ import annotations

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, decimal GB/s
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix-core peak (no sparsity)

# (16-byte accesses in flight per stream and thread, workgroups) of the
# streaming-probe sweep that sets each read:write mix's ceiling
STREAM_CONFIGS = ((2, 16384), (2, 32768), (4, 8192), (4, 16384), (4, 32768), (8, 16384))


def _layouts(layout: int) -> int:
    return (layout & 1) + ((layout >> 1) & 1)


def swiglu_fwd_bytes(M: int, N: int, layout: int) -> int:
    """gate + up read (2 x 2 bytes per element), h cast once per layout."""
    return 4 * M * N + _layouts(layout) * (M * N + M * N // 32)


def swiglu_bwd_bytes(M: int, N: int, layout: int) -> int:
    """dh + gate + up read, [dgate | dup] (2N wide) cast once per layout."""
    return 6 * M * N + _layouts(layout) * (2 * M * N + 2 * M * N // 32)


def quant_2d_bytes(M: int, K: int, layout: int) -> int:
    return 2 * M * K + _layouts(layout) * (M * K + M * K // 32)


def quant_3d_bytes(E: int, N: int, K: int) -> int:
    return E * N * K * 2 + E * N * K + E * N * K // 32


def gbps(nbytes: float, seconds: float) -> float:
    return nbytes / seconds / 1e9
