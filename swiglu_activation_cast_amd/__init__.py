"""MI355X (gfx950) fused SwiGLU + MXFP8 cast.

The work happens in libmxfp8.so (hand-written HIP kernels behind a C ABI,
declared in include/mxfp8.h).  This package is its thin ctypes binding,
the in-tree build step, the byte model used for roofline reporting and the
seeded synthetic workloads.
"""
from ._binding import (
    BOTH,
    COLWISE,
    ROWWISE,
    Mxfp8Error,
    alloc_outputs,
    gated_act_mxfp8_backward,
    gated_act_mxfp8_forward,
    lib,
    mxfp8_quant_2d,
    mxfp8_quant_3d_colwise,
    mxfp8_swiglu_bwd,
    mxfp8_swiglu_bwd_bf16,
    mxfp8_swiglu_fwd,
    mxfp8_swiglu_fwd_bf16,
    status_str,
)

__all__ = [
    "BOTH",
    "COLWISE",
    "ROWWISE",
    "Mxfp8Error",
    "alloc_outputs",
    "gated_act_mxfp8_backward",
    "gated_act_mxfp8_forward",
    "lib",
    "mxfp8_quant_2d",
    "mxfp8_quant_3d_colwise",
    "mxfp8_swiglu_bwd",
    "mxfp8_swiglu_bwd_bf16",
    "mxfp8_swiglu_fwd",
    "mxfp8_swiglu_fwd_bf16",
    "status_str",
]
