"""ctypes binding of libmxfp8.so (argument marshalling only).

Every function here takes torch tensors that live on the GPU, checks
dtypes and devices, allocates the outputs with torch when the caller does
not pass them, and calls the C entry point of the same name on torch's
current stream.  All computation happens in the HIP kernels; there is no
CPU or PyTorch fallback: if the library is missing or a call fails, an
exception is raised.

Output tuple order follows the pages' API ("Add swiglu + MXFP8 fused CuTe
DSL kernel", API): (output_rowwise, output_colwise, scales_rowwise,
scales_colwise); a layout that was not asked for comes back as an empty
tensor.  E4M3 data and E8M0 scales are returned as uint8 tensors (use
``.view(torch.float8_e4m3fn)`` / ``.view(torch.float8_e8m0fnu)`` to
reinterpret).  The colwise data is the [W, M] row-major tensor, i.e. the
column-major storage of the [M, W] result (``q_col.t()`` is that view).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

ROWWISE = 1
COLWISE = 2
BOTH = 3

# gate activations of mxfp8_gated_fwd / mxfp8_gated_bwd (MXFP8_ACT_* in mxfp8.h)
ACT_SILU, ACT_GELU_TANH, ACT_GELU, ACT_RELU = 0, 1, 2, 3
ACTIVATIONS = {"silu": ACT_SILU, "gelu_tanh": ACT_GELU_TANH, "gelu": ACT_GELU, "relu": ACT_RELU}

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmxfp8.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_int = ctypes.c_int

_SIGNATURES = {
    "mxfp8_swiglu_fwd": [_p, _i64, _p, _i64, _i64, _i64, _int] + [_p, _i64] * 4 + [_p],
    "mxfp8_swiglu_bwd": [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _int] + [_p, _i64] * 4 + [_p],
    "mxfp8_gated_fwd": [_int, _p, _i64, _p, _i64, _i64, _i64, _int] + [_p, _i64] * 4 + [_p],
    "mxfp8_gated_bwd": [_int, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _int] + [_p, _i64] * 4 + [_p],
    "mxfp8_quant_2d": [_p, _i64, _i64, _i64, _int] + [_p, _i64] * 4 + [_p],
    "mxfp8_quant_3d_colwise": [_p, _i64, _i64, _i64, _i64, _i64, _p, _p, _p],
    "mxfp8_swiglu_fwd_bf16": [_p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p],
    "mxfp8_gemm": [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64, _p],
    "mxfp8_grouped_gemm": [_p, _i64, _p, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64,
                           _p],
    "mxfp8_swiglu_bwd_bf16": [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p],
    "mxfp8_gated_fwd_grouped": [_int, _p, _i64, _p, _i64, _i64, _i64, _int] + [_p, _i64] * 4 + [_p, _i64, _p],
    "mxfp8_gated_bwd_grouped": [_int, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _int] + [_p, _i64] * 4
                               + [_p, _i64, _p],
    "mxfp8_quant_2d_grouped": [_p, _i64, _i64, _i64, _int] + [_p, _i64] * 4 + [_p, _i64, _p],
    "mxfp8_grouped_gemm_k": [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64, _i64, _p],
}

_lib = None


class Mxfp8Error(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libmxfp8.so with argument types set (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m swiglu_activation_cast_amd._build` "
            "(or __graft_entry__.build()) first"
        )
    handle = ctypes.CDLL(LIB_PATH)
    for name, argtypes in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.argtypes = argtypes
        fn.restype = _int
    handle.mxfp8_status_str.argtypes = [_int]
    handle.mxfp8_status_str.restype = ctypes.c_char_p
    _lib = handle
    return handle


def status_str(status: int) -> str:
    return lib().mxfp8_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Mxfp8Error(fn, status, status_str(status))


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _bf16_matrix(t: torch.Tensor, name: str) -> Tuple[int, int]:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.data_ptr(), t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _layout(rowwise: bool, colwise: bool) -> int:
    layout = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    if layout == 0:
        raise ValueError("at least one of rowwise / colwise must be set")
    return layout


def alloc_outputs(M: int, W: int, layout: int, device, n_groups: int = 0) -> Tuple[torch.Tensor, ...]:
    """Empty (q_row, q_col, s_row, s_col) for an [M, W] result.  With token
    groups (n_groups > 0) s_col is [W, M/32 + 16 n_groups], the per-group
    padded layout (positions no block maps to are zero), in rows whose
    stride is rounded up to 16 bytes, so that the grouped GEMMs read every
    group's scales 16 bytes at a time."""
    empty = torch.empty(0, dtype=torch.uint8, device=device)
    q_row = torch.empty((M, W), dtype=torch.uint8, device=device) if layout & ROWWISE else empty
    s_row = torch.empty((M, W // 32), dtype=torch.uint8, device=device) if layout & ROWWISE else empty
    q_col = torch.empty((W, M), dtype=torch.uint8, device=device) if layout & COLWISE else empty
    if layout & COLWISE and n_groups:
        width = M // 32 + 16 * n_groups
        s_col = torch.zeros((W, -(-width // 16) * 16), dtype=torch.uint8, device=device)[:, :width]
    elif layout & COLWISE:
        s_col = torch.empty((W, M // 32), dtype=torch.uint8, device=device)
    else:
        s_col = empty
    return q_row, q_col, s_row, s_col


def _out_args(outs: Sequence[torch.Tensor], layout: int, M: int, W: int, device, n_groups: int = 0):
    """(pointer, leading dimension) pairs of the four outputs of an [M, W]
    result.  The C ABI cannot see buffer sizes, so every enabled output is
    checked here against its full extent: q_row [M, W], s_row [M, W/32],
    q_col [W, M], s_col [W, M/32] (with token groups [W, M/32 + 16
    n_groups], the per-group padded layout), uint8, on the inputs' device,
    unit column stride (a larger row stride is allowed)."""
    if len(outs) != 4:
        raise ValueError("out must be (q_row, q_col, s_row, s_col)")
    q_row, q_col, s_row, s_col = outs
    device = torch.device(device)

    def mat(t, on, name, rows, cols):
        if not on:
            return [None, 0]
        if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D uint8 tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
        if tuple(t.shape) != (rows, cols):
            raise ValueError(f"{name} must have shape {(rows, cols)}, got {tuple(t.shape)}")
        if cols > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must have unit column stride")
        return [t.data_ptr(), t.stride(0) if rows > 1 else max(t.stride(0), cols)]

    rows, cols = layout & ROWWISE, layout & COLWISE
    return (mat(q_row, rows, "q_row", M, W) + mat(s_row, rows, "s_row", M, W // 32)
            + mat(q_col, cols, "q_col", W, M) + mat(s_col, cols, "s_col", W, M // 32 + 16 * n_groups))


def mxfp8_swiglu_fwd(gate: torch.Tensor, up: torch.Tensor, *, rowwise: bool = True, colwise: bool = False,
                     out: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """MXFP8 cast of silu(gate) * up; returns (q_row, q_col, s_row, s_col)."""
    layout = _layout(rowwise, colwise)
    pg, ldg = _bf16_matrix(gate, "gate")
    pu, ldu = _bf16_matrix(up, "up")
    if gate.shape != up.shape or gate.device != up.device:
        raise ValueError("gate and up must have the same shape and device")
    M, N = gate.shape
    outs = out if out is not None else alloc_outputs(M, N, layout, gate.device)
    st = lib().mxfp8_swiglu_fwd(pg, ldg, pu, ldu, M, N, layout, *_out_args(outs, layout, M, N, gate.device),
                                _stream(gate.device, stream))
    _check("mxfp8_swiglu_fwd", st)
    return tuple(outs)


def mxfp8_swiglu_bwd(dh: torch.Tensor, gate: torch.Tensor, up: torch.Tensor, *, rowwise: bool = True,
                     colwise: bool = False, out: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """MXFP8 cast of [dgate | dup]; returns (q_row, q_col, s_row, s_col) of width 2N."""
    layout = _layout(rowwise, colwise)
    pd, ldd = _bf16_matrix(dh, "dh")
    pg, ldg = _bf16_matrix(gate, "gate")
    pu, ldu = _bf16_matrix(up, "up")
    if not (dh.shape == gate.shape == up.shape) or not (dh.device == gate.device == up.device):
        raise ValueError("dh, gate and up must have the same shape and device")
    M, N = gate.shape
    outs = out if out is not None else alloc_outputs(M, 2 * N, layout, gate.device)
    st = lib().mxfp8_swiglu_bwd(pd, ldd, pg, ldg, pu, ldu, M, N, layout, *_out_args(outs, layout, M, 2 * N, gate.device),
                                _stream(gate.device, stream))
    _check("mxfp8_swiglu_bwd", st)
    return tuple(outs)


def _act_code(act) -> int:
    """Activation name ("silu", "gelu_tanh", "gelu", "relu") or MXFP8_ACT_* code."""
    if isinstance(act, str):
        if act not in ACTIVATIONS:
            raise ValueError(f"unknown activation {act!r}; expected one of {sorted(ACTIVATIONS)}")
        return ACTIVATIONS[act]
    return int(act)


def mxfp8_gated_fwd(gate: torch.Tensor, up: torch.Tensor, *, act="silu", rowwise: bool = True,
                    colwise: bool = False, out: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """MXFP8 cast of act(gate) * up; returns (q_row, q_col, s_row, s_col)."""
    code = _act_code(act)
    layout = _layout(rowwise, colwise)
    pg, ldg = _bf16_matrix(gate, "gate")
    pu, ldu = _bf16_matrix(up, "up")
    if gate.shape != up.shape or gate.device != up.device:
        raise ValueError("gate and up must have the same shape and device")
    M, N = gate.shape
    outs = out if out is not None else alloc_outputs(M, N, layout, gate.device)
    st = lib().mxfp8_gated_fwd(code, pg, ldg, pu, ldu, M, N, layout, *_out_args(outs, layout, M, N, gate.device),
                               _stream(gate.device, stream))
    _check("mxfp8_gated_fwd", st)
    return tuple(outs)


def mxfp8_gated_bwd(dh: torch.Tensor, gate: torch.Tensor, up: torch.Tensor, *, act="silu", rowwise: bool = True,
                    colwise: bool = False, out: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """MXFP8 cast of [dgate | dup] of act(gate) * up; returns (q_row, q_col, s_row, s_col) of width 2N."""
    code = _act_code(act)
    layout = _layout(rowwise, colwise)
    pd, ldd = _bf16_matrix(dh, "dh")
    pg, ldg = _bf16_matrix(gate, "gate")
    pu, ldu = _bf16_matrix(up, "up")
    if not (dh.shape == gate.shape == up.shape) or not (dh.device == gate.device == up.device):
        raise ValueError("dh, gate and up must have the same shape and device")
    M, N = gate.shape
    outs = out if out is not None else alloc_outputs(M, 2 * N, layout, gate.device)
    st = lib().mxfp8_gated_bwd(code, pd, ldd, pg, ldg, pu, ldu, M, N, layout, *_out_args(outs, layout, M, 2 * N, gate.device),
                               _stream(gate.device, stream))
    _check("mxfp8_gated_bwd", st)
    return tuple(outs)


def mxfp8_quant_2d(x: torch.Tensor, *, rowwise: bool = True, colwise: bool = False,
                   out: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """Plain MXFP8 cast of a bf16 [M, K] matrix; returns (q_row, q_col, s_row, s_col)."""
    layout = _layout(rowwise, colwise)
    px, ldx = _bf16_matrix(x, "x")
    M, K = x.shape
    outs = out if out is not None else alloc_outputs(M, K, layout, x.device)
    st = lib().mxfp8_quant_2d(px, ldx, M, K, layout, *_out_args(outs, layout, M, K, x.device), _stream(x.device, stream))
    _check("mxfp8_quant_2d", st)
    return tuple(outs)


def mxfp8_quant_3d_colwise(w: torch.Tensor, *, out: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """3D per-expert colwise cast of bf16 w (E, N, K); returns (q (E, K, N), s (E, K, N/32))."""
    if w.dtype != torch.bfloat16 or not w.is_cuda or w.dim() != 3:
        raise ValueError("w must be a 3-D bfloat16 GPU tensor")
    E, N, K = w.shape
    if K > 1 and w.stride(2) != 1:
        raise ValueError("w must have unit stride along K")
    if out is None:
        q = torch.empty((E, K, N), dtype=torch.uint8, device=w.device)
        s = torch.empty((E, K, N // 32), dtype=torch.uint8, device=w.device)
    else:
        q, s = out
        if not (q.is_contiguous() and s.is_contiguous() and q.dtype == s.dtype == torch.uint8):
            raise ValueError("3D outputs must be contiguous uint8 tensors")
        if q.numel() != E * K * N or s.numel() != E * K * (N // 32):
            raise ValueError("3D output sizes do not match (E, K, N) and (E, K, N/32)")
    ld_w = w.stride(1) if N > 1 else K
    stride_e = w.stride(0) if E > 1 else N * ld_w
    st = lib().mxfp8_quant_3d_colwise(w.data_ptr(), E, N, K, stride_e, ld_w, q.data_ptr(), s.data_ptr(),
                                      _stream(w.device, stream))
    _check("mxfp8_quant_3d_colwise", st)
    return q, s


def _bf16_out(t, M, W, device):
    if t is None:
        return torch.empty((M, W), dtype=torch.bfloat16, device=device)
    if t.dtype != torch.bfloat16 or tuple(t.shape) != (M, W) or (W > 1 and t.stride(1) != 1):
        raise ValueError(f"output must be a bf16 [{M}, {W}] tensor with unit column stride")
    return t


def mxfp8_swiglu_fwd_bf16(gate: torch.Tensor, up: torch.Tensor, *, out: Optional[torch.Tensor] = None, stream=None):
    """h = bf16(bf16(silu(gate)) * up) written as bf16 (the unfused pipeline's activation)."""
    pg, ldg = _bf16_matrix(gate, "gate")
    pu, ldu = _bf16_matrix(up, "up")
    if gate.shape != up.shape or gate.device != up.device:
        raise ValueError("gate and up must have the same shape and device")
    M, N = gate.shape
    h = _bf16_out(out, M, N, gate.device)
    st = lib().mxfp8_swiglu_fwd_bf16(pg, ldg, pu, ldu, M, N, h.data_ptr(), h.stride(0) if M > 1 else max(N, 8),
                                     _stream(gate.device, stream))
    _check("mxfp8_swiglu_fwd_bf16", st)
    return h


def mxfp8_swiglu_bwd_bf16(dh: torch.Tensor, gate: torch.Tensor, up: torch.Tensor, *,
                          out: Optional[torch.Tensor] = None, stream=None):
    """[dgate | dup] of silu(gate) * up for upstream dh, written as bf16 [M, 2N]."""
    pd, ldd = _bf16_matrix(dh, "dh")
    pg, ldg = _bf16_matrix(gate, "gate")
    pu, ldu = _bf16_matrix(up, "up")
    if not (dh.shape == gate.shape == up.shape) or not (dh.device == gate.device == up.device):
        raise ValueError("dh, gate and up must have the same shape and device")
    M, N = gate.shape
    y = _bf16_out(out, M, 2 * N, gate.device)
    st = lib().mxfp8_swiglu_bwd_bf16(pd, ldd, pg, ldg, pu, ldu, M, N, y.data_ptr(),
                                     y.stride(0) if M > 1 else max(2 * N, 8), _stream(gate.device, stream))
    _check("mxfp8_swiglu_bwd_bf16", st)
    return y


def gated_act_mxfp8_forward(gated_input: torch.Tensor, *, rowwise: bool = True, colwise: bool = False,
                            activation="silu", out=None, stream=None):
    """Forward on the packed [M, 2N] = [gate | up] projection (the pages' API name)."""
    N = gated_input.shape[1] // 2
    return mxfp8_gated_fwd(gated_input[:, :N], gated_input[:, N:], act=activation, rowwise=rowwise,
                           colwise=colwise, out=out, stream=stream)


def gated_act_mxfp8_backward(grad_h: torch.Tensor, gated_input: torch.Tensor, *, rowwise: bool = True,
                             colwise: bool = False, activation="silu", out=None, stream=None):
    """Backward on the packed [M, 2N] = [gate | up] projection; outputs [dgate | dup]."""
    N = gated_input.shape[1] // 2
    return mxfp8_gated_bwd(grad_h, gated_input[:, :N], gated_input[:, N:], act=activation, rowwise=rowwise,
                           colwise=colwise, out=out, stream=stream)


def _u8_matrix(t: torch.Tensor, name: str) -> Tuple[int, int]:
    if t.dtype != torch.uint8 or not t.is_cuda or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D uint8 GPU tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.data_ptr(), t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def mxfp8_gemm(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor, *,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """C = A B^T (fp32) of MXFP8 operands a [M, K], b [N, K] (uint8 E4M3 codes)
    with E8M0 scales sa [M, K/32], sb [N, K/32]; K-contiguous, as the casts
    emit them."""
    pa, lda = _u8_matrix(a, "a")
    pb, ldb = _u8_matrix(b, "b")
    psa, ld_sa = _u8_matrix(sa, "sa")
    psb, ld_sb = _u8_matrix(sb, "sb")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or tuple(sa.shape) != (M, K // 32) or tuple(sb.shape) != (N, K // 32):
        raise ValueError("operand shapes do not match a [M, K], sa [M, K/32], b [N, K], sb [N, K/32]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError(f"out must be a float32 [{M}, {N}] tensor with unit column stride")
    ldc = out.stride(0) if M > 1 else max(N, 1)
    st = lib().mxfp8_gemm(pa, lda, psa, ld_sa, pb, ldb, psb, ld_sb, M, N, K, out.data_ptr(), ldc,
                          _stream(a.device, stream))
    _check("mxfp8_gemm", st)
    return out


def mxfp8_grouped_gemm(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                       offsets: torch.Tensor, *, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Grouped C = A B_g^T (fp32): rows of a [M, K] split into groups by the
    cumulative end offsets (int32 GPU tensor [G]); group g against b[g]
    [N, K] with scales sb[g] [N, K/32].  Rows past the last offset are left
    as they are in `out` (uninitialized when `out` is None)."""
    pa, lda = _u8_matrix(a, "a")
    psa, ld_sa = _u8_matrix(sa, "sa")
    if b.dtype != torch.uint8 or not b.is_cuda or b.dim() != 3 or sb.dtype != torch.uint8 or sb.dim() != 3:
        raise ValueError("b and sb must be 3-D uint8 GPU tensors [G, N, K] and [G, N, K/32]")
    if b.stride(2) != 1 or sb.stride(2) != 1:
        raise ValueError("b and sb must have unit stride along K")
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.dim() != 1:
        raise ValueError("offsets must be a 1-D int32 GPU tensor")
    M, K = a.shape
    G, N, _ = b.shape
    if tuple(b.shape) != (G, N, K) or tuple(sb.shape) != (G, N, K // 32) or tuple(sa.shape) != (M, K // 32):
        raise ValueError("shapes must be a [M, K], sa [M, K/32], b [G, N, K], sb [G, N, K/32]")
    if offsets.shape[0] != G or (G > 1 and offsets.stride(0) != 1):
        raise ValueError("offsets must hold G contiguous entries")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError(f"out must be a float32 [{M}, {N}] tensor with unit column stride")
    ldb = b.stride(1) if N > 1 else K
    ld_sb = sb.stride(1) if N > 1 else K // 32
    stride_b = b.stride(0) if G > 1 else N * ldb
    stride_sb = sb.stride(0) if G > 1 else N * ld_sb
    ldc = out.stride(0) if M > 1 else max(N, 1)
    st = lib().mxfp8_grouped_gemm(pa, lda, psa, ld_sa, b.data_ptr(), ldb, stride_b, sb.data_ptr(), ld_sb, stride_sb,
                                  offsets.data_ptr(), G, M, N, K, out.data_ptr(), ldc, _stream(a.device, stream))
    _check("mxfp8_grouped_gemm", st)
    return out


# ------------------------------------------------------------ token groups
def _group_ends(group_ends: torch.Tensor, device) -> Tuple[int, int]:
    if group_ends.dtype != torch.int32 or group_ends.dim() != 1 or group_ends.device != torch.device(device):
        raise ValueError("group_ends must be a 1-D int32 tensor on the inputs' device")
    if group_ends.shape[0] > 1 and group_ends.stride(0) != 1:
        raise ValueError("group_ends must be contiguous")
    return group_ends.data_ptr(), group_ends.shape[0]


def mxfp8_gated_fwd_grouped(gate: torch.Tensor, up: torch.Tensor, group_ends: torch.Tensor, *, act="silu",
                            rowwise: bool = True, colwise: bool = True, out: Optional[Sequence[torch.Tensor]] = None,
                            stream=None):
    """mxfp8_gated_fwd with token groups: colwise scales in the per-group
    padded layout [N, M/32 + 16 G] (group_ends: device int32 [G], cumulative
    row ends); returns (q_row, q_col, s_row, s_col)."""
    code = _act_code(act)
    layout = _layout(rowwise, colwise)
    pg, ldg = _bf16_matrix(gate, "gate")
    pu, ldu = _bf16_matrix(up, "up")
    if gate.shape != up.shape or gate.device != up.device:
        raise ValueError("gate and up must have the same shape and device")
    M, N = gate.shape
    pe, G = _group_ends(group_ends, gate.device)
    outs = out if out is not None else alloc_outputs(M, N, layout, gate.device, G)
    st = lib().mxfp8_gated_fwd_grouped(code, pg, ldg, pu, ldu, M, N, layout,
                                       *_out_args(outs, layout, M, N, gate.device, G), pe, G,
                                       _stream(gate.device, stream))
    _check("mxfp8_gated_fwd_grouped", st)
    return tuple(outs)


def mxfp8_gated_bwd_grouped(dh: torch.Tensor, gate: torch.Tensor, up: torch.Tensor, group_ends: torch.Tensor, *,
                            act="silu", rowwise: bool = True, colwise: bool = True,
                            out: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """mxfp8_gated_bwd with token groups: colwise scales of [dgate | dup] in
    the per-group padded layout [2N, M/32 + 16 G]."""
    code = _act_code(act)
    layout = _layout(rowwise, colwise)
    pd, ldd = _bf16_matrix(dh, "dh")
    pg, ldg = _bf16_matrix(gate, "gate")
    pu, ldu = _bf16_matrix(up, "up")
    if not (dh.shape == gate.shape == up.shape) or not (dh.device == gate.device == up.device):
        raise ValueError("dh, gate and up must have the same shape and device")
    M, N = gate.shape
    pe, G = _group_ends(group_ends, gate.device)
    outs = out if out is not None else alloc_outputs(M, 2 * N, layout, gate.device, G)
    st = lib().mxfp8_gated_bwd_grouped(code, pd, ldd, pg, ldg, pu, ldu, M, N, layout,
                                       *_out_args(outs, layout, M, 2 * N, gate.device, G), pe, G,
                                       _stream(gate.device, stream))
    _check("mxfp8_gated_bwd_grouped", st)
    return tuple(outs)


def mxfp8_quant_2d_grouped(x: torch.Tensor, group_ends: torch.Tensor, *, rowwise: bool = False, colwise: bool = True,
                           out: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """mxfp8_quant_2d with token groups along M: colwise scales in the
    per-group padded layout [K, M/32 + 16 G]."""
    layout = _layout(rowwise, colwise)
    px, ldx = _bf16_matrix(x, "x")
    M, K = x.shape
    pe, G = _group_ends(group_ends, x.device)
    outs = out if out is not None else alloc_outputs(M, K, layout, x.device, G)
    st = lib().mxfp8_quant_2d_grouped(px, ldx, M, K, layout, *_out_args(outs, layout, M, K, x.device, G), pe, G,
                                      _stream(x.device, stream))
    _check("mxfp8_quant_2d_grouped", st)
    return tuple(outs)


def mxfp8_grouped_gemm_k(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                         group_ends: torch.Tensor, *, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """K-grouped C_g = A_g B_g^T (fp32 [G, M, N]): a [M, T] and b [N, T]
    E4M3 codes (the colwise outputs of [T, M] and [T, N] matrices), scales
    sa [M, >= T/32 + 16 G] and sb [N, ...] in the per-group padded layout of
    group_ends (device int32 [G])."""
    pa, lda = _u8_matrix(a, "a")
    pb, ldb = _u8_matrix(b, "b")
    psa, ld_sa = _u8_matrix(sa, "sa")
    psb, ld_sb = _u8_matrix(sb, "sb")
    M, T = a.shape
    N = b.shape[0]
    pe, G = _group_ends(group_ends, a.device)
    if b.shape[1] != T or sa.shape[0] != M or sb.shape[0] != N:
        raise ValueError("shapes must be a [M, T], b [N, T], sa [M, *], sb [N, *]")
    if sa.shape[1] < T // 32 + 16 * G or sb.shape[1] < T // 32 + 16 * G:
        raise ValueError(f"padded scale rows need at least T/32 + 16 G = {T // 32 + 16 * G} columns")
    if out is None:
        out = torch.empty((G, M, N), dtype=torch.float32, device=a.device)
    elif (out.dtype != torch.float32 or tuple(out.shape) != (G, M, N) or (N > 1 and out.stride(2) != 1)
          or out.device != a.device):
        raise ValueError(f"out must be a float32 [{G}, {M}, {N}] tensor with unit column stride")
    ldc = out.stride(1) if M > 1 else max(N, 1)
    stride_c = out.stride(0) if G > 1 else max(ldc * M, 1)
    st = lib().mxfp8_grouped_gemm_k(pa, lda, psa, ld_sa, pb, ldb, psb, ld_sb, pe, G, M, N, T, out.data_ptr(), ldc,
                                    stride_c, _stream(a.device, stream))
    _check("mxfp8_grouped_gemm_k", st)
    return out
