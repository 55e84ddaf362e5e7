"""CPU oracle for the fused SwiGLU (and gated-activation) + MXFP8 cast --
TEST INFRASTRUCTURE ONLY.

A plain, slow, single-threaded definition (``mxfp8_oracle.c``, IEEE double)
of what the GPU path computes.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product path never
does.  It shares no code with the HIP library.

Arrays are numpy: bf16 inputs are ``uint16`` bit patterns (2-D, any row
stride, unit column stride), outputs are ``uint8`` (E4M3 codes, E8M0 bytes).

Pages (title, section):
  "Add swiglu + MXFP8 fused CuTe DSL kernel": Summary, API, Numerics and
  tests, commit message; "[mxfp8 moe training] update 3d quant colwise
  scaling kernel to use single input/output TMA descriptors": Summary.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

ROWWISE = 1
COLWISE = 2
BOTH = 3

# gate activations of the gated family: act(g) * up
SILU, GELU_TANH, GELU, RELU = 0, 1, 2, 3
ACTS = {"silu": SILU, "gelu_tanh": GELU_TANH, "gelu": GELU, "relu": RELU}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxfp8_oracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"oracle library not built: run `make -C {_HERE}`")
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "orc_bf16_decode": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_bf16_round": (ctypes.c_uint16, [ctypes.c_double]),
        "orc_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
        "orc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_double]),
        "orc_e8m0_rceil": (ctypes.c_uint8, [ctypes.c_double]),
        "orc_e8m0_decode": (ctypes.c_double, [ctypes.c_uint8]),
        "orc_sigmoid": (ctypes.c_double, [ctypes.c_double]),
        "orc_silu": (ctypes.c_double, [ctypes.c_double]),
        "orc_block_scale": (ctypes.c_uint8, [_p, _i64, _i64]),
        "orc_quant_block_at": (None, [_p, _i64, _i64, ctypes.c_uint8, _p, _i64]),
        "orc_quant_block": (None, [_p, _i64, _i64, _p, _i64, _p]),
        "orc_act": (ctypes.c_double, [ctypes.c_int, ctypes.c_double]),
        "orc_act_grad": (ctypes.c_double, [ctypes.c_int, ctypes.c_double]),
        "orc_gated_fwd_values": (ctypes.c_int, [ctypes.c_int, _p, _p, _i64, _p]),
        "orc_gated_bwd_values": (ctypes.c_int, [ctypes.c_int, _p, _p, _p, _i64, _p, _p]),
        "orc_gated_fwd": (ctypes.c_int, [ctypes.c_int, _p, _i64, _p, _i64, _i64, _i64, ctypes.c_int] + [_p, _i64] * 4),
        "orc_gated_bwd": (ctypes.c_int, [ctypes.c_int, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, ctypes.c_int]
                          + [_p, _i64] * 4),
        "orc_swiglu_fwd_values": (None, [_p, _p, _i64, _p]),
        "orc_swiglu_bwd_values": (None, [_p, _p, _p, _i64, _p, _p]),
        "orc_quant_2d": (ctypes.c_int, [_p, _i64, _i64, _i64, ctypes.c_int] + [_p, _i64] * 4),
        "orc_swiglu_fwd": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _i64, ctypes.c_int] + [_p, _i64] * 4),
        "orc_swiglu_bwd": (ctypes.c_int, [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, ctypes.c_int] + [_p, _i64] * 4),
        "orc_quant_3d_colwise": (ctypes.c_int, [_p, _i64, _i64, _i64, _i64, _i64, _p, _p]),
        "orc_mx_gemm": (ctypes.c_int, [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64, _p, _i64]),
        "orc_mx_grouped_gemm": (ctypes.c_int, [_p, _i64, _p, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64,
                                               _i64, _p, _i64, _p, _i64]),
        "orc_group_bounds": (ctypes.c_int, [_p, _i64, _i64, _p, _p]),
        "orc_group_scale_base": (_i64, [_i64, _i64]),
        "orc_pad_group_scales": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64]),
        "orc_mx_grouped_gemm_k": (ctypes.c_int, [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64,
                                                 _p, _i64, _i64, _p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def lib():
    return _load()


# ----------------------------------------------------------------- scalars
def bf16_decode(b: int) -> float:
    return _load().orc_bf16_decode(int(b))


def bf16_round(v: float) -> int:
    return _load().orc_bf16_round(float(v))


def e4m3_decode(c: int) -> float:
    return _load().orc_e4m3_decode(int(c))


def e4m3_encode(v: float) -> int:
    return _load().orc_e4m3_encode(float(v))


def e8m0_rceil(amax: float) -> int:
    return _load().orc_e8m0_rceil(float(amax))


def e8m0_decode(b: int) -> float:
    return _load().orc_e8m0_decode(int(b))


def sigmoid(x: float) -> float:
    return _load().orc_sigmoid(float(x))


def silu(x: float) -> float:
    return _load().orc_silu(float(x))


def act(a: int, x: float) -> float:
    """The gate activation `a` (SILU, GELU_TANH, GELU, RELU) at x, in double."""
    return _load().orc_act(int(a), float(x))


def act_grad(a: int, x: float) -> float:
    """Its derivative at x, in double."""
    return _load().orc_act_grad(int(a), float(x))


# ------------------------------------------------------------------ blocks
def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def block_scale(y) -> int:
    y = np.ascontiguousarray(y, dtype=np.float64)
    return _load().orc_block_scale(_ptr(y), y.size, 1)


def quant_block_at(y, scale: int) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    q = np.empty(y.size, np.uint8)
    _load().orc_quant_block_at(_ptr(y), y.size, 1, int(scale), _ptr(q), 1)
    return q


def quant_block(y):
    y = np.ascontiguousarray(y, dtype=np.float64)
    q = np.empty(y.size, np.uint8)
    s = np.zeros(1, np.uint8)
    _load().orc_quant_block(_ptr(y), y.size, 1, _ptr(q), 1, _ptr(s))
    return q, int(s[0])


# ------------------------------------------------------------------ values
def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bit patterns, got {a.dtype}")
    return a


def gated_fwd_values(g, u, act: int = SILU) -> np.ndarray:
    """h = bf16(bf16(act(g)) * u), elementwise, as uint16 bits."""
    g = np.ascontiguousarray(_u16(g))
    u = np.ascontiguousarray(_u16(u))
    assert g.shape == u.shape
    h = np.empty_like(g)
    _check(_load().orc_gated_fwd_values(int(act), _ptr(g), _ptr(u), g.size, _ptr(h)), "gated_fwd_values")
    return h


def gated_bwd_values(dh, g, u, act: int = SILU):
    """(dg, du) of h = act(g) * u for upstream gradient dh, as uint16 bits."""
    dh = np.ascontiguousarray(_u16(dh))
    g = np.ascontiguousarray(_u16(g))
    u = np.ascontiguousarray(_u16(u))
    assert dh.shape == g.shape == u.shape
    dg = np.empty_like(g)
    du = np.empty_like(g)
    _check(_load().orc_gated_bwd_values(int(act), _ptr(dh), _ptr(g), _ptr(u), g.size, _ptr(dg), _ptr(du)),
           "gated_bwd_values")
    return dg, du


def swiglu_fwd_values(g, u) -> np.ndarray:
    """h = bf16(bf16(silu(g)) * u), elementwise, as uint16 bits."""
    return gated_fwd_values(g, u, SILU)


def swiglu_bwd_values(dh, g, u):
    """(dg, du) of h = silu(g) * u for upstream gradient dh, as uint16 bits."""
    return gated_bwd_values(dh, g, u, SILU)


# ------------------------------------------------------------------ matrices
def _mat(a) -> tuple[np.ndarray, int]:
    """2-D uint16 view with unit column stride; returns (array, row stride)."""
    a = _u16(a)
    if a.ndim != 2:
        raise ValueError("expected a 2-D array")
    if a.strides[1] != 2 or a.strides[0] % 2 != 0 or a.strides[0] < 2 * a.shape[1]:
        a = np.ascontiguousarray(a)
    return a, a.strides[0] // 2


def _outputs(M: int, W: int, layout: int):
    q_row = np.zeros((M, W), np.uint8) if layout & ROWWISE else np.zeros((0, 0), np.uint8)
    s_row = np.zeros((M, W // 32), np.uint8) if layout & ROWWISE else np.zeros((0, 0), np.uint8)
    q_col = np.zeros((W, M), np.uint8) if layout & COLWISE else np.zeros((0, 0), np.uint8)
    s_col = np.zeros((W, M // 32), np.uint8) if layout & COLWISE else np.zeros((0, 0), np.uint8)
    return q_row, s_row, q_col, s_col


def _out_args(q_row, s_row, q_col, s_col):
    return [
        _ptr(q_row), q_row.shape[1], _ptr(s_row), s_row.shape[1],
        _ptr(q_col), q_col.shape[1], _ptr(s_col), s_col.shape[1],
    ]


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def quant_2d(x, layout: int = ROWWISE):
    """MXFP8 cast of a bf16 [M, K] matrix; returns (q_row, s_row, q_col, s_col)."""
    x, ld = _mat(x)
    M, K = x.shape
    outs = _outputs(M, K, layout)
    _check(_load().orc_quant_2d(_ptr(x), ld, M, K, layout, *_out_args(*outs)), "quant_2d")
    return outs


def gated_fwd(gate, up, layout: int = ROWWISE, act: int = SILU):
    """Fused forward: MXFP8 cast of h = act(gate) * up; returns (q_row, s_row, q_col, s_col)."""
    g, ldg = _mat(gate)
    u, ldu = _mat(up)
    assert g.shape == u.shape
    M, N = g.shape
    outs = _outputs(M, N, layout)
    _check(_load().orc_gated_fwd(int(act), _ptr(g), ldg, _ptr(u), ldu, M, N, layout, *_out_args(*outs)),
           "gated_fwd")
    return outs


def gated_bwd(dh, gate, up, layout: int = ROWWISE, act: int = SILU):
    """Fused backward: MXFP8 cast of [dg | du]; returns (q_row, s_row, q_col, s_col), width 2N."""
    d, ldd = _mat(dh)
    g, ldg = _mat(gate)
    u, ldu = _mat(up)
    assert d.shape == g.shape == u.shape
    M, N = g.shape
    outs = _outputs(M, 2 * N, layout)
    _check(
        _load().orc_gated_bwd(int(act), _ptr(d), ldd, _ptr(g), ldg, _ptr(u), ldu, M, N, layout, *_out_args(*outs)),
        "gated_bwd",
    )
    return outs


def swiglu_fwd(gate, up, layout: int = ROWWISE):
    """Fused forward: MXFP8 cast of h = silu(gate) * up; returns (q_row, s_row, q_col, s_col)."""
    return gated_fwd(gate, up, layout, SILU)


def swiglu_bwd(dh, gate, up, layout: int = ROWWISE):
    """Fused backward: MXFP8 cast of [dg | du]; returns (q_row, s_row, q_col, s_col), width 2N."""
    return gated_bwd(dh, gate, up, layout, SILU)


def quant_3d_colwise(w):
    """3D per-expert colwise cast of bf16 w [E, N, K]; returns (q [E, K, N], s [E, K, N/32])."""
    w = _u16(w)
    if w.ndim != 3:
        raise ValueError("expected a 3-D array")
    if w.strides[2] != 2 or w.strides[1] % 2 or w.strides[0] % 2:
        w = np.ascontiguousarray(w)
    E, N, K = w.shape
    q = np.zeros((E, K, N), np.uint8)
    s = np.zeros((E, K, N // 32), np.uint8)
    _check(
        _load().orc_quant_3d_colwise(_ptr(w), E, N, K, w.strides[0] // 2, w.strides[1] // 2, _ptr(q), _ptr(s)),
        "quant_3d_colwise",
    )
    return q, s


# ------------------------------------------------------------- MX GEMM
def _u8_mat(x) -> tuple[np.ndarray, int]:
    x = np.asarray(x)
    if x.dtype != np.uint8 or x.ndim != 2:
        raise TypeError("expected a 2-D uint8 array")
    if x.strides[1] != 1 or x.strides[0] < x.shape[1]:
        x = np.ascontiguousarray(x)
    return x, x.strides[0]


def mx_gemm(a, sa, b, sb):
    """C = A B^T of MXFP8 operands stored K-contiguous: a [M, K] and b [N, K]
    E4M3 codes with E8M0 scales sa [M, K/32], sb [N, K/32].  Returns (C,
    sum |products|), both float64 [M, N]."""
    a, lda = _u8_mat(a)
    b, ldb = _u8_mat(b)
    sa, ld_sa = _u8_mat(sa)
    sb, ld_sb = _u8_mat(sb)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K and sa.shape == (M, K // 32) and sb.shape == (N, K // 32)
    c = np.zeros((M, N), np.float64)
    cabs = np.zeros((M, N), np.float64)
    _check(_load().orc_mx_gemm(_ptr(a), lda, _ptr(sa), ld_sa, _ptr(b), ldb, _ptr(sb), ld_sb, M, N, K,
                               _ptr(c), N, _ptr(cabs), N), "mx_gemm")
    return c, cabs


def mx_grouped_gemm(a, sa, b, sb, offsets):
    """Grouped C = A B_g^T: rows of a [M, K] split by the cumulative end
    offsets (int32, length G) into groups, group g against b[g] [N, K] with
    scales sb[g] [N, K/32].  Returns (C, sum |products|) as float64 [M, N];
    rows no group covers are NaN (never written)."""
    a, lda = _u8_mat(a)
    sa, ld_sa = _u8_mat(sa)
    b = np.ascontiguousarray(np.asarray(b, np.uint8))
    sb = np.ascontiguousarray(np.asarray(sb, np.uint8))
    offs = np.ascontiguousarray(np.asarray(offsets, np.int32))
    M, K = a.shape
    G, N, Kb = b.shape
    assert Kb == K and sb.shape == (G, N, K // 32) and offs.shape == (G,)
    c = np.full((M, N), np.nan)
    cabs = np.full((M, N), np.nan)
    _check(_load().orc_mx_grouped_gemm(_ptr(a), lda, _ptr(sa), ld_sa, _ptr(b), K, N * K, _ptr(sb), K // 32,
                                       N * (K // 32), _ptr(offs), G, M, N, K, _ptr(c), N, _ptr(cabs), N),
           "mx_grouped_gemm")
    return c, cabs


# ------------------------------------------------- token groups (wgrad)
def _offs(offsets):
    return np.ascontiguousarray(np.asarray(offsets, np.int32).reshape(-1))


def group_bounds(offsets, T):
    """(starts, ends) of the G token groups plus the tail group G, after
    rounding each cumulative end down to a multiple of 32 and clamping the
    ends to be non-decreasing and at most T.  int64 arrays of length G + 1."""
    offs = _offs(offsets)
    G = offs.size
    st = np.zeros(G + 1, np.int64)
    en = np.zeros(G + 1, np.int64)
    _check(_load().orc_group_bounds(_ptr(offs), G, int(T), _ptr(st), _ptr(en)), "group_bounds")
    return st, en


def group_scale_base(g, start):
    """Position of group g's first scale block in a per-group padded row."""
    return int(_load().orc_group_scale_base(int(g), int(start)))


def pad_group_scales(s, T, offsets, ld_out=None, fill=0):
    """Per-group padded layout of colwise scales s [rows, T/32]; returns
    [rows, ld_out] (default T/32 + 16 G) with unused positions = fill."""
    s, ld_s = _u8_mat(s)
    offs = _offs(offsets)
    G = offs.size
    rows = s.shape[0]
    ld_out = T // 32 + 16 * G if ld_out is None else int(ld_out)
    out = np.full((rows, ld_out), fill, np.uint8)
    _check(_load().orc_pad_group_scales(_ptr(s), rows, ld_s, int(T), _ptr(offs), G, _ptr(out), ld_out),
           "pad_group_scales")
    return out


def mx_grouped_gemm_k(a, sa, b, sb, offsets):
    """K-grouped C_g = A_g B_g^T over each token group's columns of a [M, T]
    and b [N, T] (E4M3 codes), scales sa [M, ld], sb [N, ld] in the per-group
    padded layout.  Returns (C, sum |products|) as float64 [G, M, N]."""
    a, lda = _u8_mat(a)
    b, ldb = _u8_mat(b)
    sa, ld_sa = _u8_mat(sa)
    sb, ld_sb = _u8_mat(sb)
    offs = _offs(offsets)
    G = offs.size
    M, T = a.shape
    N = b.shape[0]
    assert b.shape[1] == T and sa.shape[0] == M and sb.shape[0] == N
    c = np.zeros((G, M, N), np.float64)
    cabs = np.zeros((G, M, N), np.float64)
    _check(_load().orc_mx_grouped_gemm_k(_ptr(a), lda, _ptr(sa), ld_sa, _ptr(b), ldb, _ptr(sb), ld_sb, _ptr(offs), G,
                                         M, N, T, _ptr(c), N, M * N, _ptr(cabs)), "mx_grouped_gemm_k")
    return c, cabs
