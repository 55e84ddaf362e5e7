"""The C ABI without a GPU: the library loads, exports every declared entry
point, and every argument check returns its status before any HIP call.

Mirrors the launcher guards of "Add swiglu + MXFP8 fused CuTe DSL kernel"
(Numerics and tests: each error path exercised without allocating).  Every
call below is invalid or empty, so nothing is launched.
"""
import ctypes
import os
import re

import pytest

import swiglu_activation_cast_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, STRIDE, ALIGN, LAYOUT, OVERFLOW, LAUNCH, ACT = range(9)

A = 1 << 20  # a fake, 16-byte aligned "device address" (never dereferenced)


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mxfp8.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(mxfp8_\w+)\s*\(", text))


def test_library_exports_every_declared_symbol():
    lib = mx.lib()
    names = declared_functions()
    assert names == {"mxfp8_swiglu_fwd", "mxfp8_swiglu_bwd", "mxfp8_gated_fwd", "mxfp8_gated_bwd",
                     "mxfp8_quant_2d", "mxfp8_quant_3d_colwise", "mxfp8_swiglu_fwd_bf16", "mxfp8_swiglu_bwd_bf16",
                     "mxfp8_gemm", "mxfp8_grouped_gemm", "mxfp8_status_str", "mxfp8_gated_fwd_grouped",
                     "mxfp8_gated_bwd_grouped", "mxfp8_quant_2d_grouped", "mxfp8_grouped_gemm_k"}
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings():
    for st in range(9):
        assert len(mx.status_str(st)) >= 2
    assert mx.status_str(99) == "unknown status"


def fwd(**kw):
    a = dict(gate=A, ld_gate=256, up=A + 256, ld_up=256, M=64, N=128, layout=3,
             q_row=A, ld_q_row=128, s_row=A, ld_s_row=4, q_col=A, ld_q_col=64, s_col=A, ld_s_col=2)
    a.update(kw)
    return mx.lib().mxfp8_swiglu_fwd(a["gate"], a["ld_gate"], a["up"], a["ld_up"], a["M"], a["N"], a["layout"],
                                     a["q_row"], a["ld_q_row"], a["s_row"], a["ld_s_row"], a["q_col"],
                                     a["ld_q_col"], a["s_col"], a["ld_s_col"], None)


def bwd(**kw):
    a = dict(dh=A, ld_dh=128, gate=A, ld_gate=256, up=A + 256, ld_up=256, M=64, N=128, layout=3,
             q_row=A, ld_q_row=256, s_row=A, ld_s_row=8, q_col=A, ld_q_col=64, s_col=A, ld_s_col=2)
    a.update(kw)
    return mx.lib().mxfp8_swiglu_bwd(a["dh"], a["ld_dh"], a["gate"], a["ld_gate"], a["up"], a["ld_up"], a["M"],
                                     a["N"], a["layout"], a["q_row"], a["ld_q_row"], a["s_row"], a["ld_s_row"],
                                     a["q_col"], a["ld_q_col"], a["s_col"], a["ld_s_col"], None)


def gfwd(act=0, **kw):
    a = dict(gate=A, ld_gate=256, up=A + 256, ld_up=256, M=64, N=128, layout=3,
             q_row=A, ld_q_row=128, s_row=A, ld_s_row=4, q_col=A, ld_q_col=64, s_col=A, ld_s_col=2)
    a.update(kw)
    return mx.lib().mxfp8_gated_fwd(act, a["gate"], a["ld_gate"], a["up"], a["ld_up"], a["M"], a["N"], a["layout"],
                                    a["q_row"], a["ld_q_row"], a["s_row"], a["ld_s_row"], a["q_col"],
                                    a["ld_q_col"], a["s_col"], a["ld_s_col"], None)


def gbwd(act=0, **kw):
    a = dict(dh=A, ld_dh=128, gate=A, ld_gate=256, up=A + 256, ld_up=256, M=64, N=128, layout=3,
             q_row=A, ld_q_row=256, s_row=A, ld_s_row=8, q_col=A, ld_q_col=64, s_col=A, ld_s_col=2)
    a.update(kw)
    return mx.lib().mxfp8_gated_bwd(act, a["dh"], a["ld_dh"], a["gate"], a["ld_gate"], a["up"], a["ld_up"], a["M"],
                                    a["N"], a["layout"], a["q_row"], a["ld_q_row"], a["s_row"], a["ld_s_row"],
                                    a["q_col"], a["ld_q_col"], a["s_col"], a["ld_s_col"], None)


def q2d(**kw):
    a = dict(x=A, ld_x=128, M=64, K=128, layout=3, q_row=A, ld_q_row=128, s_row=A, ld_s_row=4, q_col=A,
             ld_q_col=64, s_col=A, ld_s_col=2)
    a.update(kw)
    return mx.lib().mxfp8_quant_2d(a["x"], a["ld_x"], a["M"], a["K"], a["layout"], a["q_row"], a["ld_q_row"],
                                   a["s_row"], a["ld_s_row"], a["q_col"], a["ld_q_col"], a["s_col"], a["ld_s_col"],
                                   None)


def q3d(**kw):
    a = dict(w=A, E=4, N=64, K=40, stride_e=64 * 40, ld_w=40, q=A, s=A)
    a.update(kw)
    return mx.lib().mxfp8_quant_3d_colwise(a["w"], a["E"], a["N"], a["K"], a["stride_e"], a["ld_w"], a["q"], a["s"],
                                           None)


@pytest.mark.parametrize("call", [fwd, bwd, q2d])
def test_layout_errors(call):
    for layout in (0, 4, -1, 7):
        assert call(layout=layout) == LAYOUT


@pytest.mark.parametrize("call", [fwd, bwd])
def test_swiglu_shape_errors(call):
    assert call(M=-1) == SHAPE
    assert call(N=-32) == SHAPE
    assert call(N=48) == SHAPE                     # width not a multiple of 32
    assert call(M=40, layout=2) == SHAPE           # colwise rows not a multiple of 32
    assert call(M=40, layout=3) == SHAPE


def test_quant_2d_shape_errors():
    assert q2d(K=40, layout=1) == SHAPE            # rowwise blocks run along K
    assert q2d(K=36, layout=2, ld_x=40) == SHAPE   # colwise needs K % 8 == 0
    assert q2d(M=33, layout=2) == SHAPE


@pytest.mark.parametrize("call", [fwd, bwd, q2d])
def test_empty_is_ok_without_pointers(call):
    nul = dict(q_row=None, s_row=None, q_col=None, s_col=None)
    if call is q2d:
        assert call(M=0, x=None, **nul) == OK
        assert call(K=0, x=None, **nul) == OK
    else:
        assert call(M=0, gate=None, up=None, **nul) == OK
        assert call(N=0, gate=None, up=None, **nul) == OK


def test_null_errors():
    assert fwd(gate=None) == NULL
    assert fwd(up=None) == NULL
    assert fwd(q_row=None) == NULL
    assert fwd(s_col=None) == NULL
    assert bwd(dh=None) == NULL
    assert q2d(x=None) == NULL
    assert q2d(s_row=None, layout=1) == NULL
    # pointers of a layout that is not requested may be NULL; the call then
    # fails later on purpose (bad stride) so that nothing launches
    assert fwd(q_col=None, s_col=None, layout=1, ld_gate=100) == STRIDE


def test_stride_errors():
    assert fwd(ld_gate=64) == STRIDE               # smaller than N
    assert fwd(ld_up=132) == STRIDE                # not a multiple of 8 elements
    assert fwd(ld_q_row=120) == STRIDE             # smaller than W
    assert fwd(ld_q_row=136) == STRIDE             # not a multiple of 16 bytes
    assert fwd(ld_s_row=3) == STRIDE
    assert fwd(ld_q_col=40) == STRIDE              # smaller than M
    assert fwd(ld_s_col=1) == STRIDE
    assert bwd(ld_q_row=128) == STRIDE             # W = 2N = 256
    assert bwd(ld_s_row=4) == STRIDE
    assert bwd(ld_dh=120) == STRIDE


def test_alignment_errors():
    assert fwd(gate=A + 2) == ALIGN
    assert fwd(up=A + 8) == ALIGN
    assert fwd(q_row=A + 4) == ALIGN
    assert fwd(q_col=A + 1) == ALIGN
    assert bwd(dh=A + 2) == ALIGN
    assert q2d(x=A + 6) == ALIGN
    # scale pointers have no alignment requirement: the call proceeds to the
    # next check (made to fail here so that nothing launches)
    assert fwd(s_row=A + 1, ld_gate=100) == STRIDE


def test_overflow_errors():
    big = 1 << 61
    assert fwd(M=big, ld_gate=big) == OVERFLOW or fwd(M=big, ld_gate=big) == STRIDE
    assert q2d(M=1 << 40, K=1 << 24, ld_x=1 << 24, ld_q_row=1 << 24, ld_s_row=1 << 19, layout=1) == OVERFLOW


def test_3d_errors():
    assert q3d(E=-1) == SHAPE
    assert q3d(N=48) == SHAPE
    assert q3d(K=36, ld_w=40) == SHAPE
    assert q3d(E=0, w=None, q=None, s=None) == OK
    assert q3d(w=None) == NULL
    assert q3d(q=None) == NULL
    assert q3d(ld_w=36) == STRIDE
    assert q3d(ld_w=44) == STRIDE
    assert q3d(stride_e=64 * 40 - 8) == STRIDE
    assert q3d(w=A + 2) == ALIGN
    assert q3d(q=A + 8) == ALIGN
    assert q3d(E=1 << 40, stride_e=1 << 30) == OVERFLOW


def test_colwise_stride_limits():
    # the colwise kernel addresses a tile with 32-bit offsets: oversized
    # strides are refused before anything launches
    assert q2d(layout=2, ld_x=1 << 24) == OVERFLOW
    assert q2d(layout=2, ld_q_col=1 << 25) == OVERFLOW
    assert fwd(layout=3, ld_q_row=1 << 25) == OVERFLOW
    assert q3d(ld_w=1 << 24, stride_e=(1 << 24) * 64) == OVERFLOW
    assert q3d(N=1 << 25, stride_e=(1 << 25) * 40) == OVERFLOW
    # rowwise-only calls have no such limit (stride check fails first here)
    assert q2d(layout=1, ld_x=(1 << 24) + 4) == STRIDE


def test_bf16_value_entry_points_errors():
    lib = mx.lib()
    f = lib.mxfp8_swiglu_fwd_bf16
    b = lib.mxfp8_swiglu_bwd_bf16
    assert f(A, 128, A, 128, 64, 128, None, 128, None) == NULL
    assert f(None, 128, A, 128, 64, 128, A, 128, None) == NULL
    assert f(A, 128, A, 128, 64, 12, A, 128, None) == SHAPE        # N % 8 != 0
    assert f(A, 128, A, 128, -1, 128, A, 128, None) == SHAPE
    assert f(A, 128, A, 128, 64, 128, A, 120, None) == STRIDE      # ld_h < N
    assert f(A, 100, A, 128, 64, 96, A, 128, None) == STRIDE       # ld not a multiple of 8
    assert f(A + 2, 128, A, 128, 64, 128, A, 128, None) == ALIGN
    assert f(A, 128, A, 128, 64, 128, A + 8, 128, None) == ALIGN
    assert f(None, 128, None, 128, 0, 128, None, 128, None) == OK  # empty
    assert b(A, 128, A, 128, A, 128, 64, 128, A, 128, None) == STRIDE   # [dg|du] needs ld >= 2N
    assert b(A, 128, A, 128, None, 128, 64, 128, A, 256, None) == NULL
    assert b(A, 128, A, 128, A, 128, 64, 128, A + 4, 256, None) == ALIGN



@pytest.mark.parametrize("call", [gfwd, gbwd])
def test_gated_activation_errors(call):
    # an unknown activation is refused before any other check, even on an
    # empty or otherwise invalid call
    for act in (-1, 4, 99):
        assert call(act=act) == ACT
        assert call(act=act, M=0) == ACT
        assert call(act=act, layout=0) == ACT


@pytest.mark.parametrize("call", [gfwd, gbwd])
@pytest.mark.parametrize("act", [0, 1, 2, 3])
def test_gated_checks_match_swiglu(call, act):
    """Every activation runs the same argument checks as the SwiGLU calls."""
    plain = fwd if call is gfwd else bwd
    cases = [dict(layout=0), dict(M=-1), dict(N=48), dict(M=40, layout=2), dict(gate=None), dict(ld_gate=64),
             dict(ld_q_row=136), dict(gate=A + 2), dict(q_col=A + 1), dict(layout=3, ld_q_row=1 << 25)]
    for kw in cases:
        assert call(act=act, **kw) == plain(**kw), kw
    nul = dict(q_row=None, s_row=None, q_col=None, s_col=None)
    assert call(act=act, M=0, gate=None, up=None, **nul) == OK


def test_binding_activation_names():
    assert mx.ACTIVATIONS == {"silu": 0, "gelu_tanh": 1, "gelu": 2, "relu": 3}
    from swiglu_activation_cast_amd._binding import _act_code

    with pytest.raises(ValueError):
        _act_code("swish")
    assert _act_code("gelu") == 2 and _act_code(3) == 3


def gemm(**kw):
    a = dict(a=A, lda=128, sa=A, ld_sa=4, b=A, ldb=128, sb=A, ld_sb=4, M=64, N=48, K=128, c=A, ldc=48)
    a.update(kw)
    return mx.lib().mxfp8_gemm(a["a"], a["lda"], a["sa"], a["ld_sa"], a["b"], a["ldb"], a["sb"], a["ld_sb"], a["M"],
                               a["N"], a["K"], a["c"], a["ldc"], None)


def test_gemm_errors():
    assert gemm(K=48) == SHAPE                      # partial block
    assert gemm(M=-1) == SHAPE
    assert gemm(M=0, a=None, c=None) == OK          # empty result: nothing to do
    assert gemm(N=0, b=None) == OK
    assert gemm(a=None) == NULL
    assert gemm(sb=None) == NULL
    assert gemm(c=None) == NULL
    assert gemm(lda=120) == STRIDE                  # < K
    assert gemm(ldb=136) == STRIDE                  # not a multiple of 16
    assert gemm(ld_sa=3) == STRIDE
    assert gemm(ldc=40) == STRIDE
    assert gemm(a=A + 8) == ALIGN
    assert gemm(b=A + 4) == ALIGN
    assert gemm(c=A + 2) == ALIGN
    assert gemm(sa=A + 1, lda=120) == STRIDE        # scales need no alignment
    assert gemm(M=1 << 62, K=1 << 20, lda=1 << 20, ldb=1 << 20, ld_sa=1 << 15, ld_sb=1 << 15) == OVERFLOW


def ggemm(**kw):
    a = dict(a=A, lda=128, sa=A, ld_sa=4, b=A, ldb=128, stride_b=48 * 128, sb=A, ld_sb=4, stride_sb=48 * 4, offs=A,
             G=3, M=64, N=48, K=128, c=A, ldc=48)
    a.update(kw)
    return mx.lib().mxfp8_grouped_gemm(a["a"], a["lda"], a["sa"], a["ld_sa"], a["b"], a["ldb"], a["stride_b"], a["sb"],
                                       a["ld_sb"], a["stride_sb"], a["offs"], a["G"], a["M"], a["N"], a["K"], a["c"],
                                       a["ldc"], None)


def test_grouped_gemm_errors():
    assert ggemm(G=0, offs=None) == OK               # no groups: nothing to do
    assert ggemm(G=-1) == SHAPE
    assert ggemm(G=1025) == SHAPE
    assert ggemm(K=40) == SHAPE
    assert ggemm(offs=None) == NULL
    assert ggemm(stride_b=47 * 128) == STRIDE        # experts would overlap
    assert ggemm(stride_b=48 * 128 + 8) == STRIDE    # not a multiple of 16
    assert ggemm(stride_sb=47 * 4) == STRIDE
    assert ggemm(offs=A + 2) == ALIGN
    assert ggemm(lda=120) == STRIDE
    assert ggemm(M=0, a=None) == OK


def kgemm(**kw):
    a = dict(a=A, lda=256, sa=A, ld_sa=8 + 48, b=A, ldb=256, sb=A, ld_sb=8 + 48, offs=A, G=3, M=64, N=48, T=256,
             c=A, ldc=48, stride_c=64 * 48)
    a.update(kw)
    return mx.lib().mxfp8_grouped_gemm_k(a["a"], a["lda"], a["sa"], a["ld_sa"], a["b"], a["ldb"], a["sb"], a["ld_sb"],
                                         a["offs"], a["G"], a["M"], a["N"], a["T"], a["c"], a["ldc"], a["stride_c"],
                                         None)


def test_grouped_gemm_k_errors():
    assert kgemm(G=0, offs=None) == OK                # no groups: nothing to do
    assert kgemm(G=-1) == SHAPE
    assert kgemm(G=1025) == SHAPE
    assert kgemm(T=240) == SHAPE                      # tokens not a multiple of 32
    assert kgemm(offs=None) == NULL
    assert kgemm(ld_sa=8 + 47) == STRIDE              # padded scale rows need T/32 + 16 G
    assert kgemm(ld_sb=8 + 47) == STRIDE
    assert kgemm(lda=248) == STRIDE
    assert kgemm(stride_c=63 * 48) == STRIDE          # group results would overlap
    assert kgemm(offs=A + 2) == ALIGN
    assert kgemm(c=A + 2) == ALIGN
    assert kgemm(M=0, a=None) == OK


def grouped_cast(fn, **kw):
    lib = mx.lib()
    a = dict(gate=A, ld_gate=256, up=A + 256, ld_up=256, dh=A, ld_dh=128, M=64, N=128, layout=3,
             q_row=A, ld_q_row=256, s_row=A, ld_s_row=8, q_col=A, ld_q_col=64, s_col=A, ld_s_col=2 + 16 * 2,
             offs=A, G=2, act=0)
    a.update(kw)
    common = (a["M"], a["N"], a["layout"], a["q_row"], a["ld_q_row"], a["s_row"], a["ld_s_row"], a["q_col"],
              a["ld_q_col"], a["s_col"], a["ld_s_col"], a["offs"], a["G"], None)
    if fn == "fwd":
        return lib.mxfp8_gated_fwd_grouped(a["act"], a["gate"], a["ld_gate"], a["up"], a["ld_up"], *common)
    if fn == "bwd":
        return lib.mxfp8_gated_bwd_grouped(a["act"], a["dh"], a["ld_dh"], a["gate"], a["ld_gate"], a["up"],
                                           a["ld_up"], *common)
    return lib.mxfp8_quant_2d_grouped(a["gate"], a["ld_gate"], *common)


@pytest.mark.parametrize("fn", ["fwd", "bwd", "quant"])
def test_grouped_cast_errors(fn):
    """The token-group checks come on top of the ungrouped casts' checks;
    colwise scale rows must hold M/32 + 16 groups."""
    assert grouped_cast(fn, G=0) == SHAPE
    assert grouped_cast(fn, G=1025) == SHAPE
    assert grouped_cast(fn, offs=None) == NULL
    assert grouped_cast(fn, offs=A + 2) == ALIGN
    assert grouped_cast(fn, ld_s_col=2 + 16 * 2 - 1) == STRIDE
    # rowwise only: the colwise scale row is not checked (the call fails on
    # the NULL input instead, before any launch)
    assert grouped_cast(fn, layout=1, ld_s_col=0, gate=None, dh=None) == NULL
    assert grouped_cast(fn, M=1 << 31, ld_q_col=1 << 31) == OVERFLOW
    if fn != "quant":
        assert grouped_cast(fn, act=9) == ACT
    assert grouped_cast(fn, M=0) == OK


def test_stream_probe_exports_and_checks():
    """libmxstream.so (the bandwidth probe) exports what include/mxstream.h
    declares and rejects bad arguments before any launch."""
    from swiglu_activation_cast_amd import stream_probe

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mxstream.h")).read(), flags=re.S)
    names = set(re.findall(r"\b(mxstream_\w+)\s*\(", text))
    assert names == {"mxstream_mix"}
    lib = stream_probe.lib()
    bufs = (ctypes.c_void_p * 4)(A, A + 4096, A + 8192, A + 12288)
    assert lib.mxstream_mix(None, 1, bufs, 1, 32768, 8, 1, None) == 1
    assert lib.mxstream_mix(bufs, 0, bufs, 1, 32768, 8, 1, None) == 2
    assert lib.mxstream_mix(bufs, 5, bufs, 1, 32768, 8, 1, None) == 2
    assert lib.mxstream_mix(bufs, 3, bufs, 3, 32768, 8, 1, None) == 2
    assert lib.mxstream_mix(bufs, 3, bufs, 2, 32768 + 16, 8, 1, None) == 2
    assert lib.mxstream_mix(bufs, 3, bufs, 2, 32768, 6, 1, None) == 2
    assert lib.mxstream_mix(bufs, 3, bufs, 2, 32768, 8, 0, None) == 2
    odd = (ctypes.c_void_p * 2)(A + 8, A)
    assert lib.mxstream_mix(odd, 2, bufs, 1, 32768, 8, 1, None) == 2
