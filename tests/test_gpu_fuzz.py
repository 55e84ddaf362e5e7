"""Seeded random cases of the casts against the oracle (GPU).

The 2D cases: each draws an operation (the plain cast, the SwiGLU forward or
backward, or a gated forward or backward with another activation), a launch
layout, a shape and padded input row strides from its own seed, so that the
cases reach the tile-order paths the fixed-shape tests meet only at large
sizes: bands of 8, 32 and 128 row tiles, each with a ragged last band, one
ragged last row tile and one ragged last column tile, and inputs read
through row strides wider than the row ("Add swiglu + MXFP8 fused CuTe DSL
kernel", Summary: the packed w13 input whose halves are gate and up).

The 3D cases draw expert counts, shapes and padded strides; the grouped
cases draw token-group ends (unsorted, negative, past the end, empty
groups), for the grouped casts and for the K-grouped GEMM.

Same bar as the fixed-shape tests: the plain cast bit-exact, the fused casts
within oracle/parity.py's tolerance (codes within one E4M3 step, scales
bit-exact except next to a power-of-two boundary).
"""
import numpy as np
import pytest
import torch

import swiglu_activation_cast_amd as mx
from swiglu_activation_cast_amd import synth

from helpers import torch_bf16_to_bits
from oracle.parity import assert_exact, compare_fused

ROW, COL, BOTH = 1, 2, 3
OPS = ("quant", "swiglu_fwd", "swiglu_bwd", "gated_fwd", "gated_bwd")
OTHER = ("gelu", "gelu_tanh", "relu")
BUCKETS = ("few tiles", "up to 128 row tiles", "past 128 row tiles")
N_CASES = len(OPS) * 3 * len(BUCKETS)  # every (operation, layout, size bucket) once


def draw(idx):
    """The case's parameters: its operation, layout and size bucket from its
    index, the rest from its own seed."""
    rng = np.random.default_rng(9000 + idx)
    op = OPS[idx % len(OPS)]
    layout = (ROW, COL, BOTH)[(idx // len(OPS)) % 3]
    bucket = idx // (3 * len(OPS))
    if bucket == 0:  # a few tiles
        M, W = int(rng.integers(1, 700)), 32 * int(rng.integers(1, 33))
    elif bucket == 1:  # up to 128 row tiles: the both-layout launch takes bands of 8
        M, W = int(rng.integers(700, 16385)), 32 * int(rng.integers(1, 9))
    else:  # more than 128 row tiles: bands of 32 (both layouts) and 128 (colwise only)
        M, W = int(rng.integers(16385, 36001)), 32 * int(rng.integers(1, 4))
    if layout & COL:
        M = max(32, M // 32 * 32)
    if op == "quant" and layout == COL and rng.random() < 0.5:
        W -= 8 * int(rng.integers(0, 4))  # colwise only: the row needs K % 8 == 0 only
    pad = 8 * int(rng.integers(0, 5))
    act = OTHER[int(rng.integers(len(OTHER)))]
    return dict(op=op, layout=layout, bucket=BUCKETS[bucket], M=M, W=W, pad=pad, act=act,
                seed=int(rng.integers(1 << 30)))


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _flags(layout):
    return dict(rowwise=bool(layout & ROW), colwise=bool(layout & COL))


def _gpu(outs):
    q_row, q_col, s_row, s_col = outs
    return tuple(t.cpu().numpy() for t in (q_row, s_row, q_col, s_col))


def _padded(bits, pad, dev):
    """bits [M, W] on the device inside a [M, W + pad] buffer (row stride W + pad)."""
    M, W = bits.shape
    buf = np.zeros((M, W + pad), dtype=np.uint16)
    buf[:, :W] = bits
    return torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).to(dev)[:, :W]


def _w13(g_bits, u_bits, pad, dev):
    """gate and up as the two halves of one [M, 2N + pad] buffer."""
    M, N = g_bits.shape
    buf = np.zeros((M, 2 * N + pad), dtype=np.uint16)
    buf[:, :N], buf[:, N:2 * N] = g_bits, u_bits
    t = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).to(dev)
    return t[:, :N], t[:, N:2 * N]


@pytest.mark.gpu
@pytest.mark.parametrize("idx", range(N_CASES))
def test_random_case(oracle_mod, idx):
    dev = _dev()
    c = draw(idx)
    op, layout, M, W, pad, act = c["op"], c["layout"], c["M"], c["W"], c["pad"], c["act"]
    print(f"case {idx}: {c}", flush=True)
    name = f"fuzz{idx}/{op}"
    if op == "quant":
        x = torch_bf16_to_bits(synth.normal_bf16((M, W), 2.0, seed=c["seed"]))
        gpu = _gpu(mx.mxfp8_quant_2d(_padded(x, pad, dev), **_flags(layout)))
        orc = oracle_mod.quant_2d(x, layout)
        if layout & ROW:
            assert_exact(name + "/q_row", gpu[0], orc[0])
            assert_exact(name + "/s_row", gpu[1], orc[1])
        if layout & COL:
            assert_exact(name + "/q_col", gpu[2], orc[2])
            assert_exact(name + "/s_col", gpu[3], orc[3])
        return
    inp = synth.swiglu_inputs(M, W, seed=c["seed"], std=3.0)
    g, u, dh = (torch_bf16_to_bits(t) for t in (inp.gate, inp.up, inp.dh))
    g_d, u_d = _w13(g, u, pad, dev)
    oa = oracle_mod.ACTS[act]
    if op == "swiglu_fwd":
        outs = mx.mxfp8_swiglu_fwd(g_d, u_d, **_flags(layout))
        orc, vals = oracle_mod.swiglu_fwd(g, u, layout), oracle_mod.swiglu_fwd_values(g, u)
    elif op == "gated_fwd":
        outs = mx.mxfp8_gated_fwd(g_d, u_d, act=act, **_flags(layout))
        orc, vals = oracle_mod.gated_fwd(g, u, layout, oa), oracle_mod.gated_fwd_values(g, u, oa)
    elif op == "swiglu_bwd":
        outs = mx.mxfp8_swiglu_bwd(_padded(dh, pad, dev), g_d, u_d, **_flags(layout))
        orc = oracle_mod.swiglu_bwd(dh, g, u, layout)
        vals = np.concatenate(oracle_mod.swiglu_bwd_values(dh, g, u), axis=1)
    else:
        outs = mx.mxfp8_gated_bwd(_padded(dh, pad, dev), g_d, u_d, act=act, **_flags(layout))
        orc = oracle_mod.gated_bwd(dh, g, u, layout, oa)
        vals = np.concatenate(oracle_mod.gated_bwd_values(dh, g, u, oa), axis=1)
    compare_fused(oracle_mod, name, _gpu(outs), orc, vals, layout)


@pytest.mark.gpu
@pytest.mark.parametrize("idx", range(12))
def test_random_3d_case(oracle_mod, idx):
    """The 3D per-expert colwise cast ("[mxfp8 moe training] update 3d quant
    colwise scaling kernel ...", Summary) on a drawn expert count, shape and
    padded expert and row strides: bit-exact against the oracle."""
    dev = _dev()
    rng = np.random.default_rng(9500 + idx)
    E, N, K = int(rng.integers(1, 13)), 32 * int(rng.integers(1, 13)), 8 * int(rng.integers(1, 41))
    pn, pk = int(rng.integers(0, 3)), 8 * int(rng.integers(0, 3))
    print(f"case 3d {idx}: E={E} N={N} K={K} row pad {pk} expert pad {pn} rows", flush=True)
    w = torch_bf16_to_bits(synth.expert_weights(E, N + pn, K + pk, seed=int(rng.integers(1 << 30)), std=1.0))
    w_dev = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev)[:, :N, :K]
    q, s_ = mx.mxfp8_quant_3d_colwise(w_dev)
    qo, so = oracle_mod.quant_3d_colwise(np.ascontiguousarray(w[:, :N, :K]))
    assert_exact(f"q3d#{idx}", q.cpu().numpy(), qo)
    assert_exact(f"s3d#{idx}", s_.cpu().numpy(), so)


@pytest.mark.gpu
@pytest.mark.parametrize("idx", range(12))
def test_random_grouped_cast(oracle_mod, idx):
    """The casts with token groups on drawn group ends (sorted or not, some
    negative, some past the end, empty groups, up to 80 groups): every
    output equals the ungrouped cast's, and the colwise scales sit where
    the oracle's per-group padded layout puts them."""
    from test_gpu_grouped import _expected_padded
    dev = _dev()
    rng = np.random.default_rng(9700 + idx)
    kind = ("quant", "fwd", "bwd")[idx % 3]
    M, N, G = 32 * int(rng.integers(1, 400)), 32 * int(rng.integers(1, 6)), int(rng.integers(1, 81))
    ends = np.sort(rng.integers(-40, M + 100, G))
    if rng.random() < 0.3:
        rng.shuffle(ends)
    offs = [int(e) for e in ends]
    print(f"case grouped {idx}: {kind} M={M} N={N} G={G}", flush=True)
    offs_t = torch.tensor(offs, dtype=torch.int32, device=dev)
    inp = synth.swiglu_inputs(M, N, seed=int(rng.integers(1 << 30)), std=2.0, device=dev)
    if kind == "quant":
        grouped = mx.mxfp8_quant_2d_grouped(inp.gate, offs_t, rowwise=True, colwise=True)
        plain = mx.mxfp8_quant_2d(inp.gate, rowwise=True, colwise=True)
    elif kind == "fwd":
        grouped = mx.mxfp8_gated_fwd_grouped(inp.gate, inp.up, offs_t, rowwise=True, colwise=True)
        plain = mx.mxfp8_swiglu_fwd(inp.gate, inp.up, rowwise=True, colwise=True)
    else:
        grouped = mx.mxfp8_gated_bwd_grouped(inp.dh, inp.gate, inp.up, offs_t, rowwise=True, colwise=True)
        plain = mx.mxfp8_swiglu_bwd(inp.dh, inp.gate, inp.up, rowwise=True, colwise=True)
    for i, name in ((0, "q_row"), (1, "q_col"), (2, "s_row")):
        assert torch.equal(grouped[i], plain[i]), name
    s_pad = grouped[3].cpu().numpy()
    assert s_pad.shape[1] == M // 32 + 16 * G
    assert_exact(f"s_col padded#{idx}", s_pad, _expected_padded(oracle_mod, plain[3].cpu().numpy(), M, offs, s_pad.shape[1]))


@pytest.mark.gpu
@pytest.mark.parametrize("idx", range(10))
def test_random_grouped_gemm_k(oracle_mod, idx):
    """The K-grouped GEMM (the weight gradient over token groups) on drawn
    token counts and group ends, through the same check as its fixed cases
    (every group against the oracle, empty groups zero)."""
    from test_gpu_grouped import test_grouped_gemm_k_random as check_case
    rng = np.random.default_rng(9900 + idx)
    T, G = 32 * int(rng.integers(1, 121)), int(rng.integers(1, 13))
    ends = np.sort(rng.integers(-40, T + 100, G))
    if rng.random() < 0.3:
        rng.shuffle(ends)
    check_case(oracle_mod, T, [int(e) for e in ends])


def test_cases_reach_every_band():
    """Every (operation, layout) pair runs past 128 row tiles (bands of 32
    for both layouts, 128 for colwise only) with a ragged last band, and
    with at most 128 row tiles; the shapes leave ragged last tiles."""
    cs = [draw(i) for i in range(N_CASES)]
    assert len({(c["op"], c["layout"], c["bucket"]) for c in cs}) == N_CASES
    for c in cs:
        n_rt = -(-c["M"] // 128)
        if c["bucket"] == BUCKETS[2]:
            assert n_rt > 128 and n_rt % (32 if c["layout"] == BOTH else 128) != 0, c
        else:
            assert n_rt <= 128, c
    assert sum(c["M"] % 128 != 0 for c in cs) > N_CASES // 2
    assert sum(c["W"] % 128 != 0 for c in cs) > N_CASES // 2
