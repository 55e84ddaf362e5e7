"""Structural invariants of the oracle's matrix-level routines.

Layouts from "Add swiglu + MXFP8 fused CuTe DSL kernel" (Summary: rowwise
1x32, colwise 32x1 or both in one pass; API: [gate | up] input, [dGate |
dUp] output; Numerics and tests: both-mode equals rowwise plus colwise) and
"[mxfp8 moe training] update 3d quant colwise scaling kernel to use single
input/output TMA descriptors" (Summary: column-major per expert).  The 3D
routine is a separate loop in the oracle, so its agreement with the 2D
colwise cast is a real check.
"""
import numpy as np
import torch

from helpers import torch_bf16_to_bits

ROW, COL, BOTH = 1, 2, 3


def _bf16(rng, shape, scale=1.0):
    return torch_bf16_to_bits(torch.from_numpy(rng.standard_normal(shape) * scale).to(torch.bfloat16))


def test_colwise_is_rowwise_of_transpose(oracle_mod):
    rng = np.random.default_rng(0)
    x = _bf16(rng, (96, 160), 3.0)
    _, _, q_col, s_col = oracle_mod.quant_2d(x, COL)
    q_row_t, s_row_t, _, _ = oracle_mod.quant_2d(np.ascontiguousarray(x.T), ROW)
    assert (q_col == q_row_t).all() and (s_col == s_row_t).all()


def test_both_equals_row_and_col(oracle_mod):
    rng = np.random.default_rng(1)
    g = _bf16(rng, (64, 96))
    u = _bf16(rng, (64, 96))
    dh = _bf16(rng, (64, 96))
    for fn, args in ((oracle_mod.quant_2d, (g,)), (oracle_mod.swiglu_fwd, (g, u)),
                     (oracle_mod.swiglu_bwd, (dh, g, u))):
        both = fn(*args, BOTH)
        row = fn(*args, ROW)
        col = fn(*args, COL)
        assert (both[0] == row[0]).all() and (both[1] == row[1]).all()
        assert (both[2] == col[2]).all() and (both[3] == col[3]).all()


def test_fused_forward_is_quant_of_values(oracle_mod):
    rng = np.random.default_rng(2)
    g = _bf16(rng, (64, 128), 2.0)
    u = _bf16(rng, (64, 128))
    h = oracle_mod.swiglu_fwd_values(g, u)
    fused = oracle_mod.swiglu_fwd(g, u, BOTH)
    plain = oracle_mod.quant_2d(h, BOTH)
    for a, b in zip(fused, plain):
        assert (a == b).all()


def test_fused_backward_is_quant_of_concatenated_grads(oracle_mod):
    rng = np.random.default_rng(3)
    g = _bf16(rng, (32, 64), 2.0)
    u = _bf16(rng, (32, 64))
    dh = _bf16(rng, (32, 64))
    dg, du = oracle_mod.swiglu_bwd_values(dh, g, u)
    y = np.concatenate([dg, du], axis=1)  # [dGate | dUp]
    fused = oracle_mod.swiglu_bwd(dh, g, u, BOTH)
    plain = oracle_mod.quant_2d(y, BOTH)
    for a, b in zip(fused, plain):
        assert (a == b).all()
    assert fused[0].shape == (32, 128) and fused[2].shape == (128, 32)


def test_w13_halves_equal_separate_tensors(oracle_mod):
    rng = np.random.default_rng(4)
    w13 = _bf16(rng, (64, 2 * 96))
    gate, up = w13[:, :96], w13[:, 96:]
    assert gate.strides[0] == 2 * 192  # a strided view, not a copy
    a = oracle_mod.swiglu_fwd(gate, up, BOTH)
    b = oracle_mod.swiglu_fwd(np.ascontiguousarray(gate), np.ascontiguousarray(up), BOTH)
    for x, y in zip(a, b):
        assert (x == y).all()


def test_3d_matches_2d_colwise_per_expert(oracle_mod):
    rng = np.random.default_rng(5)
    w = _bf16(rng, (3, 64, 40), 0.02)
    q, s = oracle_mod.quant_3d_colwise(w)
    assert q.shape == (3, 40, 64) and s.shape == (3, 40, 2)
    for e in range(3):
        _, _, q_col, s_col = oracle_mod.quant_2d(w[e], COL)
        assert (q[e] == q_col).all() and (s[e] == s_col).all()


def test_3d_with_padded_strides(oracle_mod):
    rng = np.random.default_rng(6)
    big = _bf16(rng, (2, 70, 48))
    w = big[:, :64, :40]  # stride_e = 70*48, ld_w = 48
    q, s = oracle_mod.quant_3d_colwise(w)
    q2, s2 = oracle_mod.quant_3d_colwise(np.ascontiguousarray(w))
    assert (q == q2).all() and (s == s2).all()


def test_rowwise_allows_ragged_row_count(oracle_mod):
    rng = np.random.default_rng(7)
    g = _bf16(rng, (37, 64))
    u = _bf16(rng, (37, 64))
    q, s, _, _ = oracle_mod.swiglu_fwd(g, u, ROW)
    q_full, s_full, _, _ = oracle_mod.swiglu_fwd(np.vstack([g, g[:27]]), np.vstack([u, u[:27]]), ROW)
    assert (q == q_full[:37]).all() and (s == s_full[:37]).all()


def test_special_value_blocks_in_a_matrix(oracle_mod):
    x = np.zeros((32, 64), np.uint16)
    x[0, 5] = 0x7FC0           # NaN: invalidates row block (0, 0) and column block 5
    x[3, 40] = 0xFF80          # -Inf: row block (3, 1) and column block 40
    x[10, 33] = 0x0001         # smallest subnormal alone in its column
    q_row, s_row, q_col, s_col = oracle_mod.quant_2d(x, BOTH)
    assert s_row[0, 0] == 255 and (q_row[0, :32] == 0x7F).all()
    assert s_row[0, 1] == 0 and (q_row[0, 32:] == 0).all()
    assert s_row[3, 1] == 255 and s_col[40, 0] == 255 and (q_col[40] == 0x7F).all()
    assert s_col[5, 0] == 255
    assert s_col[33, 0] == 0 and q_col[33, 10] == 0x08  # 2^-133 * 2^127 = 2^-6
    assert s_col[0, 0] == 0 and (q_col[0] == 0).all()


def test_rejects_bad_shapes(oracle_mod):
    import pytest

    x = np.zeros((40, 64), np.uint16)
    with pytest.raises(ValueError):
        oracle_mod.quant_2d(x, COL)        # colwise needs rows % 32 == 0
    with pytest.raises(ValueError):
        oracle_mod.swiglu_fwd(x[:, :48], x[:, :48], ROW)  # width % 32 != 0
