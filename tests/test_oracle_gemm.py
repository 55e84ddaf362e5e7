"""Pins of the oracle's MX GEMM (C = A B^T of MXFP8 operands stored with K
contiguous), the consumer the casts produce operands for ("[mxfp8 moe
training] add compile support", Perf analysis: a scaled grouped GEMM on the
cast outputs; "Add swiglu + MXFP8 fused CuTe DSL kernel", Summary).

Each pin is fixed by the MX definition, not by the oracle's own code:
closed forms (all-ones blocks, identity operands, power-of-two scale
shifts), an independent decode path (torch's float8_e4m3fn cast) feeding
numpy's float64 matmul, symmetry C(A, B) = C(B, A)^T, and NaN propagation
from a NaN code or a NaN scale.
"""
import numpy as np
import pytest
import torch

ONE = 0x38  # E4M3 1.0


def _dequant_torch(q, s):
    """Independent decode: torch's E4M3 cast, times 2^(s - 127) per 32-block."""
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    scale = np.ldexp(1.0, np.repeat(s.astype(np.int64), 32, axis=1) - 127)
    return v * scale


def _rand_operands(rng, rows, K, lo=120, hi=135):
    codes = rng.integers(0, 256, (rows, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A  # no NaN codes here
    scales = rng.integers(lo, hi, (rows, K // 32)).astype(np.uint8)
    return codes, scales


def test_all_ones_closed_form(oracle_mod):
    M, N, K = 5, 7, 96
    a = np.full((M, K), ONE, np.uint8)
    b = np.full((N, K), ONE, np.uint8)
    for ea, eb in ((127, 127), (130, 120), (0, 254), (140, 100)):
        c, cabs = oracle_mod.mx_gemm(a, np.full((M, 3), ea, np.uint8), b, np.full((N, 3), eb, np.uint8))
        want = K * 2.0 ** (ea - 127) * 2.0 ** (eb - 127)
        assert (c == want).all() and (cabs == want).all()


def test_identity_operand_returns_the_other(oracle_mod):
    """A = I (code 1.0 on the diagonal, scale 2^0): C[m][n] = value of B[n][m]."""
    rng = np.random.default_rng(1)
    K = 64
    a = np.zeros((K, K), np.uint8)
    np.fill_diagonal(a, ONE)
    sa = np.full((K, K // 32), 127, np.uint8)
    b, sb = _rand_operands(rng, 9, K)
    c, _ = oracle_mod.mx_gemm(a, sa, b, sb)
    assert np.array_equal(c, _dequant_torch(b, sb).T)


def test_against_independent_decode_and_matmul(oracle_mod):
    rng = np.random.default_rng(2)
    for M, N, K in ((3, 4, 32), (17, 9, 160), (33, 40, 512)):
        a, sa = _rand_operands(rng, M, K)
        b, sb = _rand_operands(rng, N, K)
        c, cabs = oracle_mod.mx_gemm(a, sa, b, sb)
        da, db = _dequant_torch(a, sa), _dequant_torch(b, sb)
        ref = da @ db.T
        # both sums of exact products in double: they differ by rounding only
        assert np.all(np.abs(c - ref) <= 1e-13 * cabs)
        assert np.allclose(cabs, np.abs(da) @ np.abs(db).T, rtol=1e-13, atol=0)


def test_scale_shift_doubles_exactly(oracle_mod):
    rng = np.random.default_rng(3)
    a, sa = _rand_operands(rng, 6, 128)
    b, sb = _rand_operands(rng, 5, 128)
    c, _ = oracle_mod.mx_gemm(a, sa, b, sb)
    sa2 = sa.copy()
    sa2[2] += 1  # every block of row 2 doubles
    c2, _ = oracle_mod.mx_gemm(a, sa2, b, sb)
    assert np.array_equal(c2[2], 2 * c[2])
    assert np.array_equal(np.delete(c2, 2, 0), np.delete(c, 2, 0))


def test_symmetry(oracle_mod):
    rng = np.random.default_rng(4)
    a, sa = _rand_operands(rng, 11, 96)
    b, sb = _rand_operands(rng, 13, 96)
    c, _ = oracle_mod.mx_gemm(a, sa, b, sb)
    ct, _ = oracle_mod.mx_gemm(b, sb, a, sa)
    assert np.array_equal(c, ct.T)


def test_nan_code_or_scale_poisons_its_row(oracle_mod):
    rng = np.random.default_rng(5)
    a, sa = _rand_operands(rng, 4, 64)
    b, sb = _rand_operands(rng, 3, 64)
    a[1, 40] = 0x7F          # NaN code
    sa[3, 0] = 255           # NaN scale
    c, _ = oracle_mod.mx_gemm(a, sa, b, sb)
    assert np.isnan(c[1]).all() and np.isnan(c[3]).all()
    assert np.isfinite(c[0]).all() and np.isfinite(c[2]).all()


def test_rejects_partial_blocks(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.lib()  # loaded
        c = np.zeros((1, 1))
        oracle_mod._check(oracle_mod.lib().orc_mx_gemm(0, 40, 0, 1, 0, 40, 0, 1, 1, 1, 40, c.ctypes.data, 1, 0, 1),
                          "mx_gemm")


def test_grouped_matches_independent_per_group_products(oracle_mod):
    """Grouped form: each group's rows against its own expert, checked with
    the independent decode; an empty group, and rows past the last offset
    left unwritten."""
    rng = np.random.default_rng(6)
    M, N, K, G = 90, 20, 96, 4
    a, sa = _rand_operands(rng, M, K)
    bs = [_rand_operands(rng, N, K) for _ in range(G)]
    b = np.stack([x[0] for x in bs])
    sb = np.stack([x[1] for x in bs])
    offs = np.array([17, 17, 60, 81], np.int32)  # group 1 empty; rows 81.. uncovered
    c, cabs = oracle_mod.mx_grouped_gemm(a, sa, b, sb, offs)
    da = _dequant_torch(a, sa)
    start = 0
    for g in range(G):
        end = offs[g]
        ref = da[start:end] @ _dequant_torch(b[g], sb[g]).T
        assert np.all(np.abs(c[start:end] - ref) <= 1e-13 * cabs[start:end])
        start = end
    assert np.isnan(c[81:]).all()


def test_grouped_offsets_are_clamped(oracle_mod):
    """Decreasing or too-large offsets are clamped into ordered groups
    within [0, M]: no row is read or written outside A and C."""
    rng = np.random.default_rng(7)
    M, N, K = 40, 8, 64
    a, sa = _rand_operands(rng, M, K)
    b, sb = _rand_operands(rng, 3 * N, K)
    b, sb = b.reshape(3, N, K), sb.reshape(3, N, K // 32)
    c, _ = oracle_mod.mx_grouped_gemm(a, sa, b, sb, np.array([25, 10, 1000], np.int32))
    # groups: [0, 25) expert 0, [25, 25) expert 1 (clamped up), [25, 40) expert 2 (clamped down)
    c0, _ = oracle_mod.mx_gemm(a[:25], sa[:25], b[0], sb[0])
    c2, _ = oracle_mod.mx_gemm(a[25:], sa[25:], b[2], sb[2])
    assert np.array_equal(c[:25], c0) and np.array_equal(c[25:], c2)
