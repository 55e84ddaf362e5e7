"""Pins of the oracle's token-group pieces: the group bounds, the per-group
padded layout of colwise scales, and the K-grouped (weight-gradient) MX GEMM.

"[mxfp8 moe training] add compile support", Perf analysis (the grouped GEMMs
of a mixture-of-experts step, the weight gradient contracting over each
expert's tokens) and Summary with its review comments (per-group scale
buffers sized by an upper bound on their padding).  The pages fix no
layout; the padded positions are this build's reading, pinned here by the
properties that make them usable (every group's run starts on a 16-byte
boundary, runs never overlap, the upper bound T/32 + 16 G holds, the
relayout loses nothing) rather than by restating their formula.  The GEMM
is pinned against the plain (ungrouped) GEMM, which has its own pins, and
against an independent decode with numpy's float64 matmul.
"""
import numpy as np
import pytest
import torch


def _dequant_torch(q, s):
    """Independent decode: torch's E4M3 cast, times 2^(s - 127) per 32-block."""
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v * np.ldexp(1.0, np.repeat(s.astype(np.int64), 32, axis=1) - 127)


def _rand_codes(rng, rows, T):
    codes = rng.integers(0, 256, (rows, T)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    return codes


def _rand_offsets(rng, T, G, valid):
    if valid:
        return np.sort(rng.integers(0, T // 32 + 1, G) * 32).astype(np.int32)
    return rng.integers(-100, T + 200, G).astype(np.int32)


def test_group_bounds_worked_example(oracle_mod):
    """Ends 100, 64, 300, 2000 over T = 512 tokens: 100 rounds down to 96;
    64 rounds to 64 and is lifted to 96 (ends never decrease); 300 rounds to
    288; 2000 is capped at 512; the tail group [512, 512) is empty."""
    st, en = oracle_mod.group_bounds([100, 64, 300, 2000], 512)
    assert st.tolist() == [0, 96, 96, 288, 512]
    assert en.tolist() == [96, 96, 288, 512, 512]
    st, en = oracle_mod.group_bounds([-5, 40], 128)
    assert st.tolist() == [0, 0, 32] and en.tolist() == [0, 32, 128]


@pytest.mark.parametrize("valid", [True, False])
def test_padded_layout_properties(oracle_mod, valid):
    rng = np.random.default_rng(1 if valid else 2)
    for trial in range(300):
        T = int(rng.integers(0, 80)) * 32
        G = int(rng.integers(1, 40))
        offs = _rand_offsets(rng, T, G, valid) if T else np.zeros(G, np.int32)
        st, en = oracle_mod.group_bounds(offs, T)
        assert st[0] == 0 and en[-1] == T and np.all(st[1:] == en[:-1]) and np.all(en >= st)
        assert np.all(st % 32 == 0) and np.all(en % 32 == 0)
        prev_end = 0
        for g in range(G + 1):
            base = oracle_mod.group_scale_base(g, st[g])
            nb = (en[g] - st[g]) // 32
            assert base % 16 == 0, (trial, g)
            assert base >= prev_end, (trial, g)  # after the previous group's last block
            prev_end = base + nb
        assert prev_end <= T // 32 + 16 * G
        # lossless: block b of the plain row lands exactly once, in its group
        nblk = T // 32
        s = (np.arange(nblk) % 251 + 1).astype(np.uint8)[None].repeat(2, 0)
        s[1] = 255 - s[1]
        out = oracle_mod.pad_group_scales(s, T, offs, fill=0)
        assert out.shape == (2, T // 32 + 16 * G)
        used = np.zeros(out.shape[1], bool)
        for g in range(G + 1):
            base = oracle_mod.group_scale_base(g, st[g])
            for b in range(st[g] // 32, en[g] // 32):
                p = base + b - st[g] // 32
                assert not used[p]
                used[p] = True
                assert out[0, p] == s[0, b] and out[1, p] == s[1, b]
        assert used.sum() == nblk and np.all(out[:, ~used] == 0)


def test_one_group_is_the_plain_layout(oracle_mod):
    rng = np.random.default_rng(3)
    s = rng.integers(0, 256, (5, 24)).astype(np.uint8)
    out = oracle_mod.pad_group_scales(s, 768, [768], fill=7)
    assert np.array_equal(out[:, :24], s) and np.all(out[:, 24:] == 7)


def test_pad_rejects_a_short_row(oracle_mod):
    s = np.zeros((2, 4), np.uint8)
    with pytest.raises(ValueError):
        oracle_mod.pad_group_scales(s, 128, [64, 128], ld_out=4 + 31)


def _padded_operands(oracle_mod, rng, rows, T, offs):
    codes = _rand_codes(rng, rows, T)
    plain = rng.integers(118, 137, (rows, T // 32)).astype(np.uint8)
    return codes, plain, oracle_mod.pad_group_scales(plain, T, offs, fill=0)


def test_grouped_k_one_group_equals_the_plain_gemm(oracle_mod):
    rng = np.random.default_rng(4)
    T = 320
    a, sa, sap = _padded_operands(oracle_mod, rng, 19, T, [T])
    b, sb, sbp = _padded_operands(oracle_mod, rng, 23, T, [T])
    c, cabs = oracle_mod.mx_grouped_gemm_k(a, sap, b, sbp, [T])
    c0, cabs0 = oracle_mod.mx_gemm(a, sa, b, sb)
    assert np.array_equal(c[0], c0) and np.array_equal(cabs[0], cabs0)


def test_grouped_k_against_independent_decode(oracle_mod):
    """Each group's result is the float64 product of the decoded columns of
    that group (torch's E4M3 decode, plain scales), empty groups are zero,
    and the groups together sum to the plain GEMM over all grouped tokens."""
    rng = np.random.default_rng(5)
    T = 640
    for offs in ([64, 64, 320, 608], [0, 640], [96, 50, 700], [-3, 128, 128, 1000]):
        a, sa, sap = _padded_operands(oracle_mod, rng, 21, T, offs)
        b, sb, sbp = _padded_operands(oracle_mod, rng, 17, T, offs)
        c, cabs = oracle_mod.mx_grouped_gemm_k(a, sap, b, sbp, offs)
        va, vb = _dequant_torch(a, sa), _dequant_torch(b, sb)
        st, en = oracle_mod.group_bounds(offs, T)
        total = np.zeros((21, 17))
        for g in range(len(offs)):
            want = va[:, st[g]:en[g]] @ vb[:, st[g]:en[g]].T
            mag = np.abs(va[:, st[g]:en[g]]) @ np.abs(vb[:, st[g]:en[g]]).T
            assert np.all(np.abs(c[g] - want) <= 1e-12 * mag + 1e-300), (offs, g)
            assert np.allclose(cabs[g], mag, rtol=1e-12, atol=0)
            if en[g] == st[g]:
                assert np.all(c[g] == 0)
            total += c[g]
        full, fmag = oracle_mod.mx_gemm(a[:, :en[-2]], sa[:, :en[-2] // 32], b[:, :en[-2]], sb[:, :en[-2] // 32])
        assert np.all(np.abs(total - full) <= 1e-12 * fmag)
