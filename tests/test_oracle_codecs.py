"""Pins of the oracle's number formats against things other than itself.

Each check ties one oracle routine to a library routine (torch's CPU casts),
to closed forms from the format definitions (tests/golden), or to brute
force.  Formats named on "Add swiglu + MXFP8 fused CuTe DSL kernel"
(Summary; Numerics and tests; commit message).
"""
import math
import os

import numpy as np
import pytest
import torch

from helpers import all_bf16_bits, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_value(tok: str) -> float:
    if "p" in tok and not tok.startswith("0x"):
        m, e = tok.split("p")
        return math.ldexp(float(m), int(e))
    return float(tok)


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((parts[0], parts[1]))
    return rows


# ------------------------------------------------------------------- bf16
def test_bf16_decode_matches_torch_all_patterns(oracle_mod):
    bits = all_bf16_bits()
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    lib = oracle_mod.lib()
    got = np.array([lib.orc_bf16_decode(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    # signs of zeros too
    assert math.copysign(1.0, oracle_mod.bf16_decode(0x8000)) == -1.0


def test_bf16_round_matches_torch_on_float32_inputs(oracle_mod):
    rng = np.random.default_rng(11)
    # float32 values across the whole range, including subnormals and near-overflow
    raw = rng.integers(0, 2**32, size=40000, dtype=np.uint64).astype(np.uint32)
    vals = raw.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # add values that sit exactly on bf16 rounding midpoints
    mid = (all_bf16_bits().astype(np.uint32) << 16 | 0x8000).view(np.float32)
    vals = np.concatenate([vals, mid[np.isfinite(mid)]])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lib = oracle_mod.lib()
    got = np.array([lib.orc_bf16_round(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_bf16_round_closed_forms(oracle_mod):
    r = oracle_mod.bf16_round
    assert r(1.0 + 2**-8) == 0x3F80                 # tie -> even (1.0)
    assert r(1.0 + 2**-7 + 2**-8) == 0x3F82         # tie from odd 0x3F81 -> even 0x3F82
    assert r(1.0 + 2**-8 + 2**-30) == 0x3F81        # just above the tie rounds up
    assert r(math.ldexp(255, 120)) == 0x7F7F        # largest finite
    assert r(math.ldexp(255.5, 120)) == 0x7F80      # tie above the largest finite -> Inf
    assert r(-math.ldexp(256, 120)) == 0xFF80
    assert r(2.0**-133) == 0x0001                   # smallest subnormal
    assert r(2.0**-134) == 0x0000                   # tie with zero -> even (zero)
    assert r(3 * 2.0**-134) == 0x0002               # tie between 1 and 2 quanta -> 2
    assert r(-2.0**-140) == 0x8000                  # underflow keeps the sign
    assert r(float("nan")) == 0x7FC0
    assert r(float("-inf")) == 0xFF80


# ------------------------------------------------------------------- E4M3
def test_e4m3_decode_matches_torch_all_codes(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle_mod.e4m3_decode(int(c)) for c in codes])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.nanmax(got) == 448.0
    assert np.sum(np.isnan(got)) == 2


def test_e4m3_golden_points(oracle_mod):
    rows = _golden("e4m3_points.txt")
    assert len(rows) >= 15
    for v, code in rows:
        val = float(v)
        assert oracle_mod.e4m3_encode(val) == int(code, 16), (v, code)


def test_e4m3_encode_matches_torch_exhaustive_bf16_times_scales(oracle_mod):
    """Every finite bf16 value times 2^s (s in -10..10) against torch's cast.

    torch's float8_e4m3fn cast rounds to nearest-even but returns NaN above
    464 instead of saturating, so values above 464 are checked separately.
    """
    lib = oracle_mod.lib()
    bits = all_bf16_bits()
    base = bf16_bits_to_f32(bits).astype(np.float64)
    base = base[np.isfinite(base)]
    rng = np.random.default_rng(5)
    for s in range(-10, 11):
        v = base * 2.0**s
        v = v[np.abs(v) < 2.0**-12 + 600]  # keep the interesting range plus saturation
        sub = v if v.size <= 6000 else rng.choice(v, 6000, replace=False)
        sub = np.concatenate([sub, v[(np.abs(v) > 400) & (np.abs(v) < 600)]])
        got = np.array([lib.orc_e4m3_encode(float(x)) for x in sub], dtype=np.uint8)
        f32 = sub.astype(np.float32)
        assert (f32.astype(np.float64) == sub).all()
        ref = torch.from_numpy(f32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        inrange = np.abs(sub) <= 464  # 464 is the tie that rounds down to 448
        assert (got[inrange] == ref[inrange]).all(), s
        sat = ~inrange
        assert (got[sat] & 0x7F == 0x7E).all()
        assert ((got[sat] & 0x80) == np.where(sub[sat] < 0, 0x80, 0)).all()


def test_e4m3_encode_is_nearest_by_brute_force(oracle_mod):
    table = np.array([oracle_mod.e4m3_decode(c) for c in range(256)])
    finite = [c for c in range(256) if not np.isnan(table[c])]
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.uniform(-450, 450, 3000),
        rng.uniform(-0.05, 0.05, 3000),
        np.ldexp(rng.uniform(-1, 1, 2000), rng.integers(-12, 9, 2000)),
    ])
    for v in vals:
        c = oracle_mod.e4m3_encode(float(v))
        d = abs(table[c] - v)
        best = min(abs(table[k] - v) for k in finite)
        assert d == best, (v, c)
        if v != 0:
            assert (c & 0x80 != 0) == (v < 0)
    assert oracle_mod.e4m3_encode(float("nan")) == 0x7F


# ------------------------------------------------------------------- E8M0
def test_e8m0_golden_points(oracle_mod):
    for v, b in _golden("e8m0_points.txt"):
        assert oracle_mod.e8m0_rceil(_parse_value(v)) == int(b), (v, b)


def test_e8m0_rceil_matches_closed_form_for_every_bf16_amax(oracle_mod):
    """Closed form 2^ceil(log2(amax/448)), clamped to the E8M0 range, with
    numpy's float64 log2.  The float64 quotient amax/448 never lands on a
    power of two unless it is exactly one (a bf16 amax is (1 + m/128) 2^e and
    (1 + m/128)/1.75 is a power of two only for m = 96), and log2 is exact
    at powers of two, so the ceiling is exact."""
    bits = all_bf16_bits()[:0x7F80]  # +0 .. largest finite
    amax = bf16_bits_to_f32(bits).astype(np.float64)
    with np.errstate(divide="ignore"):
        k = np.ceil(np.log2(amax / 448.0))
    ref = np.clip(k + 127, 0, 254).astype(np.uint8)
    lib = oracle_mod.lib()
    got = np.array([lib.orc_e8m0_rceil(float(a)) for a in amax], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(amax[i]), got[i], ref[i]) for i in bad[:5]]
    # torch's float8_e8m0fnu cast rounds to the nearest power of two, so it
    # agrees with RCEIL exactly where amax/448 is already a power of two.
    pw = np.ldexp(1.0, np.arange(-126, 120)).astype(np.float32)
    tref = torch.from_numpy(pw).to(torch.float8_e8m0fnu).view(torch.uint8).numpy()
    tgot = np.array([oracle_mod.e8m0_rceil(float(p) * 448.0) for p in pw], dtype=np.uint8)
    assert (tgot == tref).all()


def test_e8m0_minimality_brute_force(oracle_mod):
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        np.ldexp(rng.uniform(0, 2, 3000), rng.integers(-140, 128, 3000)),
        np.ldexp(448.0, np.arange(-127, 128)).astype(np.float64),
    ])
    for a in vals:
        b = oracle_mod.e8m0_rceil(float(a))
        assert 0 <= b <= 254
        scale = math.ldexp(1.0, b - 127)
        assert a <= 448.0 * scale
        if b > 0:
            assert a > 448.0 * scale / 2


def test_e8m0_decode(oracle_mod):
    assert oracle_mod.e8m0_decode(127) == 1.0
    assert oracle_mod.e8m0_decode(0) == 2.0**-127
    assert math.isnan(oracle_mod.e8m0_decode(255))


# ------------------------------------------------------------------ blocks
def _descale(b):
    return math.ldexp(1.0, 127 - b)


def test_block_quant_brute_force_dequantize(oracle_mod):
    """Tiny random blocks: minimal scale, every scaled value within +-448,
    every code the nearest E4M3 value of the scaled element."""
    table = np.array([oracle_mod.e4m3_decode(c) for c in range(256)])
    finite = np.array([c for c in range(256) if not np.isnan(table[c])])
    rng = np.random.default_rng(9)
    for trial in range(300):
        mag = 2.0 ** rng.integers(-135, 120)
        y = rng.standard_normal(32) * mag
        if trial % 7 == 0:
            y[rng.integers(0, 32, 5)] = 0.0
        y = np.array([oracle_mod.bf16_decode(oracle_mod.bf16_round(v)) for v in y])
        q, b = oracle_mod.quant_block(y)
        amax = np.abs(y).max()
        assert amax <= 448 * math.ldexp(1.0, b - 127)
        assert b == 0 or amax > 448 * math.ldexp(1.0, b - 128)
        scaled = y * _descale(b)
        assert np.abs(scaled).max() <= 448
        for v, c in zip(scaled, q):
            best = np.min(np.abs(table[finite] - v))
            assert abs(table[c] - v) == best


def test_block_special_values(oracle_mod):
    y = np.ones(32)
    y[3] = np.nan
    q, b = oracle_mod.quant_block(y)
    assert b == 255 and (q == 0x7F).all()
    y = np.ones(32)
    y[31] = -np.inf
    q, b = oracle_mod.quant_block(y)
    assert b == 255 and (q == 0x7F).all()
    y = np.zeros(32)
    y[::2] = -0.0
    q, b = oracle_mod.quant_block(y)
    assert b == 0
    assert (q[::2] == 0x80).all() and (q[1::2] == 0x00).all()
    # amax exactly a power of two: that element's code is 256 (0x78)
    y = np.full(32, 0.25)
    y[0] = 4.0
    q, b = oracle_mod.quant_block(y)
    assert b == 119 + 2 and q[0] == 0x78
    # amax at the E4M3 boundary 448 * 2^k: scale 2^k, code 0x7E
    y = np.zeros(32)
    y[5] = -448 * 2.0**-3
    q, b = oracle_mod.quant_block(y)
    assert b == 124 and q[5] == 0xFE
    # subnormal-tiny: byte-0 scale descales by 2^127
    y = np.zeros(32)
    y[0] = 2.0**-133
    q, b = oracle_mod.quant_block(y)
    assert b == 0 and q[0] == oracle_mod.e4m3_encode(2.0**-6) == 0x08


def test_quant_block_at_matches_quant_block(oracle_mod):
    rng = np.random.default_rng(2)
    for _ in range(50):
        y = rng.standard_normal(32) * 10
        q, b = oracle_mod.quant_block(y)
        assert (oracle_mod.quant_block_at(y, b) == q).all()
