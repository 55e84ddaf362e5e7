"""Pins of the oracle's SwiGLU forward/backward values.

The pages ("Add swiglu + MXFP8 fused CuTe DSL kernel", Numerics and tests)
fix the forward as the eager bf16 activation followed by the quantizer and
the backward as its autograd.  Checks here: torch's float64 sigmoid/silu and
autograd (library routines), a finite-difference derivative, closed-form
special cases, and the eager bf16 CPU ops (which round in float32, so they
may differ by one bf16 step on rare elements -- a low rate pins where the
roundings sit).
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

from helpers import all_bf16_bits, bf16_bits_to_f32, bits_to_torch_bf16, torch_bf16_to_bits


def _finite_bf16(rng, n, scale):
    x = torch.from_numpy(rng.standard_normal(n) * scale).to(torch.bfloat16)
    return torch_bf16_to_bits(x)


def test_sigmoid_silu_match_torch_float64(oracle_mod):
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.standard_normal(3000) * 4, rng.uniform(-700, 700, 1000),
                         [0.0, -0.0, 1e-300, -1e-300, 30.0, -30.0, -745.0, 709.0]])
    t = torch.from_numpy(xs)
    ref_sig = torch.sigmoid(t).numpy()
    ref_silu = F.silu(t).numpy()
    for x, rs, rl in zip(xs, ref_sig, ref_silu):
        s = oracle_mod.sigmoid(float(x))
        l = oracle_mod.silu(float(x))
        # torch underflows sigmoid to 0 below about -709; the oracle's stable
        # split keeps a subnormal there, so allow an absolute 1e-300 as well
        assert abs(s - rs) <= 2e-15 * abs(rs) + 1e-300, x
        assert abs(l - rl) <= 2e-15 * abs(rl) + 1e-300, x


def test_silu_special_values(oracle_mod):
    assert oracle_mod.silu(0.0) == 0.0
    assert math.isnan(oracle_mod.silu(float("-inf")))
    assert oracle_mod.silu(float("inf")) == float("inf")
    assert math.isnan(oracle_mod.silu(float("nan")))
    # far-negative gate: tiny but not zero (no overflow in the stable split)
    v = oracle_mod.silu(-95.0)
    assert v < 0 and abs(v - (-95.0 * math.exp(-95.0))) <= 1e-15 * abs(v)


def test_forward_values_match_float64_definition(oracle_mod):
    """h = bf16(bf16(silu(g)) * u) with torch's float64 silu and the oracle's
    pinned bf16 rounding: bit-exact."""
    rng = np.random.default_rng(2)
    g = _finite_bf16(rng, 20000, 3.0)
    u = _finite_bf16(rng, 20000, 1.0)
    got = oracle_mod.swiglu_fwd_values(g, u)
    g64 = torch.from_numpy(bf16_bits_to_f32(g).astype(np.float64))
    u64 = bf16_bits_to_f32(u).astype(np.float64)
    silu64 = F.silu(g64).numpy()
    s = np.array([oracle_mod.bf16_round(v) for v in silu64], dtype=np.uint16)
    ref = np.array([oracle_mod.bf16_round(v) for v in bf16_bits_to_f32(s) * u64], dtype=np.uint16)
    assert (got == ref).all()


def test_forward_values_vs_eager_bf16_exhaustive_gate(oracle_mod):
    """All 65536 bf16 gates with u = 1: h = bf16(silu(g)).  Eager torch CPU
    computes silu in float32, so a few rounding-boundary cases may differ by
    one bf16 step; NaN/Inf cases must agree."""
    g = all_bf16_bits()
    u = np.full_like(g, 0x3F80)  # 1.0
    got = oracle_mod.swiglu_fwd_values(g, u)
    ref = torch_bf16_to_bits(F.silu(bits_to_torch_bf16(g)) * bits_to_torch_bf16(u))
    gv = bf16_bits_to_f32(got).astype(np.float64)
    rv = bf16_bits_to_f32(ref).astype(np.float64)
    nan = np.isnan(gv) | np.isnan(rv)
    assert (np.isnan(gv) == np.isnan(rv)).all()
    diff = got[~nan] != ref[~nan]
    # one bf16 step apart at most
    steps = np.abs(got[~nan].astype(np.int32) - ref[~nan].astype(np.int32))
    # signs may only differ at zero (eager underflows far-negative gates to -0)
    far = bf16_bits_to_f32(g[~nan]) < -87
    assert (steps[~far] <= 1).all()
    rate = diff[~far].mean()
    assert rate < 2e-3, rate


def test_forward_rounding_sites_vs_eager_random(oracle_mod):
    """Random g, u: the oracle's two-rounding forward matches eager bf16 on
    nearly all elements.  A one-rounding variant would differ on a large
    fraction, so the low rate pins the intermediate rounding."""
    rng = np.random.default_rng(4)
    g = _finite_bf16(rng, 50000, 2.0)
    u = _finite_bf16(rng, 50000, 1.0)
    got = oracle_mod.swiglu_fwd_values(g, u)
    eager = torch_bf16_to_bits(F.silu(bits_to_torch_bf16(g)) * bits_to_torch_bf16(u))
    rate = (got != eager).mean()
    assert rate < 2e-3, rate
    # the single-rounding alternative, for contrast
    one = torch_bf16_to_bits((F.silu(bits_to_torch_bf16(g).float()) * bits_to_torch_bf16(u).float()).bfloat16())
    assert (one != eager).mean() > 20 * max(rate, 1e-4)


def test_backward_values_match_float64_autograd(oracle_mod):
    """du = bf16(dh * bf16(silu(g))), dg = bf16(bf16(dh * u) * silu'(g)) with
    silu' from torch's float64 autograd: bit-exact."""
    rng = np.random.default_rng(6)
    n = 20000
    g = _finite_bf16(rng, n, 3.0)
    u = _finite_bf16(rng, n, 1.0)
    dh = _finite_bf16(rng, n, 1.0)
    dg, du = oracle_mod.swiglu_bwd_values(dh, g, u)
    g64 = torch.from_numpy(bf16_bits_to_f32(g).astype(np.float64)).requires_grad_(True)
    u64 = bf16_bits_to_f32(u).astype(np.float64)
    dh64 = bf16_bits_to_f32(dh).astype(np.float64)
    rnd = np.vectorize(oracle_mod.bf16_round, otypes=[np.uint16])
    ds = rnd(dh64 * u64)
    (grad,) = torch.autograd.grad(F.silu(g64), g64, torch.from_numpy(bf16_bits_to_f32(ds).astype(np.float64)))
    dg_ref = rnd(grad.numpy())
    s = rnd(F.silu(g64.detach()).numpy())
    du_ref = rnd(dh64 * bf16_bits_to_f32(s))
    assert (du == du_ref).all()
    assert (dg == dg_ref).all()


def test_backward_derivative_finite_difference(oracle_mod):
    """silu'(g) recovered from the oracle's dg (ds = 1) against a central
    difference of the oracle's own silu, in double."""
    rng = np.random.default_rng(8)
    g = _finite_bf16(rng, 400, 3.0)
    one = np.full_like(g, 0x3F80)
    dg, _ = oracle_mod.swiglu_bwd_values(one, g, one)  # ds = bf16(1 * 1) = 1
    for gi, d in zip(bf16_bits_to_f32(g).astype(np.float64), bf16_bits_to_f32(dg).astype(np.float64)):
        h = 1e-5
        fd = (oracle_mod.silu(gi + h) - oracle_mod.silu(gi - h)) / (2 * h)
        # dg is fd rounded to bf16: within half a bf16 step plus fd error
        assert abs(d - fd) <= abs(fd) * 2**-8 + 1e-9, (gi, d, fd)


def test_backward_special_cases(oracle_mod):
    # g = 0: sigmoid = 1/2, silu = 0, silu' = 1/2
    zero = np.zeros(1, np.uint16)
    u = torch_bf16_to_bits(torch.tensor([3.0], dtype=torch.bfloat16))
    dh = torch_bf16_to_bits(torch.tensor([-1.5], dtype=torch.bfloat16))
    dg, du = oracle_mod.swiglu_bwd_values(dh, zero, u)
    assert du[0] in (0x0000, 0x8000)
    assert bf16_bits_to_f32(dg)[0] == np.float32(-4.5 * 0.5)


def test_backward_vs_eager_bf16_autograd(oracle_mod):
    rng = np.random.default_rng(10)
    n = 30000
    g = _finite_bf16(rng, n, 2.0)
    u = _finite_bf16(rng, n, 1.0)
    dh = _finite_bf16(rng, n, 1.0)
    dg, du = oracle_mod.swiglu_bwd_values(dh, g, u)
    gt = bits_to_torch_bf16(g).clone().requires_grad_(True)
    ut = bits_to_torch_bf16(u).clone().requires_grad_(True)
    (F.silu(gt) * ut).backward(bits_to_torch_bf16(dh))
    dg_e = torch_bf16_to_bits(gt.grad)
    du_e = torch_bf16_to_bits(ut.grad)
    assert (np.abs(dg.astype(np.int32) - dg_e.astype(np.int32)) <= 1).all()
    assert (np.abs(du.astype(np.int32) - du_e.astype(np.int32)) <= 1).all()
    assert (dg != dg_e).mean() < 5e-3
    assert (du != du_e).mean() < 2e-3
