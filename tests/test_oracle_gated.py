"""Pins of the oracle's other gated activations: GELU (exact, x * Phi(x)),
GELU in the tanh form, and ReLU, each in place of silu in act(g) * up.

"Add swiglu + MXFP8 fused CuTe DSL kernel" (API) makes the activation a
compile-time policy; its Follow-ups plan more activations without naming
them, so these three are definitions taken here.  Checks: scipy's normal cdf
(Cephes, not the C library's erfc the oracle uses), torch's float64 GELU in
both forms and its autograd, textbook normal-cdf values, the identity
act(x) - act(-x) = x that holds for all four, central differences of the
derivative, and the eager bf16 CPU ops (exact for ReLU, which rounds
nothing but products of bf16 values).
"""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch
import torch.nn.functional as F

from helpers import all_bf16_bits, bf16_bits_to_f32, bits_to_torch_bf16, torch_bf16_to_bits

ACTS = ("silu", "gelu_tanh", "gelu", "relu")


def _xs(seed):
    rng = np.random.default_rng(seed)
    return np.concatenate([rng.standard_normal(3000) * 3, rng.uniform(-30, 30, 1000),
                           [0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 1e-30, -1e-30, 5.0, -5.0]])


def _torch_act(name, t):
    if name == "silu":
        return F.silu(t)
    if name == "gelu_tanh":
        return F.gelu(t, approximate="tanh")
    if name == "gelu":
        return F.gelu(t, approximate="none")
    return F.relu(t)


def test_gelu_is_x_times_normal_cdf(oracle_mod):
    """GELU(x) = x * Phi(x) against scipy's ndtr, including the far tail where
    1 + erf(x / sqrt 2) would cancel (the oracle uses erfc)."""
    xs = np.concatenate([_xs(1), -np.linspace(5, 37, 200)])
    for x in xs:
        ref = x * sps.ndtr(x)
        got = oracle_mod.act(oracle_mod.GELU, float(x))
        # Phi in the tail has condition number about x^2: an argument
        # rounding of 2^-53 alone moves it by x^2 * 2^-53 relative
        assert abs(got - ref) <= (4e-15 + 4e-16 * x * x) * abs(ref) + 1e-300, (x, got, ref)


def test_gelu_textbook_values(oracle_mod):
    """Phi(1) = 0.841344746068543, Phi(2) = 0.977249868051821 (normal tables);
    GELU(0) = 0 and GELU'(0) = 1/2."""
    G = oracle_mod.GELU
    for x, phi in ((1.0, 0.841344746068543), (2.0, 0.977249868051821)):
        assert oracle_mod.act(G, x) == pytest.approx(x * phi, rel=1e-14)
        assert oracle_mod.act(G, -x) == pytest.approx(-x * (1 - phi), rel=1e-13)
    assert oracle_mod.act(G, 0.0) == 0.0
    assert oracle_mod.act_grad(G, 0.0) == 0.5
    # GELU'(x) = Phi(x) + x phi(x); at 1: 0.841344746068543 + 0.241970724519143
    assert oracle_mod.act_grad(G, 1.0) == pytest.approx(0.841344746068543 + 0.241970724519143, rel=1e-14)


@pytest.mark.parametrize("name", ("gelu_tanh", "gelu"))
def test_gelu_forms_match_torch_float64(oracle_mod, name):
    """Both GELU forms against torch's float64 implementation (tanh form
    evaluated as 0.5 x (1 + tanh(.)), which cancels for negative x: an
    absolute allowance of a few double ulps of |x| covers that)."""
    a = oracle_mod.ACTS[name]
    xs = _xs(2)
    ref = _torch_act(name, torch.from_numpy(xs)).numpy()
    for x, r in zip(xs, ref):
        got = oracle_mod.act(a, float(x))
        assert abs(got - r) <= 4e-15 * abs(r) + 4e-16 * abs(x) + 1e-300, (name, x, got, r)


@pytest.mark.parametrize("name", ("gelu_tanh", "gelu"))
def test_gelu_derivatives_match_torch_autograd(oracle_mod, name):
    a = oracle_mod.ACTS[name]
    xs = _xs(3)
    t = torch.from_numpy(xs).requires_grad_(True)
    (grad,) = torch.autograd.grad(_torch_act(name, t).sum(), t)
    for x, r in zip(xs, grad.numpy()):
        got = oracle_mod.act_grad(a, float(x))
        assert abs(got - r) <= 1e-14 * abs(r) + 1e-14, (name, x, got, r)


def test_gelu_tanh_equals_the_tanh_formula_where_it_is_accurate(oracle_mod):
    """The oracle evaluates x * sigmoid(2 c (x + 0.044715 x^3)); the printed
    textbook form 0.5 x (1 + tanh(c (x + 0.044715 x^3))) agrees with it where
    1 + tanh does not cancel."""
    c = math.sqrt(2 / math.pi)
    for x in np.linspace(-3, 6, 301):
        ref = 0.5 * x * (1 + math.tanh(c * (x + 0.044715 * x ** 3)))
        assert oracle_mod.act(oracle_mod.GELU_TANH, float(x)) == pytest.approx(ref, rel=1e-13, abs=1e-15)


@pytest.mark.parametrize("name", ACTS)
def test_odd_part_identity(oracle_mod, name):
    """act(x) - act(-x) = x for all four (sigmoid(w) + sigmoid(-w) = 1,
    Phi(x) + Phi(-x) = 1, relu(x) - relu(-x) = x)."""
    a = oracle_mod.ACTS[name]
    for x in _xs(4):
        d = oracle_mod.act(a, float(x)) - oracle_mod.act(a, float(-x))
        assert d == pytest.approx(x, rel=1e-14, abs=1e-300), (name, x, d)


@pytest.mark.parametrize("name", ("silu", "gelu_tanh", "gelu"))
def test_derivative_central_difference(oracle_mod, name):
    a = oracle_mod.ACTS[name]
    rng = np.random.default_rng(5)
    for x in rng.standard_normal(400) * 3:
        h = 1e-5
        fd = (oracle_mod.act(a, x + h) - oracle_mod.act(a, x - h)) / (2 * h)
        assert oracle_mod.act_grad(a, float(x)) == pytest.approx(fd, rel=1e-8, abs=1e-9), (name, x)


def test_relu_closed_form(oracle_mod):
    R = oracle_mod.RELU
    for x in _xs(6):
        assert oracle_mod.act(R, float(x)) == max(float(x), 0.0)
        assert oracle_mod.act_grad(R, float(x)) == (1.0 if x > 0 else 0.0)
    assert math.copysign(1.0, oracle_mod.act(R, -0.0)) == 1.0  # +0
    assert math.isnan(oracle_mod.act(R, float("nan")))
    assert oracle_mod.act_grad(R, float("nan")) == 1.0  # NaN passes the gradient
    assert oracle_mod.act(R, float("-inf")) == 0.0


def test_silu_policy_equals_swiglu(oracle_mod):
    rng = np.random.default_rng(7)
    g, u, dh = (torch_bf16_to_bits(torch.from_numpy(rng.standard_normal(5000) * 3).to(torch.bfloat16))
                for _ in range(3))
    assert (oracle_mod.gated_fwd_values(g, u, oracle_mod.SILU) == oracle_mod.swiglu_fwd_values(g, u)).all()
    for a, b in zip(oracle_mod.gated_bwd_values(dh, g, u, oracle_mod.SILU), oracle_mod.swiglu_bwd_values(dh, g, u)):
        assert (a == b).all()


@pytest.mark.parametrize("name", ("gelu_tanh", "gelu", "relu"))
def test_values_vs_eager_bf16(oracle_mod, name):
    """Forward and backward values against eager torch bf16 on the CPU (which
    rounds the activation from float32): ReLU bit-exact; the GELUs within one
    bf16 step and on a small fraction of elements, for gates above -3 (below
    that eager float32 forms 1 + erf or 1 + tanh, which cancels)."""
    a = oracle_mod.ACTS[name]
    rng = np.random.default_rng(8)
    n = 30000
    g, u, dh = (torch_bf16_to_bits(torch.from_numpy(rng.standard_normal(n) * s).to(torch.bfloat16))
                for s in (2.5, 1.0, 1.0))
    h = oracle_mod.gated_fwd_values(g, u, a)
    dg, du = oracle_mod.gated_bwd_values(dh, g, u, a)
    gt = bits_to_torch_bf16(g).clone().requires_grad_(True)
    ut = bits_to_torch_bf16(u).clone().requires_grad_(True)
    ht = _torch_act(name, gt) * ut
    ht.backward(bits_to_torch_bf16(dh))
    keep = (bf16_bits_to_f32(g) > -3) if name != "relu" else np.ones(n, bool)
    for mine, eager, rate in ((h, torch_bf16_to_bits(ht.detach()), 2e-3), (dg, torch_bf16_to_bits(gt.grad), 5e-3),
                              (du, torch_bf16_to_bits(ut.grad), 2e-3)):
        mine, eager = mine[keep], eager[keep]
        steps = np.abs(mine.astype(np.int32) - eager.astype(np.int32))
        zero = ((mine & 0x7FFF) == 0) & ((eager & 0x7FFF) == 0)
        steps[zero] = 0
        if name == "relu":
            assert (steps == 0).all()
        else:
            assert steps.max() <= 1
            assert (steps > 0).mean() < rate


@pytest.mark.parametrize("name", ("gelu_tanh", "gelu"))
def test_exhaustive_gate_vs_eager_bf16(oracle_mod, name):
    """Every bf16 gate with u = 1: h = bf16(act(g)) within one step of eager
    bf16 (float32) wherever eager does not underflow or cancel."""
    a = oracle_mod.ACTS[name]
    g = all_bf16_bits()
    one = np.full_like(g, 0x3F80)
    got = oracle_mod.gated_fwd_values(g, one, a)
    ref = torch_bf16_to_bits(_torch_act(name, bits_to_torch_bf16(g)) * bits_to_torch_bf16(one))
    x = bf16_bits_to_f32(g)
    # eager CPU GELU returns NaN at +Inf; x * Phi(x) -> +Inf, which the oracle
    # (and IEEE Inf * 1) gives
    inf = x == np.inf
    assert bf16_bits_to_f32(got)[inf][0] == np.inf
    got, ref, x, g = got[~inf], ref[~inf], x[~inf], g[~inf]
    gv, rv = bf16_bits_to_f32(got), bf16_bits_to_f32(ref)
    assert (np.isnan(gv) == np.isnan(rv)).all()
    # eager float32 loses the negative tail (1 + erf / 1 + tanh cancel, or
    # underflow), flushes results in the subnormal range to 0 and overflows
    # an intermediate above about 1.7e38: compare where the gate is in
    # (-3, 1e38) and not within 1e-37 of 0
    ok = ~np.isnan(gv) & (x > -3) & (x < 1e38) & (np.abs(x) > 1e-37)
    steps = np.abs(got[ok].astype(np.int32) - ref[ok].astype(np.int32))
    zero = ((got[ok] & 0x7FFF) == 0) & ((ref[ok] & 0x7FFF) == 0)
    steps[zero] = 0
    assert steps.max() <= 1
    assert (steps > 0).mean() < 2e-3


@pytest.mark.parametrize("name", ACTS)
def test_fused_equals_plain_cast_of_values(oracle_mod, name):
    a = oracle_mod.ACTS[name]
    rng = np.random.default_rng(9)
    M, N = 64, 96
    g, u, dh = (torch_bf16_to_bits(torch.from_numpy(rng.standard_normal((M, N)) * 2).to(torch.bfloat16))
                for _ in range(3))
    fused = oracle_mod.gated_fwd(g, u, oracle_mod.BOTH, a)
    plain = oracle_mod.quant_2d(oracle_mod.gated_fwd_values(g, u, a), oracle_mod.BOTH)
    for x, y in zip(fused, plain):
        assert (x == y).all()
    fused = oracle_mod.gated_bwd(dh, g, u, oracle_mod.BOTH, a)
    dg, du = oracle_mod.gated_bwd_values(dh, g, u, a)
    plain = oracle_mod.quant_2d(np.concatenate([dg, du], axis=1), oracle_mod.BOTH)
    for x, y in zip(fused, plain):
        assert (x == y).all()


def test_unknown_activation_is_rejected(oracle_mod):
    g = np.zeros((32, 32), np.uint16)
    with pytest.raises(ValueError):
        oracle_mod.gated_fwd(g, g, oracle_mod.BOTH, 7)
    with pytest.raises(ValueError):
        oracle_mod.gated_fwd_values(g, g, -1)
