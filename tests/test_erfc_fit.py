"""The exact-GELU gate's erfc polynomials (host-side checks, no GPU).

- The constants in csrc/mx_ops.hpp are exactly what gen_erfc_fit.py prints.
- The kernel's float32 evaluation, emulated step by step in numpy float32,
  stays within 1e-5 relative of the normal cdf (scipy) for GELU's value
  over every finite bf16 gate whose result is a normal float, for the
  forward's form t e^(-z^2 + P(x)) and the backward's t e^(-z^2) Q(x)
  alike, and within 1e-4 (relative, absolute near its zero) for the
  derivative, which only the backward's form evaluates.  (The hardware
  exp2 and reciprocal carry about one ulp more than numpy's correctly
  rounded ones; the bounds leave room for that.)
"""
import importlib.util
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "swiglu_activation_cast_amd", "csrc")

scipy_special = pytest.importorskip("scipy.special")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_erfc_fit", os.path.join(CSRC, "gen_erfc_fit.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def header_coefficients(which="P"):
    text = open(os.path.join(CSRC, "mx_ops.hpp")).read()
    m = re.search(r"kErfc%s\[(\d+)\]\s*=\s*\{([^}]*)\}" % which, text)
    assert m, f"kErfc{which} not found in mx_ops.hpp"
    lits = [s.strip() for s in m.group(2).split(",")]
    assert len(lits) == int(m.group(1))
    return lits


@pytest.mark.parametrize("which,bound", [("P", 2e-6), ("Q", 6e-6)])
def test_header_constants_are_the_generated_fit(which, bound):
    gen = _gen()
    assert header_coefficients(which) == gen.c_literals(which)
    _, err = gen.fit(which)
    assert err < bound


def _emulate(which, g):
    """float32 steps of ActGelu: (act, derivative), each already rescaled.
    "P": the forward's act, t e^(-z^2 + P(x)) (its derivative is the same
    cdf plus a separate Gaussian); "Q": the backward's act and derivative,
    t e^(-z^2) Q(x) with e^(-z^2) shared with the Gaussian.  P = u R_P(u),
    Q = 1 + u R_Q(u) with u = x - 1, R_* the header's coefficients."""
    f32 = np.float32
    c = [f32(float.fromhex(s.rstrip("f"))) for s in header_coefficients(which)]
    l2e = f32(1.4426950408889634)
    with np.errstate(all="ignore"):
        far = g < f32(-8.0)
        sc = np.where(far, f32(64.0), f32(0.0)).astype(f32)
        th = (f32(1.0) / (f32(2.0) + np.abs(g) * f32(0.7071067811865476))).astype(f32)
        u = (th * f32(4.0) - f32(2.0)).astype(f32)  # x - 1
        r = np.full_like(u, c[-1])
        for ci in c[-2::-1]:
            r = (r * u + ci).astype(f32)
        gauss = np.exp2((((g * g).astype(f32) * f32(-0.5 * l2e)) + sc).astype(f32)).astype(f32)
        if which == "P":
            e = ((f32(-0.5) * g) * g + (u * r).astype(f32)).astype(f32)
            q = (th * np.exp2((e * l2e + sc).astype(f32))).astype(f32)
        else:
            q = ((th * (u * r + f32(1.0))).astype(f32) * gauss).astype(f32)
        cdf = np.where(g < 0, q, f32(1.0) - q).astype(f32)
        act = (g * cdf).astype(np.float64)
        grad = (cdf + g * (f32(0.3989422804014327) * gauss)).astype(np.float64)
    scale = np.where(far, 2.0 ** -64, 1.0)
    return act * scale, grad * scale


@pytest.mark.parametrize("which", ["P", "Q"])
def test_float32_evaluation_error_over_every_bf16_gate(which):
    bits = np.arange(65536, dtype=np.uint32)
    g = (bits << 16).view(np.float32)
    g = g[np.isfinite(g)]
    act, grad = _emulate(which, g)
    gd = g.astype(np.float64)
    cdf = scipy_special.ndtr(gd)
    want_act = gd * cdf
    want_grad = cdf + gd * np.exp(-0.5 * gd * gd) / np.sqrt(2.0 * np.pi)
    m = np.abs(want_act) > 1e-37
    rel = np.abs(act[m] - want_act[m]) / np.abs(want_act[m])
    assert rel.max() < 1e-5, rel.max()
    # below the normal range the result is a bf16 subnormal at most: absolute
    tiny = ~m
    assert np.abs(act[tiny] - want_act[tiny]).max() < 1e-42
    # the derivative crosses zero near g = -0.75: absolute error there.  Only
    # the backward (the Q form) evaluates the derivative; the forward's P
    # form computes the activation alone, so its derivative is not bounded.
    err = np.abs(grad - want_grad) / np.maximum(np.abs(want_grad), 1e-3)
    ok = np.abs(want_grad) > 1e-37
    if which == "Q":
        assert err[ok].max() < 1e-4, err[ok].max()
    print(f"  {which}: act max rel error {rel.max():.2e}, derivative {err[ok].max():.2e}")


def test_emulated_forward_casts_like_the_oracle_for_every_gate(oracle_mod):
    """The kernel's float32 forward (emulated), rounded to bf16 and cast by
    the oracle's quantizer, against the oracle's own exact forward for every
    finite bf16 gate (up = 1), 32 consecutive patterns per block: codes
    within one step, scales equal.  Subnormal gates make g Phi(g) = g / 2 a
    bf16 rounding tie, which only an exact cdf of 1/2 at g -> 0 rounds as
    the definition does."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = bits[(bits & 0x7FFF) < 0x7F80]
    fin = np.resize(fin, (fin.size // (32 * 64) + 1) * 32 * 64).reshape(-1, 64)
    g = (fin.astype(np.uint32) << 16).view(np.float32)
    act, _ = _emulate("P", g.ravel())
    a32 = act.reshape(g.shape).astype(np.float32)
    u = a32.view(np.uint32).astype(np.uint64)
    hb = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # bf16, round to nearest even
    one = np.full_like(fin, 0x3F80)
    exact = oracle_mod.gated_fwd(fin, one, 1, oracle_mod.ACTS["gelu"])
    emu = oracle_mod.quant_2d(hb, 1)
    assert np.array_equal(exact[1], emu[1])
    c_e = emu[0].astype(np.int32)
    c_o = exact[0].astype(np.int32)
    ord_e = np.where(c_e & 0x80, -(c_e & 0x7F), c_e & 0x7F)
    ord_o = np.where(c_o & 0x80, -(c_o & 0x7F), c_o & 0x7F)
    assert np.abs(ord_e - ord_o).max() <= 1
