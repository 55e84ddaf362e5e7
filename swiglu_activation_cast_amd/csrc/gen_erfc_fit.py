"""Generates the erfc polynomials used by the exact-GELU gate (mx_ops.hpp).

For z >= 0 the kernel evaluates, with t = 2 / (2 + z), x = 2t - 1 in (-1, 1]
and u = x - 1 = 2t - 2 in (-2, 0],

    erfc(z) = t * exp(-z^2 + P(x))    (forward: one exponential)
    erfc(z) = t * exp(-z^2) * Q(x)    (backward: the exponential is shared
                                       with the Gaussian in the derivative)

the change of variable of Schonfelder's Chebyshev expansions of the error
function ("Chebyshev expansions for the error and related functions", Math.
Comp. 32, 1978), which maps the whole half-line onto one interval on which
Q(x) = erfcx(z) (2 + z) / 2 (between 1/(2 sqrt(pi)) and 1) and its logarithm
P(x) are smooth.  At z = 0 (x = 1) they are exactly Q = 1 and P = 0, and the
fits keep that exactly: each is written P = u R(u), Q = 1 + u R(u), so that
erfc(0) = 1 in float32 whatever the rounding of the coefficients (tiny gates
then give the cdf 1/2 exactly, as the definition does, and ties of g / 2 round
as the exact values do).  R is fitted by least squares on Chebyshev nodes of
x in double precision (scipy's erfcx as the target), expressed in powers of u
for Horner evaluation, and rounded to float32.

Run `python gen_erfc_fit.py` to print the constants; `tests/test_erfc_fit.py`
checks that the header holds exactly these values and bounds the float32
evaluation error.
"""
from __future__ import annotations

import numpy as np

DEGREE = {"P": 8, "Q": 7}
NODES = 40001


def fit(which: str = "P") -> tuple[np.ndarray, float]:
    """Power-basis coefficients in u (lowest first, float64) of R, with
    P = u R(u) or Q = 1 + u R(u), and the max fit error of P or Q once the
    coefficients are rounded to float32 (absolute in P, relative in Q:
    relative in erfc either way)."""
    from scipy.special import erfcx

    x = np.cos(np.linspace(0.0, np.pi, NODES))
    x = x[x > -1.0 + 1e-12]                  # x = -1 is z = infinity
    z = 2.0 * (1.0 - x) / (1.0 + x)          # inverse of x = 4 / (2 + z) - 1
    q = erfcx(z) * (2.0 + z) / 2.0
    y = np.log(q) if which == "P" else q - 1.0
    u = x - 1.0
    deg = DEGREE[which]                      # of P or Q; R has one less
    # y = u R(u), R in the Chebyshev basis of x: least squares on the nodes
    basis = np.stack([u * np.polynomial.chebyshev.chebval(x, np.eye(deg)[k]) for k in range(deg)], axis=1)
    cheb, *_ = np.linalg.lstsq(basis, y, rcond=None)
    r_x = np.polynomial.Polynomial(np.polynomial.chebyshev.cheb2poly(cheb))
    r_u = r_x(np.polynomial.Polynomial([1.0, 1.0])).coef  # R as a polynomial in u = x - 1
    r32 = r_u.astype(np.float32).astype(np.float64)
    val = u * np.polynomial.polynomial.polyval(u, r32)
    err = np.abs(val - y)
    return r_u, float((err if which == "P" else err / q).max())


def float32_coefficients(which: str = "P") -> list[float]:
    power, _ = fit(which)
    return [float(np.float32(c)) for c in power]


def c_literals(which: str = "P") -> list[str]:
    """The coefficients as C hexadecimal float literals (exact float32 values)."""
    out = []
    for c in float32_coefficients(which):
        mant, exp = c.hex().split("p")
        mant = mant.rstrip("0").rstrip(".")
        out.append(f"{mant}p{exp}f")
    return out


if __name__ == "__main__":
    for which in ("P", "Q"):
        _, err = fit(which)
        print(f"// {which}: degree {DEGREE[which]}, max fit error {err:.2e} (relative in erfc)")
        print("constexpr float kErfc%s[%d] = {%s};" % (which, DEGREE[which], ", ".join(c_literals(which))))
