"""Generates the erfc polynomial used by the exact-GELU gate (mx_ops.hpp).

For z >= 0 the kernel evaluates

    erfc(z) = t * exp(-z^2 + P(x)),   t = 2 / (2 + z),   x = 2t - 1 in (-1, 1],

the change of variable of Schonfelder's Chebyshev expansions of the error
function ("Chebyshev expansions for the error and related functions", Math.
Comp. 32, 1978), which maps the whole half-line onto one interval on which
P(x) = ln(erfcx(z) (2 + z) / 2) is smooth.  P is fitted here by least squares
on Chebyshev nodes in double precision (scipy's erfcx as the target),
converted to the power basis for Horner evaluation, and rounded to float32.

Run `python gen_erfc_fit.py` to print the constants; `tests/test_erfc_fit.py`
checks that the header holds exactly these values and bounds the float32
evaluation error.
"""
from __future__ import annotations

import numpy as np

DEGREE = 9
NODES = 40001


def fit(degree: int = DEGREE) -> tuple[np.ndarray, float]:
    """Power-basis coefficients (lowest first, float64) and the max fit error."""
    from scipy.special import erfcx

    x = np.cos(np.linspace(0.0, np.pi, NODES))
    x = x[x > -1.0 + 1e-12]                  # x = -1 is z = infinity
    z = 2.0 * (1.0 - x) / (1.0 + x)          # inverse of x = 4 / (2 + z) - 1
    y = np.log(erfcx(z) * (2.0 + z) / 2.0)
    cheb = np.polynomial.chebyshev.chebfit(x, y, degree)
    power = np.polynomial.chebyshev.cheb2poly(cheb)
    err = float(np.abs(np.polynomial.polynomial.polyval(x, power) - y).max())
    return power, err


def float32_coefficients(degree: int = DEGREE) -> list[float]:
    power, _ = fit(degree)
    return [float(np.float32(c)) for c in power]


def c_literals(degree: int = DEGREE) -> list[str]:
    """The coefficients as C hexadecimal float literals (exact float32 values)."""
    out = []
    for c in float32_coefficients(degree):
        mant, exp = c.hex().split("p")
        mant = mant.rstrip("0").rstrip(".")
        out.append(f"{mant}p{exp}f")
    return out


if __name__ == "__main__":
    _, err = fit()
    print(f"// degree {DEGREE}, max |fit error| {err:.2e} (absolute in P, relative in erfc)")
    print("constexpr float kErfcP[%d] = {%s};" % (DEGREE + 1, ", ".join(c_literals())))
