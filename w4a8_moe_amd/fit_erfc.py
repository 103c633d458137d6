"""Generator of the erfc polynomial in csrc/common.h (gelu_erf's fast fp32 path).

The form is the one of the erfcc routine of Numerical Recipes: with z = |g| / sqrt 2
and t = 1 / (1 + z / 2),

    erfc(z) = t * exp(-z^2 + P(t)),

P a polynomial in t. Here P is written in base 2, Q(t) = log2(erfc(z) / t) + z^2 log2(e),
and refitted: degree 9, least squares in Chebyshev form at 20000 Chebyshev nodes of t
over |g| in [0, 17] (t in [1 / (1 + 17 / (2 sqrt 2)), 1]; beyond 17, erfc(z) / 2 < 1e-64
and the result is max(g, 0)).
The kernel evaluates erfc / 2 = th 2^(Q(t) - z^2 log2 e) with th = t / 2, so the
coefficient of t^k is scaled by 2^k and Q is evaluated in th by Horner's rule in fp32
(one fma per coefficient).

    python -m w4a8_moe_amd.fit_erfc      prints the fp32 coefficients (highest degree
                                         first, the order of common.h) and the fit's
                                         largest error in log2 units and relative to erfc

Uses only NumPy and SciPy's erfc (the target function); it reads nothing of the oracle.
"""
import numpy as np
from numpy.polynomial import chebyshev as C
from scipy.special import erfc

DEG = 9
GMAX = 17.0
NODES = 20000
L2E = 1.4426950408889634


def _q_of_g(g):
    z = g / np.sqrt(2.0)
    t = 1.0 / (1.0 + 0.5 * z)
    return t, np.log2(erfc(z) / t) + z * z * L2E


def fit():
    lo, hi = 1.0 / (1.0 + GMAX / (2.0 * np.sqrt(2.0))), 1.0
    x = np.cos(np.pi * (np.arange(NODES) + 0.5) / NODES)      # Chebyshev nodes in [-1, 1]
    t = lo + (x + 1.0) * 0.5 * (hi - lo)
    z = 2.0 * (1.0 / t - 1.0)
    q = np.log2(erfc(z) / t) + z * z * L2E
    cheb = C.chebfit(x, q, DEG)
    # power series in t: x = s t + o
    s, o = 2.0 / (hi - lo), -2.0 * lo / (hi - lo) - 1.0
    p = np.polynomial.Polynomial(C.cheb2poly(cheb))(np.polynomial.Polynomial([o, s])).coef
    # coefficients of th = t / 2, highest degree first, rounded to fp32
    return np.array([p[k] * 2.0 ** k for k in range(DEG, -1, -1)], dtype=np.float32)


def evaluate(coef, g):
    """The kernel's arithmetic for erfc(|g| / sqrt 2) / 2, emulated in fp32 (fma rounded once)."""
    a = np.abs(np.asarray(g, np.float32))
    th = (np.float32(1.0) / (a * np.float32(0.70710678118654746) + np.float32(2.0))).astype(np.float32)
    acc = np.full_like(th, coef[0])
    for c in coef[1:]:
        acc = (acc.astype(np.float64) * th + np.float64(c)).astype(np.float32)
    e = (-(a.astype(np.float64) ** 2) * np.float32(0.7213475204444817) + acc).astype(np.float32)
    return th.astype(np.float64) * np.exp2(e.astype(np.float64)), acc


def main():
    coef = fit()
    g = np.linspace(0.0, GMAX, 200001)
    t, q = _q_of_g(g)
    _, acc = evaluate(coef, g)
    th = t / 2.0
    # log2 error of Q alone (the fp32 Horner evaluation included)
    qk = np.polyval(coef.astype(np.float64), th)
    print("coefficients (highest degree first):")
    for c in coef:
        print(f"  {float(c)!r}f")
    print(f"max |Q_fp64 - log2 target| = {np.max(np.abs(qk - q)):.3g} (log2 units)")
    half, _ = evaluate(coef, g)
    ref = erfc(g / np.sqrt(2.0)) / 2.0
    ok = ref > 1e-30
    print(f"max relative error of erfc/2 (fp32 Horner, exact exp2): {np.max(np.abs(half[ok] / ref[ok] - 1)):.3g}")


if __name__ == "__main__":
    main()
