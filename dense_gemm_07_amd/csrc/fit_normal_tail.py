"""Fits the normal-tail approximation used by the GELU activation of the kernels.

Q(x) = Phi(-x) = erfc(x / sqrt 2) / 2 for x >= 0 is written as
    Q(x) = exp(-x^2 / 2) * t * P(t),   t = 1 / (1 + 0.3 x),
with P a degree-9 polynomial (degree 6 for results rounded to 16 bits). The
exp factor carries the Gaussian decay, so P varies slowly on t in (0, 1] and
a low degree fits it to ~3.5e-9 (degree 9) or ~3.8e-6 (degree 6) relative
error over x in [0, 14] (beyond, Q is below fp32's normal range). Coefficients
come from least squares on the relative error, reweighted toward minimax;
the reference values are computed to 40 digits with mpmath. Run it to
reproduce the constants in dg_kernels.hpp (needs numpy and mpmath; it is not
part of any build or run path).
"""
import mpmath as mp
import numpy as np

A, DEG = 0.3, 9


def fit():
    mp.mp.dps = 40
    xs = np.concatenate([np.linspace(0, 2, 4000), np.linspace(2, 14, 12000)])
    q = np.array([float(0.5 * mp.erfc(x / mp.sqrt(2))) for x in xs])
    t = 1.0 / (1.0 + A * xs)
    y = q * np.exp(xs * xs / 2) / t  # the P(t) to fit
    V = np.vander(t, DEG + 1, increasing=True)
    w = 1.0 / y
    for _ in range(60):
        c, *_ = np.linalg.lstsq(V * w[:, None], y * w, rcond=None)
        rel = (V @ c - y) / y
        w = w * (1 + 50 * np.abs(rel) / np.abs(rel).max())
    return c, float(np.abs(rel).max())


if __name__ == "__main__":
    import sys
    # --degree N: the degree of P (9 for the fp32 tail, 6 for the 16-bit one)
    if "--degree" in sys.argv:
        DEG = int(sys.argv[sys.argv.index("--degree") + 1])
    c, err = fit()
    print(f"max relative fit error {err:.3e}")
    print(", ".join(f"{float(np.float32(v)):.9g}f" for v in c))
