"""Prints the coefficients of the FP32 erfc approximation used by the erf-GELU kernels.

erfc(z) = t * exp(-z^2 + Q(t)) with t = 1 / (1 + z/2) (the change of variable of the
classic Chebyshev-fitted erfc of Press et al., Numerical Recipes, 6.2), here with Q a
degree-7 polynomial fitted by least squares on Chebyshev nodes to ln(erfc(z)/t) + z^2 over
the range the kernels use, z in [0, 12.75/sqrt 2] (|x| <= 12.75 in x = -z sqrt 2).
Q(0) tends to ln(1/(2 sqrt pi)) as z -> inf.  Run: python gen_erfc_poly.py
"""
import mpmath as mp
import numpy as np

mp.mp.dps = 40
ZMAX = 12.75 / np.sqrt(2.0)
TMIN = 1.0 / (1.0 + 0.5 * ZMAX)
DEG = 7


def q_exact(t):
    t = mp.mpf(t)
    z = 2 * (1 / t - 1)
    return mp.log(mp.erfc(z) / t) + z * z


def fit():
    """Least squares on Chebyshev nodes; the coefficients are rounded to FP32 one at a
    time, lowest degree first, each time refitting the higher ones to the residual."""
    n = 800
    k = np.arange(n)
    ts = 0.5 * (1 + TMIN) + 0.5 * (1 - TMIN) * np.cos(np.pi * (k + 0.5) / n)
    qs = np.array([float(q_exact(t)) for t in ts])
    fixed = {}
    for d in range(DEG + 1):
        resid = qs - sum(v * ts ** i for i, v in fixed.items())
        free = [i for i in range(DEG + 1) if i not in fixed]
        A = np.stack([ts ** i for i in free], axis=1)
        sol = np.linalg.lstsq(A, resid, rcond=None)[0]
        fixed[d] = float(np.float32(sol[free.index(d)]))
    return np.array([fixed[i] for i in range(DEG + 1)], np.float32)


def main():
    c = fit()
    grid = np.linspace(TMIN, 1.0, 5001)
    err = max(abs(float(np.polyval(c[::-1].astype(np.float64), t)) - float(q_exact(t))) for t in grid)
    print(f"// degree {DEG}, t in [{TMIN:.6f}, 1], max |Q error| {err:.2e} (FP32 coefficients)")
    print("constexpr float ERFC_Q[%d] = {" % (DEG + 1))
    print(",\n".join(f"    {float(v):.9e}f" for v in c))
    print("};")


if __name__ == "__main__":
    main()
