"""Coefficients of the 16-bit GELU (gelu2_tail in kcommon.h: the fused post-attention kernel and the
GEMM's GELU epilogue).

GELU(x) = x Phi(x) = max(x, 0) - |x| Q(|x|), Q the upper tail of the standard normal distribution.
The kernel takes Q(a) = 2^(p(a) - 1), p(a) = c3 a^3 + c2 a^2 + c1 a (so Q(0) = 1/2 exactly), and this
script finds c3, c2, c1 by minimising max over a in [0, 10] of max(a, 1) |2^(p(a) - 1) - Q(a)|: the
GELU's absolute error for |x| >= 1 and its error relative to |x| below.  Run it with numpy and scipy;
it prints the coefficients and the resulting GELU error in fp32 arithmetic.
"""
import numpy as np
from scipy.optimize import minimize
from scipy.special import erf, erfc


def fit():
    a = np.linspace(0.0, 10.0, 100001)
    q = 0.5 * erfc(a / np.sqrt(2.0))
    w = np.maximum(a, 1.0)

    def cost(c):
        return np.max(w * np.abs(np.exp2(np.polyval(np.append(c, -1.0), a)) - q))

    c = np.array([-0.0292, -0.4838, -1.1434])
    for _ in range(8):
        c = minimize(cost, c, method="Nelder-Mead", options={"maxiter": 60000, "xatol": 1e-14, "fatol": 1e-15}).x
    return c.astype(np.float32)


def gelu_error(c):
    x = np.linspace(-12.0, 12.0, 1200001).astype(np.float32)
    a = np.abs(x)
    p = (((c[0] * a + c[1]) * a + c[2]) * a).astype(np.float32)
    g = 0.5 * (x + a * (np.float32(1.0) - np.exp2(p)))
    exact = 0.5 * x.astype(np.float64) * (1.0 + erf(x.astype(np.float64) / np.sqrt(2.0)))
    err = np.abs(g - exact)
    return err.max(), (err / np.abs(x))[np.abs(x) > 1e-4].max()


if __name__ == "__main__":
    c = fit()
    e_abs, e_rel = gelu_error(c)
    print("c3, c2, c1 =", [float(v) for v in c])
    print(f"GELU error: {e_abs:.3e} absolute, {e_rel:.3e} |x|")
