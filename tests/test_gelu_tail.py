"""The 16-bit GELU of the kernels (gelu2_tail in csrc/kcommon.h): the coefficients written there give,
in fp32 arithmetic, a GELU within the bound its comment states of the erf GELU (x Phi(x)), at
every x of a fine grid over [-12, 12] and at the special points 0 and the far tails."""
import math
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
KCOMMON = os.path.join(HERE, "..", "axial_band_split_amd", "csrc", "kcommon.h")


def coefficients():
    src = open(KCOMMON).read()
    body = src[src.index("float gelu2_tail(float x)"):]
    body = body[:body.index("}")]
    nums = [float(v) for v in re.findall(r"(-?\d+\.\d+)f", body)]
    c3, c2, c1 = nums[0], nums[1], nums[2]
    return np.float32(c3), np.float32(c2), np.float32(c1)


def gelu_tail(x):
    c3, c2, c1 = coefficients()
    x = x.astype(np.float32)
    a = np.abs(x)
    p = (c3 * a + c2).astype(np.float32)
    p = (p * a + c1).astype(np.float32)
    p = (p * a).astype(np.float32)
    return (np.float32(0.5) * (a * (np.float32(1.0) - np.exp2(p)) + x)).astype(np.float64)


def gelu_exact(x):
    erf = np.vectorize(math.erf)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def test_coefficients_are_negative_so_the_tail_falls():
    assert all(c < 0 for c in coefficients())


def test_gelu_tail_within_its_stated_bound():
    x = np.linspace(-12.0, 12.0, 240001)
    err = np.abs(gelu_tail(x) - gelu_exact(x))
    assert err.max() <= 1.35e-4
    nz = np.abs(x) > 1e-3
    assert (err[nz] / np.abs(x[nz])).max() <= 1.35e-4


def test_gelu_tail_special_points():
    x = np.array([0.0, 30.0, -30.0, 1e4, -1e4])
    g = gelu_tail(x)
    assert g[0] == 0.0
    assert abs(g[1] - 30.0) < 1e-5 and abs(g[3] - 1e4) < 1e-2
    assert abs(g[2]) < 1e-5 and abs(g[4]) < 1e-2
