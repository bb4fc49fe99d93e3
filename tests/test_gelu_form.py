"""CPU check of the GPU epilogue's GELU: the erfc polynomial constants in
csrc/common.hpp and the fp32 operation sequence of gelu_erf, replayed in
numpy, against GELU(z) = z/2 * erfc(-z/sqrt 2) from scipy in binary64."""
import os
import re

import numpy as np
import pytest
from scipy.special import erfc

HDR = os.path.join(os.path.dirname(__file__), "..", "block_scaled_fp4_add_amd", "csrc", "common.hpp")
f32 = np.float32


def poly():
    src = open(HDR).read()
    m = re.search(r"kGeluErfcPoly\[10\]\s*=\s*\{([^}]*)\}", src)
    assert m, "kGeluErfcPoly not found"
    c = [float(v.strip().rstrip("f")) for v in m.group(1).split(",")]
    assert len(c) == 10
    return np.array(c)


def fma32(a, b, c):
    # a single rounding of a*b + c (binary64 holds the product of two fp32 exactly)
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(f32)


def gelu_gpu_form(z, c):
    z = np.asarray(z, f32)
    cf = c.astype(f32)
    x = (np.abs(z) * f32(0.70710678118654752440)).astype(f32)
    t = (f32(1.0) / fma32(f32(0.5), x, f32(1.0))).astype(f32)
    g = np.full_like(t, cf[9])
    for k in range(8, -1, -1):
        g = fma32(g, t, cf[k])
    arg = fma32((f32(-0.5) * z).astype(f32), z, g)
    e = (t * np.exp2((arg * f32(1.44269504088896340736)).astype(f32).astype(np.float64)).astype(f32)).astype(f32)
    fac = np.where(z >= 0, (f32(2.0) - e).astype(f32), e)
    return ((f32(0.5) * z).astype(f32) * fac).astype(f32)


def gelu_ref(z):
    z = np.asarray(z, np.float64)
    return 0.5 * z * erfc(-z / np.sqrt(2.0))


def test_erfc_fit_relative_error():
    c = poly()
    x = np.concatenate([np.linspace(0.0, 10.0, 200001), np.linspace(10.0, 26.0, 1601)])
    t = 1.0 / (1.0 + 0.5 * x)
    approx = t * np.exp(-x * x + np.polyval(c[::-1], t))
    rel = np.abs(approx / erfc(x) - 1.0)
    assert rel.max() < 1.1e-7, rel.max()


@pytest.mark.parametrize("lo,hi,bound", [(-6.0, -4.0, 2e-6), (-4.0, -2.0, 1.2e-6), (-2.0, 0.0, 6e-7),
                                         (0.0, 2.0, 6e-7), (2.0, 12.0, 2e-7)])
def test_gelu_fp32_sequence(lo, hi, bound):
    z = np.linspace(lo, hi, 200001, dtype=np.float64).astype(f32)
    z = z[z != 0]
    got = gelu_gpu_form(z, poly()).astype(np.float64)
    ref = gelu_ref(z)
    rel = np.abs(got - ref) / np.abs(ref)
    assert rel.max() < bound, (lo, hi, rel.max())


def test_gelu_special_values():
    c = poly()
    z = np.array([0.0, -0.0, 1e-30, -1e-30, 30.0, -30.0, 200.0, -200.0], f32)
    g = gelu_gpu_form(z, c)
    assert g[0] == 0 and g[1] == 0
    assert g[4] == f32(30.0) and g[6] == f32(200.0)       # erfc(-x) -> 2: gelu(z) = z
    assert g[5] == 0 and np.signbit(g[5])                  # deep negative tail: -0, the sign kept
    assert g[7] == 0 and np.signbit(g[7])
    np.testing.assert_allclose(g[2:4].astype(np.float64), [5e-31, -5e-31], rtol=1e-6)
