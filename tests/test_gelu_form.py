"""CPU check of the GPU epilogue's GELU: the erfc polynomial constants in
csrc/common.hpp and the fp32 operation sequence of gelu_erf, replayed in
numpy, against GELU(z) = z/2 * erfc(-z/sqrt 2) from scipy in binary64.

The device evaluates the reciprocal and the power of two with v_rcp_f32 and
v_exp_f32, which the CDNA instruction set documents as accurate to one ulp.
The hardware model below lets each of those two results sit one ulp either
side of the correctly rounded value; its worst case over a dense sweep is
the GELU error bound (checkers.GELU_REL) that the FP4-output comparison
window carries."""
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


def _ulp_step(v, d):
    """v moved d (-1, 0, +1) ulps (fp32)."""
    return v if d == 0 else np.nextafter(v, f32(np.inf * d)).astype(f32)


def gelu_gpu_form(z, c, d_rcp=0, d_exp=0):
    """gelu_erf's fp32 sequence; d_rcp / d_exp shift the reciprocal and the
    power of two by that many ulps (the one-ulp hardware model)."""
    z = np.asarray(z, f32)
    cf = c.astype(f32)
    x = (np.abs(z) * f32(0.70710678118654752440)).astype(f32)
    t = _ulp_step((f32(1.0) / fma32(f32(0.5), x, f32(1.0))).astype(f32), d_rcp)
    g = np.full_like(t, cf[9])
    for k in range(8, -1, -1):
        g = fma32(g, t, cf[k])
    arg = fma32((f32(-0.5) * z).astype(f32), z, g)
    p2 = _ulp_step(np.exp2((arg * f32(1.44269504088896340736)).astype(f32).astype(np.float64)).astype(f32), d_exp)
    e = (t * p2).astype(f32)
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


@pytest.mark.parametrize("lo,hi,bound", [(-9.0, -6.0, 4.5e-6), (-6.0, -4.0, 2.6e-6), (-4.0, -2.0, 1.6e-6),
                                         (-2.0, 2.0, 1.0e-6), (2.0, 16.0, 2e-7)])
def test_gelu_hardware_model_bound(lo, hi, bound):
    """With v_rcp_f32 and v_exp_f32 each one ulp off in either direction the
    relative error stays inside the bound the FP4-output window uses (the
    whole-range bound is checkers.GELU_REL)."""
    from .checkers import GELU_REL
    assert bound <= GELU_REL
    z = np.linspace(lo, hi, 200001, dtype=np.float64).astype(f32)
    z = z[z != 0]
    ref = gelu_ref(z)
    worst = 0.0
    for dr in (-1, 0, 1):
        for de in (-1, 0, 1):
            got = gelu_gpu_form(z, poly(), dr, de).astype(np.float64)
            worst = max(worst, float((np.abs(got - ref) / np.abs(ref)).max()))
    assert worst < bound, (lo, hi, worst)


def test_gelu_deep_tail_is_negligible():
    """Below z = -9 the bound is not needed: |gelu(z)| < 1.1e-18 there, so
    any value scaled by an FP4 block inverse of at most 2^9 * gs_out stays
    far below the first E2M1 boundary (0.25) for any gs_out < 4e14."""
    z = np.linspace(-200.0, -9.0, 100001)
    assert np.abs(gelu_ref(z)).max() < 1.1e-18
