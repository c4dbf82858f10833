"""CPU checks of constants the HIP kernels compute with (no GPU): the
device GELU's polynomial, evaluated step by step in float32 as the kernel
does, against the exact t * Phi(t) from math.erfc."""
import math
import os

import numpy as np
# The device GELU's formula (not the oracle's, which is math.erfc in fp64):
# its committed coefficients, evaluated step by step in float32, against the
# exact t * Phi(t).  Pins the constants in csrc/igemm_kernel.h on the CPU.
def _device_gelu_coefficients(fn="gelu_erf", degree=7):
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..", "convolution_forward_implicit_amd", "csrc",
                            "igemm_kernel.h")).read()
    body = src[src.index("__device__ __forceinline__ float %s(float v)" % fn):]
    body = body[:body.index("\n}\n")]
    coef = [float(c) for c in re.findall(r"([-+]?\d\.\d+e[-+]\d+)f", body)]
    assert len(coef) == degree + 1, coef
    return coef


def _device_gelu_f32(v):
    f = np.float32
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    c = _device_gelu_coefficients()
    r = np.full(v.shape, c[0], dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        for k in c[1:]:   # fmaf: one rounding of the exact a*r + k
            r = (a.astype(np.float64) * r.astype(np.float64) + np.float64(np.float32(k))).astype(np.float32)
        p = np.exp2(r.astype(np.float64)).astype(np.float32)
        q = np.where(np.signbit(v), p, (f(1.0) - p).astype(np.float32))
        return (v * q).astype(np.float32)


def test_device_gelu_special_values():
    v = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e30, -1e30], dtype=np.float32)
    g = _device_gelu_f32(v)
    # -inf: -inf * Phi(-inf) = -inf * 0, NaN as in t/2 * erfc(-t/sqrt 2)
    assert np.isnan(g[0]) and g[1] == np.inf and np.isnan(g[2])
    assert g[3] == 0.0 and g[4] == 0.0
    assert g[5] == np.float32(1e30) and g[6] == 0.0


def test_device_gelu_polynomial_accuracy():
    t = np.concatenate([np.linspace(-40.0, 40.0, 800001), np.linspace(-1e-3, 1e-3, 2001)]).astype(np.float32)
    exact = np.array([0.5 * float(x) * math.erfc(-float(x) / math.sqrt(2.0)) for x in t.astype(np.float64)])
    got = _device_gelu_f32(t).astype(np.float64)
    err = np.abs(got - exact)
    # relative accuracy wherever the value is not tiny; where it is (the
    # negative tail beyond the fitted range, where R extrapolates) within
    # 1e-9 |t|, far inside the error bound the parity tests grade with
    big = np.abs(exact) > 1e-6
    assert np.max(err[big] / np.abs(exact[big])) < 1.2e-5
    assert np.max(err[~big] / np.maximum(np.abs(t[~big].astype(np.float64)), 1.0)) < 1.1e-9
    # the fit itself (not the float32 evaluation): log2 Phi(-a) within 6e-6 on [0, 6]
    a = np.linspace(0.0, 6.0, 60001)
    c = _device_gelu_coefficients()
    r = np.polyval(c, a)
    ref_log2 = np.log2([0.5 * math.erfc(x / math.sqrt(2.0)) for x in a])
    assert np.max(np.abs(r - ref_log2)) < 6e-6
    # closed forms carried through: GELU(0) = 0, GELU(t) - GELU(-t) = t
    assert _device_gelu_f32(np.float32(0.0)) == 0.0
    s = np.linspace(0.0, 5.0, 501).astype(np.float32)
    assert np.max(np.abs((_device_gelu_f32(s) - _device_gelu_f32(-s)) - s) / np.maximum(s, 1e-30)) < 1e-6 + 1e-5


# The variant for results rounded to bfloat16: degree-5 R, and
# t/2 + |t| (1/2 - Phi(-|t|)) in one fused multiply-add.
def _device_gelu_bf16out_f32(v):
    f = np.float32
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    c = _device_gelu_coefficients("gelu_erf_bf16out", 5)
    r = np.full(v.shape, c[0], dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        for k in c[1:]:
            r = (a.astype(np.float64) * r.astype(np.float64) + np.float64(np.float32(k))).astype(np.float32)
    p = np.exp2(r.astype(np.float64)).astype(np.float32)
    h = (f(0.5) - p).astype(np.float32)
    half = (f(0.5) * v).astype(np.float32)
    with np.errstate(invalid="ignore"):
        return (np.abs(v).astype(np.float64) * h.astype(np.float64) + half.astype(np.float64)).astype(np.float32)


def test_device_gelu_bf16out_special_values():
    v = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e30, -1e30], dtype=np.float32)
    g = _device_gelu_bf16out_f32(v)
    assert np.isnan(g[0]) and g[1] == np.inf and np.isnan(g[2])
    assert g[3] == 0.0 and g[4] == 0.0
    assert g[5] == np.float32(1e30) and g[6] == 0.0


def test_device_gelu_bf16out_accuracy():
    t = np.concatenate([np.linspace(-40.0, 40.0, 800001), np.linspace(-1e-3, 1e-3, 2001)]).astype(np.float32)
    exact = np.array([0.5 * float(x) * math.erfc(-float(x) / math.sqrt(2.0)) for x in t.astype(np.float64)])
    got = _device_gelu_bf16out_f32(t).astype(np.float64)
    err = np.abs(got - exact)
    # a tenth of bfloat16's relative rounding step (2^-9), plus the
    # absolute 2^-25 |t| of the cancelling negative side
    assert np.all(err <= 4.2e-4 * np.abs(exact) + 2.0 ** -24 * np.abs(t.astype(np.float64)))
    # the fit itself: log2 Phi(-a) within 6e-4 on [0, 6]
    a = np.linspace(0.0, 6.0, 60001)
    r = np.polyval(_device_gelu_coefficients("gelu_erf_bf16out", 5), a)
    ref_log2 = np.log2([0.5 * math.erfc(x / math.sqrt(2.0)) for x in a])
    assert np.max(np.abs(r - ref_log2)) < 6e-4
    # GELU(t) - GELU(-t) = t, to fp32 rounding
    s = np.linspace(0.0, 5.0, 501).astype(np.float32)
    d = _device_gelu_bf16out_f32(s).astype(np.float64) - _device_gelu_bf16out_f32(-s)
    assert np.max(np.abs(d - s)) <= 2.0 ** -22 * 5.0


def test_device_gelu_fits_extrapolate_downwards():
    """Neither fit is clamped at |t| = 6: evaluated in float32 as the device
    does, R stays below its value at 6 (log2 Phi(-6) = -29.9) and keeps
    decreasing for every larger a, up to overflow to -inf, so Phi(-a) =
    2^R only shrinks towards 0 there."""
    a = np.concatenate([np.linspace(6.0, 100.0, 200001), np.geomspace(100.0, 3e38, 20001)]).astype(np.float32)
    for fn, deg in (("gelu_erf", 7), ("gelu_erf_bf16out", 5)):
        c = _device_gelu_coefficients(fn, deg)
        r = np.full(a.shape, c[0], dtype=np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            for k in c[1:]:
                r = (a.astype(np.float64) * r.astype(np.float64) + np.float64(np.float32(k))).astype(np.float32)
        assert not np.isnan(r).any()
        assert np.all(r <= -29.9) and np.all(r[1:] <= r[:-1]), fn
        assert r[-1] == -np.inf
