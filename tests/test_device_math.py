"""CPU checks of constants the HIP kernels compute with (no GPU): the
device GELU's polynomial, evaluated step by step in float32 as the kernel
does, against the exact t * Phi(t) from math.erfc."""
import math
import os

import numpy as np
# The device GELU's formula (not the oracle's, which is math.erfc in fp64):
# its committed coefficients, evaluated step by step in float32, against the
# exact t * Phi(t).  Pins the constants in csrc/igemm_kernel.h on the CPU.
def _device_gelu_coefficients():
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..", "convolution_forward_implicit_amd", "csrc",
                            "igemm_kernel.h")).read()
    body = src[src.index("__device__ __forceinline__ float gelu_erf(float v)"):]
    body = body[:body.index("\n}\n")]
    coef = [float(c) for c in re.findall(r"([-+]?\d\.\d+e[-+]\d+)f", body)]
    assert len(coef) == 8, coef
    return coef


def _device_gelu_f32(v):
    f = np.float32
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v), f(6.0))
    c = _device_gelu_coefficients()
    r = np.full(v.shape, c[0], dtype=np.float32)
    for k in c[1:]:   # fmaf: one rounding of the exact a*r + k
        r = (a.astype(np.float64) * r.astype(np.float64) + np.float64(np.float32(k))).astype(np.float32)
    p = np.exp2(r.astype(np.float64)).astype(np.float32)
    q = np.where(np.signbit(v), p, (f(1.0) - p).astype(np.float32))
    return (v * q).astype(np.float32)


def test_device_gelu_special_values():
    v = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e30], dtype=np.float32)
    g = _device_gelu_f32(v)
    assert np.isnan(g[0]) and g[1] == np.inf and g[2] == -np.inf
    assert g[3] == 0.0 and g[4] == 0.0
    assert g[5] == np.float32(1e30)


def test_device_gelu_polynomial_accuracy():
    t = np.concatenate([np.linspace(-12.0, 12.0, 480001), np.linspace(-1e-3, 1e-3, 2001)]).astype(np.float32)
    exact = np.array([0.5 * float(x) * math.erfc(-float(x) / math.sqrt(2.0)) for x in t.astype(np.float64)])
    got = _device_gelu_f32(t).astype(np.float64)
    err = np.abs(got - exact)
    # relative accuracy wherever the value is not tiny; where it is (the
    # negative tail, Phi clamped at Phi(-6) = 1e-9 beyond |t| = 6) within
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
