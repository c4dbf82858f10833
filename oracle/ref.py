"""Python face of the fp64 CPU oracle (oracle/conv_oracle.c).

TEST INFRASTRUCTURE ONLY -- imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library.

A problem is described by a plain dict (keys below), the same for 1-D, 2-D
and 3-D convolution: a 1-D conv is the 3-D problem with D = H = 1, which is
how the ExecuTorch conv1d issue ("Suggested fix") re-expresses nn.Conv1d as
nn.Conv2d with a singleton height.  C and K are per group (layouts NHWGC x
GKYXC -> NHWGK of the Composable Kernel grouped-conv note, intro).

    {"N", "G", "C", "K", "in": (Di, Hi, Wi), "filt": (Z, Y, X),
     "stride": (sd, sh, sw), "pad": (pd, ph, pw), "dil": (dd, dh, dw)}

Pins (tests/test_oracle_pins.py): output extents against every configured
shape and the page's dispatch shapes; an independent numpy brute force
(explicit zero padding, zero-inserted dilated kernel); torch fp64 conv;
conv1d == conv2d(H=1) == conv3d(D=H=1); grouped == G independent convs;
delta kernel; all-ones border counts; 1x1 conv == matmul; single-channel
conv == numpy.correlate; linearity; GELU closed forms.
"""
import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


class _Desc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("G", ctypes.c_int64),
                ("C", ctypes.c_int64), ("K", ctypes.c_int64),
                ("in_", ctypes.c_int64 * 3), ("filt", ctypes.c_int64 * 3),
                ("stride", ctypes.c_int64 * 3), ("pad", ctypes.c_int64 * 3),
                ("dil", ctypes.c_int64 * 3)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_out_dims.argtypes = [ctypes.POINTER(_Desc), ip]
        lib.oracle_out_dims.restype = ctypes.c_int
        lib.oracle_conv_fwd.argtypes = [ctypes.POINTER(_Desc), dp, dp, dp,
                                        ctypes.c_int, dp, dp]
        lib.oracle_conv_fwd.restype = ctypes.c_int
        lib.oracle_conv_fwd_points.argtypes = [ctypes.POINTER(_Desc), dp, dp, dp,
                                               ctypes.c_int, ctypes.c_int64, ip, dp, dp]
        lib.oracle_conv_fwd_points.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _mk_desc(p):
    d = _Desc()
    d.N, d.G, d.C, d.K = int(p["N"]), int(p["G"]), int(p["C"]), int(p["K"])
    for i in range(3):
        d.in_[i] = int(p["in"][i])
        d.filt[i] = int(p["filt"][i])
        d.stride[i] = int(p["stride"][i])
        d.pad[i] = int(p["pad"][i])
        d.dil[i] = int(p["dil"][i])
    return d


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def out_dims(p):
    """(Do, Ho, Wo) = floor((I + 2p - d(F-1) - 1)/s) + 1 per dim; raises on an
    empty output."""
    o = (ctypes.c_int64 * 3)()
    rc = _load().oracle_out_dims(ctypes.byref(_mk_desc(p)), o)
    if rc != 0:
        raise ValueError("degenerate convolution descriptor: %r" % (p,))
    return tuple(int(v) for v in o)


def shapes(p):
    """Library-layout shapes (x, w, b, y) of a problem."""
    Do, Ho, Wo = out_dims(p)
    Di, Hi, Wi = p["in"]
    Z, Y, X = p["filt"]
    return ((p["N"], Di, Hi, Wi, p["G"], p["C"]),
            (p["G"], p["K"], Z, Y, X, p["C"]),
            (p["G"], p["K"]),
            (p["N"], Do, Ho, Wo, p["G"], p["K"]))


def _as_f64(a, shape, name):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if a.size != int(np.prod(shape)):
        raise ValueError("%s has %d elements, expected shape %r" % (name, a.size, shape))
    return a.reshape(shape)


def conv_fwd(p, x, w, b=None, gelu=False, want_absdot=True):
    """Full output y (library layout, float64) and, if asked, the per-element
    sum |b| + sum |x*w| used by the error bound."""
    xs, ws, bs, ys = shapes(p)
    x = _as_f64(x, xs, "x")
    w = _as_f64(w, ws, "w")
    bb = None if b is None else _as_f64(b, bs, "b")
    y = np.empty(ys, dtype=np.float64)
    ad = np.empty(ys, dtype=np.float64) if want_absdot else None
    rc = _load().oracle_conv_fwd(ctypes.byref(_mk_desc(p)), _dptr(x), _dptr(w),
                                 None if bb is None else _dptr(bb), int(bool(gelu)),
                                 _dptr(y), None if ad is None else _dptr(ad))
    if rc != 0:
        raise ValueError("oracle_conv_fwd failed (%d)" % rc)
    return (y, ad) if want_absdot else y


def conv_fwd_points(p, x, w, b, gelu, flat_idx):
    """Outputs at flat indices of the y layout: (values, absdot)."""
    xs, ws, bs, ys = shapes(p)
    x = _as_f64(x, xs, "x")
    w = _as_f64(w, ws, "w")
    bb = None if b is None else _as_f64(b, bs, "b")
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    y = np.empty(idx.shape, dtype=np.float64)
    ad = np.empty(idx.shape, dtype=np.float64)
    rc = _load().oracle_conv_fwd_points(
        ctypes.byref(_mk_desc(p)), _dptr(x), _dptr(w),
        None if bb is None else _dptr(bb), int(bool(gelu)), idx.size,
        idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(y), _dptr(ad))
    if rc != 0:
        raise ValueError("oracle_conv_fwd_points failed (%d)" % rc)
    return y, ad


def max_threads():
    return int(_load().oracle_max_threads())


def gelu(v):
    """Exact GELU t*Phi(t) written as 0.5*t*erfc(-t/sqrt(2)), in float64
    (erf-GELU of the Whisper conv frontend; the erfc form has no
    cancellation for negative t)."""
    v = np.asarray(v, dtype=np.float64)
    erfc = np.vectorize(math.erfc, otypes=[np.float64])
    return 0.5 * v * erfc(-v / math.sqrt(2.0))


def useful_flop(p):
    """2 * MACs counting padded taps: 2*N*G*K*C*prod(O)*prod(F).  This is how
    the ExecuTorch conv1d issue (third table) turns dispatch times into
    'useful throughput' (552.96 MFLOP / 17.7 ms = 31.3 GFLOP/s)."""
    Do, Ho, Wo = out_dims(p)
    Z, Y, X = p["filt"]
    return 2 * p["N"] * p["G"] * p["K"] * p["C"] * Do * Ho * Wo * Z * Y * X
