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
conv == numpy.correlate; linearity; GELU closed forms; bf16 rounding against
IEEE bit patterns and hand-worked ties; the two-conv chain against delta
filters (closed form) and against the composed 5-tap kernel (interior); the
backward passes as the adjoints of the forward sum (<conv(x,w), dy> =
<x, dgrad> = <w, wgrad> on the exhaustive tiny grid, plus one-hot forward
probes), against torch's fp64 autograd, a delta kernel's scatter and the
all-ones valid-output counts.
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
        for name in ("oracle_conv_bwd_data", "oracle_conv_bwd_weight"):
            getattr(lib, name).argtypes = [ctypes.POINTER(_Desc), dp, dp, dp, dp]
            getattr(lib, name).restype = ctypes.c_int
        for name in ("oracle_conv_bwd_data_points", "oracle_conv_bwd_weight_points"):
            getattr(lib, name).argtypes = [ctypes.POINTER(_Desc), dp, dp, ctypes.c_int64, ip, dp, dp]
            getattr(lib, name).restype = ctypes.c_int
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


def conv_bwd_data(p, dy, w):
    """Gradient with respect to the input (x's layout, float64) of the
    forward sum for output gradient dy, and the per-element sum of |terms|:
    (dx, absdot).  No bias or activation (the backward of the linear conv)."""
    xs, ws, _, ys = shapes(p)
    dy = _as_f64(dy, ys, "dy")
    w = _as_f64(w, ws, "w")
    dx = np.empty(xs, dtype=np.float64)
    ad = np.empty(xs, dtype=np.float64)
    rc = _load().oracle_conv_bwd_data(ctypes.byref(_mk_desc(p)), _dptr(dy), _dptr(w), _dptr(dx), _dptr(ad))
    if rc != 0:
        raise ValueError("oracle_conv_bwd_data failed (%d)" % rc)
    return dx, ad


def conv_bwd_data_points(p, dy, w, flat_idx):
    """conv_bwd_data at flat indices of the x layout: (values, absdot)."""
    xs, ws, _, ys = shapes(p)
    dy = _as_f64(dy, ys, "dy")
    w = _as_f64(w, ws, "w")
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    v = np.empty(idx.shape, dtype=np.float64)
    ad = np.empty(idx.shape, dtype=np.float64)
    rc = _load().oracle_conv_bwd_data_points(ctypes.byref(_mk_desc(p)), _dptr(dy), _dptr(w), idx.size,
                                             idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(v),
                                             _dptr(ad))
    if rc != 0:
        raise ValueError("oracle_conv_bwd_data_points failed (%d)" % rc)
    return v, ad


def conv_bwd_weight(p, x, dy):
    """Gradient with respect to the weights (w's layout, float64) for input
    x and output gradient dy, and the per-element sum of |terms|: (dw,
    absdot)."""
    xs, ws, _, ys = shapes(p)
    x = _as_f64(x, xs, "x")
    dy = _as_f64(dy, ys, "dy")
    dw = np.empty(ws, dtype=np.float64)
    ad = np.empty(ws, dtype=np.float64)
    rc = _load().oracle_conv_bwd_weight(ctypes.byref(_mk_desc(p)), _dptr(x), _dptr(dy), _dptr(dw), _dptr(ad))
    if rc != 0:
        raise ValueError("oracle_conv_bwd_weight failed (%d)" % rc)
    return dw, ad


def conv_bwd_weight_points(p, x, dy, flat_idx):
    """conv_bwd_weight at flat indices of the w layout: (values, absdot)."""
    xs, ws, _, ys = shapes(p)
    x = _as_f64(x, xs, "x")
    dy = _as_f64(dy, ys, "dy")
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    v = np.empty(idx.shape, dtype=np.float64)
    ad = np.empty(idx.shape, dtype=np.float64)
    rc = _load().oracle_conv_bwd_weight_points(ctypes.byref(_mk_desc(p)), _dptr(x), _dptr(dy), idx.size,
                                               idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(v),
                                               _dptr(ad))
    if rc != 0:
        raise ValueError("oracle_conv_bwd_weight_points failed (%d)" % rc)
    return v, ad


def round_bf16(v):
    """Exact values -> the nearest bfloat16 (ties to even), as float64:
    8 significant bits, float32's exponent range (normal from 2^-126,
    subnormals in steps of 2^-133), overflow to infinity.  Rounds the exact
    value once (no detour through float32)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    a = np.abs(v)
    big = a >= 2.0 ** -126
    m, e = np.frexp(v[big])                       # v = m * 2^e, 0.5 <= |m| < 1
    out[big] = np.ldexp(np.rint(m * 256.0), e - 8)  # numpy rint: half to even
    out[~big] = np.rint(v[~big] * 2.0 ** 133) * 2.0 ** -133
    maxb = (2.0 - 2.0 ** -7) * 2.0 ** 127
    # beyond the largest finite bf16 (after rounding) the result is infinite
    out[np.abs(out) > maxb] = np.copysign(np.inf, v[np.abs(out) > maxb])
    return out


def chain_problems(p1, p2):
    """Check that p2 reads p1's output (same batch, p2.C == p1.K, p2's input
    extent == p1's output extent, one group)."""
    if p1["G"] != 1 or p2["G"] != 1 or p1["N"] != p2["N"] or p2["C"] != p1["K"]:
        raise ValueError("second conv must read the first one's output")
    if tuple(p2["in"]) != tuple(out_dims(p1)):
        raise ValueError("second conv's input extent %r != first conv's output %r"
                         % (tuple(p2["in"]), tuple(out_dims(p1))))


def conv_chain(p1, p2, x, w1, b1, w2, b2, gelu):
    """Two convolutions in a row, the way the conv frontend of the ExecuTorch
    conv1d issue (table of the two-conv frontend) runs them: h = conv1(x)
    (+ b1, GELU), rounded to bfloat16 (the intermediate has the call's
    dtype), then y = conv2(h) (+ b2, GELU), unrounded.
    Returns (y, absdot2, carry): absdot2 = |b2| + sum|w2 h| per output, and
    carry = sum|w2| * absdot1 over the h values each output reads (absdot1 =
    |b1| + sum|w1 x| of that h value), which bounds how the fp32
    accumulation error of h propagates into y."""
    chain_problems(p1, p2)
    h, ad1 = conv_fwd(p1, x, w1, b1, gelu)
    hr = round_bf16(h)
    y, ad2 = conv_fwd(p2, hr, w2, b2, gelu)
    carry = conv_fwd(p2, ad1, np.abs(np.asarray(w2, dtype=np.float64)), None, False, want_absdot=False)
    return y, ad2, carry


def conv_chain_points(p1, p2, x, w1, b1, w2, b2, gelu, flat_idx):
    """conv_chain at flat output indices of y: only the h values those
    outputs read are computed (the rest of h stays zero and is never read)."""
    chain_problems(p1, p2)
    idx = np.asarray(flat_idx, dtype=np.int64)
    _, ws2, _, ys2 = shapes(p2)
    _, _, _, hs = shapes(p1)
    N, Do, Ho, Wo, _, K2 = ys2
    Z, Y, X = p2["filt"]
    sd, sh, sw = p2["stride"]
    pd, ph, pw = p2["pad"]
    dd, dh, dw = p2["dil"]
    Dh, Hh, Wh = hs[1], hs[2], hs[3]
    rest, ow = np.divmod(idx // K2, Wo)
    rest, oh = np.divmod(rest, Ho)
    nb, od = np.divmod(rest, Do)
    pix = set()
    for z in range(Z):
        for yy in range(Y):
            for xx in range(X):
                di, hi, wi = od * sd - pd + z * dd, oh * sh - ph + yy * dh, ow * sw - pw + xx * dw
                ok = (di >= 0) & (di < Dh) & (hi >= 0) & (hi < Hh) & (wi >= 0) & (wi < Wh)
                pix.update(((nb[ok] * Dh + di[ok]) * Hh + hi[ok]) * Wh + wi[ok])
    pix = np.array(sorted(pix), dtype=np.int64)
    C2 = p2["C"]
    hidx = (pix[:, None] * C2 + np.arange(C2)[None, :]).ravel()
    hv, ad1 = conv_fwd_points(p1, x, w1, b1, gelu, hidx)
    h = np.zeros(int(np.prod(hs)), dtype=np.float64)
    a1 = np.zeros_like(h)
    h[hidx] = round_bf16(hv)
    a1[hidx] = ad1
    y, ad2 = conv_fwd_points(p2, h, w2, b2, gelu, idx)
    carry, _ = conv_fwd_points(p2, a1, np.abs(np.asarray(w2, dtype=np.float64)), None, False, idx)
    return y, ad2, carry


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
