"""Parity checks against the fp64 oracle.  TEST INFRASTRUCTURE ONLY.

Per-element bound (a reading of "max relative error 1e-4 for fp32 and 2 bf16
ulps, relative 8e-3, for bf16 outputs"; a purely relative bound cannot hold
where a sum cancels to ~0, because fp32 accumulation error scales with the
sum of |terms| whatever the result):

    |g - r| <= rtol * |r| + L * gamma_n * absdot

  rtol    = 1e-4 for fp32 outputs, 8e-3 for bf16 outputs
  gamma_n = n u / (1 - n u), u = 2^-24, n = C*Z*Y*X + has_bias (Higham's
            bound for an n-term fp32 dot product in any order)
  absdot  = |b| + sum |x*w|  (from the oracle)
  L       = 1.13 with GELU (max |GELU'| is 1.1289), else 1

Pinned by tests/test_oracle_pins.py (bound holds for an fp32 numpy sum and
fails for a perturbed one; bf16 rounding against IEEE bit patterns).
"""
import numpy as np

RTOL = {"f32": 1e-4, "bf16": 8e-3}


def gamma(n):
    u = 2.0 ** -24
    return n * u / (1.0 - n * u)


def reduction_length(p, has_bias):
    Z, Y, X = p["filt"]
    return int(p["C"] * Z * Y * X + (1 if has_bias else 0))


def bound(ref, absdot, p, dtype, has_bias, gelu):
    lip = 1.13 if gelu else 1.0
    return RTOL[dtype] * np.abs(ref) + lip * gamma(reduction_length(p, has_bias)) * absdot


def check(got, ref, absdot, p, dtype, has_bias, gelu):
    """Returns a dict of statistics; 'ok' is the graded verdict."""
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    absdot = np.asarray(absdot, dtype=np.float64).ravel()
    if got.shape != ref.shape:
        raise ValueError("shape mismatch %r vs %r" % (got.shape, ref.shape))
    err = np.abs(got - ref)
    lim = bound(ref, absdot, p, dtype, has_bias, gelu)
    finite = np.isfinite(got)
    ratio = np.where(lim > 0, err / np.where(lim > 0, lim, 1.0), np.where(err > 0, np.inf, 0.0))
    ok = bool(finite.all() and (err <= lim).all())
    big = np.abs(ref) >= 1e-3 * (np.abs(ref).max() if ref.size else 0.0)
    rel_big = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    denom = float(np.linalg.norm(got) * np.linalg.norm(ref))
    cos = float(np.dot(got, ref) / denom) if denom > 0 else 1.0
    worst = int(np.argmax(ratio)) if ratio.size else -1
    return {
        "ok": ok,
        "n": int(got.size),
        "n_fail": int((~(err <= lim)).sum() + (~finite).sum()),
        "max_ratio": float(ratio.max()) if ratio.size else 0.0,
        "worst_index": worst,
        "max_abs_diff": float(err.max()) if err.size else 0.0,
        "max_rel_err_big": rel_big,
        "normwise": float(err.max() / np.abs(ref).max()) if ref.size and np.abs(ref).max() > 0 else 0.0,
        "cosine": cos,
    }


def check_chain(got, ref, absdot2, carry, p1, p2, gelu):
    """Parity of a fused two-conv chain (bf16), whose intermediate h never
    leaves the device, so the oracle rounds its own exact h to bf16.  The
    device's h may then differ from the oracle's by the fp32 accumulation
    error of conv1 plus one bf16 rounding step (2^-7 relative), and conv2
    carries that into y:

        |g - r| <= rtol |r| + L gamma_n2 absdot2
                   + L (2^-7 (absdot2 - |b2|) + L gamma_n1 carry)

    with absdot2 = |b2| + sum |w2 h| and carry = sum |w2| absdot1 (from
    oracle.ref.conv_chain).  The |b2| part is left in the 2^-7 term (a
    slightly looser bound)."""
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    absdot2 = np.asarray(absdot2, dtype=np.float64).ravel()
    carry = np.asarray(carry, dtype=np.float64).ravel()
    lip = 1.13 if gelu else 1.0
    lim = (RTOL["bf16"] * np.abs(ref) + lip * gamma(reduction_length(p2, True)) * absdot2
           + lip * (2.0 ** -7 * absdot2 + lip * gamma(reduction_length(p1, True)) * carry))
    err = np.abs(got - ref)
    finite = np.isfinite(got)
    plain = bound(ref, absdot2, p2, "bf16", True, gelu)
    return {
        "ok": bool(finite.all() and (err <= lim).all()),
        "n": int(got.size),
        "n_fail": int((~(err <= lim)).sum() + (~finite).sum()),
        "max_ratio": float((err / np.where(lim > 0, lim, 1.0)).max()) if got.size else 0.0,
        "within_single_call_bound": float((err <= plain).mean()) if got.size else 1.0,
        "max_abs_diff": float(err.max()) if got.size else 0.0,
        "limit": lim,
    }


def round_to_bf16_bits(v):
    """IEEE round-to-nearest-even of float32-exact values to bfloat16, as
    uint16 bit patterns (NaN stays NaN).  Used to form the expected output of
    integer-valued cases, whose fp32 result is exact and so has one correct
    bf16 rounding."""
    f = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    f32 = f.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), f, equal_nan=True):
        raise ValueError("round_to_bf16_bits expects float32-exact values")
    bits = f32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f32)
    if nan.any():
        rounded[nan] = ((bits[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
