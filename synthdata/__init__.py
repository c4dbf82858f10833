"""Seeded synthetic inputs for the forward-convolution workloads.

This module is shared by both sides of every parity check (the fp64 oracle
and the HIP library) and therefore holds none of the convolution's
arithmetic: it only draws random numbers, lays them out and rounds inputs to
the stated storage precision.

Workloads (all inputs in the library's channels-innermost layouts,
x: N x Di x Hi x Wi x G x C, w: G x K x Z x Y x X x C, b: G x K):

  conv1d_80to384_f32_b1     one conv1d 80->384, k=3, s=1, p=1, batch 1, fp32,
                            input [1,80,3000] (the first conv of the Whisper-tiny
                            encoder the ExecuTorch conv1d issue profiles)
  whisper_frontend_f32_b1   conv1d 80->384 k3 s1 p1 + bias + GELU, then
                            conv1d 384->384 k3 s2 p1 + bias + GELU, batch 1, fp32
  whisper_frontend_bf16_b32 the same two convs, batch 32, bf16 inputs/weights
  grouped_conv2d_bf16       N=8, 56x56, G=4, C=K=64 per group, 3x3, s1 p1 d1
  grouped_conv3d_bf16_dil2  N=2, 16x28x28, G=8, C=K=32 per group, 3x3x3, s1 p2 d2

Recipe: numpy Generator(PCG64(1000 + workload id)); draws in the order
x, w1, b1, w2, b2; inputs uniform[-1, 1); weights normal(0, 1/sqrt(C*taps))
(sigma is the standard deviation); biases normal(0, 0.02); values sampled in
float64, cast to float32, then rounded to bfloat16 (nearest-even) for bf16
workloads.  Conv1d tensors are drawn in PyTorch's NCL / KCX shapes and
transposed to the channels-last layouts (W x C, K x X x C).
"""
import numpy as np

WORKLOADS = {
    1: "conv1d_80to384_f32_b1",
    2: "whisper_frontend_f32_b1",
    3: "whisper_frontend_bf16_b32",
    4: "grouped_conv2d_bf16",
    5: "grouped_conv3d_bf16_dil2",
}
BY_NAME = {v: k for k, v in WORKLOADS.items()}


def problem(N, G, C, K, inp, filt, stride=(1, 1, 1), pad=(0, 0, 0), dil=(1, 1, 1)):
    """A problem dict (3-D canonical form; unit leading dims for 1-D/2-D)."""
    return {"N": int(N), "G": int(G), "C": int(C), "K": int(K),
            "in": tuple(int(v) for v in inp), "filt": tuple(int(v) for v in filt),
            "stride": tuple(int(v) for v in stride), "pad": tuple(int(v) for v in pad),
            "dil": tuple(int(v) for v in dil)}


def conv1d_problem(N, C, K, L, k, s, p, d=1):
    return problem(N, 1, C, K, (1, 1, L), (1, 1, k), (1, 1, s), (0, 0, p), (1, 1, d))


def round_bf16(a):
    """float32 -> nearest-even bfloat16, returned as bf16-exact float32."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    r = (((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32).reshape(f.shape)


def _store(a, dtype):
    a = np.asarray(a, dtype=np.float64).astype(np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def layers(wid):
    """[(problem, has_bias, gelu)] of a workload, in execution order."""
    if wid == 1:
        return [(conv1d_problem(1, 80, 384, 3000, 3, 1, 1), True, False)]
    if wid in (2, 3):
        n = 1 if wid == 2 else 32
        return [(conv1d_problem(n, 80, 384, 3000, 3, 1, 1), True, True),
                (conv1d_problem(n, 384, 384, 3000, 3, 2, 1), True, True)]
    if wid == 4:
        return [(problem(8, 4, 64, 64, (1, 56, 56), (1, 3, 3), (1, 1, 1), (0, 1, 1)), False, False)]
    if wid == 5:
        return [(problem(2, 8, 32, 32, (16, 28, 28), (3, 3, 3), (1, 1, 1), (2, 2, 2), (2, 2, 2)),
                 False, False)]
    raise KeyError(wid)


def dtype_of(wid):
    return "f32" if wid in (1, 2) else "bf16"


def workload(wid):
    """Seeded inputs of a workload: {"dtype", "layers": [(problem, has_bias,
    gelu)], "x": first input, "w": [per layer], "b": [per layer or None]}.
    Arrays are float32 (bf16-exact for bf16 workloads), library layout."""
    if isinstance(wid, str):
        wid = BY_NAME[wid]
    rng = np.random.Generator(np.random.PCG64(1000 + wid))
    dt = dtype_of(wid)
    ls = layers(wid)
    out = {"id": wid, "name": WORKLOADS[wid], "dtype": dt, "layers": ls, "w": [], "b": []}
    p0 = ls[0][0]
    if wid in (1, 2, 3):
        L = p0["in"][2]
        x = rng.uniform(-1.0, 1.0, size=(p0["N"], p0["C"], L))          # N, C, L
        out["x"] = _store(x.transpose(0, 2, 1), dt).reshape(p0["N"], 1, 1, L, 1, p0["C"])
        for p, hb, _ in ls:
            kx = p["filt"][2]
            fan = p["C"] * kx
            w = rng.normal(0.0, 1.0 / np.sqrt(fan), size=(p["K"], p["C"], kx))  # K, C, X
            out["w"].append(_store(w.transpose(0, 2, 1), dt).reshape(1, p["K"], 1, 1, kx, p["C"]))
            b = rng.normal(0.0, 0.02, size=(p["K"],))
            out["b"].append(_store(b, dt).reshape(1, p["K"]) if hb else None)
    else:
        p = p0
        Di, Hi, Wi = p["in"]
        Z, Y, X = p["filt"]
        x = rng.uniform(-1.0, 1.0, size=(p["N"], Di, Hi, Wi, p["G"], p["C"]))
        out["x"] = _store(x, dt)
        w = rng.normal(0.0, 1.0 / np.sqrt(p["C"] * Z * Y * X),
                       size=(p["G"], p["K"], Z, Y, X, p["C"]))
        out["w"].append(_store(w, dt))
        out["b"].append(None)
    return out


def random_inputs(p, dtype, seed, has_bias, kind="float", imax=2):
    """Inputs for an arbitrary problem: kind="float" draws x ~ U[-1,1),
    w ~ N(0, 1/sqrt(fan_in)), b ~ N(0, 0.02); kind="int" draws integers in
    {-imax..imax} for x, w and b (with the default 2 the sums stay far below
    2^24, so any fp32 summation order gives the exact result)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Di, Hi, Wi = p["in"]
    Z, Y, X = p["filt"]
    xs = (p["N"], Di, Hi, Wi, p["G"], p["C"])
    ws = (p["G"], p["K"], Z, Y, X, p["C"])
    bs = (p["G"], p["K"])
    if kind == "int":
        x = rng.integers(-imax, imax + 1, size=xs).astype(np.float32)
        w = rng.integers(-imax, imax + 1, size=ws).astype(np.float32)
        b = rng.integers(-imax, imax + 1, size=bs).astype(np.float32) if has_bias else None
        return x, w, b
    x = _store(rng.uniform(-1.0, 1.0, size=xs), dtype)
    w = _store(rng.normal(0.0, 1.0 / np.sqrt(p["C"] * Z * Y * X), size=ws), dtype)
    b = _store(rng.normal(0.0, 0.02, size=bs), dtype) if has_bias else None
    return x, w, b


def random_int8(shape, seed):
    """Integers in {-2..2} as int8 (one byte per element, for inputs of
    several GiB; exact in bf16 and fp32 once converted)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(-2, 3, size=shape, dtype=np.int8)
