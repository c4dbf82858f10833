"""Fits the selector's cost model to a sweep table and writes the
coefficients compiled into the library.

    python -m convolution_forward_implicit_amd.tuning.fit SWEEP.csv [--write]

Model, per tile configuration c and problem s (the unit is milliseconds):
    t_c(s) = a_c + b_c * r + d_c * r * nk + e_c * nk + f_c * gelu * r
    r  = ceil(tiles / CUs)          workgroups each compute unit runs
    nk = ceil(C*Z*Y*X / BK_c)       K-steps per workgroup
    gelu = 1 with the bias + GELU epilogue (its VALU time per workgroup), else 0
    tiles = ceil(M / BM_c) * ceil(K / BN_c) * G
(an input-patch configuration: tiles = boxes x channel tiles x planes x
groups, nk = Z * C / CC) fitted by least squares on relative error.  Reported: leave-one-problem-out
mean efficiency (best time / time of the pick), top-1 and top-5 hit rates --
the measures the Composable Kernel grouped-conv heuristic note uses for its
kernel selector -- with every problem held out of its own fit.
"""
import csv
import math
import os
import re
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(os.path.dirname(HERE), "csrc", "selector_coef.inc")
OUT_DB = os.path.join(os.path.dirname(HERE), "csrc", "selector_db.inc")
CUS = 256


def cfg_tile(name):
    """(BM, BN, BK, KG) of an implicit-GEMM configuration (KG reduction
    groups per workgroup), or ("patch", TH, TW, BN, CC) of an input-patch
    one."""
    m = re.match(r"bf16_patch_(\d+)x(\d+)x(\d+)_c(\d+)_s\d_p\d+x\d+_d\d$", name)
    if m:
        return ("patch",) + tuple(int(v) for v in m.groups())
    m = re.match(r"bf16_pfix_(\d+)x(\d+)x(\d+)_c(\d+)_s\d_f\d+x\d+_d\d+x\d+_w\d+_l\d_r\d_rr\d$", name)
    if m:
        return ("patch",) + tuple(int(v) for v in m.groups())
    m = re.match(r"(f32|bf16)_dma_(\d+)x(\d+)_w\dx\d_s\d_m\d+_k(\d)(_g\d)?(_f\d)?$", name)
    if m:
        esz = 2 if m.group(1) == "bf16" else 4
        return int(m.group(2)), int(m.group(3)), int(m.group(4)) * 128 // esz, int(m.group(5)[2:]) if m.group(5) else 1
    m = re.match(r"(f32|bf16)_(\d+)x(\d+)x(\d+)_w\dx\d_v\d$", name)
    return int(m.group(2)), int(m.group(3)), int(m.group(4)), 1


def features(prob, name):
    """[1, r, r*nk, nk, gelu*r] of a problem (dict with a "gelu" flag) for one
    configuration."""
    t = cfg_tile(name)
    o = [(prob["in"][i] + 2 * prob["pad"][i] - prob["dil"][i] * (prob["filt"][i] - 1) - 1) // prob["stride"][i] + 1
         for i in range(3)]
    if t[0] == "patch":
        _, TH, TW, BN, CC = t
        tiles = prob["N"] * o[0] * math.ceil(o[1] / TH) * math.ceil(o[2] / TW) * math.ceil(prob["K"] / BN) * prob["G"]
        nk = prob["filt"][0] * (prob["C"] // CC)
    else:
        BM, BN, BK, KG = t
        M = prob["N"] * o[0] * o[1] * o[2]
        tiles = math.ceil(M / BM) * math.ceil(prob["K"] / BN) * prob["G"]
        nk = math.ceil(math.ceil(prob["C"] * prob["filt"][0] * prob["filt"][1] * prob["filt"][2] / BK) / KG)
    r = math.ceil(tiles / CUS)
    g = 1.0 if prob.get("gelu") else 0.0
    return [1.0, float(r), float(r * nk), float(nk), g * r]


def load(path):
    probs = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            key = tuple(row[k] for k in ("dtype", "N", "G", "C", "K", "Di", "Hi", "Wi", "Z", "Y", "X",
                                         "sd", "sh", "sw", "pd", "ph", "pw", "dd", "dh", "dw", "gelu"))
            if key not in probs:
                v = [int(x) for x in key[1:]]
                probs[key] = {"dtype": key[0], "N": v[0], "G": v[1], "C": v[2], "K": v[3],
                              "in": v[4:7], "filt": v[7:10], "stride": v[10:13], "pad": v[13:16],
                              "dil": v[16:19], "gelu": v[19], "times": {}, "ptimes": {}}
            probs[key]["times"][row["config"]] = float(row["ms"])
            if row.get("ms_packed"):
                probs[key]["ptimes"][row["config"]] = float(row["ms_packed"])
    return list(probs.values())


def fit(probs, skip=None):
    """Per-configuration least squares; `skip` holds out one problem shape
    (both of its epilogue variants)."""
    coef = {}
    names = sorted({n for p in probs for n in p["times"]})
    held = None if skip is None else shape_key(probs[skip])
    for name in names:
        X, y = [], []
        for i, p in enumerate(probs):
            if (held is not None and shape_key(p) == held) or name not in p["times"]:
                continue
            X.append(features(p, name))
            y.append(p["times"][name])
        if len(y) < 6:
            continue
        X, y = np.array(X), np.array(y)
        w = 1.0 / y
        coef[name], *_ = np.linalg.lstsq(X * w[:, None], y * w, rcond=None)
    return coef


def shape_key(p):
    return (p["dtype"], p["N"], p["G"], p["C"], p["K"], tuple(p["in"]), tuple(p["filt"]),
            tuple(p["stride"]), tuple(p["pad"]), tuple(p["dil"]))


def pick(coef, p):
    pred = {n: float(np.dot(coef[n], features(p, n))) for n in p["times"] if n in coef}
    return min(pred, key=pred.get)


def quality(probs):
    eff, top1, top5 = [], 0, 0
    for i, p in enumerate(probs):
        c = pick(fit(probs, skip=i), p)
        order = sorted(p["times"], key=p["times"].get)
        eff.append(p["times"][order[0]] / p["times"][c])
        top1 += c == order[0]
        top5 += c in order[:5]
    n = len(probs)
    return {"problems": n, "mean_eff": float(np.mean(eff)), "min_eff": float(np.min(eff)),
            "top1": top1 / n, "top5": top5 / n}


def write(coef, path=OUT):
    with open(path, "w") as f:
        f.write("// Generated by convolution_forward_implicit_amd/tuning/fit.py from a sweep of every\n"
                "// configuration over the calibration grid: predicted milliseconds\n"
                "// t = a + b*r + d*r*nk + e*nk + f*gelu*r (r = workgroups per compute unit,\n"
                "// nk = K-steps, gelu = 1 with the GELU epilogue).\n")
        for name in sorted(coef):
            a, b, d, e, g = coef[name]
            f.write('    {"%s", %.6e, %.6e, %.6e, %.6e, %.6e},\n' % (name, a, b, d, e, g))


PACK_TOLERANCE = 1.03   # a configuration with a prepacked-weight form wins within 3% of the fastest


def packable(name):
    """The direct-to-LDS and fixed-filter patch kernels can run from
    prepacked weights (conv_fwd_run_packed); the others cannot."""
    return "_dma_" in name or "_pfix_" in name


def record(p):
    """The tuning record of one swept (problem, epilogue): (configuration,
    prepacked-weight configuration).  With prepacked timings in the sweep:
    the fastest configuration from natural weights and, separately, the
    fastest from prepacked weights (a plan holds both).  Without them: the
    fastest configuration, or the fastest one with a prepacked form when it
    is within PACK_TOLERANCE of it, serving both entry points."""
    times, ptimes = p["times"], p.get("ptimes", {})
    best = min(times, key=times.get)
    if ptimes:
        return best, min(ptimes, key=ptimes.get)
    if not packable(best):
        pk = [n for n in times if packable(n)]
        if pk:
            alt = min(pk, key=times.get)
            if times[alt] <= PACK_TOLERANCE * times[best]:
                best = alt
    return best, best if packable(best) else ""


def write_db(probs, path=OUT_DB):
    """Exact-shape tuning records: per swept (problem, epilogue), the
    fastest measured configurations (see record)."""
    with open(path, "w") as f:
        f.write("// Generated by convolution_forward_implicit_amd/tuning/fit.py: the configurations\n"
                "// measured fastest for each problem of the calibration sweep (MI355X, 256 CUs),\n"
                "// from natural and from prepacked weights (\"\": none has a prepacked form).\n"
                "// {dtype, gelu, N, G, C, K, in, filt, stride, pad, dil, config, packed config}\n")
        for p in probs:
            best, pbest = record(p)
            t = lambda v: "{%d, %d, %d}" % tuple(v)
            f.write('    {%d, %d, %d, %d, %d, %d, %s, %s, %s, %s, %s, "%s", "%s"},\n' % (
                0 if p["dtype"] == "f32" else 1, p["gelu"], p["N"], p["G"], p["C"], p["K"], t(p["in"]),
                t(p["filt"]), t(p["stride"]), t(p["pad"]), t(p["dil"]), best, pbest))


if __name__ == "__main__":
    probs = load(sys.argv[1])
    print(quality(probs))
    if "--write" in sys.argv:
        write(fit(probs))
        write_db(probs)
        print("wrote", OUT, OUT_DB)
