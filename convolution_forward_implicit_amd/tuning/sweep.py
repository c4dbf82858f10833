"""Times every eligible tile configuration on a grid of convolution problems
through the C ABI and writes one CSV row per (problem, configuration).

    python -m convolution_forward_implicit_amd.tuning.sweep OUT.csv [PASSES]

Needs a GPU.  Every problem is timed with the two epilogues the workloads
use: none, and bias + GELU (the erf-GELU costs VALU time per output, which
matters for thin reductions); the "gelu" column says which.  Timing: cold
caches as in the benchmark (consecutive launches rotate through copies of
x, w, bias and y that together exceed the 256 MB last-level cache), 40
launches to raise the clock, then per configuration 3 untimed launches and
the median of 21, each timed by HIP events that the launch records when the
kernel starts and ends; all configurations are timed PASSES times (default
2), alternating between opposite orders, and the lowest median is kept.  A configuration with a
prepacked-weight form is timed the same way from its prepacked weights too
("ms_packed"; empty for the others).  Inputs are random (values do not
affect the timing).
"""
import csv
import itertools
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COLD_BYTES = 512 << 20    # buffer sets per problem: at least twice the last-level cache
FIELDS = ["dtype", "N", "G", "C", "K", "Di", "Hi", "Wi", "Z", "Y", "X", "sd", "sh", "sw",
          "pd", "ph", "pw", "dd", "dh", "dw", "gelu", "config", "ms", "ms_packed"]


def problem(N, G, C, K, inp, filt, stride, pad, dil):
    return {"N": N, "G": G, "C": C, "K": K, "in": tuple(inp), "filt": tuple(filt),
            "stride": tuple(stride), "pad": tuple(pad), "dil": tuple(dil)}


def grid():
    """The calibration grid: audio-style 1-D convs (the Whisper frontend
    shapes and neighbours), plain and grouped 2-D convs, grouped 3-D convs
    with and without dilation (enough dilation-2 shapes that every
    fixed-filter configuration compiled for it gets calibrated)."""
    out = []
    for N, C, K, L, k, s in [(1, 80, 384, 3000, 3, 1), (1, 384, 384, 3000, 3, 2), (4, 80, 384, 3000, 3, 1),
                             (32, 80, 384, 3000, 3, 1), (32, 384, 384, 3000, 3, 2), (8, 256, 256, 1000, 3, 1),
                             (1, 512, 512, 1500, 3, 1), (16, 128, 64, 2048, 5, 1), (2, 64, 128, 4096, 7, 2),
                             (64, 384, 384, 500, 3, 1)]:
        out.append(problem(N, 1, C, K, (1, 1, L), (1, 1, k), (1, 1, s), (0, 0, k // 2), (1, 1, 1)))
    for N, G, C, K, H, k, s, p, d in [(8, 4, 64, 64, 56, 3, 1, 1, 1), (8, 1, 64, 64, 56, 3, 1, 1, 1),
                                      (4, 1, 128, 128, 28, 3, 1, 1, 1), (16, 1, 256, 256, 14, 3, 1, 1, 1),
                                      (8, 8, 32, 32, 56, 3, 1, 1, 1), (2, 32, 16, 16, 112, 3, 1, 1, 1),
                                      (8, 1, 64, 128, 56, 1, 1, 0, 1), (4, 2, 128, 128, 28, 3, 2, 1, 1),
                                      (8, 4, 64, 64, 56, 3, 1, 2, 2), (1, 1, 256, 256, 64, 3, 1, 1, 1),
                                      (32, 1, 64, 64, 32, 3, 1, 1, 1), (8, 1, 512, 512, 7, 3, 1, 1, 1)]:
        out.append(problem(N, G, C, K, (1, H, H), (1, k, k), (1, s, s), (0, p, p), (1, d, d)))
    for N, G, C, K, D, H, k, p, d in [(2, 8, 32, 32, 16, 28, 3, 2, 2), (2, 1, 64, 64, 16, 28, 3, 1, 1),
                                      (1, 4, 32, 32, 8, 56, 3, 1, 1), (4, 1, 32, 64, 8, 28, 3, 1, 1),
                                      (2, 16, 16, 16, 16, 28, 3, 1, 1), (1, 2, 64, 64, 32, 32, 3, 1, 1),
                                      (1, 8, 32, 32, 16, 28, 3, 2, 2), (4, 8, 32, 32, 8, 28, 3, 2, 2),
                                      (2, 4, 32, 32, 16, 32, 3, 2, 2), (2, 16, 32, 32, 8, 28, 3, 2, 2)]:
        out.append(problem(N, G, C, K, (D, H, H), (k, k, k), (1, 1, 1), (p, p, p), (d, d, d)))
    return out


def main(path, passes=2):
    import torch
    from convolution_forward_implicit_amd import ConvFwd, ConvError, capi
    dev = torch.device("cuda:0")
    names = [capi.conv_fwd_config_name(i) for i in range(capi.conv_fwd_num_configs())]
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(FIELDS)
        for p, dt, ge in itertools.product(grid(), ["bf16", "f32"], [False, True]):
            if dt == "f32" and p["in"][1] > 1 and p["N"] > 4:
                continue   # keep the fp32 part of the grid small
            tdt = torch.float32 if dt == "f32" else torch.bfloat16
            ref = ConvFwd(p, dt, ge, ge)
            esz = 4 if dt == "f32" else 2
            set_bytes = esz * sum(math.prod(sh) for sh in (ref.x_shape, ref.w_shape, ref.y_shape))
            nsets = max(2, -(-COLD_BYTES // set_bytes))
            sets = []
            for _ in range(nsets):
                sets.append((torch.randn(ref.x_shape, device=dev).to(tdt), torch.randn(ref.w_shape, device=dev).to(tdt),
                             torch.randn(ref.b_shape, device=dev).to(tdt) if ge else None,
                             torch.empty(ref.y_shape, dtype=tdt, device=dev)))
            turn = [0]

            def nxt():
                turn[0] = (turn[0] + 1) % nsets
                return sets[turn[0]]

            plans = []
            for ci, name in enumerate(names):
                try:
                    c = ConvFwd(p, dt, ge, ge, config=ci)
                except ConvError:
                    continue

                def run(e=None, c=c):
                    x, w, b, y = nxt()
                    c(x, w, b, out=y, events=e)
                plans.append((name, c, run))
                try:
                    wps = [c.pack(w) for _, w, _, _ in sets]
                except ConvError:
                    continue

                def run_packed(e=None, c=c, wps=wps):
                    x, _, b, y = nxt()
                    c.run_packed(x, wps[turn[0]], b, out=y, events=e)
                plans.append((name + " packed", c, run_packed))
            for _ in range(40):           # bring the clock up before anything is timed
                x, w, b, y = nxt()
                ref(x, w, b, out=y)
            best = {}
            # passes in alternating opposite orders, the lowest median kept: a clock that
            # is still rising favours no particular position in the table
            for order in [plans, plans[::-1]] * ((passes + 1) // 2):
                for name, c, run in order:
                    for _ in range(3):
                        run()
                    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                           for _ in range(21)]
                    for a, e in evs:      # create the event handles the launches record
                        a.record()
                        e.record()
                    torch.cuda.synchronize()
                    for a, e in evs:      # kernel start/stop, without the launch gap
                        run((a, e))
                    torch.cuda.synchronize()
                    ts = sorted(a.elapsed_time(e) for a, e in evs)
                    med = ts[len(ts) // 2]
                    best[name] = min(best.get(name, med), med)
            for name, _, _ in plans:
                if name.endswith(" packed"):
                    continue
                pk = best.get(name + " packed")
                wr.writerow([dt, p["N"], p["G"], p["C"], p["K"], *p["in"], *p["filt"], *p["stride"],
                             *p["pad"], *p["dil"], int(ge), name, "%.6f" % best[name],
                             "" if pk is None else "%.6f" % pk])
            f.flush()
            del sets, plans
            print("swept", dt, "gelu" if ge else "", p, flush=True)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "sweep.csv", int(sys.argv[2]) if len(sys.argv) > 2 else 2)
