"""Throughput of forward convolution (implicit im2col + MFMA GEMM) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole workload (every conv layer, with its bias
and GELU epilogue) over one batch of seeded synthetic input already resident
in HBM.  Default workload: the Whisper-tiny conv frontend at batch 1 in fp32
(conv1d 80->384 k3 s1 p1 + bias + GELU, then 384->384 k3 s2 p1 + bias +
GELU on a [1, 80, 3000] input).  Other workloads (--workload):
conv1d_80to384_f32_b1, whisper_frontend_bf16_b32, grouped_conv2d_bf16,
grouped_conv3d_bf16_dil2.

Prints ONE JSON line.  value = useful TFLOP/s of the whole step (2*MACs
counting padded taps, over the wall time of K steps bracketed by device
synchronisation).  roofline = the dominant (most flop) kernel: its useful
flop per launch over its mean duration, from HIP events that the launch
itself records when the kernel starts and ends (on the stream it runs on),
against the MI355X dense MFMA peak of its dtype.  Those events are taken on
every --event-every'th step of the timed region (default 8): a launch that
records them costs the host ~10 us more, which at every step would show up
in the step time of the small workloads.  cpu_baseline = the fp64
oracle on the host cores over a bounded sample of the same workload.

    python bench.py --copy-bytes B [--steps K]

runs only a device-to-device copy of B bytes K times (the reference kernel
that scales the FETCH_SIZE / WRITE_SIZE counters to bytes).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}   # MI355X dense MFMA
HBM_GBS = 8000.0
METRIC = "conv fwd useful TFLOP/s and % of MFMA peak (Whisper frontend, grouped bf16)"
DEFAULT_WORKLOAD = "whisper_frontend_f32_b1"


def kernel_source_hash():
    """Hash of every source the HIP library is built from (kernels, host
    code, selector coefficients)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "convolution_forward_implicit_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, layer_index, launches_bytes):
    """HBM bytes per launch of the dominant kernel, from the committed
    counter summary (profiles/traffic_<workload>.json), or None when there
    is none or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("layer") != layer_index:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(W, target_s):
    """Times the fp64 oracle on the host cores over a bounded sample of the
    workload: whole layers (repeated to fill the time budget) when a layer is
    small, otherwise a random sample of its outputs; the rate is useful flop
    of the sample over its time."""
    import numpy as np
    from oracle import ref
    flop, secs, parts = 0.0, 0.0, []
    budget = target_s / len(W["layers"])
    x = W["x"]
    for li, (p, hb, ge) in enumerate(W["layers"]):
        w, b = W["w"][li], W["b"][li]
        _, _, _, ys = ref.shapes(p)
        xin = np.ascontiguousarray(x, dtype=np.float64) if x is not None else None
        if xin is None:
            xin = np.zeros(ref.shapes(p)[0])
        per_out = ref.useful_flop(p) / float(np.prod(ys))
        # calibrate on a small sample, then size the timed sample to the budget
        rng = np.random.Generator(np.random.PCG64(li))
        idx = rng.integers(0, int(np.prod(ys)), 2000)
        t0 = time.perf_counter()
        ref.conv_fwd_points(p, xin, w, b, ge, idx)
        t_cal = max(time.perf_counter() - t0, 1e-4)
        n = int(min(np.prod(ys), max(2000, 2000 * budget / t_cal)))
        if n >= np.prod(ys):
            reps, dt = 0, 0.0
            while reps == 0 or dt < budget:
                t0 = time.perf_counter()
                y = ref.conv_fwd(p, xin, w, b, ge, want_absdot=False)
                dt += time.perf_counter() - t0
                reps += 1
            parts.append("layer %d: all %d outputs x %d" % (li + 1, int(np.prod(ys)), reps))
            flop += ref.useful_flop(p) * reps
            x = y
        else:
            idx = rng.integers(0, int(np.prod(ys)), n)
            t0 = time.perf_counter()
            ref.conv_fwd_points(p, xin, w, b, ge, idx)
            dt = time.perf_counter() - t0
            parts.append("layer %d: %d random outputs of %d" % (li + 1, n, int(np.prod(ys))))
            flop += per_out * n
            x = None
        secs += dt
    return {"value": flop / secs / 1e12, "unit": "TFLOP/s", "cores": ref.max_threads(),
            "kind": "oracle", "sample": "; ".join(parts) + " (fp64 direct loops, %.1f s)" % secs}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--event-every", type=int, default=8,
                    help="record the dominant kernel's start/stop events on every N-th timed step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the oracle CPU baseline (0 = skip)")
    ap.add_argument("--fused", action="store_true",
                    help="run a two-conv frontend workload as one fused kernel from prepacked weights "
                         "(conv_chain_pack_weights once, then conv_chain_run_packed per step)")
    ap.add_argument("--fused-natural", action="store_true",
                    help="run a two-conv frontend workload as one fused kernel from the natural weights "
                         "(conv_chain_run)")
    ap.add_argument("--pass", dest="pass_", default="fwd", choices=["fwd", "bwd_data", "bwd_weight"],
                    help="which pass of the workload's convolutions to time (backward: synthetic dy ~ U[-1,1))")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a device copy of this many bytes --steps times")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (--gpus 1); a %d-GPU run is not "
              "supported -- the path needs no collective and would shard by batch" % max(args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synthdata as sd
    from convolution_forward_implicit_amd import ConvFwd, ConvChain

    if args.copy_bytes:
        a = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel() * 4, "launches": args.steps}), flush=True)
        return

    W = sd.workload(args.workload)
    dt = W["dtype"]
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dt == "f32" else torch.bfloat16

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(tdt).contiguous()

    convs, ws, bs, outs = [], [], [], []
    x0 = up(W["x"])
    stream = torch.cuda.current_stream(dev)
    esz = 4 if dt == "f32" else 2
    fused = args.fused or args.fused_natural
    prepack = None
    if args.pass_ != "fwd":
        if fused:
            print("bench.py: --fused is a forward path", file=sys.stderr)
            sys.exit(2)
        return bench_backward(args, W, dt, tdt, dev, up)
    if fused:
        if len(W["layers"]) != 2:
            print("bench.py: --fused needs a two-conv workload", file=sys.stderr)
            sys.exit(2)
        (p1, hb, ge), (p2, _, _) = W["layers"]
        chain = ConvChain(p1, p2, dt, hb, ge)
        w1, w2 = up(W["w"][0]), up(W["w"][1])
        b1, b2 = (up(W["b"][0]), up(W["b"][1])) if hb else (None, None)
        y = torch.empty(chain.y_shape, dtype=tdt, device=dev)
        convs = [chain]
        flops = [chain.useful_flop()]
        dom = 0
        dom_alg_bytes = esz * (int(np.prod(chain.x_shape)) + int(np.prod(chain.w1_shape)) +
                               int(np.prod(chain.w2_shape)) + (2 * int(np.prod(chain.b_shape)) if hb else 0) +
                               int(np.prod(chain.y_shape)))

        if args.fused:
            # weights are constant across steps: prepack once, as a model load would
            wp = chain.pack(w1, w2, stream=stream)
            pe = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            torch.cuda.synchronize()
            pe[0].record(stream)
            chain.pack(w1, w2, out=wp, stream=stream)
            pe[1].record(stream)
            torch.cuda.synchronize()
            prepack = {"ms": round(pe[0].elapsed_time(pe[1]), 5), "bytes": int(wp.numel()),
                       "when": "once, before the timed steps (weights are constant)"}

            def step(ev=None, i=0):
                kev = (ev[0][i], ev[1][i]) if ev is not None else None
                chain.run_packed(x0, wp, b1, b2, out=y, stream=stream, events=kev)
        else:
            def step(ev=None, i=0):
                kev = (ev[0][i], ev[1][i]) if ev is not None else None
                chain(x0, w1, b1, w2, b2, out=y, stream=stream, events=kev)
    else:
        for li, (p, hb, ge) in enumerate(W["layers"]):
            c = ConvFwd(p, dt, hb, ge)
            convs.append(c)
            ws.append(up(W["w"][li]))
            bs.append(up(W["b"][li]) if hb else None)
            outs.append(torch.empty(c.y_shape, dtype=tdt, device=dev))
        flops = [c.useful_flop() for c in convs]
        dom = int(np.argmax(flops))
        dom_alg_bytes = esz * (int(np.prod(convs[dom].x_shape)) + int(np.prod(convs[dom].w_shape)) +
                               (int(np.prod(convs[dom].b_shape)) if convs[dom].has_bias else 0) +
                               int(np.prod(convs[dom].y_shape)))

        def step(ev=None, i=0):
            x = x0
            for li, c in enumerate(convs):
                kev = (ev[0][i], ev[1][i]) if ev is not None and li == dom else None
                c(x, ws[li], bs[li], out=outs[li], stream=stream, events=kev)
                x = outs[li]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    E = max(1, args.event_every)
    NE = (K + E - 1) // E             # steps whose dominant launch records events
    ev = ([torch.cuda.Event(enable_timing=True) for _ in range(NE)],
          [torch.cuda.Event(enable_timing=True) for _ in range(NE)])
    for e in ev[0] + ev[1]:
        e.record(stream)              # creates the event handles the kernel launch records
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        if i % E == 0:
            step(ev, i // E)
        else:
            step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / K
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(*ev)]))

    total_flop = float(sum(flops))
    value = total_flop / (ms_step * 1e-3) / 1e12
    achieved = flops[dom] / (dom_ms * 1e-3) / 1e12
    alg_bytes = dom_alg_bytes
    roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_TFLOPS[dt],
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[dt], 4),
            "traffic": recorded_traffic(args.workload + ("_fused" if args.fused else "_fused_natural" if args.fused_natural
                                                         else ""), dom, alg_bytes),
            "kernel": "layer %d: %s" % (dom + 1, convs[dom].describe()),
            "kernel_ms": round(dom_ms, 5), "kernel_launches_timed": NE, "algorithmic_bytes": alg_bytes,
            "hbm_GBs_algorithmic": round(alg_bytes / (dom_ms * 1e-3) / 1e9, 1)}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(W, args.cpu_seconds)
        cpu["value"] = round(cpu["value"], 6)

    line = {
        "metric": METRIC, "value": round(value, 4), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": args.workload, "fused": "prepacked" if args.fused else "natural" if args.fused_natural
                   else False, "batch": W["layers"][0][0]["N"],
                   "layers": [c.describe() for c in convs], "useful_gflop_per_step": round(total_flop / 1e9, 4),
                   "wall_s_timed": round(t_wall, 4), "parallelism": "single GPU",
                   "weight_prepack": prepack},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_backward(args, W, dt, tdt, dev, up):
    """Times one backward pass (input or weight gradient) of every layer of
    the workload: a step is that pass over all layers, on synthetic output
    gradients dy ~ U[-1, 1) (seeded) and, for the weight gradient of a layer
    after the first, a synthetic input of that layer's shape.  Each layer's
    call (its small preparation kernels included) is bracketed by stream
    events on every --event-every-th step; the roofline entry is the
    dominant layer's call."""
    import numpy as np
    import torch
    from convolution_forward_implicit_amd import ConvBwdData, ConvBwdWeight
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    rnd = lambda shape: (torch.rand(shape, generator=gen, device=dev) * 2 - 1).to(tdt).contiguous()
    ops, args_ = [], []
    for li, (p, _, _) in enumerate(W["layers"]):
        if args.pass_ == "bwd_data":
            c = ConvBwdData(p, dt)
            a = (rnd(c.dy_shape), up(W["w"][li]))
        else:
            c = ConvBwdWeight(p, dt)
            a = (up(W["x"]) if li == 0 else rnd(c.x_shape), rnd(c.dy_shape))
        ops.append(c)
        args_.append(a)
    outs = [None] * len(ops)
    flops = [c.useful_flop() for c in ops]
    dom = int(np.argmax(flops))

    def step():
        for li, c in enumerate(ops):
            outs[li] = c(*args_[li], out=outs[li], stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    E = max(1, args.event_every)
    lay = [[] for _ in ops]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    evs = []
    for i in range(K):
        if i % E == 0:
            for li, c in enumerate(ops):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                outs[li] = c(*args_[li], out=outs[li], stream=stream)
                e1.record(stream)
                evs.append((li, e0, e1))
        else:
            step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / K
    for li, e0, e1 in evs:
        lay[li].append(e0.elapsed_time(e1))
    dom_ms = float(np.mean(lay[dom]))
    value = float(sum(flops)) / (ms_step * 1e-3) / 1e12
    achieved = flops[dom] / (dom_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_TFLOPS[dt], "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS[dt], 4), "traffic": None,
            "kernel": "layer %d %s (whole call): %s" % (dom + 1, args.pass_, ops[dom].describe()),
            "kernel_ms": round(dom_ms, 5), "layer_ms": [round(float(np.mean(v)), 5) for v in lay]}
    line = {
        "metric": METRIC, "value": round(value, 4), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": args.workload, "pass": args.pass_, "batch": W["layers"][0][0]["N"],
                   "layers": [c.describe() for c in ops], "useful_gflop_per_step": round(sum(flops) / 1e9, 4),
                   "wall_s_timed": round(t_wall, 4), "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
