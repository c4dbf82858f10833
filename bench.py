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
in the step time of the small workloads.  The warm-cache figures (value,
roofline) run every step on one buffer set; cold = the same measurement
rotating through device copies of the inputs, weights and outputs that
total at least 512 MiB (twice the MALL), so no step finds its data in the
L2 or the MALL.  cpu_baseline = the fp64 oracle on the host cores over a
bounded sample of the same workload.

    python bench.py --copy-bytes B [--steps K]

runs only a device-to-device copy of B bytes K times (the reference kernel
that scales the FETCH_SIZE / WRITE_SIZE counters to bytes).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}   # MI355X dense MFMA
HBM_GBS = 8000.0
COLD_POOL_BYTES = 512 << 20   # rotated buffer sets: twice the 256 MB MALL
METRIC = "conv fwd useful TFLOP/s and % of MFMA peak (Whisper frontend, grouped bf16)"
DEFAULT_WORKLOAD = "whisper_frontend_f32_b1"


_COMMENT = re.compile(rb"//[^\n]*|/\*.*?\*/", re.S)


def kernel_source_hash():
    """Hash of every source the HIP library is built from (kernels, host
    code, selector coefficients), with comments and whitespace taken out so
    that an edit that cannot change the compiled code keeps the hash."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "convolution_forward_implicit_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            code = b" ".join(_COMMENT.sub(b" ", f.read()).split())
        h.update(name.encode())
        h.update(code)
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
    ap.add_argument("--cold-steps", type=int, default=64,
                    help="steps of the cold-cache measurement (rotating buffer sets); 0 skips it")
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

    stream = torch.cuda.current_stream(dev)
    esz = 4 if dt == "f32" else 2
    fused = args.fused or args.fused_natural
    prepack = None
    if args.pass_ != "fwd":
        if fused:
            print("bench.py: --fused is a forward path", file=sys.stderr)
            sys.exit(2)
        return bench_backward(args, W, dt, tdt, dev, up)

    # Buffer sets: set 0 holds the workload's seeded arrays; further sets are
    # device copies of them, used by the cold-cache measurement, which
    # rotates through enough sets that no step finds its inputs, weights or
    # outputs in the L2 or the 256 MB MALL.
    def clone(t):
        return None if t is None else t.clone()

    if fused:
        if len(W["layers"]) != 2:
            print("bench.py: --fused needs a two-conv workload", file=sys.stderr)
            sys.exit(2)
        (p1, hb, ge), (p2, _, _) = W["layers"]
        chain = ConvChain(p1, p2, dt, hb, ge)
        base = {"x": up(W["x"]), "w1": up(W["w"][0]), "w2": up(W["w"][1]),
                "b1": up(W["b"][0]) if hb else None, "b2": up(W["b"][1]) if hb else None,
                "y": torch.empty(chain.y_shape, dtype=tdt, device=dev)}
        convs = [chain]
        flops = [chain.useful_flop()]
        dom = 0
        dom_alg_bytes = esz * (int(np.prod(chain.x_shape)) + int(np.prod(chain.w1_shape)) +
                               int(np.prod(chain.w2_shape)) + (2 * int(np.prod(chain.b_shape)) if hb else 0) +
                               int(np.prod(chain.y_shape)))

        def make_set(first):
            st = base if first else {k: clone(v) for k, v in base.items()}
            if args.fused:
                # weights are constant across steps: prepack once per set, as a model load would
                st["wp"] = chain.pack(st["w1"], st["w2"], stream=stream)
            return st

        def step(st, kev=None):
            if args.fused:
                chain.run_packed(st["x"], st["wp"], st["b1"], st["b2"], out=st["y"], stream=stream, events=kev)
            else:
                chain(st["x"], st["w1"], st["b1"], st["w2"], st["b2"], out=st["y"], stream=stream, events=kev)
    else:
        convs = [ConvFwd(p, dt, hb, ge) for p, hb, ge in W["layers"]]
        base = {"x": up(W["x"]), "w": [up(w) for w in W["w"]],
                "b": [up(b) if hb else None for b, (_, hb, _) in zip(W["b"], W["layers"])],
                "outs": [torch.empty(c.y_shape, dtype=tdt, device=dev) for c in convs]}
        flops = [c.useful_flop() for c in convs]
        dom = int(np.argmax(flops))
        dom_alg_bytes = esz * (int(np.prod(convs[dom].x_shape)) + int(np.prod(convs[dom].w_shape)) +
                               (int(np.prod(convs[dom].b_shape)) if convs[dom].has_bias else 0) +
                               int(np.prod(convs[dom].y_shape)))

        def make_set(first):
            if first:
                return base
            return {"x": clone(base["x"]), "w": [clone(w) for w in base["w"]], "b": [clone(b) for b in base["b"]],
                    "outs": [torch.empty_like(o) for o in base["outs"]]}

        def step(st, kev=None):
            x = st["x"]
            for li, c in enumerate(convs):
                c(x, st["w"][li], st["b"][li], out=st["outs"][li], stream=stream, events=kev if li == dom else None)
                x = st["outs"][li]

    def set_bytes(st):
        tot = 0
        for v in st.values():
            for t in (v if isinstance(v, list) else [v]):
                if t is not None:
                    tot += t.numel() * t.element_size()
        return tot

    sets = [make_set(True)]
    if args.fused:
        wp0 = sets[0]["wp"]
        pe = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        torch.cuda.synchronize()
        pe[0].record(stream)
        chain.pack(sets[0]["w1"], sets[0]["w2"], out=wp0, stream=stream)
        pe[1].record(stream)
        torch.cuda.synchronize()
        prepack = {"ms": round(pe[0].elapsed_time(pe[1]), 5), "bytes": int(wp0.numel()),
                   "when": "once, before the timed steps (weights are constant)"}

    def timed(K, E, pick):
        """K steps (step i on buffer set pick(i)) between two device
        synchronisations; the dominant kernel records start/stop events on
        every E-th step.  Returns (ms per step, mean dominant-kernel ms,
        launches timed, wall seconds)."""
        NE = (K + E - 1) // E
        ev = ([torch.cuda.Event(enable_timing=True) for _ in range(NE)],
              [torch.cuda.Event(enable_timing=True) for _ in range(NE)])
        for e in ev[0] + ev[1]:
            e.record(stream)              # creates the event handles the kernel launch records
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(K):
            st = sets[pick(i)]
            if i % E == 0:
                step(st, (ev[0][i // E], ev[1][i // E]))
            else:
                step(st)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return (start.elapsed_time(end) / K, float(np.mean([a.elapsed_time(b) for a, b in zip(*ev)])), NE, wall)

    for _ in range(args.warmup):
        step(sets[0])
    torch.cuda.synchronize()

    K = args.steps
    E = max(1, args.event_every)
    ms_step, dom_ms, NE, t_wall = timed(K, E, lambda i: 0)

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

    # Cold caches: rotate through sets totalling at least 2x the MALL, so
    # each step's buffers were last touched several hundred MB earlier.
    cold = None
    if args.cold_steps > 0:
        sb = set_bytes(sets[0])
        nsets = max(2, -(-COLD_POOL_BYTES // sb))
        while len(sets) < nsets:
            sets.append(make_set(False))
        for i in range(nsets):
            step(sets[i])
        torch.cuda.synchronize()
        Kc = args.cold_steps
        c_step, c_dom, c_ne, _ = timed(Kc, E, lambda i: (i + 1) % nsets)
        c_ach = flops[dom] / (c_dom * 1e-3) / 1e12
        cold = {"value": round(total_flop / (c_step * 1e-3) / 1e12, 4), "ms_per_step": round(c_step, 5),
                "kernel_ms": round(c_dom, 5), "achieved": round(c_ach, 3), "frac": round(c_ach / PEAK_TFLOPS[dt], 4),
                "hbm_GBs_algorithmic": round(alg_bytes / (c_dom * 1e-3) / 1e9, 1),
                "kernel_launches_timed": c_ne, "steps": Kc, "buffer_sets": nsets, "bytes_per_set": sb}

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
        "roofline": roof, "cold": cold, "cpu_baseline": cpu,
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
