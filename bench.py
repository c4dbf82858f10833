"""Throughput of forward convolution (implicit im2col + MFMA GEMM) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-suite]

One step = one pass of the whole workload (every conv layer, with its bias
and GELU epilogue) over one batch of seeded synthetic input already resident
in HBM.  The headline workload (--workload, default: the Whisper-tiny conv
frontend at batch 1 in fp32 -- conv1d 80->384 k3 s1 p1 + bias + GELU, then
384->384 k3 s2 p1 + bias + GELU on a [1, 80, 3000] input) gives `value`;
the same measurement of every workload (the single conv1d, both frontends,
the fused batch-32 frontend, the grouped 2-D and 3-D convs) is reported in
`workloads` of the same line.

Prints ONE JSON line:

* value: useful TFLOP/s of the headline step (2*MACs counting padded taps)
  over the wall time of K steps bracketed by device synchronisation, with
  cold caches: the steps rotate through device copies of the inputs,
  weights and outputs totalling at least 512 MiB (twice the MALL), so no
  step finds its data in the L2 or the MALL.  `warm` repeats it on one
  buffer set.
* workloads[name].layers[i]: each layer kernel's duration from HIP events
  that the launch itself records when the kernel starts and ends (on the
  stream it runs on), over a dedicated pass of --launches cold launches
  (median and mean), its useful TFLOP/s, the fraction of the MFMA peak of
  its dtype, its bound (MFMA or HBM, from its arithmetic intensity against
  the ridge), the fraction of that attainable roofline min(peak, AI * BW),
  and the HBM rate of its algorithmic bytes.
* roofline: the headline workload's dominant (most flop) kernel, from the
  same dedicated pass; traffic = HBM bytes per launch from the committed
  FETCH_SIZE / WRITE_SIZE counter summary while the kernel sources are
  unchanged, else null.
* peaks: spec peaks and the rates the peak probes reach on this GPU.
* cpu_baseline: the fp64 oracle timed on the host cores over a bounded
  sample of the headline workload, its one-thread rate on the single
  conv1d, the CPU model; and the parity of the outputs the timed GPU runs
  produced, on sampled elements, against the oracle.

    python bench.py --copy-bytes B [--steps K]

runs only a device-to-device copy of B bytes K times (the reference kernel
that scales the FETCH_SIZE / WRITE_SIZE counters to bytes).
"""
import argparse
import hashlib
import json
import os
import re
import subprocess
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
SUITE = ["conv1d_80to384_f32_b1", "whisper_frontend_f32_b1", "whisper_frontend_bf16_b32",
         "whisper_frontend_bf16_b32_fused", "grouped_conv2d_bf16", "grouped_conv3d_bf16_dil2"]
# the convolutions the >= 50%-of-bf16-peak target names (batch-32 384->384 layer, grouped convs)
TARGET_LAYERS = {("whisper_frontend_bf16_b32", 1), ("grouped_conv2d_bf16", 0), ("grouped_conv3d_bf16_dil2", 0)}
FUSED = "_fused"


_COMMENT = re.compile(rb"//[^\n]*|/\*.*?\*/", re.S)


def kernel_source_hash():
    """Hash of every source the HIP library is built from (kernels, host
    code, selector coefficients), with comments and whitespace taken out so
    that an edit that cannot change the compiled code keeps the hash."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "convolution_forward_implicit_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name == "peak_probe.hip":
            continue
        with open(os.path.join(d, name), "rb") as f:
            code = b" ".join(_COMMENT.sub(b" ", f.read()).split())
        h.update(name.encode())
        h.update(code)
    return h.hexdigest()[:16]


def recorded_traffic(workload, layer_index):
    """HBM bytes per launch of one layer's kernel, from the committed counter
    summary (profiles/traffic_<workload>.json), or None when there is none or
    the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    for lay in rec.get("layers", []):
        if lay.get("layer") == layer_index:
            return lay.get("hbm_bytes_per_launch")
    return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def one_thread_oracle():
    """The oracle over the whole single conv1d (80->384, L=3000, fp32) on one
    thread, in a child process started before this one touches the GPU."""
    code = ("import time, sys; sys.path.insert(0, %r)\n"
            "import synthdata as sd\nfrom oracle import ref\n"
            "W = sd.workload(1); p, hb, ge = W['layers'][0]\n"
            "t0 = time.perf_counter(); ref.conv_fwd(p, W['x'], W['w'][0], W['b'][0], ge, want_absdot=False)\n"
            "dt = time.perf_counter() - t0\n"
            "print(ref.max_threads(), dt, ref.useful_flop(p))\n" % ROOT)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       env=env, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr[-400:]}
    th, dt, fl = r.stdout.split()[-3:]
    return {"workload": "conv1d_80to384_f32_b1 (all 1152000 outputs)", "threads": int(th),
            "seconds": round(float(dt), 3), "value": round(float(fl) / float(dt) / 1e12, 6), "unit": "TFLOP/s"}


# ---------------------------------------------------------------------------
# Workload runners: plans, buffer sets and one step
class Runner:
    """Plans and device buffers of one workload; step(set, events) enqueues
    one pass of every layer on the stream."""

    def __init__(self, name, stream, fused_mode=None):
        import numpy as np
        import torch
        import synthdata as sd
        from convolution_forward_implicit_amd import ConvFwd, ConvChain
        self.name = name
        base_name = name[:-len(FUSED)] if name.endswith(FUSED) else name
        self.fused = fused_mode if fused_mode else ("prepacked" if name.endswith(FUSED) else None)
        W = sd.workload(base_name)
        self.W = W
        self.dt = dt = W["dtype"]
        self.esz = 4 if dt == "f32" else 2
        self.stream = stream
        dev = torch.device("cuda:0")
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        self.tdt = tdt

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(tdt).contiguous()

        if self.fused:
            (p1, hb, ge), (p2, _, _) = W["layers"]
            self.chain = ConvChain(p1, p2, dt, hb, ge)
            self.kernels = [self.chain]
            self.base = {"x": up(W["x"]), "w1": up(W["w"][0]), "w2": up(W["w"][1]),
                         "b1": up(W["b"][0]) if hb else None, "b2": up(W["b"][1]) if hb else None,
                         "y": torch.empty(self.chain.y_shape, dtype=tdt, device=dev)}
            self.flops = [self.chain.useful_flop()]
            c = self.chain
            self.alg_bytes = [self.esz * (int(np.prod(c.x_shape)) + int(np.prod(c.w1_shape)) +
                                          int(np.prod(c.w2_shape)) + (2 * int(np.prod(c.b_shape)) if hb else 0) +
                                          int(np.prod(c.y_shape)))]
        else:
            self.convs = [ConvFwd(p, dt, hb, ge) for p, hb, ge in W["layers"]]
            self.kernels = self.convs
            self.base = {"x": up(W["x"]), "w": [up(w) for w in W["w"]],
                         "b": [up(b) if hb else None for b, (_, hb, _) in zip(W["b"], W["layers"])],
                         "outs": [torch.empty(c.y_shape, dtype=tdt, device=dev) for c in self.convs]}
            self.flops = [c.useful_flop() for c in self.convs]
            self.alg_bytes = [self.esz * (int(np.prod(c.x_shape)) + int(np.prod(c.w_shape)) +
                                          (int(np.prod(c.b_shape)) if c.has_bias else 0) + int(np.prod(c.y_shape)))
                              for c in self.convs]
        self.sets = [self._prepare(self.base)]
        self.prepack = None
        if self.fused == "prepacked":
            pe = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            torch.cuda.synchronize()
            pe[0].record(stream)
            self.chain.pack(self.base["w1"], self.base["w2"], out=self.base["wp"], stream=stream)
            pe[1].record(stream)
            torch.cuda.synchronize()
            self.prepack = {"ms": round(pe[0].elapsed_time(pe[1]), 5), "bytes": int(self.base["wp"].numel()),
                            "when": "once per weight set, before the timed steps (weights are constant)"}

    def _prepare(self, st):
        if self.fused == "prepacked":
            # weights are constant across steps: prepack once per set, as a model load would
            st["wp"] = self.chain.pack(st["w1"], st["w2"], stream=self.stream)
        elif not self.fused:
            # each layer's weights in its plan's prepacked form, where the plan's kernel has one
            from convolution_forward_implicit_amd import ConvError
            st["wp"] = []
            for li, c in enumerate(self.convs):
                try:
                    st["wp"].append(c.pack(st["w"][li], stream=self.stream))
                except ConvError:
                    st["wp"].append(None)
        return st

    def packable(self):
        return (not self.fused) and any(v is not None for v in self.sets[0]["wp"])

    def set_bytes(self, st):
        tot = 0
        for v in st.values():
            for t in (v if isinstance(v, list) else [v]):
                if t is not None:
                    tot += t.numel() * t.element_size()
        return tot

    def make_cold_sets(self):
        """Device copies of the buffer set until the sets total at least
        COLD_POOL_BYTES."""
        import torch
        sb = self.set_bytes(self.sets[0])
        nsets = max(2, -(-COLD_POOL_BYTES // sb))
        clone = lambda t: None if t is None else t.clone()
        while len(self.sets) < nsets:
            b = self.base
            if self.fused:
                st = {k: clone(v) for k, v in b.items() if k != "wp"}
            else:
                st = {"x": clone(b["x"]), "w": [clone(w) for w in b["w"]], "b": [clone(v) for v in b["b"]],
                      "outs": [torch.empty_like(o) for o in b["outs"]]}
            self.sets.append(self._prepare(st))
        for st in self.sets:
            self.step(st)
        torch.cuda.synchronize()
        return nsets, sb

    def step(self, st, evs=None, packed=False):
        """evs: None, or one (start, stop) event pair per kernel; packed: run
        the layers that have prepacked weights from them."""
        s = self.stream
        if self.fused == "prepacked":
            self.chain.run_packed(st["x"], st["wp"], st["b1"], st["b2"], out=st["y"], stream=s,
                                  events=evs[0] if evs else None)
        elif self.fused:
            self.chain(st["x"], st["w1"], st["b1"], st["w2"], st["b2"], out=st["y"], stream=s,
                       events=evs[0] if evs else None)
        else:
            x = st["x"]
            for li, c in enumerate(self.convs):
                ev = evs[li] if evs else None
                if packed and st["wp"][li] is not None:
                    c.run_packed(x, st["wp"][li], st["b"][li], out=st["outs"][li], stream=s, events=ev)
                else:
                    c(x, st["w"][li], st["b"][li], out=st["outs"][li], stream=s, events=ev)
                x = st["outs"][li]

    def outputs(self, st):
        return [st["y"]] if self.fused else st["outs"]


def timed_steps(r, K, pick):
    """K steps (step i on buffer set pick(i)) between two device
    synchronisations: (ms per step, wall seconds)."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(r.stream)
    for i in range(K):
        r.step(r.sets[pick(i)])
    end.record(r.stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / K, time.perf_counter() - t0


def kernel_pass(r, L, pick, packed=False):
    """L steps, each kernel recording start/stop events from inside its own
    launch: per-kernel durations in microseconds, [kernel][launch]."""
    import torch
    import numpy as np
    nk = len(r.kernels)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nk)]
          for _ in range(L)]
    for row in ev:
        for a, b in row:
            a.record(r.stream)     # creates the event handles the kernel launches record
            b.record(r.stream)
    torch.cuda.synchronize()
    for i in range(L):
        r.step(r.sets[pick(i)], ev[i], packed)
    torch.cuda.synchronize()
    return np.array([[ev[i][k][0].elapsed_time(ev[i][k][1]) * 1e3 for i in range(L)] for k in range(nk)])


def layer_record(r, k, us, workload):
    import numpy as np
    dt = r.dt
    flop, ab = r.flops[k], r.alg_bytes[k]
    med, mean = float(np.median(us)), float(np.mean(us))
    peak = PEAK_TFLOPS[dt]
    ai = flop / ab
    roof = min(peak, ai * HBM_GBS / 1e3)          # TFLOP/s
    bound = "mfma" if ai * HBM_GBS / 1e3 >= peak else "hbm"
    ach = flop / (med * 1e-6) / 1e12
    rec = {"kernel": r.kernels[k].describe(), "useful_gflop": round(flop / 1e9, 4), "algorithmic_bytes": ab,
           "flop_per_byte": round(ai, 1), "bound": bound, "us_median": round(med, 3), "us_mean": round(mean, 3),
           "us_min": round(float(np.min(us)), 3), "launches": int(len(us)), "tflops": round(ach, 2),
           "frac_of_mfma_peak": round(ach / peak, 4), "attainable_tflops": round(roof, 1),
           "frac_of_attainable": round(ach / roof, 4), "hbm_GBs_algorithmic": round(ab / (med * 1e-6) / 1e9, 1),
           "hbm_traffic_bytes": recorded_traffic(workload, k)}
    if (workload, k) in TARGET_LAYERS:
        lim = flop / (0.5 * peak * 1e12) * 1e6
        rec["target"] = {"frac_of_mfma_peak": 0.5, "us_at_most": round(lim, 2), "met": med <= lim}
    return rec


def measure(r, steps, warmup, launches, workload):
    """Warm-up, the timed cold steps, the timed warm steps and the dedicated
    cold per-kernel pass of one workload."""
    import numpy as np
    for _ in range(warmup):
        r.step(r.sets[0])
    nsets, sb = r.make_cold_sets()
    ms_cold, wall = timed_steps(r, steps, lambda i: (i + 1) % nsets)
    ms_warm, _ = timed_steps(r, steps, lambda i: 0)
    us = kernel_pass(r, launches, lambda i: (i + 1) % nsets)
    total = float(sum(r.flops))
    layers = [layer_record(r, k, us[k], workload) for k in range(len(r.kernels))]
    if r.packable():
        # the same layers run from their plan-time prepacked weights (A/B)
        usp = kernel_pass(r, launches, lambda i: (i + 1) % nsets, packed=True)
        for k, lay in enumerate(layers):
            if r.sets[0]["wp"][k] is None:
                lay["prepacked"] = None
                continue
            med = float(np.median(usp[k]))
            ach = r.flops[k] / (med * 1e-6) / 1e12
            from convolution_forward_implicit_amd import capi
            lay["prepacked"] = {"config": capi.conv_fwd_config_name(r.convs[k].packed_config()),
                                "us_median": round(med, 3), "us_mean": round(float(np.mean(usp[k])), 3),
                                "tflops": round(ach, 2), "frac_of_mfma_peak": round(ach / PEAK_TFLOPS[r.dt], 4),
                                "bytes": int(r.sets[0]["wp"][k].numel())}
            if "target" in lay:
                lay["target"]["met_prepacked"] = med <= lay["target"]["us_at_most"]
    rec = {"dtype": r.dt, "batch": r.W["layers"][0][0]["N"], "useful_gflop_per_step": round(total / 1e9, 4),
           "step_tflops_cold": round(total / (ms_cold * 1e-3) / 1e12, 3), "ms_per_step_cold": round(ms_cold, 5),
           "step_tflops_warm": round(total / (ms_warm * 1e-3) / 1e12, 3), "ms_per_step_warm": round(ms_warm, 5),
           "kernel_sum_us_median": round(sum(l["us_median"] for l in layers), 3),
           "buffer_sets": nsets, "bytes_per_set": sb, "layers": layers}
    if r.prepack:
        rec["weight_prepack"] = r.prepack
    return rec, ms_cold, wall


# ---------------------------------------------------------------------------
# Measured peaks
def measured_peaks(stream):
    import torch
    from convolution_forward_implicit_amd import capi
    dev = torch.device("cuda:0")
    out = {}
    grid = 1024
    sink = torch.empty(grid * capi.conv_probe_threads(), dtype=torch.float32, device=dev)
    for kind, key, iters in ((0, "mfma_bf16_32x32x16_tflops", 4000), (1, "mfma_f32_16x16x4_tflops", 4000)):
        capi.conv_probe_mfma(kind, 200, grid, sink.data_ptr(), stream.cuda_stream)
        best = 0.0
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fl = capi.conv_probe_mfma(kind, iters, grid, sink.data_ptr(), stream.cuda_stream)
            b.record(stream)
            torch.cuda.synchronize()
            best = max(best, fl / (a.elapsed_time(b) * 1e-3) / 1e12)
        out[key] = round(best, 1)
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    rsink = torch.empty(8192 * capi.conv_probe_threads(), dtype=torch.int32, device=dev)
    best, best_grid = 0.0, 0
    for rgrid in (1024, 2048, 4096, 8192):
        for i in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            capi.conv_probe_hbm_read(buf.data_ptr(), nbytes, rgrid, rsink.data_ptr(), stream.cuda_stream)
            b.record(stream)
            torch.cuda.synchronize()
            rate = nbytes / (a.elapsed_time(b) * 1e-3) / 1e9
            if i and rate > best:
                best, best_grid = rate, rgrid
    out["hbm_read_GBs"] = round(best, 1)
    out["hbm_read_grid"] = best_grid
    dst = torch.empty_like(buf)
    best = 0.0
    for i in range(4):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(buf)
        b.record(stream)
        torch.cuda.synchronize()
        if i:
            best = max(best, 2 * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    out["hbm_copy_GBs_read_plus_write"] = round(best, 1)
    del buf, dst
    return {"spec": {"mfma_bf16_tflops": PEAK_TFLOPS["bf16"], "mfma_f32_tflops": PEAK_TFLOPS["f32"],
                     "hbm_GBs": HBM_GBS},
            "measured": out,
            "how": "MFMA: 1024 workgroups of 4 waves, each wave running 8 independent accumulator chains back "
                   "to back (best of 3 launches); HBM: a streaming read of 1 GiB (16-byte vectors, 8 in flight "
                   "per lane; best over grids of 1024-8192 workgroups) and a 1 GiB device copy; timed with "
                   "events"}


# ---------------------------------------------------------------------------
# CPU baseline (the only leg that runs the oracle) and the parity of the
# outputs the timed GPU runs produced
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


def parity_of_outputs(r, host_outs, npts):
    """Sampled elements of the outputs a timed GPU run produced against the
    oracle on the same inputs (each layer after the first fed the device's
    own intermediate; the fused frontend against the oracle's chain, which
    rounds its own intermediate to bf16)."""
    import numpy as np
    from oracle import ref, check
    W = r.W
    res = []
    if r.fused:
        (p1, _, ge), (p2, _, _) = W["layers"]
        ys = ref.shapes(p2)[3]
        idx = np.random.Generator(np.random.PCG64(7)).integers(0, int(np.prod(ys)), npts)
        v, a2, cy = ref.conv_chain_points(p1, p2, W["x"], W["w"][0], W["b"][0], W["w"][1], W["b"][1], ge, idx)
        st = check.check_chain(host_outs[0].ravel()[idx], v, a2, cy, p1, p2, ge)
        res.append({"layer": "fused", "n": st["n"], "ok": st["ok"], "max_ratio": round(st["max_ratio"], 4),
                    "max_abs_diff": st["max_abs_diff"]})
        return res
    x = W["x"]
    for li, (p, hb, ge) in enumerate(W["layers"]):
        ys = ref.shapes(p)[3]
        idx = np.random.Generator(np.random.PCG64(11 + li)).integers(0, int(np.prod(ys)), npts)
        v, a = ref.conv_fwd_points(p, x, W["w"][li], W["b"][li], ge, idx)
        st = check.check(host_outs[li].ravel()[idx], v, a, p, r.dt, hb, ge)
        res.append({"layer": li, "n": st["n"], "ok": st["ok"], "max_ratio": round(st["max_ratio"], 4),
                    "max_abs_diff": st["max_abs_diff"], "cosine": round(st["cosine"], 9)})
        x = host_outs[li]
    return res


def host_copies(r):
    import numpy as np
    return [o.float().cpu().numpy().astype(np.float64) for o in r.outputs(r.sets[0])]


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of each workload (cold and warm)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, help="headline workload (value, roofline)")
    ap.add_argument("--launches", type=int, default=64,
                    help="cold launches of each kernel in the dedicated event-timed pass")
    ap.add_argument("--no-suite", action="store_true", help="measure the headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the oracle CPU baseline (0 = skip the oracle leg: no parity, no baseline)")
    ap.add_argument("--parity-points", type=int, default=1500,
                    help="sampled output elements per layer checked against the oracle in the CPU leg")
    ap.add_argument("--no-peaks", action="store_true", help="skip the peak probes")
    ap.add_argument("--fused", action="store_true",
                    help="run a two-conv headline workload as one fused kernel from prepacked weights")
    ap.add_argument("--fused-natural", action="store_true",
                    help="run a two-conv headline workload as one fused kernel from the natural weights")
    ap.add_argument("--pass", dest="pass_", default="fwd", choices=["fwd", "bwd_data", "bwd_weight"],
                    help="which pass of the workload's convolutions to time (backward: synthetic dy ~ U[-1,1))")
    ap.add_argument("--event-every", type=int, default=8, help="(backward passes) event-timed step interval")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a device copy of this many bytes --steps times")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (--gpus 1); a %d-GPU run is not "
              "supported -- the path needs no collective and would shard by batch" % max(args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    # the one-thread oracle runs in a child process before this process touches the GPU
    one_thread = one_thread_oracle() if (args.cpu_seconds > 0 and not args.copy_bytes and args.pass_ == "fwd") \
        else None

    import torch
    import synthdata as sd

    if args.copy_bytes:
        a = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel() * 4, "launches": args.steps}), flush=True)
        return

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.pass_ != "fwd":
        if args.fused or args.fused_natural:
            print("bench.py: --fused is a forward path", file=sys.stderr)
            sys.exit(2)
        return bench_backward(args, sd.workload(args.workload), dev)

    head = args.workload
    fused_mode = "prepacked" if args.fused else "natural" if args.fused_natural else None
    if fused_mode and len(sd.layers(sd.BY_NAME[head[:-len(FUSED)] if head.endswith(FUSED) else head])) != 2:
        print("bench.py: --fused needs a two-conv workload", file=sys.stderr)
        sys.exit(2)
    head_key = head + ("" if not fused_mode or head.endswith(FUSED) else FUSED if fused_mode == "prepacked"
                       else "_fused_natural")

    peaks = None if args.no_peaks else measured_peaks(stream)

    names = [head_key] + ([n for n in SUITE if n != head_key] if not args.no_suite else [])
    records, outs, runners = {}, {}, {}
    for name in names:
        print("bench: %s ..." % name, file=sys.stderr, flush=True)
        r = Runner(name, stream, fused_mode if name == head_key else None)
        rec, ms_cold, wall = measure(r, args.steps, args.warmup, args.launches, name)
        records[name] = rec
        runners[name] = r
        if name == head_key:
            head_ms, head_wall, head_runner = ms_cold, wall, r
        if args.cpu_seconds > 0:
            outs[name] = host_copies(r)      # set 0: written by the timed warm steps
        r.sets = r.sets[:1]                  # drop the cold copies before the next workload
        torch.cuda.synchronize()

    hr = records[head_key]
    total = float(sum(head_runner.flops))
    value = total / (head_ms * 1e-3) / 1e12
    dom = max(range(len(head_runner.flops)), key=lambda k: head_runner.flops[k])
    dl = hr["layers"][dom]
    dt = head_runner.dt
    ach_mean = head_runner.flops[dom] / (dl["us_mean"] * 1e-6) / 1e12
    roof = {"bound": dl["bound"], "achieved": round(ach_mean, 3), "peak": PEAK_TFLOPS[dt], "unit": "TFLOP/s",
            "frac": round(ach_mean / PEAK_TFLOPS[dt], 4), "traffic": dl["hbm_traffic_bytes"],
            "kernel": "layer %d: %s" % (dom + 1, dl["kernel"]), "kernel_us_mean": dl["us_mean"],
            "kernel_us_median": dl["us_median"], "kernel_launches_timed": dl["launches"],
            "caches": "cold (rotating buffer sets)", "algorithmic_bytes": dl["algorithmic_bytes"],
            "attainable_tflops": dl["attainable_tflops"], "frac_of_attainable": dl["frac_of_attainable"]}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(head_runner.W, args.cpu_seconds)
        cpu["value"] = round(cpu["value"], 6)
        cpu["cpu_model"] = cpu_model()
        cpu["one_thread"] = one_thread
        t0 = time.perf_counter()
        par = {name: parity_of_outputs(runners[name], outs[name], args.parity_points) for name in names}
        cpu["parity_of_timed_outputs"] = par
        cpu["parity_all_ok"] = all(l["ok"] for v in par.values() for l in v)
        cpu["parity_seconds"] = round(time.perf_counter() - t0, 2)

    line = {
        "metric": METRIC, "value": round(value, 4), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": head_key, "batch": hr["batch"], "layers": [l["kernel"] for l in hr["layers"]],
                   "useful_gflop_per_step": hr["useful_gflop_per_step"], "caches": "cold (rotating buffer sets)",
                   "wall_s_timed": round(head_wall, 4), "parallelism": "single GPU",
                   "warm": {"value": hr["step_tflops_warm"], "ms_per_step": hr["ms_per_step_warm"]}},
        "roofline": roof, "peaks": peaks, "workloads": records, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_backward(args, W, dev):
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
    dt = W["dtype"]
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(tdt).contiguous()
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
