"""The library's entry points under HIP graph capture.

conv_fwd_run, conv_fwd_run_packed, conv_chain_run_packed and the backward
passes (with a caller workspace) allocate nothing and enqueue only kernels
on the caller's stream, so a caller can capture them in a HIP graph and
replay it.  Each graph is captured once,
then replayed several times with other eager work of the library between
the replays; every replay's output is compared bit for bit with the eager
run of the same inputs (the eager path itself is checked against the
oracle in test_parity_gpu.py)."""
import numpy as np
import pytest
import torch

import synthdata as sd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _up(a, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return t if dtype == "f32" else t.to(torch.bfloat16)


def _replays_match(dev, launch, y, eager_work, replays=3):
    """Captures launch() (which writes y) in a graph, then replays it
    `replays` times, clearing y before and running eager_work() after each
    replay; returns the outputs of every replay."""
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        launch(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    outs = []
    for _ in range(replays):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        outs.append(y.clone())
        eager_work()
        torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("packed", [False, True], ids=["natural", "prepacked"])
def test_conv_fwd_graph_replays_match_eager(dev, wid, packed):
    from convolution_forward_implicit_amd import ConvFwd, ConvError
    W = sd.workload(wid)
    dt = W["dtype"]
    p, hb, ge = W["layers"][-1]          # the last layer (the 384-channel one of the frontends)
    c = ConvFwd(p, dt, hb, ge)
    print("case: graph", wid, "packed" if packed else "natural", c.describe(), flush=True)
    rng = np.random.Generator(np.random.PCG64(91 + wid))
    x = _up(rng.uniform(-1, 1, c.x_shape), dt, dev)
    w = _up(rng.normal(0, 0.05, c.w_shape), dt, dev)
    b = _up(rng.normal(0, 0.02, c.b_shape), dt, dev) if hb else None
    if packed:
        try:
            wp = c.pack(w)
        except ConvError:
            pytest.skip("this plan's kernel has no prepacked form")
        run = lambda xx, yy, s=None: c.run_packed(xx, wp, b, out=yy, stream=s)
    else:
        run = lambda xx, yy, s=None: c(xx, w, b, out=yy, stream=s)
    y_eager = run(x, torch.empty(c.y_shape, dtype=x.dtype, device=dev))
    torch.cuda.synchronize()
    y = torch.empty_like(y_eager)
    # eager work between the replays: the same plan on other inputs
    x2 = _up(rng.uniform(-1, 1, c.x_shape), dt, dev)
    y2 = torch.empty_like(y_eager)
    outs = _replays_match(dev, lambda s: run(x, y, s), y, lambda: run(x2, y2))
    for k, o in enumerate(outs):
        assert torch.equal(o.view(torch.int16) if dt == "bf16" else o.view(torch.int32),
                           y_eager.view(torch.int16) if dt == "bf16" else y_eager.view(torch.int32)), k


def test_chain_graph_replays_match_eager(dev):
    """The fused batch-32 frontend from prepacked weights under capture."""
    from convolution_forward_implicit_amd import ConvChain
    W = sd.workload(3)
    (p1, hb, ge), (p2, _, _) = W["layers"]
    ch = ConvChain(p1, p2, "bf16", hb, ge)
    print("case: graph chain", ch.describe(), flush=True)
    x = _up(W["x"], "bf16", dev)
    w1, w2 = _up(W["w"][0], "bf16", dev), _up(W["w"][1], "bf16", dev)
    b1, b2 = _up(W["b"][0], "bf16", dev), _up(W["b"][1], "bf16", dev)
    wp = ch.pack(w1, w2)
    y_eager = ch.run_packed(x, wp, b1, b2)
    torch.cuda.synchronize()
    y = torch.empty_like(y_eager)
    x2 = torch.flip(x, dims=[1]).contiguous()
    y2 = torch.empty_like(y_eager)
    outs = _replays_match(dev, lambda s: ch.run_packed(x, wp, b1, b2, out=y, stream=s), y,
                          lambda: ch.run_packed(x2, wp, b1, b2, out=y2))
    for k, o in enumerate(outs):
        assert torch.equal(o.view(torch.int16), y_eager.view(torch.int16)), k


BWD_DATA_CASES = {
    "strided_1d_bf16": (sd.conv1d_problem(4, 96, 64, 600, 3, 2, 1), "bf16"),       # stride phases of dy
    "strided_2d_bf16": (sd.problem(2, 2, 16, 24, (1, 13, 11), (1, 3, 3), (1, 2, 2), (0, 1, 2), (1, 1, 2)), "bf16"),  # spread dy
    "unit_2d_f32": (sd.problem(2, 2, 16, 24, (1, 20, 18), (1, 3, 3), (1, 1, 1), (0, 1, 1)), "f32"),
    "dilated_3d_bf16": (sd.problem(1, 4, 32, 32, (6, 14, 14), (3, 3, 3), (1, 1, 1), (2, 2, 2), (2, 2, 2)), "bf16"),
}


@pytest.mark.parametrize("case", sorted(BWD_DATA_CASES))
def test_bwd_data_graph_replays_match_eager(dev, case):
    """Backward-data (weight flip or the stride phases' filters, dy spread
    for strided problems the phases do not cover, the forward
    kernels) captured with a caller workspace."""
    from convolution_forward_implicit_amd import ConvBwdData
    p, dt = BWD_DATA_CASES[case]
    bd = ConvBwdData(p, dt)
    print("case: graph bwd_data", case, bd.describe(), flush=True)
    rng = np.random.Generator(np.random.PCG64(7))
    dy = _up(rng.uniform(-1, 1, bd.dy_shape), dt, dev)
    w = _up(rng.normal(0, 0.05, bd.w_shape), dt, dev)
    ws = torch.empty(max(bd.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    dx_eager = bd(dy, w, workspace=ws)
    torch.cuda.synchronize()
    dx = torch.empty_like(dx_eager)
    dy2 = _up(rng.uniform(-1, 1, bd.dy_shape), dt, dev)
    dx2 = torch.empty_like(dx_eager)
    outs = _replays_match(dev, lambda s: bd(dy, w, out=dx, stream=s, workspace=ws), dx,
                          lambda: bd(dy2, w, out=dx2, workspace=ws))
    view = torch.int16 if dt == "bf16" else torch.int32
    for k, o in enumerate(outs):
        assert torch.equal(o.view(view), dx_eager.view(view)), k


def test_bwd_weight_graph_replays_match_eager(dev):
    """Backward-weight (split partials in the workspace, then their ordered
    sum) captured with a caller workspace."""
    from convolution_forward_implicit_amd import ConvBwdWeight
    p = sd.problem(4, 4, 64, 64, (1, 28, 28), (1, 3, 3), (1, 1, 1), (0, 1, 1))
    bw = ConvBwdWeight(p)
    print("case: graph bwd_weight", bw.describe(), flush=True)
    rng = np.random.Generator(np.random.PCG64(8))
    x = _up(rng.uniform(-1, 1, bw.x_shape), "bf16", dev)
    dy = _up(rng.uniform(-1, 1, bw.dy_shape), "bf16", dev)
    ws = torch.empty(max(bw.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    dw_eager = bw(x, dy, workspace=ws)
    torch.cuda.synchronize()
    dw = torch.empty_like(dw_eager)
    dy2 = _up(rng.uniform(-1, 1, bw.dy_shape), "bf16", dev)
    dw2 = torch.empty_like(dw_eager)
    outs = _replays_match(dev, lambda s: bw(x, dy, out=dw, stream=s, workspace=ws), dw,
                          lambda: bw(x, dy2, out=dw2, workspace=ws))
    for k, o in enumerate(outs):
        assert torch.equal(o.view(torch.int16), dw_eager.view(torch.int16)), k
