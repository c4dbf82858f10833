"""The forward entry points under HIP graph capture.

conv_fwd_run, conv_fwd_run_packed and conv_chain_run_packed allocate
nothing and enqueue only kernels on the caller's stream, so a caller can
capture them in a HIP graph and replay it.  Each graph is captured once,
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
