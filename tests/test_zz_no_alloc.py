"""The allocation-free backward-data entry point (conv_bwd_data_run_noalloc,
workspace in the library's static per-GPU array) against the entry point
that takes a caller workspace (conv_bwd_data_run), through the C ABI: the
same kernels run on the same inputs, so the results must be bit-identical.
Two calls in a row, the second on a smaller problem, then the first problem
again (nothing may carry over through the shared array); a plan whose
workspace exceeds the array is refused before any launch."""
import numpy as np
import pytest

import synthdata as sd

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(p, dtype, seed):
    from convolution_forward_implicit_amd import capi, desc_from_problem, ConvFwd
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    f = ConvFwd(p, dtype)
    dy_shape, w_shape, dx_shape = f.y_shape, f.w_shape, f.x_shape
    f.close()
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    dy = (torch.rand(dy_shape, generator=g, device=dev) * 2 - 1).to(tdt).contiguous()
    w = (torch.randn(w_shape, generator=g, device=dev) * 0.05).to(tdt).contiguous()
    plan = capi.conv_bwd_data_create(desc_from_problem(p, dtype))
    return plan, dy, w, dx_shape, tdt


def _with_workspace(plan, dy, w, dx_shape, tdt):
    from convolution_forward_implicit_amd import capi
    nbytes = capi.conv_bwd_data_workspace_bytes(plan)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dy.device)
    dx = torch.full(dx_shape, 3.0, dtype=tdt, device=dy.device)
    capi.conv_bwd_data_run(plan, dy.data_ptr(), w.data_ptr(), dx.data_ptr(), ws.data_ptr(), ws.numel(),
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return dx


def _noalloc(plan, dy, w, dx_shape, tdt):
    from convolution_forward_implicit_amd import capi
    dx = torch.full(dx_shape, 5.0, dtype=tdt, device=dy.device)
    capi.conv_bwd_data_run_noalloc(plan, dy.data_ptr(), w.data_ptr(), dx.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return dx


def _same(a, b):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


def test_noalloc_matches_caller_workspace_two_calls_second_smaller():
    from convolution_forward_implicit_amd import capi
    big = sd.conv1d_problem(8, 384, 384, 3000, 3, 2, 1)                   # strided: the stride phases' filters
    small = sd.problem(2, 4, 16, 8, (1, 13, 11), (1, 3, 3), (1, 1, 1), (0, 1, 1))   # stride 1: weights only
    cases = [(big, "bf16", 1), (small, "f32", 2)]
    plans = []
    try:
        results = []
        for p, dt, seed in cases:
            plan, dy, w, dxs, tdt = _case(p, dt, seed)
            plans.append(plan)
            assert capi.conv_bwd_data_workspace_bytes(plan) <= capi.CONV_BWD_DATA_SCRATCH_BYTES
            print("case: noalloc", p, dt, capi.conv_bwd_data_describe(plan), flush=True)
            got = _noalloc(plan, dy, w, dxs, tdt)
            results.append((plan, dy, w, dxs, tdt, got))
        assert capi.conv_bwd_data_workspace_bytes(plans[1]) < capi.conv_bwd_data_workspace_bytes(plans[0])
        for plan, dy, w, dxs, tdt, got in results:
            want = _with_workspace(plan, dy, w, dxs, tdt)
            assert _same(got, want)
        # the first problem again, after the smaller one used the array
        plan, dy, w, dxs, tdt, first = results[0]
        assert _same(_noalloc(plan, dy, w, dxs, tdt), first)
    finally:
        for plan in plans:
            capi.conv_bwd_data_destroy(plan)


def test_noalloc_refuses_a_workspace_beyond_the_array():
    from convolution_forward_implicit_amd import capi, desc_from_problem, ConvError
    p = sd.problem(48, 1, 64, 64, (1, 112, 112), (1, 3, 3), (1, 2, 2), (0, 1, 1))   # 2-D strided: spread dy of 80 MB
    plan = capi.conv_bwd_data_create(desc_from_problem(p, "bf16"))
    try:
        assert capi.conv_bwd_data_workspace_bytes(plan) > capi.CONV_BWD_DATA_SCRATCH_BYTES
        with pytest.raises(ConvError) as e:
            capi.conv_bwd_data_run_noalloc(plan, 16, 16, 16, 0)
        assert e.value.status == capi.CONV_ERR_UNSUPPORTED
    finally:
        capi.conv_bwd_data_destroy(plan)


def test_noalloc_under_graph_capture():
    """The allocation-free entry point is meant for code under graph
    capture: captured once, replayed three times with eager calls of it on
    other inputs between the replays (the shared array is rewritten each
    time), every replay bit-identical to the eager result."""
    from convolution_forward_implicit_amd import capi
    p = sd.conv1d_problem(4, 96, 64, 600, 3, 2, 1)       # strided: the stride phases' filters in the array
    plan, dy, w, dx_shape, tdt = _case(p, "bf16", 21)
    try:
        ref = _noalloc(plan, dy, w, dx_shape, tdt)
        dy2 = (dy.float() * -0.5).to(tdt).contiguous()
        dx = torch.empty(dx_shape, dtype=tdt, device=dy.device)
        side = torch.cuda.Stream(dy.device)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            capi.conv_bwd_data_run_noalloc(plan, dy.data_ptr(), w.data_ptr(), dx.data_ptr(),
                                           torch.cuda.current_stream(dy.device).cuda_stream)
        torch.cuda.synchronize()
        for k in range(3):
            dx.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert _same(dx, ref), k
            _noalloc(plan, dy2, w, dx_shape, tdt)      # eager work on the same array between replays
    finally:
        capi.conv_bwd_data_destroy(plan)
