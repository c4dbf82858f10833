"""convfwd: forward convolution as implicit im2col + tiled MFMA GEMM on MI355X.

The computation lives in the HIP library libconvfwd.so (C ABI in
include/convfwd.h); this package only marshals arguments.  PyTorch supplies
device memory and streams:

    from convolution_forward_implicit_amd import ConvFwd
    conv = ConvFwd(problem, "bf16", has_bias=True, gelu=True)
    y = conv(x, w, bias)          # x, w, bias: contiguous cuda tensors in the
                                  # library layouts (NDHWGC, GKZYXC, GK)

A problem is a dict {"N", "G", "C", "K", "in": (D, H, W), "filt": (Z, Y, X),
"stride", "pad", "dil"} (C and K per group); a 1-D convolution has
D = H = 1, a 2-D one D = 1.

ConvChain(first, second, "bf16", has_bias, gelu) runs two 1-D convs back to
back in one kernel (the conv frontend), the intermediate kept on chip;
ConvChain.pack(w1, w2) prepacks the weights once and ConvChain.run_packed
runs the chain from them.

ConvBwdData(problem, dtype) is the input gradient of a forward problem,
ConvBwdWeight(problem) its weight gradient (bf16).
"""
from . import capi
from .capi import ConvError  # noqa: F401

__all__ = ["ConvFwd", "ConvChain", "ConvBwdData", "ConvBwdWeight", "ConvError", "capi", "desc_from_problem"]


def _ndim(p):
    triv = lambda i: (p["in"][i] == 1 and p["filt"][i] == 1 and p["stride"][i] == 1
                      and p["pad"][i] == 0 and p["dil"][i] == 1)
    if not triv(0):
        return 3
    return 2 if not triv(1) else 1


def desc_from_problem(p, dtype, has_bias=False, gelu=False):
    return capi.make_desc(_ndim(p), dtype, p["N"], p["G"], p["C"], p["K"], p["in"], p["filt"],
                          p["stride"], p["pad"], p["dil"], has_bias, gelu)


class ConvFwd:
    """A plan for one problem.  Calling it enqueues the kernel on the current
    torch stream (or `stream`) and returns y."""

    def __init__(self, problem, dtype, has_bias=False, gelu=False, config=None):
        self.problem = dict(problem)
        self.dtype = dtype
        self.has_bias = bool(has_bias)
        self.gelu = bool(gelu)
        self._desc = desc_from_problem(problem, dtype, has_bias, gelu)
        self._plan = (capi.conv_fwd_create(self._desc) if config is None
                      else capi.conv_fwd_create_with_config(self._desc, config))
        self.out_dims = capi.conv_fwd_out_dims(self._plan)
        p = self.problem
        self.x_shape = (p["N"],) + tuple(p["in"]) + (p["G"], p["C"])
        self.w_shape = (p["G"], p["K"]) + tuple(p["filt"]) + (p["C"],)
        self.b_shape = (p["G"], p["K"])
        self.y_shape = (p["N"],) + self.out_dims + (p["G"], p["K"])

    def useful_flop(self):
        """2 * multiply-adds counting padded taps (the library's count)."""
        return capi.conv_fwd_useful_flop(self._plan)

    def describe(self):
        return capi.conv_fwd_describe(self._plan)

    def packed_config(self):
        """Index of the tile configuration pack / run_packed use (the
        plan's own, or the one a tuning record names for prepacked
        weights)."""
        return capi.conv_fwd_packed_config(self._plan)

    def packed_bytes(self):
        """Size of this plan's prepacked weights (ConvError UNSUPPORTED when
        the plan's kernel reads natural weights only)."""
        return capi.conv_fwd_packed_bytes(self._plan)

    def pack(self, w, out=None, stream=None):
        """This plan's prepacked weights (a uint8 cuda tensor) from w,
        enqueued on `stream`; pack once, reuse for every run_packed."""
        import torch
        wp = self._tensor(w, self.w_shape, "w", torch)
        nbytes = self.packed_bytes()
        if out is None:
            out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
        if out.device.type != "cuda" or out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() != nbytes:
            raise ValueError("packed must be a contiguous cuda uint8 tensor of %d bytes" % nbytes)
        s = stream if stream is not None else torch.cuda.current_stream(w.device)
        capi.conv_fwd_pack_weights(self._plan, wp, out.data_ptr(), s.cuda_stream)
        return out

    def run_packed(self, x, packed, bias=None, out=None, stream=None, events=None):
        """As __call__, with the weights from pack()."""
        import torch
        xp = self._tensor(x, self.x_shape, "x", torch)
        if packed.device.type != "cuda" or packed.dtype != torch.uint8 or not packed.is_contiguous():
            raise ValueError("packed must be a contiguous cuda uint8 tensor (from pack)")
        if packed.numel() != self.packed_bytes():
            raise ValueError("packed has %d bytes, expected %d" % (packed.numel(), self.packed_bytes()))
        bp = None
        if self.has_bias:
            if bias is None:
                raise ValueError("this plan has a bias")
            bp = self._tensor(bias, self.b_shape, "bias", torch)
        elif bias is not None:
            raise ValueError("this plan has no bias")
        if out is None:
            out = torch.empty(self.y_shape, dtype=x.dtype, device=x.device)
        yp = self._tensor(out, self.y_shape, "out", torch)
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        if events is None:
            capi.conv_fwd_run_packed(self._plan, xp, packed.data_ptr(), bp, yp, s.cuda_stream)
        else:
            capi.conv_fwd_run_packed_events(self._plan, xp, packed.data_ptr(), bp, yp, s.cuda_stream,
                                            events[0].cuda_event, events[1].cuda_event)
        return out

    def close(self):
        if getattr(self, "_plan", None):
            capi.conv_fwd_destroy(self._plan)
            self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _tensor(self, t, shape, name, torch):
        tdt = torch.float32 if self.dtype == "f32" else torch.bfloat16
        if t.device.type != "cuda":
            raise ValueError("%s must be a cuda tensor" % name)
        if t.dtype != tdt:
            raise ValueError("%s must be %s, got %s" % (name, tdt, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        n = 1
        for s in shape:
            n *= s
        if t.numel() != n:
            raise ValueError("%s has %d elements, expected shape %r" % (name, t.numel(), shape))
        return t.data_ptr()

    def __call__(self, x, w, bias=None, out=None, stream=None, events=None):
        """events: optional (start, stop) torch.cuda.Event pair recorded when
        the kernel itself starts and ends (each must have been recorded once,
        so that its handle exists)."""
        import torch
        xp = self._tensor(x, self.x_shape, "x", torch)
        wp = self._tensor(w, self.w_shape, "w", torch)
        bp = None
        if self.has_bias:
            if bias is None:
                raise ValueError("this plan has a bias")
            bp = self._tensor(bias, self.b_shape, "bias", torch)
        elif bias is not None:
            raise ValueError("this plan has no bias")
        if out is None:
            out = torch.empty(self.y_shape, dtype=x.dtype, device=x.device)
        yp = self._tensor(out, self.y_shape, "out", torch)
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        if events is None:
            capi.conv_fwd_run(self._plan, xp, wp, bp, yp, s.cuda_stream)
        else:
            capi.conv_fwd_run_events(self._plan, xp, wp, bp, yp, s.cuda_stream,
                                     events[0].cuda_event, events[1].cuda_event)
        return out


class ConvChain:
    """A fused two-conv 1-D plan (conv_chain_create): y = act(conv2(h) + b2),
    h = round_bf16(act(conv1(x) + b1)).  Raises ConvError (UNSUPPORTED) for a
    chain outside the supported set (see include/convfwd.h)."""

    def __init__(self, first, second, dtype="bf16", has_bias=False, gelu=False):
        self.first, self.second = dict(first), dict(second)
        self.dtype = dtype
        self.has_bias = bool(has_bias)
        self.gelu = bool(gelu)
        self._plan = capi.conv_chain_create(desc_from_problem(first, dtype, has_bias, gelu),
                                            desc_from_problem(second, dtype, has_bias, gelu))
        p1, p2 = self.first, self.second
        self.x_shape = (p1["N"],) + tuple(p1["in"]) + (p1["G"], p1["C"])
        self.w1_shape = (p1["G"], p1["K"]) + tuple(p1["filt"]) + (p1["C"],)
        self.w2_shape = (p2["G"], p2["K"]) + tuple(p2["filt"]) + (p2["C"],)
        self.b_shape = (p1["G"], p1["K"])
        self.out_dims = capi.conv_chain_out_dims(self._plan)
        self.y_shape = (p2["N"],) + self.out_dims + (p2["G"], p2["K"])

    def useful_flop(self):
        """Both convs' 2 * multiply-adds, counting padded taps (the
        library's count)."""
        return capi.conv_chain_useful_flop(self._plan)

    def describe(self):
        return capi.conv_chain_describe(self._plan)

    def close(self):
        if getattr(self, "_plan", None):
            capi.conv_chain_destroy(self._plan)
            self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _tensor(self, t, shape, name, torch):
        if t.device.type != "cuda":
            raise ValueError("%s must be a cuda tensor" % name)
        if t.dtype != torch.bfloat16:
            raise ValueError("%s must be torch.bfloat16, got %s" % (name, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        n = 1
        for s in shape:
            n *= s
        if t.numel() != n:
            raise ValueError("%s has %d elements, expected shape %r" % (name, t.numel(), shape))
        return t.data_ptr()

    def __call__(self, x, w1, b1, w2, b2, out=None, stream=None, events=None):
        import torch
        xp = self._tensor(x, self.x_shape, "x", torch)
        w1p = self._tensor(w1, self.w1_shape, "w1", torch)
        w2p = self._tensor(w2, self.w2_shape, "w2", torch)
        if self.has_bias:
            if b1 is None or b2 is None:
                raise ValueError("this chain has biases")
            b1p = self._tensor(b1, self.b_shape, "b1", torch)
            b2p = self._tensor(b2, self.b_shape, "b2", torch)
        else:
            if b1 is not None or b2 is not None:
                raise ValueError("this chain has no bias")
            b1p = b2p = None
        if out is None:
            out = torch.empty(self.y_shape, dtype=x.dtype, device=x.device)
        yp = self._tensor(out, self.y_shape, "out", torch)
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        if events is None:
            capi.conv_chain_run(self._plan, xp, w1p, b1p, w2p, b2p, yp, s.cuda_stream)
        else:
            capi.conv_chain_run_events(self._plan, xp, w1p, b1p, w2p, b2p, yp, s.cuda_stream,
                                       events[0].cuda_event, events[1].cuda_event)
        return out

    def packed_bytes(self):
        """Size of the prepacked weights (ConvError UNSUPPORTED beyond the
        prepacked kernel's channel limit)."""
        return capi.conv_chain_packed_bytes(self._plan)

    def pack(self, w1, w2, out=None, stream=None):
        """Prepacked weights (a uint8 cuda tensor) from w1 and w2, enqueued on
        `stream`; do it once and reuse the result for every run_packed."""
        import torch
        w1p = self._tensor(w1, self.w1_shape, "w1", torch)
        w2p = self._tensor(w2, self.w2_shape, "w2", torch)
        nbytes = self.packed_bytes()
        if out is None:
            out = torch.empty(nbytes, dtype=torch.uint8, device=w1.device)
        if out.device.type != "cuda" or out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() != nbytes:
            raise ValueError("packed must be a contiguous cuda uint8 tensor of %d bytes" % nbytes)
        s = stream if stream is not None else torch.cuda.current_stream(w1.device)
        capi.conv_chain_pack_weights(self._plan, w1p, w2p, out.data_ptr(), s.cuda_stream)
        return out

    def run_packed(self, x, packed, b1, b2, out=None, stream=None, events=None):
        import torch
        xp = self._tensor(x, self.x_shape, "x", torch)
        if packed.device.type != "cuda" or packed.dtype != torch.uint8 or not packed.is_contiguous():
            raise ValueError("packed must be a contiguous cuda uint8 tensor (from pack)")
        if packed.numel() != self.packed_bytes():
            raise ValueError("packed has %d bytes, expected %d" % (packed.numel(), self.packed_bytes()))
        if self.has_bias:
            if b1 is None or b2 is None:
                raise ValueError("this chain has biases")
            b1p = self._tensor(b1, self.b_shape, "b1", torch)
            b2p = self._tensor(b2, self.b_shape, "b2", torch)
        else:
            if b1 is not None or b2 is not None:
                raise ValueError("this chain has no bias")
            b1p = b2p = None
        if out is None:
            out = torch.empty(self.y_shape, dtype=x.dtype, device=x.device)
        yp = self._tensor(out, self.y_shape, "out", torch)
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        if events is None:
            capi.conv_chain_run_packed(self._plan, xp, packed.data_ptr(), b1p, b2p, yp, s.cuda_stream)
        else:
            capi.conv_chain_run_packed_events(self._plan, xp, packed.data_ptr(), b1p, b2p, yp, s.cuda_stream,
                                              events[0].cuda_event, events[1].cuda_event)
        return out


class ConvBwdData:
    """Input gradient of a forward convolution problem (conv_bwd_data_*):
    dx = the gradient of <conv(x, w), dy> with respect to x.  `problem` is
    the forward problem; no bias or GELU.  The workspace it needs is
    allocated once here (torch, caller-side) and reused by every call."""

    def __init__(self, problem, dtype):
        self.problem = dict(problem)
        self.dtype = dtype
        self._plan = capi.conv_bwd_data_create(desc_from_problem(problem, dtype, False, False))
        fwd = ConvFwd(problem, dtype)
        self.dy_shape, self.w_shape, self.dx_shape = fwd.y_shape, fwd.w_shape, fwd.x_shape
        self._flop = fwd.useful_flop()
        fwd.close()
        self.workspace_bytes = capi.conv_bwd_data_workspace_bytes(self._plan)
        self._ws = None

    def useful_flop(self):
        """2 * multiply-adds of the gradient sum: the forward's count."""
        return self._flop

    def describe(self):
        return capi.conv_bwd_data_describe(self._plan)

    def close(self):
        if getattr(self, "_plan", None):
            capi.conv_bwd_data_destroy(self._plan)
            self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __call__(self, dy, w, out=None, stream=None, workspace=None):
        import torch
        tdt = torch.float32 if self.dtype == "f32" else torch.bfloat16
        for t, shape, name in ((dy, self.dy_shape, "dy"), (w, self.w_shape, "w")):
            if t.device.type != "cuda" or t.dtype != tdt or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError("%s must be a contiguous cuda %s tensor of shape %r" % (name, tdt, shape))
        if out is None:
            out = torch.empty(self.dx_shape, dtype=tdt, device=dy.device)
        if workspace is None:
            if self._ws is None or self._ws.device != dy.device:
                self._ws = torch.empty(max(self.workspace_bytes, 16), dtype=torch.uint8, device=dy.device)
            workspace = self._ws
        s = stream if stream is not None else torch.cuda.current_stream(dy.device)
        capi.conv_bwd_data_run(self._plan, dy.data_ptr(), w.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                               workspace.numel(), s.cuda_stream)
        return out


class ConvBwdWeight:
    """Weight gradient of a forward convolution problem (conv_bwd_weight_*):
    dw = the gradient of <conv(x, w), dy> with respect to w, bf16.  The
    workspace it needs is allocated once here (torch, caller-side)."""

    def __init__(self, problem, dtype="bf16"):
        self.problem = dict(problem)
        self.dtype = dtype
        self._plan = capi.conv_bwd_weight_create(desc_from_problem(problem, dtype, False, False))
        fwd = ConvFwd(problem, dtype)
        self.x_shape, self.dy_shape, self.dw_shape = fwd.x_shape, fwd.y_shape, fwd.w_shape
        self._flop = fwd.useful_flop()
        fwd.close()
        self.workspace_bytes = capi.conv_bwd_weight_workspace_bytes(self._plan)
        self._ws = None

    def useful_flop(self):
        """2 * multiply-adds of the gradient sum: the forward's count."""
        return self._flop

    def describe(self):
        return capi.conv_bwd_weight_describe(self._plan)

    def close(self):
        if getattr(self, "_plan", None):
            capi.conv_bwd_weight_destroy(self._plan)
            self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __call__(self, x, dy, out=None, stream=None, workspace=None):
        import torch
        for t, shape, name in ((x, self.x_shape, "x"), (dy, self.dy_shape, "dy")):
            if t.device.type != "cuda" or t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError("%s must be a contiguous cuda bfloat16 tensor of shape %r" % (name, shape))
        if out is None:
            out = torch.empty(self.dw_shape, dtype=torch.bfloat16, device=x.device)
        if workspace is None:
            if self._ws is None or self._ws.device != x.device:
                self._ws = torch.empty(max(self.workspace_bytes, 16), dtype=torch.uint8, device=x.device)
            workspace = self._ws
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        capi.conv_bwd_weight_run(self._plan, x.data_ptr(), dy.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                 workspace.numel(), s.cuda_stream)
        return out
