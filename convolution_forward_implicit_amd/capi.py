"""ctypes binding of the C ABI in include/convfwd.h -- argument marshalling
only; every step of the computation runs in the HIP library.

The functions keep the C names.  Pointers are plain integers (device
addresses) and the stream is a hipStream_t handle as an integer (0 = null
stream).  Errors come back as ConvError carrying the status and the
library's message.  Loading fails loudly if libconvfwd.so has not been built.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libconvfwd.so")

CONV_DT_F32 = 0
CONV_DT_BF16 = 1
DTYPES = {"f32": CONV_DT_F32, "bf16": CONV_DT_BF16}

CONV_OK = 0
CONV_ERR_INVALID_ARG = 1
CONV_ERR_UNSUPPORTED = 2
CONV_ERR_HIP = 3
CONV_ERR_NOMEM = 4
STATUS_NAMES = {0: "CONV_OK", 1: "CONV_ERR_INVALID_ARG", 2: "CONV_ERR_UNSUPPORTED",
                3: "CONV_ERR_HIP", 4: "CONV_ERR_NOMEM"}

EXPORTED = ["conv_fwd_create", "conv_fwd_create_with_config", "conv_fwd_out_dims", "conv_fwd_useful_flop",
            "conv_fwd_packed_config", "conv_fwd_packed_bytes", "conv_fwd_pack_weights", "conv_fwd_run_packed", "conv_fwd_run_packed_events",
            "conv_fwd_run", "conv_fwd_run_events", "conv_fwd_destroy", "conv_fwd_describe", "conv_fwd_num_configs",
            "conv_fwd_config_name", "conv_fwd_config_dtype", "conv_fwd_last_error",
            "conv_chain_create", "conv_chain_run", "conv_chain_run_events", "conv_chain_destroy",
            "conv_chain_describe", "conv_chain_out_dims", "conv_chain_useful_flop", "conv_chain_packed_bytes", "conv_chain_pack_weights", "conv_chain_run_packed",
            "conv_chain_run_packed_events", "conv_bwd_data_create", "conv_bwd_data_workspace_bytes",
            "conv_bwd_data_run", "conv_bwd_data_run_noalloc", "conv_bwd_data_destroy", "conv_bwd_data_describe", "conv_bwd_weight_create",
            "conv_bwd_weight_workspace_bytes", "conv_bwd_weight_run", "conv_bwd_weight_destroy",
            "conv_bwd_weight_describe"]


class conv_fwd_desc_t(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("N", ctypes.c_int64), ("G", ctypes.c_int64),
                ("C", ctypes.c_int64), ("K", ctypes.c_int64),
                ("in_", ctypes.c_int64 * 3), ("filt", ctypes.c_int64 * 3),
                ("stride", ctypes.c_int64 * 3), ("pad", ctypes.c_int64 * 3),
                ("dilation", ctypes.c_int64 * 3),
                ("has_bias", ctypes.c_int32), ("gelu", ctypes.c_int32)]


class ConvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status
        self.message = message


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("convfwd HIP library not built: %s is missing "
                              "(run python -m convolution_forward_implicit_amd.build)" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        D = ctypes.POINTER(conv_fwd_desc_t)
        L.conv_fwd_create.argtypes = [D, ctypes.POINTER(P)]
        L.conv_fwd_create.restype = ctypes.c_int
        L.conv_fwd_create_with_config.argtypes = [D, ctypes.c_int32, ctypes.POINTER(P)]
        L.conv_fwd_create_with_config.restype = ctypes.c_int
        L.conv_fwd_out_dims.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.conv_fwd_out_dims.restype = ctypes.c_int
        L.conv_fwd_useful_flop.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.conv_fwd_useful_flop.restype = ctypes.c_int
        L.conv_fwd_packed_config.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
        L.conv_fwd_packed_config.restype = ctypes.c_int
        L.conv_fwd_packed_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.conv_fwd_packed_bytes.restype = ctypes.c_int
        L.conv_fwd_pack_weights.argtypes = [P, P, P, P]
        L.conv_fwd_pack_weights.restype = ctypes.c_int
        L.conv_fwd_run_packed.argtypes = [P, P, P, P, P, P]
        L.conv_fwd_run_packed.restype = ctypes.c_int
        L.conv_fwd_run_packed_events.argtypes = [P, P, P, P, P, P, P, P]
        L.conv_fwd_run_packed_events.restype = ctypes.c_int
        L.conv_chain_out_dims.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.conv_chain_out_dims.restype = ctypes.c_int
        L.conv_chain_useful_flop.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.conv_chain_useful_flop.restype = ctypes.c_int
        L.conv_fwd_run.argtypes = [P, P, P, P, P, P]
        L.conv_fwd_run.restype = ctypes.c_int
        L.conv_fwd_run_events.argtypes = [P, P, P, P, P, P, P, P]
        L.conv_fwd_run_events.restype = ctypes.c_int
        L.conv_fwd_destroy.argtypes = [P]
        L.conv_fwd_destroy.restype = None
        L.conv_fwd_describe.argtypes = [P]
        L.conv_fwd_describe.restype = ctypes.c_char_p
        L.conv_fwd_num_configs.argtypes = []
        L.conv_fwd_num_configs.restype = ctypes.c_int32
        L.conv_fwd_config_name.argtypes = [ctypes.c_int32]
        L.conv_fwd_config_name.restype = ctypes.c_char_p
        L.conv_fwd_config_dtype.argtypes = [ctypes.c_int32]
        L.conv_fwd_config_dtype.restype = ctypes.c_int32
        L.conv_fwd_last_error.argtypes = []
        L.conv_fwd_last_error.restype = ctypes.c_char_p
        L.conv_chain_create.argtypes = [D, D, ctypes.POINTER(P)]
        L.conv_chain_create.restype = ctypes.c_int
        L.conv_chain_run.argtypes = [P] * 8
        L.conv_chain_run.restype = ctypes.c_int
        L.conv_chain_run_events.argtypes = [P] * 10
        L.conv_chain_run_events.restype = ctypes.c_int
        L.conv_chain_destroy.argtypes = [P]
        L.conv_chain_destroy.restype = None
        L.conv_chain_describe.argtypes = [P]
        L.conv_chain_describe.restype = ctypes.c_char_p
        L.conv_chain_packed_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.conv_chain_packed_bytes.restype = ctypes.c_int
        L.conv_chain_pack_weights.argtypes = [P] * 5
        L.conv_chain_pack_weights.restype = ctypes.c_int
        L.conv_chain_run_packed.argtypes = [P] * 7
        L.conv_chain_run_packed.restype = ctypes.c_int
        L.conv_chain_run_packed_events.argtypes = [P] * 9
        L.conv_chain_run_packed_events.restype = ctypes.c_int
        L.conv_bwd_data_create.argtypes = [D, ctypes.POINTER(P)]
        L.conv_bwd_data_create.restype = ctypes.c_int
        L.conv_bwd_data_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.conv_bwd_data_workspace_bytes.restype = ctypes.c_int
        L.conv_bwd_data_run.argtypes = [P, P, P, P, P, ctypes.c_int64, P]
        L.conv_bwd_data_run.restype = ctypes.c_int
        L.conv_bwd_data_run_noalloc.argtypes = [P, P, P, P, P]
        L.conv_bwd_data_run_noalloc.restype = ctypes.c_int
        L.conv_bwd_data_destroy.argtypes = [P]
        L.conv_bwd_data_destroy.restype = None
        L.conv_bwd_data_describe.argtypes = [P]
        L.conv_bwd_data_describe.restype = ctypes.c_char_p
        L.conv_bwd_weight_create.argtypes = [D, ctypes.POINTER(P)]
        L.conv_bwd_weight_create.restype = ctypes.c_int
        L.conv_bwd_weight_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.conv_bwd_weight_workspace_bytes.restype = ctypes.c_int
        L.conv_bwd_weight_run.argtypes = [P, P, P, P, P, ctypes.c_int64, P]
        L.conv_bwd_weight_run.restype = ctypes.c_int
        L.conv_bwd_weight_destroy.argtypes = [P]
        L.conv_bwd_weight_destroy.restype = None
        L.conv_bwd_weight_describe.argtypes = [P]
        L.conv_bwd_weight_describe.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(st):
    if st != CONV_OK:
        raise ConvError(st, lib().conv_fwd_last_error().decode())


def make_desc(ndim, dtype, N, G, C, K, inp, filt, stride=(1, 1, 1), pad=(0, 0, 0),
              dilation=(1, 1, 1), has_bias=False, gelu=False):
    """A conv_fwd_desc_t; spatial tuples are (D, H, W) order, length 3."""
    d = conv_fwd_desc_t()
    d.ndim = int(ndim)
    d.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    d.N, d.G, d.C, d.K = int(N), int(G), int(C), int(K)
    for i in range(3):
        d.in_[i], d.filt[i] = int(inp[i]), int(filt[i])
        d.stride[i], d.pad[i], d.dilation[i] = int(stride[i]), int(pad[i]), int(dilation[i])
    d.has_bias, d.gelu = int(bool(has_bias)), int(bool(gelu))
    return d


def conv_fwd_create(desc):
    plan = ctypes.c_void_p()
    _check(lib().conv_fwd_create(ctypes.byref(desc), ctypes.byref(plan)))
    return plan.value


def conv_fwd_create_with_config(desc, config):
    plan = ctypes.c_void_p()
    _check(lib().conv_fwd_create_with_config(ctypes.byref(desc), int(config), ctypes.byref(plan)))
    return plan.value


def conv_fwd_out_dims(plan):
    out = (ctypes.c_int64 * 3)()
    _check(lib().conv_fwd_out_dims(plan, out))
    return tuple(int(v) for v in out)


def conv_fwd_useful_flop(plan):
    n = ctypes.c_int64()
    _check(lib().conv_fwd_useful_flop(plan, ctypes.byref(n)))
    return n.value


def conv_fwd_packed_config(plan):
    n = ctypes.c_int32()
    _check(lib().conv_fwd_packed_config(plan, ctypes.byref(n)))
    return n.value


def conv_fwd_packed_bytes(plan):
    n = ctypes.c_int64()
    _check(lib().conv_fwd_packed_bytes(plan, ctypes.byref(n)))
    return n.value


def conv_fwd_pack_weights(plan, w, packed, stream=0):
    _check(lib().conv_fwd_pack_weights(plan, w, packed, stream))


def conv_fwd_run_packed(plan, x, packed, bias, y, stream=0):
    _check(lib().conv_fwd_run_packed(plan, x, packed, bias, y, stream))


def conv_fwd_run_packed_events(plan, x, packed, bias, y, stream, start_event, stop_event):
    _check(lib().conv_fwd_run_packed_events(plan, x, packed, bias, y, stream, start_event, stop_event))


def conv_chain_out_dims(plan):
    out = (ctypes.c_int64 * 3)()
    _check(lib().conv_chain_out_dims(plan, out))
    return tuple(int(v) for v in out)


def conv_chain_useful_flop(plan):
    n = ctypes.c_int64()
    _check(lib().conv_chain_useful_flop(plan, ctypes.byref(n)))
    return n.value


def conv_fwd_run(plan, x, w, bias, y, stream=0):
    _check(lib().conv_fwd_run(plan, x, w, bias, y, stream))


def conv_fwd_run_events(plan, x, w, bias, y, stream=0, start_event=None, stop_event=None):
    _check(lib().conv_fwd_run_events(plan, x, w, bias, y, stream, start_event, stop_event))


def conv_fwd_destroy(plan):
    lib().conv_fwd_destroy(plan)


def conv_fwd_describe(plan):
    return lib().conv_fwd_describe(plan).decode()


def conv_fwd_num_configs():
    return int(lib().conv_fwd_num_configs())


def conv_fwd_config_name(config):
    r = lib().conv_fwd_config_name(int(config))
    return None if r is None else r.decode()


def conv_fwd_config_dtype(config):
    return int(lib().conv_fwd_config_dtype(int(config)))


def conv_chain_create(first, second):
    plan = ctypes.c_void_p()
    _check(lib().conv_chain_create(ctypes.byref(first), ctypes.byref(second), ctypes.byref(plan)))
    return plan.value


def conv_chain_run(plan, x, w1, b1, w2, b2, y, stream=0):
    _check(lib().conv_chain_run(plan, x, w1, b1, w2, b2, y, stream))


def conv_chain_run_events(plan, x, w1, b1, w2, b2, y, stream=0, start_event=None, stop_event=None):
    _check(lib().conv_chain_run_events(plan, x, w1, b1, w2, b2, y, stream, start_event, stop_event))


def conv_chain_destroy(plan):
    lib().conv_chain_destroy(plan)


def conv_chain_describe(plan):
    return lib().conv_chain_describe(plan).decode()


def conv_chain_packed_bytes(plan):
    n = ctypes.c_int64()
    _check(lib().conv_chain_packed_bytes(plan, ctypes.byref(n)))
    return n.value


def conv_chain_pack_weights(plan, w1, w2, packed, stream=0):
    _check(lib().conv_chain_pack_weights(plan, w1, w2, packed, stream))


def conv_chain_run_packed(plan, x, packed, b1, b2, y, stream=0):
    _check(lib().conv_chain_run_packed(plan, x, packed, b1, b2, y, stream))


def conv_chain_run_packed_events(plan, x, packed, b1, b2, y, stream=0, start_event=None, stop_event=None):
    _check(lib().conv_chain_run_packed_events(plan, x, packed, b1, b2, y, stream, start_event, stop_event))


def conv_bwd_data_create(desc):
    plan = ctypes.c_void_p()
    _check(lib().conv_bwd_data_create(ctypes.byref(desc), ctypes.byref(plan)))
    return plan.value


def conv_bwd_data_workspace_bytes(plan):
    n = ctypes.c_int64()
    _check(lib().conv_bwd_data_workspace_bytes(plan, ctypes.byref(n)))
    return n.value


def conv_bwd_data_run(plan, dy, w, dx, workspace, workspace_bytes, stream=0):
    _check(lib().conv_bwd_data_run(plan, dy, w, dx, workspace, int(workspace_bytes), stream))


CONV_BWD_DATA_SCRATCH_BYTES = 64 << 20


def conv_bwd_data_run_noalloc(plan, dy, w, dx, stream=0):
    _check(lib().conv_bwd_data_run_noalloc(plan, dy, w, dx, stream))


def conv_bwd_data_destroy(plan):
    lib().conv_bwd_data_destroy(plan)


def conv_bwd_data_describe(plan):
    return lib().conv_bwd_data_describe(plan).decode()


def conv_bwd_weight_create(desc):
    plan = ctypes.c_void_p()
    _check(lib().conv_bwd_weight_create(ctypes.byref(desc), ctypes.byref(plan)))
    return plan.value


def conv_bwd_weight_workspace_bytes(plan):
    n = ctypes.c_int64()
    _check(lib().conv_bwd_weight_workspace_bytes(plan, ctypes.byref(n)))
    return n.value


def conv_bwd_weight_run(plan, x, dy, dw, workspace, workspace_bytes, stream=0):
    _check(lib().conv_bwd_weight_run(plan, x, dy, dw, workspace, int(workspace_bytes), stream))


def conv_bwd_weight_destroy(plan):
    lib().conv_bwd_weight_destroy(plan)


def conv_bwd_weight_describe(plan):
    return lib().conv_bwd_weight_describe(plan).decode()


def conv_fwd_last_error():
    return lib().conv_fwd_last_error().decode()


# ---- peak-rate probes (include/convprobe.h), used by the benchmark ---------
PROBE_LIB_PATH = os.path.join(_HERE, "libconvprobe.so")
PROBE_EXPORTED = ["conv_probe_threads", "conv_probe_mfma", "conv_probe_hbm_read"]
_probe = None


def probe_lib():
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError("peak-probe library not built: %s is missing "
                              "(run python -m convolution_forward_implicit_amd.build)" % PROBE_LIB_PATH)
        L = ctypes.CDLL(PROBE_LIB_PATH)
        P = ctypes.c_void_p
        L.conv_probe_threads.argtypes = []
        L.conv_probe_threads.restype = ctypes.c_int32
        L.conv_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P,
                                      ctypes.POINTER(ctypes.c_double)]
        L.conv_probe_mfma.restype = ctypes.c_int32
        L.conv_probe_hbm_read.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P]
        L.conv_probe_hbm_read.restype = ctypes.c_int32
        _probe = L
    return _probe


def conv_probe_threads():
    return int(probe_lib().conv_probe_threads())


def conv_probe_mfma(kind, iters, grid, sink, stream=0):
    """Enqueues the MFMA probe; returns the useful FLOP of the launch."""
    f = ctypes.c_double()
    rc = probe_lib().conv_probe_mfma(int(kind), int(iters), int(grid), sink, stream, ctypes.byref(f))
    if rc != 0:
        raise RuntimeError("conv_probe_mfma failed: hipError %d" % rc)
    return f.value


def conv_probe_hbm_read(buf, nbytes, grid, sink, stream=0):
    rc = probe_lib().conv_probe_hbm_read(buf, int(nbytes), int(grid), sink, stream)
    if rc != 0:
        raise RuntimeError("conv_probe_hbm_read failed: hipError %d" % rc)
