"""Host-side tests of the C ABI: the library loads, exports every function
include/convfwd.h declares, validates descriptors, and rejects bad run()
arguments before launching anything.  No GPU needed."""
import ctypes
import os
import re

import numpy as np
import pytest

from convolution_forward_implicit_amd import capi, desc_from_problem, ConvFwd, ConvError
import synthdata as sd
from oracle import ref

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "convfwd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(conv_(?:fwd|chain|bwd_data|bwd_weight)_\w+)\s*\(", text)))


def test_header_declares_what_binding_expects():
    assert declared_functions() == sorted(capi.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = capi.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_probe_library_exports_what_its_header_declares():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER.replace("convfwd.h", "convprobe.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(conv_probe_\w+)\s*\(", text)))
    assert declared == sorted(capi.PROBE_EXPORTED)
    lib = capi.probe_lib()
    for name in declared:
        assert hasattr(lib, name), name
    assert capi.conv_probe_threads() == 256
    # bad arguments are refused before any launch (hipErrorInvalidValue)
    with pytest.raises(RuntimeError):
        capi.conv_probe_mfma(4, 1, 1, 16)
    with pytest.raises(RuntimeError):
        capi.conv_probe_mfma(0, 1, 1, None)
    with pytest.raises(RuntimeError):
        capi.conv_probe_hbm_read(16, 24, 1, 16)


def test_desc_struct_layout_matches_header():
    # int32 ndim, int32 dtype, 4 int64, 5 x int64[3], int32 has_bias, int32 gelu
    assert ctypes.sizeof(capi.conv_fwd_desc_t) == 8 + 4 * 8 + 15 * 8 + 8
    assert capi.conv_fwd_desc_t.N.offset == 8
    assert capi.conv_fwd_desc_t.has_bias.offset == 8 + 4 * 8 + 15 * 8


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_out_dims_match_oracle_at_every_workload(wid):
    for p, hb, ge in sd.layers(wid):
        plan = capi.conv_fwd_create(desc_from_problem(p, sd.dtype_of(wid), hb, ge))
        try:
            assert capi.conv_fwd_out_dims(plan) == ref.out_dims(p)
            assert capi.conv_fwd_describe(plan).split()[0] in ("igemm", "patch")
        finally:
            capi.conv_fwd_destroy(plan)


def test_out_dims_grid_against_oracle():
    import itertools
    for I, F, s, p, d in itertools.product((1, 2, 5, 9), (1, 2, 3), (1, 2, 3), (0, 1, 3), (1, 2)):
        prob = sd.conv1d_problem(1, 1, 1, I, F, s, p, d)
        try:
            want = ref.out_dims(prob)
        except ValueError:
            with pytest.raises(ConvError) as e:
                capi.conv_fwd_create(desc_from_problem(prob, "f32"))
            assert e.value.status == capi.CONV_ERR_INVALID_ARG
            continue
        plan = capi.conv_fwd_create(desc_from_problem(prob, "f32"))
        assert capi.conv_fwd_out_dims(plan) == want
        capi.conv_fwd_destroy(plan)


def _base(**kw):
    args = dict(ndim=2, dtype="bf16", N=2, G=1, C=8, K=8, inp=(1, 5, 5), filt=(1, 3, 3),
                stride=(1, 1, 1), pad=(0, 1, 1), dilation=(1, 1, 1))
    args.update(kw)
    return args


@pytest.mark.parametrize("kw,status", [
    (dict(ndim=0), capi.CONV_ERR_INVALID_ARG),
    (dict(ndim=4), capi.CONV_ERR_INVALID_ARG),
    (dict(dtype=7), capi.CONV_ERR_INVALID_ARG),
    (dict(N=-1), capi.CONV_ERR_INVALID_ARG),
    (dict(G=0), capi.CONV_ERR_INVALID_ARG),
    (dict(C=0), capi.CONV_ERR_INVALID_ARG),
    (dict(K=0), capi.CONV_ERR_INVALID_ARG),
    (dict(inp=(1, 0, 5)), capi.CONV_ERR_INVALID_ARG),
    (dict(filt=(1, 3, 0)), capi.CONV_ERR_INVALID_ARG),
    (dict(stride=(1, 0, 1)), capi.CONV_ERR_INVALID_ARG),
    (dict(dilation=(1, 1, 0)), capi.CONV_ERR_INVALID_ARG),
    (dict(pad=(0, -1, 0)), capi.CONV_ERR_INVALID_ARG),
    (dict(inp=(2, 5, 5)), capi.CONV_ERR_INVALID_ARG),          # unused D dim not trivial
    (dict(pad=(1, 1, 1)), capi.CONV_ERR_INVALID_ARG),
    (dict(filt=(1, 9, 3)), capi.CONV_ERR_INVALID_ARG),         # empty output
    (dict(N=1 << 20, inp=(1, 1024, 1024), C=64), capi.CONV_ERR_UNSUPPORTED),
    (dict(C=1 << 16, K=1 << 16, filt=(1, 3, 3)), capi.CONV_ERR_UNSUPPORTED),
])
def test_create_rejects_invalid(kw, status):
    a = _base(**kw)
    d = capi.make_desc(a["ndim"], a["dtype"] if isinstance(a["dtype"], str) else a["dtype"],
                       a["N"], a["G"], a["C"], a["K"], a["inp"], a["filt"], a["stride"],
                       a["pad"], a["dilation"])
    with pytest.raises(ConvError) as e:
        capi.conv_fwd_create(d)
    assert e.value.status == status
    assert capi.conv_fwd_last_error()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_largest_inputs_32bit_offset_bound(dtype):
    """The plan accepts an input whose zero-padded element count is just
    below 2^31 (a 1-D conv with 1.07e9 input elements: 2 GiB in bf16, so
    the 32-bit-byte-offset kernels are not eligible and the description
    names a register-staged configuration) and rejects one just above."""
    p = sd.conv1d_problem(16, 64, 16, 1048600, 3, 1, 1)
    plan = capi.conv_fwd_create(desc_from_problem(p, dtype, True, False))
    try:
        text = capi.conv_fwd_describe(plan)
        assert "_dma_" not in text and "_patch_" not in text
    finally:
        capi.conv_fwd_destroy(plan)
    big = sd.conv1d_problem(32, 64, 16, 1048576, 3, 1, 1)   # 32 x 1048578 x 64 > 2^31 - 1
    with pytest.raises(ConvError) as e:
        capi.conv_fwd_create(desc_from_problem(big, dtype))
    assert e.value.status == capi.CONV_ERR_UNSUPPORTED


def test_flags_must_be_boolean():
    d = desc_from_problem(sd.conv1d_problem(1, 4, 4, 8, 3, 1, 1), "f32")
    d.has_bias = 2
    with pytest.raises(ConvError):
        capi.conv_fwd_create(d)
    d.has_bias, d.gelu = 0, 5
    with pytest.raises(ConvError):
        capi.conv_fwd_create(d)


def test_null_arguments():
    lib = capi.lib()
    assert lib.conv_fwd_create(None, None) == capi.CONV_ERR_INVALID_ARG
    d = desc_from_problem(sd.conv1d_problem(1, 4, 4, 8, 3, 1, 1), "f32")
    assert lib.conv_fwd_create(ctypes.byref(d), None) == capi.CONV_ERR_INVALID_ARG
    assert lib.conv_fwd_out_dims(None, None) == capi.CONV_ERR_INVALID_ARG
    assert lib.conv_fwd_run(None, None, None, None, None, None) == capi.CONV_ERR_INVALID_ARG
    lib.conv_fwd_destroy(None)                       # no-op
    assert lib.conv_fwd_describe(None) == b""


def test_config_table():
    n = capi.conv_fwd_num_configs()
    assert n >= 2
    names = [capi.conv_fwd_config_name(i) for i in range(n)]
    assert len(set(names)) == n
    assert {capi.conv_fwd_config_dtype(i) for i in range(n)} == {0, 1}
    assert capi.conv_fwd_config_name(n) is None and capi.conv_fwd_config_dtype(-1) == -1


def test_forced_config_dtype_and_vector_rules():
    n = capi.conv_fwd_num_configs()
    d_bf16 = desc_from_problem(sd.problem(1, 1, 32, 16, (1, 6, 6), (1, 3, 3), pad=(0, 1, 1)), "bf16")
    d_odd = desc_from_problem(sd.problem(1, 1, 5, 16, (1, 6, 6), (1, 3, 3)), "bf16")
    for i in range(n):
        name = capi.conv_fwd_config_name(i)
        if capi.conv_fwd_config_dtype(i) != capi.CONV_DT_BF16:
            with pytest.raises(ConvError) as e:
                capi.conv_fwd_create_with_config(d_bf16, i)
            assert e.value.status == capi.CONV_ERR_UNSUPPORTED
            continue
        m = re.search(r"_pfix_.*_f(\d+)x(\d+)_d(\d+)x(\d+)", name)
        d_ok, d_bad = d_bf16, d_odd
        if m:   # fixed-filter patch kernels: exactly their own H/W filter and dilation
            FY, FX, DH, DW = (int(v) for v in m.groups())
            fit = sd.problem(1, 1, 32, 16, (1, 6 + DH * (FY - 1), 6 + DW * (FX - 1)), (1, FY, FX), pad=(0, 1, 1),
                             dil=(1, DH, DW))
            d_ok = desc_from_problem(fit, "bf16")
            d_bad = desc_from_problem(dict(fit, C=5), "bf16")
            other = desc_from_problem(dict(fit, dil=(1, DH + 1, DW)), "bf16")
            with pytest.raises(ConvError) as e:
                capi.conv_fwd_create_with_config(other, i)
            assert e.value.status == capi.CONV_ERR_UNSUPPORTED
        plan = capi.conv_fwd_create_with_config(d_ok, i)
        assert name in capi.conv_fwd_describe(plan)
        capi.conv_fwd_destroy(plan)
        if not name.endswith("_v1"):   # 16-byte channel vectors / slices need C % 8 (16, 32) == 0
            with pytest.raises(ConvError):
                capi.conv_fwd_create_with_config(d_bad, i)
    with pytest.raises(ConvError):
        capi.conv_fwd_create_with_config(d_bf16, n)
    with pytest.raises(ConvError):
        capi.conv_fwd_create_with_config(d_bf16, -1)


def test_selector_uses_scalar_loads_only_for_odd_channels():
    for C, dt, vec_ok in ((80, "f32", True), (6, "f32", False), (64, "bf16", True), (12, "bf16", False)):
        c = ConvFwd(sd.conv1d_problem(1, C, 8, 50, 3, 1, 1), dt)
        assert c.describe().split()[1].endswith("_v1") != vec_ok, c.describe()


def test_run_argument_checks_before_launch():
    """Every failure below is detected on the host; nothing is launched."""
    lib = capi.lib()
    p = sd.conv1d_problem(1, 8, 8, 16, 3, 1, 1)
    plan_b = capi.conv_fwd_create(desc_from_problem(p, "f32", has_bias=True))
    plan = capi.conv_fwd_create(desc_from_problem(p, "f32"))
    A = 1 << 20   # fake, well-separated, aligned addresses: never dereferenced
    try:
        assert lib.conv_fwd_run(plan_b, A, 2 * A, None, 3 * A, None) == capi.CONV_ERR_INVALID_ARG
        assert lib.conv_fwd_run(plan, A, 2 * A, 4 * A, 3 * A, None) == capi.CONV_ERR_INVALID_ARG
        assert lib.conv_fwd_run(plan, None, 2 * A, None, 3 * A, None) == capi.CONV_ERR_INVALID_ARG
        assert lib.conv_fwd_run(plan, A, None, None, 3 * A, None) == capi.CONV_ERR_INVALID_ARG
        assert lib.conv_fwd_run(plan, A, 2 * A, None, None, None) == capi.CONV_ERR_INVALID_ARG
        assert lib.conv_fwd_run(plan, A + 4, 2 * A, None, 3 * A, None) == capi.CONV_ERR_INVALID_ARG
        assert "aligned" in capi.conv_fwd_last_error()
        assert lib.conv_fwd_run(plan, A, 2 * A, None, A + 64, None) == capi.CONV_ERR_INVALID_ARG
        assert "overlap" in capi.conv_fwd_last_error()
        assert lib.conv_fwd_run(plan_b, A, 2 * A, 3 * A + 2, 4 * A, None) == capi.CONV_ERR_INVALID_ARG
    finally:
        capi.conv_fwd_destroy(plan)
        capi.conv_fwd_destroy(plan_b)


def test_empty_batch_is_a_valid_noop():
    p = sd.conv1d_problem(0, 8, 8, 16, 3, 1, 1)
    plan = capi.conv_fwd_create(desc_from_problem(p, "bf16"))
    try:
        assert capi.conv_fwd_out_dims(plan) == (1, 1, 16)
        # nothing to compute: returns before touching the device
        assert capi.lib().conv_fwd_run(plan, None, 1 << 20, None, None, None) == capi.CONV_OK
    finally:
        capi.conv_fwd_destroy(plan)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(capi, "_lib", None)
    monkeypatch.setattr(capi, "LIB_PATH", str(tmp_path / "libconvfwd.so"))
    with pytest.raises(ImportError):
        capi.lib()


def test_selector_coefficients_match_compiled_configs():
    """Every fitted cost-model entry names a configuration the library
    compiles (a stale coefficient table would silently fall back)."""
    import os
    inc = os.path.join(os.path.dirname(capi.LIB_PATH), "csrc", "selector_coef.inc")
    names = {line.split('"')[1] for line in open(inc) if line.strip().startswith('{"')}
    compiled = {capi.conv_fwd_config_name(i) for i in range(capi.conv_fwd_num_configs())}
    assert names and names <= compiled, names - compiled
    dma = {n for n in compiled if "_dma_" in n or "_patch_" in n or "_pfix_" in n}
    assert dma <= names, dma - names


def test_selector_fit_reproduces_committed_table(tmp_path):
    """tuning/fit.py applied to the committed sweep table regenerates the
    committed coefficients, and its held-out selector quality is recorded."""
    import os
    from convolution_forward_implicit_amd.tuning import fit
    here = os.path.dirname(capi.LIB_PATH)
    probs = fit.load(os.path.join(here, "tuning", "sweep_mi355x.csv"))
    out = tmp_path / "coef.inc"
    fit.write(fit.fit(probs), str(out))
    assert out.read_text() == open(os.path.join(here, "csrc", "selector_coef.inc")).read()
    q = fit.quality(probs)
    assert q["mean_eff"] > 0.9 and q["top5"] > 0.8, q


def test_tuning_records_match_sweep_and_configs(tmp_path):
    """The exact-shape tuning records are the sweep's fastest configuration
    per (problem, epilogue), regenerate from the committed sweep, and name
    compiled configurations of their own dtype."""
    import os
    from convolution_forward_implicit_amd.tuning import fit
    here = os.path.dirname(capi.LIB_PATH)
    probs = fit.load(os.path.join(here, "tuning", "sweep_mi355x.csv"))
    out = tmp_path / "db.inc"
    fit.write_db(probs, str(out))
    committed = open(os.path.join(here, "csrc", "selector_db.inc")).read()
    assert out.read_text() == committed
    dtype_of = {capi.conv_fwd_config_name(i): capi.conv_fwd_config_dtype(i)
                for i in range(capi.conv_fwd_num_configs())}
    rows = [l for l in committed.splitlines() if l.strip().startswith("{")]
    assert len(rows) == len(probs)
    for l in rows:
        name, packed = l.split('"')[1], l.split('"')[3]
        assert name in dtype_of, name
        assert dtype_of[name] == int(l.strip()[1]), l
        # the prepacked-weight configuration: none, or a compiled one of the
        # same dtype that has a prepacked form
        assert packed == "" or (dtype_of.get(packed) == int(l.strip()[1]) and fit.packable(packed)), l


def test_plans_take_the_records_prepacked_configuration():
    """A plan for a recorded shape runs the record's configuration from
    natural weights and the record's prepacked-weight configuration from
    prepacked weights (conv_fwd_packed_config); a forced plan uses its own
    configuration for both."""
    import os
    import re as _re
    from convolution_forward_implicit_amd.tuning import fit
    here = os.path.dirname(capi.LIB_PATH)
    index = {capi.conv_fwd_config_name(i): i for i in range(capi.conv_fwd_num_configs())}
    probs = fit.load(os.path.join(here, "tuning", "sweep_mi355x.csv"))
    seen_split = 0
    for p in probs:
        best, pbest = fit.record(p)
        prob = sd.problem(p["N"], p["G"], p["C"], p["K"], tuple(p["in"]), tuple(p["filt"]), tuple(p["stride"]),
                          tuple(p["pad"]), tuple(p["dil"]))
        plan = capi.conv_fwd_create(desc_from_problem(prob, p["dtype"], bool(p["gelu"]), bool(p["gelu"])))
        try:
            text = capi.conv_fwd_describe(plan)
            assert (" %s " % best) in text and "tuned" in text, text
            if pbest:
                assert capi.conv_fwd_packed_config(plan) == index[pbest]
                if pbest != best:
                    seen_split += 1
                    assert ("prepacked: %s " % pbest) in text, text
            else:
                assert capi.conv_fwd_packed_config(plan) == index[best]
        finally:
            capi.conv_fwd_destroy(plan)
    if any(p["ptimes"] for p in probs):
        assert seen_split > 0   # prepacked timings change some records
    i = _cfg_index(r"^bf16_dma_128x64_w2x2_s2_m32_k1$")
    plan = capi.conv_fwd_create_with_config(desc_from_problem(sd.conv1d_problem(2, 64, 64, 100, 3, 1, 1), "bf16"), i)
    try:
        assert capi.conv_fwd_packed_config(plan) == i
        assert "prepacked:" not in capi.conv_fwd_describe(plan)
    finally:
        capi.conv_fwd_destroy(plan)
    with pytest.raises(ConvError):
        capi.conv_fwd_packed_config(None)


# --------------------------------------------------------------------------
# Fused two-conv chain: plan-time validation (no GPU work)
def _chain_descs(N=2, C1=80, L=300, K1=384, K2=384, k1=3, s1=1, k2=3, s2=2, dtype="bf16", hb=True, ge=True,
                 hb2=None, ge2=None, L2=None):
    p1 = sd.conv1d_problem(N, C1, K1, L, k1, s1, k1 // 2)
    o1 = ref.out_dims(p1)[2]
    p2 = sd.conv1d_problem(N, K1, K2, o1 if L2 is None else L2, k2, s2, k2 // 2)
    return (desc_from_problem(p1, dtype, hb, ge),
            desc_from_problem(p2, dtype, hb if hb2 is None else hb2, ge if ge2 is None else ge2))


def test_chain_create_accepts_the_frontend_and_describes_it():
    a, b = _chain_descs()
    plan = capi.conv_chain_create(a, b)
    try:
        text = capi.conv_chain_describe(plan)
        assert "chain bf16" in text and "C1=80" in text and "Lo=150" in text and "gelu" in text
    finally:
        capi.conv_chain_destroy(plan)
    capi.conv_chain_destroy(None)
    assert capi.conv_chain_describe(None) == ""


@pytest.mark.parametrize("N,L,C1", [(1, 3000, 80), (32, 3000, 80), (2, 301, 16), (3, 2, 128), (1, 1, 224)])
def test_chain_out_dims_and_flop_come_from_the_library(N, L, C1):
    """conv_chain_out_dims / conv_chain_useful_flop against the oracle's
    extents of the two convs and the 2 x multiply-add count with padded taps
    (per conv: 2 * N * K * C * taps * Lo); the binding sizes y from them."""
    from convolution_forward_implicit_amd import ConvChain
    p1 = sd.conv1d_problem(N, C1, 384, L, 3, 1, 1)
    p2 = sd.conv1d_problem(N, 384, 384, L, 3, 2, 1)
    a, b = desc_from_problem(p1, "bf16", True, True), desc_from_problem(p2, "bf16", True, True)
    plan = capi.conv_chain_create(a, b)
    try:
        o1, o2 = ref.out_dims(p1), ref.out_dims(p2)
        assert o1 == (1, 1, L)
        assert capi.conv_chain_out_dims(plan) == o2
        want = 2 * N * 384 * C1 * 3 * o1[2] + 2 * N * 384 * 384 * 3 * o2[2]
        assert capi.conv_chain_useful_flop(plan) == want
    finally:
        capi.conv_chain_destroy(plan)
    c = ConvChain(p1, p2, "bf16", True, True)
    assert c.y_shape == (N,) + o2 + (1, 384)
    assert c.useful_flop() == want
    with pytest.raises(ConvError):
        capi.conv_chain_out_dims(None)


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_useful_flop_comes_from_the_library(wid):
    """conv_fwd_useful_flop = 2 * N * G * K * C * prod(output extents) *
    prod(filter) with the oracle's extents; the workloads' totals
    (useful GFLOP 0.553, 1.880, 60.162, 7.399, 11.098)."""
    total = 0
    for p, hb, ge in sd.layers(wid):
        plan = capi.conv_fwd_create(desc_from_problem(p, sd.dtype_of(wid), hb, ge))
        try:
            o = ref.out_dims(p)
            want = 2 * p["N"] * p["G"] * p["K"] * p["C"] * o[0] * o[1] * o[2] * \
                p["filt"][0] * p["filt"][1] * p["filt"][2]
            assert capi.conv_fwd_useful_flop(plan) == want
            total += want
        finally:
            capi.conv_fwd_destroy(plan)
    assert round(total / 1e9, 3) == {1: 0.553, 2: 1.880, 3: 60.162, 4: 7.399, 5: 11.098}[wid]
    with pytest.raises(ConvError):
        capi.conv_fwd_useful_flop(None)


def _cfg_index(pattern):
    import re as _re
    return next(i for i in range(capi.conv_fwd_num_configs()) if _re.search(pattern, capi.conv_fwd_config_name(i)))


def test_packed_bytes_sizes_and_refusals():
    """conv_fwd_packed_bytes: the direct-to-LDS image is one BN x 128-byte
    block per sub-slice and K-step of every (group, channel tile); the
    fixed-filter patch image one W_BYTES image per (group, channel tile,
    depth tap, channel slice); the register-staged kernel has none."""
    p = sd.problem(2, 2, 32, 40, (1, 13, 11), (1, 3, 3), (1, 1, 1), (0, 1, 1))
    d = desc_from_problem(p, "bf16")
    i = _cfg_index(r"^bf16_dma_128x64_w2x2_s2_m32_k1$")
    plan = capi.conv_fwd_create_with_config(d, i)
    try:
        nk = -(-(32 * 9) // 64)
        assert capi.conv_fwd_packed_bytes(plan) == 2 * 1 * nk * 1 * 64 * 128
    finally:
        capi.conv_fwd_destroy(plan)
    i = _cfg_index(r"^bf16_\d+x\d+x\d+_w\dx\d_v8$")
    plan = capi.conv_fwd_create_with_config(d, i)
    try:
        with pytest.raises(ConvError) as e:
            capi.conv_fwd_packed_bytes(plan)
        assert e.value.status == capi.CONV_ERR_UNSUPPORTED
        with pytest.raises(ConvError):
            capi.conv_fwd_pack_weights(plan, 16, 4096, 0)
        with pytest.raises(ConvError):
            capi.conv_fwd_run_packed(plan, 16, 4096, None, 8192, 0)
    finally:
        capi.conv_fwd_destroy(plan)
    with pytest.raises(ConvError):
        capi.conv_fwd_packed_bytes(None)


def test_pack_and_run_packed_refuse_bad_arguments_before_launching():
    p = sd.conv1d_problem(2, 64, 64, 100, 3, 1, 1)
    plan = capi.conv_fwd_create_with_config(desc_from_problem(p, "bf16"), _cfg_index(r"^bf16_dma_128x64_w2x2_s2_m32_k1$"))
    try:
        with pytest.raises(ConvError):
            capi.conv_fwd_pack_weights(plan, None, 4096, 0)          # w NULL
        with pytest.raises(ConvError):
            capi.conv_fwd_pack_weights(plan, 8, 4096, 0)             # misaligned
        with pytest.raises(ConvError):
            capi.conv_fwd_pack_weights(plan, 4096, 4096, 0)          # overlap
        with pytest.raises(ConvError):
            capi.conv_fwd_run_packed(plan, 16, None, None, 4096, 0)  # packed NULL
        with pytest.raises(ConvError):
            capi.conv_fwd_run_packed(plan, 8, 16, None, 4096, 0)     # misaligned x
    finally:
        capi.conv_fwd_destroy(plan)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype="f32"), capi.CONV_ERR_UNSUPPORTED),
    (dict(C1=72), capi.CONV_ERR_UNSUPPORTED),          # not a multiple of 16
    (dict(C1=368), capi.CONV_ERR_UNSUPPORTED),         # above the input-patch limit
    (dict(K1=256), capi.CONV_ERR_UNSUPPORTED),
    (dict(K2=256), capi.CONV_ERR_UNSUPPORTED),
    (dict(k1=5), capi.CONV_ERR_UNSUPPORTED),
    (dict(s2=1), capi.CONV_ERR_UNSUPPORTED),
    (dict(ge2=False), capi.CONV_ERR_UNSUPPORTED),
    (dict(hb2=False), capi.CONV_ERR_UNSUPPORTED),
    (dict(L2=299), capi.CONV_ERR_INVALID_ARG),         # second conv does not read the first's output
])
def test_chain_create_rejects(kw, status):
    a, b = _chain_descs(**kw)
    with pytest.raises(ConvError) as e:
        capi.conv_chain_create(a, b)
    assert e.value.status == status, e.value.message


def test_chain_run_rejects_bad_arguments_before_launching():
    a, b = _chain_descs()
    plan = capi.conv_chain_create(a, b)
    try:
        with pytest.raises(ConvError):
            capi.conv_chain_run(plan, 16, 16, None, 16, None, 4096)     # plan has biases
        with pytest.raises(ConvError):
            capi.conv_chain_run(plan, 16, None, 32, 16, 32, 4096)       # w1 NULL
        with pytest.raises(ConvError):
            capi.conv_chain_run(plan, 8, 16, 32, 16, 32, 4096)          # misaligned x
        with pytest.raises(ConvError):
            capi.conv_chain_run(None, 16, 16, 32, 16, 32, 4096)
    finally:
        capi.conv_chain_destroy(plan)


@pytest.mark.parametrize("C1,steps", [(80, 16 + 72), (16, 8 + 72), (128, 24 + 72), (224, 48 + 72)])
def test_chain_packed_bytes(C1, steps):
    """conv1's 3*C1/16 reduction steps rounded up to whole groups of 8, then
    conv2's 72; 12 fragments of 1 KB per step."""
    a, b = _chain_descs(C1=C1)
    plan = capi.conv_chain_create(a, b)
    try:
        assert capi.conv_chain_packed_bytes(plan) == steps * 12 * 1024
    finally:
        capi.conv_chain_destroy(plan)


def test_chain_packed_rejects_wide_input_and_bad_arguments():
    a, b = _chain_descs(C1=240)          # the unpacked chain takes it, the prepacked kernel does not
    plan = capi.conv_chain_create(a, b)
    try:
        for call in (lambda: capi.conv_chain_packed_bytes(plan),
                     lambda: capi.conv_chain_pack_weights(plan, 16, 16, 4096),
                     lambda: capi.conv_chain_run_packed(plan, 16, 4096, 32, 32, 1 << 20)):
            with pytest.raises(ConvError) as e:
                call()
            assert e.value.status == capi.CONV_ERR_UNSUPPORTED
    finally:
        capi.conv_chain_destroy(plan)
    a, b = _chain_descs()
    plan = capi.conv_chain_create(a, b)
    try:
        nb = capi.conv_chain_packed_bytes(plan)
        for call in (lambda: capi.conv_chain_pack_weights(plan, None, 16, 1 << 30),          # w1 NULL
                     lambda: capi.conv_chain_pack_weights(plan, 16, 16, (1 << 30) + 8),     # misaligned
                     lambda: capi.conv_chain_pack_weights(plan, 16, 1 << 20, (1 << 20) - 64),  # overlaps w2
                     lambda: capi.conv_chain_run_packed(plan, 16, 4096, None, 32, 1 << 30),   # plan has biases
                     lambda: capi.conv_chain_run_packed(plan, 16, None, 32, 32, 1 << 30),     # packed NULL
                     lambda: capi.conv_chain_run_packed(plan, 16, 4104, 32, 32, 1 << 30),     # misaligned
                     lambda: capi.conv_chain_run_packed(plan, 16, 1 << 30, 32, 32, (1 << 30) + nb - 16),  # overlap
                     lambda: capi.conv_chain_run_packed(None, 16, 4096, 32, 32, 1 << 30)):
            with pytest.raises(ConvError) as e:
                call()
            assert e.value.status == capi.CONV_ERR_INVALID_ARG, e.value.message
        with pytest.raises(ConvError):
            capi.conv_chain_packed_bytes(None)
    finally:
        capi.conv_chain_destroy(plan)


# --------------------------------------------------------------------------
# Backward-data: plan-time validation and argument checks (no GPU work)
def test_bwd_data_create_workspace_and_describe():
    # unit stride, pad <= d(F-1): only the flipped weights in the workspace
    p = sd.problem(8, 4, 64, 64, (1, 56, 56), (1, 3, 3), (1, 1, 1), (0, 1, 1), (1, 1, 1))
    plan = capi.conv_bwd_data_create(desc_from_problem(p, "bf16"))
    try:
        assert capi.conv_bwd_data_workspace_bytes(plan) == (4 * 64 * 9 * 64 * 2 + 255) // 256 * 256
        assert "padded dy" in capi.conv_bwd_data_describe(plan)
    finally:
        capi.conv_bwd_data_destroy(plan)
    # 1-D stride 2: the stride phases' filters only (phase 0 one tap, phase 1
    # two, each 256-byte aligned)
    p = sd.conv1d_problem(32, 384, 384, 3000, 3, 2, 1)
    plan = capi.conv_bwd_data_create(desc_from_problem(p, "f32"))
    try:
        assert capi.conv_bwd_data_workspace_bytes(plan) == 384 * 1 * 384 * 4 + 384 * 2 * 384 * 4
        assert "2 stride phases" in capi.conv_bwd_data_describe(plan)
    finally:
        capi.conv_bwd_data_destroy(plan)
    # 2-D stride 2: the spread copy of dy (N x (H + 2) x (W + 2) x K) follows the weights
    p = sd.problem(2, 1, 16, 24, (1, 13, 11), (1, 3, 3), (1, 2, 2), (0, 1, 1))
    plan = capi.conv_bwd_data_create(desc_from_problem(p, "f32"))
    try:
        wt = (24 * 9 * 16 * 4 + 255) // 256 * 256
        assert capi.conv_bwd_data_workspace_bytes(plan) == wt + 2 * 15 * 13 * 24 * 4
        assert "spread dy" in capi.conv_bwd_data_describe(plan)
    finally:
        capi.conv_bwd_data_destroy(plan)
    capi.conv_bwd_data_destroy(None)
    assert capi.conv_bwd_data_describe(None) == ""


def test_bwd_data_rejects_epilogues_and_bad_arguments():
    p = sd.problem(2, 2, 16, 8, (1, 9, 9), (1, 3, 3), (1, 2, 2), (0, 1, 1), (1, 1, 1))
    for hb, ge in ((1, 0), (0, 1)):
        with pytest.raises(ConvError) as e:
            capi.conv_bwd_data_create(desc_from_problem(p, "bf16", hb, ge))
        assert e.value.status == capi.CONV_ERR_UNSUPPORTED
    plan = capi.conv_bwd_data_create(desc_from_problem(p, "bf16"))
    try:
        ws = capi.conv_bwd_data_workspace_bytes(plan)
        base = 1 << 30
        for args in ((None, 4096, base, base + (1 << 24), ws),            # dy NULL
                     (4096, 8192, base, None, ws),                       # workspace NULL
                     (4096, 8192, base, base + (1 << 24), ws - 16),      # workspace too small
                     (4096 + 8, 8192, base, base + (1 << 24), ws),       # misaligned
                     (4096, 8192, base, base + 16, ws)):                 # workspace overlaps dx
            with pytest.raises(ConvError) as e:
                capi.conv_bwd_data_run(plan, *args)
            assert e.value.status == capi.CONV_ERR_INVALID_ARG, e.value.message
        with pytest.raises(ConvError):
            capi.conv_bwd_data_run(None, 4096, 8192, base, base + (1 << 24), ws)
    finally:
        capi.conv_bwd_data_destroy(plan)


# --------------------------------------------------------------------------
# Backward-weight: plan-time validation and argument checks (no GPU work)
def test_bwd_weight_create_and_rejects():
    p = sd.problem(8, 4, 64, 64, (1, 56, 56), (1, 3, 3), (1, 1, 1), (0, 1, 1), (1, 1, 1))
    plan = capi.conv_bwd_weight_create(desc_from_problem(p, "bf16"))
    try:
        ws = capi.conv_bwd_weight_workspace_bytes(plan)
        assert ws > 0 and ws % (4 * 64 * 9 * 64 * 4) == 0      # whole fp32 partial tiles per split
        assert "bwd_weight bf16" in capi.conv_bwd_weight_describe(plan)
        base = 1 << 30
        for args in ((4096, 8192, None, base, ws),              # dw NULL
                     (4096, 8192, base, base + (1 << 24), ws - 4),  # workspace too small
                     (4096 + 8, 8192, base, base + (1 << 24), ws),  # misaligned
                     (4096, 8192, base, base + 64, ws)):        # workspace overlaps dw
            with pytest.raises(ConvError) as e:
                capi.conv_bwd_weight_run(plan, *args)
            assert e.value.status == capi.CONV_ERR_INVALID_ARG, e.value.message
    finally:
        capi.conv_bwd_weight_destroy(plan)
    for q, dt in ((p, "f32"), (sd.problem(2, 1, 12, 16, (1, 9, 9), (1, 3, 3)), "bf16")):
        with pytest.raises(ConvError) as e:
            capi.conv_bwd_weight_create(desc_from_problem(q, dt))
        assert e.value.status == capi.CONV_ERR_UNSUPPORTED
    with pytest.raises(ConvError) as e:
        capi.conv_bwd_weight_create(desc_from_problem(p, "bf16", 1, 0))
    assert e.value.status == capi.CONV_ERR_UNSUPPORTED
    capi.conv_bwd_weight_destroy(None)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_data_strided_1d_runs_as_stride_phases(dtype):
    """A 1-D strided input gradient is planned as one forward conv of dy per
    stride phase (no spread copy) where every phase has taps, dx rows have a
    fixed pitch (N = 1 or the length a multiple of the stride) and a group
    row of dx is whole 16-byte vectors; otherwise dy is spread."""
    from convolution_forward_implicit_amd import ConvBwdData
    phases = [sd.conv1d_problem(32, 384, 384, 3000, 3, 2, 1), sd.conv1d_problem(1, 384, 384, 3000, 3, 2, 1),
              sd.conv1d_problem(2, 16, 8, 60, 5, 3, 2), sd.conv1d_problem(1, 8, 16, 50, 7, 4, 3),
              sd.conv1d_problem(2, 8, 8, 40, 3, 2, 1, 3)]
    spread = [sd.conv1d_problem(2, 64, 48, 301, 3, 2, 1),            # N > 1, length not a multiple of 2
              sd.conv1d_problem(3, 3, 5, 77, 5, 2, 2),               # 3-channel rows, and N > 1 with an odd length
              sd.problem(2, 2, 16, 24, (1, 13, 11), (1, 3, 3), (1, 2, 2), (0, 1, 2), (1, 1, 2)),   # 2-D
              sd.conv1d_problem(1, 8, 8, 40, 3, 2, 0, 2)]            # stride 2, dilation 2: one phase has no taps
    for p in phases:
        c = ConvBwdData(p, dtype)
        assert "stride phases" in c.describe(), c.describe()
        assert c.workspace_bytes >= 2 * int(np.prod(ref.shapes(p)[1]))
    for p in spread:
        assert "spread" in ConvBwdData(p, dtype).describe()
