"""Parity of the HIP path (called through the C ABI) with the fp64 oracle.

Tolerance (oracle/check.py): |g - r| <= rtol*|r| + L*gamma_n*sum|x*w|, with
rtol 1e-4 (fp32 outputs) or 8e-3 (bf16 outputs).  Integer-valued inputs in
{-2..2} make every fp32 sum exact in any order, so those cases are compared
bit for bit (bf16 outputs against the one nearest-even rounding of the exact
value)."""
import itertools
import re

import numpy as np
import pytest

import synthdata as sd
from oracle import ref, check

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(a, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return t if dtype == "f32" else t.to(torch.bfloat16)


def host(y):
    return y.float().cpu().numpy().astype(np.float64)


def bits(y):
    return y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run(dev, p, dtype, x, w, b, gelu, config=None, out=None):
    from convolution_forward_implicit_amd import ConvFwd
    c = ConvFwd(p, dtype, b is not None, gelu, config=config)
    print("case:", p, dtype, "gelu" if gelu else "", c.describe(), flush=True)
    y = c(to_dev(x, dtype, dev), to_dev(w, dtype, dev),
          None if b is None else to_dev(b, dtype, dev), out=out)
    torch.cuda.synchronize()
    return y, c


def sample_indices(p, n, seed):
    """Random flat output indices plus every combination of border/centre
    output coordinates (first, second, middle, second-to-last, last)."""
    _, _, _, ys = ref.shapes(p)
    total = int(np.prod(ys))
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = list(rng.integers(0, total, n))
    pick = lambda O: sorted({0, min(1, O - 1), O // 2, max(O - 2, 0), O - 1})
    N, Do, Ho, Wo, G, K = ys
    for nb, od, oh, ow in itertools.product(pick(N), pick(Do), pick(Ho), pick(Wo)):
        for g, k in ((0, 0), (G - 1, K - 1), (int(rng.integers(G)), int(rng.integers(K)))):
            idx.append(((((nb * Do + od) * Ho + oh) * Wo + ow) * G + g) * K + k)
    return np.unique(np.array(idx, dtype=np.int64))


def assert_close(got, p, dtype, x, w, b, gelu, idx=None):
    if idx is None:
        r, a = ref.conv_fwd(p, x, w, b, gelu)
        g = got
    else:
        r, a = ref.conv_fwd_points(p, x, w, b, gelu, idx)
        g = got.ravel()[idx]
    st = check.check(g, r, a, p, dtype, b is not None, gelu)
    print("parity:", {k: st[k] for k in ("ok", "n", "n_fail", "max_ratio", "cosine", "max_abs_diff")},
          flush=True)
    assert st["ok"], st
    return st


# --------------------------------------------------------------------------
# The five workloads at full size, in the launch configuration the benchmark
# times (the selector's choice): every output element against the oracle.
@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_workload_seeded_parity(dev, wid):
    W = sd.workload(wid)
    dt = W["dtype"]
    x = W["x"]
    for li, (p, hb, ge) in enumerate(W["layers"]):
        y, c = run(dev, p, dt, x, W["w"][li], W["b"][li], ge)
        st = assert_close(host(y), p, dt, x, W["w"][li], W["b"][li], ge)
        assert st["n"] == int(np.prod(ref.shapes(p)[3]))
        x = host(y).astype(np.float32)   # next layer is graded on the device's own input


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_workload_integer_bit_exact(dev, wid):
    """Integer-valued inputs at the workload shapes: every output element
    bit for bit (bf16 against the one nearest-even rounding of the exact
    sum)."""
    W = sd.workload(wid)
    dt = W["dtype"]
    for li, (p, hb, _) in enumerate(W["layers"]):
        x, w, b = sd.random_inputs(p, dt, 500 + wid * 10 + li, hb, kind="int")
        y, _ = run(dev, p, dt, x, w, b, False)
        r = ref.conv_fwd(p, x, w, b, False, want_absdot=False).ravel()
        if dt == "f32":
            assert np.array_equal(host(y).ravel(), r)
        else:
            assert np.array_equal(bits(y).ravel(), check.round_to_bf16_bits(r))


# --------------------------------------------------------------------------
# Every compiled tile configuration on problems that span several tiles and
# end in ragged tails along M, N (=K) and the reduction.
def _configs():
    from convolution_forward_implicit_amd import capi
    try:
        n = capi.conv_fwd_num_configs()
    except ImportError:
        return []
    return [(i, capi.conv_fwd_config_name(i)) for i in range(n)]


CONFIGS = _configs()


def _pfix_filter(name):
    """(FY, FX, DH, DW) a fixed-filter patch configuration is compiled for
    (its name carries _f<FY>x<FX>_d<DH>x<DW>), or None for other kinds."""
    m = re.search(r"_pfix_.*_f(\d+)x(\d+)_d(\d+)x(\d+)", name)
    return tuple(int(v) for v in m.groups()) if m else None


def _ragged_problem(name):
    # 2-D, 13 x 11 outputs (ragged against every tile and box), K = 40, G = 2
    pf = _pfix_filter(name)
    if pf:
        FY, FX, DH, DW = pf    # the filter the configuration is compiled for; 13 x 11 outputs
        return sd.problem(2, 2, 32, 40, (1, 13 + (FY - 1) * DH - 2, 11 + (FX - 1) * DW - 2), (1, FY, FX),
                          (1, 1, 1), (0, 1, 1), (1, DH, DW))
    if "_patch_" in name:
        C = 32        # a multiple of every patch kernel's channel slice
    else:
        C = 5 if name.endswith("_v1") else 24
    return sd.problem(2, 2, C, 40, (1, 13, 11), (1, 3, 3), (1, 1, 1), (0, 1, 1))


@pytest.mark.parametrize("cfg,name", CONFIGS, ids=[n for _, n in CONFIGS])
def test_every_config_ragged(dev, cfg, name):
    dt = "bf16" if name.startswith("bf16") else "f32"
    p = _ragged_problem(name)
    x, w, b = sd.random_inputs(p, dt, 31, True)
    y, c = run(dev, p, dt, x, w, b, True, config=cfg)
    assert name in c.describe()
    assert_close(host(y), p, dt, x, w, b, True)
    xi, wi, bi = sd.random_inputs(p, dt, 32, True, kind="int")
    y, _ = run(dev, p, dt, xi, wi, bi, False, config=cfg)
    r = ref.conv_fwd(p, xi, wi, bi, False, want_absdot=False)
    if dt == "f32":
        assert np.array_equal(host(y), r)
    else:
        assert np.array_equal(bits(y), check.round_to_bf16_bits(r))


BIG = [(i, n) for i, n in CONFIGS if re.search(r"_dma_\d+x(256|384)_", n)]


@pytest.mark.parametrize("cfg,name", BIG, ids=[n for _, n in BIG])
def test_big_tiles_several_channel_tiles(dev, cfg, name):
    """The wide-N tiles (bias staged in LDS, fragments read a quarter of
    the slice at a time) on a 1-D problem spanning several output-channel
    tiles and several row tiles, both ragged, with bias + GELU (float) and
    bit-exact in integers."""
    p = sd.conv1d_problem(3, 48, 900, 301, 3, 2, 1)
    x, w, b = sd.random_inputs(p, "bf16", 41, True)
    y, c = run(dev, p, "bf16", x, w, b, True, config=cfg)
    assert name in c.describe()
    assert_close(host(y), p, "bf16", x, w, b, True)
    xi, wi, bi = sd.random_inputs(p, "bf16", 42, True, kind="int")
    y, _ = run(dev, p, "bf16", xi, wi, bi, False, config=cfg)
    r = ref.conv_fwd(p, xi, wi, bi, False, want_absdot=False)
    assert np.array_equal(bits(y), check.round_to_bf16_bits(r))


DMA_CONFIGS = [(i, n) for i, n in CONFIGS if "_dma_" in n]


@pytest.mark.parametrize("cfg,name", DMA_CONFIGS, ids=[n for _, n in DMA_CONFIGS])
def test_dma_configs_whole_subslice_channels(dev, cfg, name):
    """Channel counts that are a whole number of 128-byte reduction
    sub-slices (64 bf16 / 32 or 64 fp32): the direct-to-LDS kernel then
    tracks the filter tap once per workgroup instead of per lane.  A 3-D
    problem with depth/height/width strides, dilations and padding (every
    tap-carry delta is used, padding taps read zeros), ragged against the
    tile in rows and output channels, with bias + GELU in floats and
    bit-exact in integers."""
    dt = "bf16" if name.startswith("bf16") else "f32"
    p = sd.problem(2, 2, 64, 40, (5, 9, 8), (3, 2, 3), (2, 1, 2), (2, 1, 3), (2, 3, 1))
    x, w, b = sd.random_inputs(p, dt, 35, True)
    y, c = run(dev, p, dt, x, w, b, True, config=cfg)
    assert name in c.describe()
    assert_close(host(y), p, dt, x, w, b, True)
    xi, wi, bi = sd.random_inputs(p, dt, 36, True, kind="int")
    y, _ = run(dev, p, dt, xi, wi, bi, False, config=cfg)
    r = ref.conv_fwd(p, xi, wi, bi, False, want_absdot=False)
    if dt == "f32":
        assert np.array_equal(host(y), r)
    else:
        assert np.array_equal(bits(y), check.round_to_bf16_bits(r))


PACKABLE = [(i, n) for i, n in CONFIGS if "_dma_" in n or "_pfix_" in n]


def run_packed(dev, p, dtype, x, w, b, gelu, config=None):
    """The plan's prepacked weights (conv_fwd_pack_weights), then
    conv_fwd_run_packed; also returns the plan."""
    from convolution_forward_implicit_amd import ConvFwd
    c = ConvFwd(p, dtype, b is not None, gelu, config=config)
    print("case: packed", p, dtype, "gelu" if gelu else "", c.describe(), flush=True)
    wt = to_dev(w, dtype, dev)
    pk = c.pack(wt)
    y = c.run_packed(to_dev(x, dtype, dev), pk, None if b is None else to_dev(b, dtype, dev))
    torch.cuda.synchronize()
    return y, c


def same_bits(a, b):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


@pytest.mark.parametrize("cfg,name", PACKABLE, ids=[n for _, n in PACKABLE])
def test_every_packable_config_prepacked_weights(dev, cfg, name):
    """Prepacked weights (f-3): on the ragged problem (several channel
    tiles, a ragged reduction), with bias + GELU, the packed run is bit for
    bit the natural run (same kernel, same order), and with integer inputs
    bit-exact against the oracle."""
    dt = "bf16" if name.startswith("bf16") else "f32"
    p = _ragged_problem(name)
    x, w, b = sd.random_inputs(p, dt, 37, True)
    yn, c = run(dev, p, dt, x, w, b, True, config=cfg)
    yp, _ = run_packed(dev, p, dt, x, w, b, True, config=cfg)
    assert same_bits(yn, yp)
    xi, wi, bi = sd.random_inputs(p, dt, 38, True, kind="int")
    y, _ = run_packed(dev, p, dt, xi, wi, bi, False, config=cfg)
    r = ref.conv_fwd(p, xi, wi, bi, False, want_absdot=False)
    if dt == "f32":
        assert np.array_equal(host(y), r)
    else:
        assert np.array_equal(bits(y), check.round_to_bf16_bits(r))


def _packed_plan_for(wid, li):
    """The selector's plan for a workload layer when its prepacked entry
    points have a kernel to run (its own configuration or the one a tuning
    record names for prepacked weights)."""
    from convolution_forward_implicit_amd import ConvFwd, ConvError
    p, hb, ge = sd.layers(wid)[li]
    c = ConvFwd(p, sd.dtype_of(wid), hb, ge)
    try:
        c.packed_bytes()
    except ConvError:
        return None
    return c


@pytest.mark.parametrize("wid", [1, 2, 4, 5])
def test_workload_prepacked_weights(dev, wid):
    """The workloads at full size with prepacked weights in the plan the
    benchmark times: every output bit for bit the natural run of the same
    configuration (the one conv_fwd_packed_config names), and against the
    oracle at the per-element bound."""
    W = sd.workload(wid)
    dt = W["dtype"]
    x = W["x"]
    for li, (p, hb, ge) in enumerate(W["layers"]):
        pl = _packed_plan_for(wid, li)
        if pl is None:
            pytest.skip("the selector's kernel for this layer reads natural weights only")
        yn, _ = run(dev, p, dt, x, W["w"][li], W["b"][li], ge, config=pl.packed_config())
        yp, c = run_packed(dev, p, dt, x, W["w"][li], W["b"][li], ge)
        assert same_bits(yn, yp)
        assert_close(host(yp), p, dt, x, W["w"][li], W["b"][li], ge)
        x = host(yp).astype(np.float32)


def _split_records(limit=4):
    """Tuning records whose prepacked-weight configuration differs from the
    natural one (read from the compiled table), smallest first, at most one
    per (dtype, natural kernel kind, prepacked kernel kind)."""
    import os
    here = os.path.join(os.path.dirname(__file__), "..", "convolution_forward_implicit_amd", "csrc", "selector_db.inc")
    out, seen = [], set()
    rows = []
    for line in open(here):
        line = line.strip()
        if not line.startswith("{"):
            continue
        nat, pk = line.split('"')[1], line.split('"')[3]
        if not pk or pk == nat:
            continue
        v = [int(t) for t in re.findall(r"-?\d+", line.split('"')[0])]
        dt = "f32" if v[0] == 0 else "bf16"
        p = sd.problem(v[2], v[3], v[4], v[5], v[6:9], v[9:12], v[12:15], v[15:18], v[18:21])
        rows.append((ref.useful_flop(p), dt, bool(v[1]), p, nat, pk))
    for flop, dt, ge, p, nat, pk in sorted(rows, key=lambda r: r[0]):
        kind = (dt, nat.split("_")[1], pk.split("_")[1])
        if kind in seen:
            continue
        seen.add(kind)
        out.append((dt, ge, p, nat, pk))
    return out[:limit]


SPLIT_RECORDS = _split_records()


@pytest.mark.parametrize("rec", SPLIT_RECORDS, ids=["%s_%s_to_%s" % (r[0], r[3], r[4]) for r in SPLIT_RECORDS])
def test_plan_runs_its_prepacked_configuration(dev, rec):
    """A recorded shape whose tuning record names another configuration for
    prepacked weights: the plan's natural run uses the record's natural
    configuration, its prepacked run the other one (conv_fwd_packed_config),
    bit for bit the natural run of a plan forced to that configuration, and
    both meet the per-element bound against the oracle."""
    dt, ge, p, nat, pk = rec
    names = {n: i for i, n in CONFIGS}
    x, w, b = sd.random_inputs(p, dt, 41, ge)
    yn, c = run(dev, p, dt, x, w, b, ge)
    assert (" %s " % nat) in c.describe()
    assert c.packed_config() == names[pk]
    yp, _ = run_packed(dev, p, dt, x, w, b, ge)
    yf, _ = run(dev, p, dt, x, w, b, ge, config=names[pk])
    assert same_bits(yp, yf)
    idx = sample_indices(p, 3000, 43) if ref.useful_flop(p) > 4e9 else None
    assert_close(host(yn), p, dt, x, w, b, ge, idx)
    assert_close(host(yp), p, dt, x, w, b, ge, idx)


@pytest.mark.parametrize("name_re", [r"_dma_", r"_pfix_"])
def test_prepacked_image_holds_every_weight_chunk(dev, name_re):
    """The packed image is a rearrangement of w with zero padding: every
    nonzero 16-byte chunk of w appears in it as often as in w times the
    number of times the kernel loads it (once per K-step image), and
    conv_fwd_packed_bytes is its size."""
    from convolution_forward_implicit_amd import ConvFwd
    cfg, name = next((i, n) for i, n in PACKABLE if re.search(name_re, n) and n.startswith("bf16"))
    p = _ragged_problem(name)
    _, w, _ = sd.random_inputs(p, "bf16", 39, False)
    c = ConvFwd(p, "bf16", config=cfg)
    wt = to_dev(w, "bf16", dev)
    pk = c.pack(wt)
    torch.cuda.synchronize()
    assert pk.numel() == c.packed_bytes() and pk.numel() % 16 == 0
    chunks = pk.cpu().numpy().view(np.uint16).reshape(-1, 8)
    nat = bits(wt).reshape(-1, 8)
    key = lambda a: np.ascontiguousarray(a).view(np.dtype((np.void, 16))).ravel()
    got = key(chunks[(chunks != 0).any(axis=1)])
    want = key(nat[(nat != 0).any(axis=1)])
    # every weight chunk is in exactly one K-step image (each K-step loads a
    # distinct slice of the reduction for a distinct channel tile)
    assert np.array_equal(np.sort(got), np.sort(want))


@pytest.mark.parametrize("cfg,name", CONFIGS, ids=[n for _, n in CONFIGS])
def test_every_config_3d_strided_dilated(dev, cfg, name):
    dt = "bf16" if name.startswith("bf16") else "f32"
    pf = _pfix_filter(name)
    if pf:
        # any depth stride/dilation/padding; in H and W the compiled filter at unit stride
        FY, FX, DH, DW = pf
        p = sd.problem(2, 2, 32, 40, (5, 10, 37), (3, FY, FX), (2, 1, 1), (2, 1, 2), (2, DH, DW))
    elif "_patch_" in name:
        # the patch kernels take any depth stride/dilation/padding; in H and W
        # a 3x3 filter at unit stride fits every configuration's patch
        p = sd.problem(2, 2, 32, 40, (5, 10, 37), (3, 3, 3), (2, 1, 1), (2, 1, 1), (2, 1, 1))
    else:
        C = 3 if name.endswith("_v1") else 16
        p = sd.problem(3, 3, C, 20, (5, 9, 8), (3, 2, 3), (2, 1, 2), (2, 1, 3), (2, 3, 1))
    x, w, b = sd.random_inputs(p, dt, 33, False)
    y, _ = run(dev, p, dt, x, w, None, False, config=cfg)
    assert_close(host(y), p, dt, x, w, None, False)


@pytest.mark.parametrize("cfg,name", CONFIGS, ids=[n for _, n in CONFIGS])
def test_every_config_gelu_range(dev, cfg, name):
    """The GELU epilogue over [-30, 30] (dense near 0 and in the negative
    tail, where Phi is tiny): a centre-tap delta filter copies input channel
    k mod C to output channel k, so each output is GELU of one input value."""
    dt = "bf16" if name.startswith("bf16") else "f32"
    p = _ragged_problem(name)
    xs, ws, _, _ = ref.shapes(p)
    n = int(np.prod(xs))
    vals = np.concatenate([np.linspace(-30.0, 30.0, n // 4), np.linspace(-12.0, -3.0, n // 4),
                           np.linspace(-1e-2, 1e-2, n // 4)])
    vals = np.concatenate([vals, np.random.Generator(np.random.PCG64(61)).uniform(-6, 6, n - vals.size)])
    x = np.random.Generator(np.random.PCG64(62)).permutation(vals).astype(np.float32).reshape(xs)
    if dt == "bf16":
        x = sd.round_bf16(x)
    w = np.zeros(ws, dtype=np.float32)
    for k in range(p["K"]):
        w[:, k, 0, p["filt"][1] // 2, p["filt"][2] // 2, k % p["C"]] = 1.0
    y, _ = run(dev, p, dt, x, w, None, True, config=cfg)
    assert_close(host(y), p, dt, x, w, None, True)


# --------------------------------------------------------------------------
# Edge cases (selector's choice)
EDGE = [
    ("c1_k1_conv1d", sd.conv1d_problem(2, 1, 1, 100, 3, 1, 1)),
    ("odd_channels", sd.conv1d_problem(3, 3, 5, 77, 5, 2, 2)),
    ("stride_gt_filter", sd.problem(2, 1, 16, 24, (1, 17, 19), (1, 2, 2), (1, 3, 3), (0, 0, 1))),
    ("one_by_one_output", sd.problem(5, 1, 32, 16, (1, 3, 3), (1, 3, 3))),
    ("pad_wider_than_filter", sd.conv1d_problem(2, 8, 8, 4, 3, 1, 3)),
    ("dilation_and_pad_3d", sd.problem(1, 2, 8, 8, (7, 6, 9), (2, 3, 2), (1, 2, 1), (3, 2, 1), (3, 1, 4))),
    ("k_not_vector_multiple", sd.problem(2, 3, 16, 13, (1, 9, 9), (1, 3, 3), (1, 1, 1), (0, 1, 1))),
    ("many_groups", sd.problem(2, 32, 8, 8, (1, 10, 10), (1, 3, 3), (1, 1, 1), (0, 1, 1))),
    ("pointwise_large_k", sd.problem(1, 1, 64, 520, (1, 7, 9), (1, 1, 1))),
    ("long_1d_batch1", sd.conv1d_problem(1, 8, 16, 5003, 7, 1, 3)),
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,p", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(dev, name, p, dt):
    x, w, b = sd.random_inputs(p, dt, 41, True)
    y, _ = run(dev, p, dt, x, w, b, True)
    assert_close(host(y), p, dt, x, w, b, True)
    xi, wi, bi = sd.random_inputs(p, dt, 42, True, kind="int")
    y, _ = run(dev, p, dt, xi, wi, bi, False)
    r = ref.conv_fwd(p, xi, wi, bi, False, want_absdot=False)
    if dt == "f32":
        assert np.array_equal(host(y), r)
    else:
        assert np.array_equal(bits(y), check.round_to_bf16_bits(r))


def _random_problems(n=48, seed=2026):
    """Seeded random problems the calibration sweep never saw: 1-D / 2-D /
    3-D, groups, strides, padding, dilation, ragged channel counts, both
    dtypes, with and without bias + GELU; small enough for the oracle."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < n:
        nd = int(rng.integers(1, 4))
        dt = "bf16" if rng.random() < 0.6 else "f32"
        G = int(rng.choice([1, 1, 2, 4, 8]))
        C = int(rng.choice([8, 16, 24, 32, 40, 64, 80, 96, 3, 13]))
        K = int(rng.choice([8, 16, 32, 48, 64, 72, 96, 128, 5, 19]))
        ins, filt, st, pad, dil = [1, 1, 1], [1, 1, 1], [1, 1, 1], [0, 0, 0], [1, 1, 1]
        for d in range(3 - nd, 3):
            ins[d] = int(rng.integers(4, 40 if nd == 3 else (64 if nd == 2 else 900)))
            filt[d] = int(rng.choice([1, 3, 3, 5]))
            st[d] = int(rng.choice([1, 1, 2, 3]))
            pad[d] = int(rng.integers(0, 3))
            dil[d] = int(rng.choice([1, 1, 2]))
        N = int(rng.integers(1, 4))
        p = sd.problem(N, G, C, K, ins, filt, st, pad, dil)
        try:
            o = ref.out_dims(p)
        except ValueError:        # a filter reaching past the padded input: no output
            continue
        if min(o) < 1 or ref.useful_flop(p) > 6e8:
            continue
        ge = bool(rng.random() < 0.5)
        out.append((dt, ge, p))
    return out


RANDOM_PROBLEMS = _random_problems()


def _random_forced(n=60, seed=4242, per=2):
    """Seeded random problems (another seed than the selector's test), each
    with `per` configurations drawn at random from those eligible for it
    (plan creation is host-only, so this runs at collection)."""
    from convolution_forward_implicit_amd import ConvFwd, ConvError
    if not CONFIGS:
        return []
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    out = []
    for k, (dt, ge, p) in enumerate(_random_problems(n=n, seed=seed)):
        cands = [i for i, nm in CONFIGS if nm.startswith(dt)]
        got = 0
        for i in rng.permutation(cands):
            try:
                ConvFwd(p, dt, ge, ge, config=int(i)).close()
            except ConvError:
                continue
            out.append((k, dt, ge, p, int(i)))
            got += 1
            if got == per:
                break
    return out


RANDOM_FORCED = _random_forced()


@pytest.mark.parametrize("k,dt,ge,p,cfg", RANDOM_FORCED,
                         ids=["f%02d_%s_c%d" % (r[0], r[1], r[4]) for r in RANDOM_FORCED])
def test_random_shapes_with_random_configs(dev, k, dt, ge, p, cfg):
    """A random eligible configuration (not the selector's pick) on a random
    shape: every output against the oracle from natural weights, and, where
    the kernel has a prepacked form, bit for bit the same from prepacked
    weights."""
    x, w, b = sd.random_inputs(p, dt, 300 + k, ge)
    y, c = run(dev, p, dt, x, w, b, ge, config=cfg)
    assert_close(host(y), p, dt, x, w, b, ge)
    from convolution_forward_implicit_amd import ConvError
    try:
        c.packed_bytes()
    except ConvError:
        return
    yp, _ = run_packed(dev, p, dt, x, w, b, ge, config=cfg)
    assert same_bits(y, yp)


@pytest.mark.parametrize("dt,ge,p", RANDOM_PROBLEMS, ids=["r%02d_%s" % (i, r[0]) for i, r in enumerate(RANDOM_PROBLEMS)])
def test_selector_on_random_shapes(dev, dt, ge, p):
    """Whatever configuration the selector (cost model or record) picks for a
    shape outside the calibration grid, every output meets the per-element
    bound against the oracle."""
    x, w, b = sd.random_inputs(p, dt, 47, ge)
    y, c = run(dev, p, dt, x, w, b, ge)
    assert_close(host(y), p, dt, x, w, b, ge)


def test_input_of_2gib_and_more_bit_exact(dev):
    """An input of 2 GiB or more (bf16 [16, 1048600, 64], 2.00005 GiB): the
    direct-to-LDS kernels address x with 32-bit byte offsets and are not
    eligible, so the plan takes the register-staged kernel, whose 64-bit
    addressing must reach the end of x.  Integer inputs, bit-exact on
    sampled outputs that include the last images (x offsets past 2^31
    bytes)."""
    from convolution_forward_implicit_amd import ConvFwd
    p = sd.conv1d_problem(16, 64, 16, 1048600, 3, 1, 1)
    xs, ws, bs, ys = ref.shapes(p)
    assert int(np.prod(xs)) * 2 >= 2 ** 31
    x8, w8, b8 = sd.random_int8(xs, 71), sd.random_int8(ws, 72), sd.random_int8(bs, 73)
    c = ConvFwd(p, "bf16", True, False)
    print("case: 2 GiB input", p, c.describe(), flush=True)
    assert "_dma_" not in c.describe() and "_patch_" not in c.describe()
    t = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)
    y = c(t(x8), t(w8), t(b8))
    torch.cuda.synchronize()
    idx = sample_indices(p, 3000, 74)
    got = y.view(torch.int16).reshape(-1)[torch.from_numpy(idx).to(dev)].cpu().numpy().view(np.uint16)
    del y
    r = ref.conv_fwd_points(p, x8, w8, b8, False, idx)[0]
    assert np.array_equal(got, check.round_to_bf16_bits(r))


def test_empty_batch_leaves_output_untouched(dev):
    from convolution_forward_implicit_amd import ConvFwd
    p = sd.conv1d_problem(0, 8, 8, 16, 3, 1, 1)
    c = ConvFwd(p, "bf16")
    x = torch.empty((0, 1, 1, 16, 1, 8), dtype=torch.bfloat16, device=dev)
    w = torch.ones((1, 8, 1, 1, 3, 8), dtype=torch.bfloat16, device=dev)
    y = torch.empty((0, 1, 1, 16, 1, 8), dtype=torch.bfloat16, device=dev)
    assert c(x, w, out=y) is y
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# Closed forms on the device: delta kernel and all-ones (exact in every dtype)
@pytest.mark.parametrize("wid", [1, 4, 5])
def test_delta_kernel_on_device(dev, wid):
    p = dict(sd.layers(wid)[0][0], N=1)
    dt = sd.dtype_of(wid)
    xs, ws, _, _ = ref.shapes(p)
    x, _, _ = sd.random_inputs(p, dt, 51, False)
    w = np.zeros(ws, dtype=np.float32)
    t0 = tuple(f - 1 for f in p["filt"])      # last tap: off-centre in every used dim
    for k in range(p["K"]):
        w[:, k, t0[0], t0[1], t0[2], k % p["C"]] = 1.0
    y, _ = run(dev, p, dt, x, w, None, False)
    r = ref.conv_fwd(p, x, w, None, False, want_absdot=False)
    assert np.array_equal(host(y), r)


@pytest.mark.parametrize("wid", [1, 4, 5])
def test_all_ones_on_device(dev, wid):
    p = dict(sd.layers(wid)[0][0], N=1)
    dt = sd.dtype_of(wid)
    xs, ws, _, _ = ref.shapes(p)
    y, _ = run(dev, p, dt, np.ones(xs, np.float32), np.ones(ws, np.float32), None, False)
    r = ref.conv_fwd(p, np.ones(xs), np.ones(ws), None, False, want_absdot=False)
    assert np.array_equal(host(y), r)


def test_repeat_runs_bitwise_identical(dev):
    W = sd.workload(4)
    p, _, _ = W["layers"][0]
    y1, c = run(dev, p, "bf16", W["x"], W["w"][0], None, False)
    y2 = c(to_dev(W["x"], "bf16", dev), to_dev(W["w"][0], "bf16", dev))
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# --------------------------------------------------------------------------
# Fused two-conv frontend (conv_chain_*): the intermediate never leaves the
# chip, so the oracle rounds its own exact intermediate to bf16
# (oracle.ref.conv_chain) and the bound carries the possible one-step
# difference of that rounding through conv2 (oracle.check.check_chain).
def _chain(N, L, C1=80):
    p1 = sd.conv1d_problem(N, C1, 384, L, 3, 1, 1)
    p2 = sd.conv1d_problem(N, 384, 384, L, 3, 2, 1)
    return p1, p2


def run_chain(dev, p1, p2, x, w1, b1, w2, b2, gelu, packed=False):
    """Runs the fused chain through the C ABI: with the natural weights
    (conv_chain_run) or prepacked ones (conv_chain_pack_weights, then
    conv_chain_run_packed)."""
    from convolution_forward_implicit_amd import ConvChain
    c = ConvChain(p1, p2, "bf16", b1 is not None, gelu)
    print("case: chain", "packed" if packed else "", p1, "gelu" if gelu else "", c.describe(), flush=True)
    t = lambda a: None if a is None else to_dev(a, "bf16", dev)
    if packed:
        y = c.run_packed(t(x), c.pack(t(w1), t(w2)), t(b1), t(b2))
    else:
        y = c(t(x), t(w1), t(b1), t(w2), t(b2))
    torch.cuda.synchronize()
    return y, c


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("N,L,C1", [(2, 300, 80), (3, 1001, 80), (1, 130, 16), (2, 257, 352), (2, 190, 224),
                                    (1, 2, 128), (1, 1, 80)])
def test_chain_integer_bit_exact(dev, N, L, C1, packed):
    """Integer inputs: conv1's fp32 sums are exact, so the device's bf16 h is
    the oracle's rounding of the exact h, conv2's sums of those bf16 values
    are exact too, and the bf16 output has one correct value."""
    if packed and C1 > 224:
        pytest.skip("the prepacked kernel takes C1 <= 224 (conv_chain_packed_bytes says UNSUPPORTED)")
    p1, p2 = _chain(N, L, C1)
    x, w1, b1 = sd.random_inputs(p1, "bf16", 81, True, kind="int")
    _, w2, b2 = sd.random_inputs(p2, "bf16", 82, True, kind="int")
    y, _ = run_chain(dev, p1, p2, x, w1, b1, w2, b2, False, packed)
    r, _, _ = ref.conv_chain(p1, p2, x, w1, b1, w2, b2, False)
    assert np.array_equal(bits(y).ravel(), check.round_to_bf16_bits(r).ravel())


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("N,L", [(2, 301), (1, 64), (2, 127)])
def test_chain_seeded_float_parity(dev, N, L, packed):
    p1, p2 = _chain(N, L)
    x, w1, b1 = sd.random_inputs(p1, "bf16", 83, True)
    _, w2, b2 = sd.random_inputs(p2, "bf16", 84, True)
    y, _ = run_chain(dev, p1, p2, x, w1, b1, w2, b2, True, packed)
    r, a2, cy = ref.conv_chain(p1, p2, x, w1, b1, w2, b2, True)
    st = check.check_chain(host(y), r, a2, cy, p1, p2, True)
    print("parity:", {k: v for k, v in st.items() if k != "limit"}, flush=True)
    assert st["ok"], {k: v for k, v in st.items() if k != "limit"}


def test_chain_packed_no_bias_no_gelu_and_pack_layout(dev):
    """Without bias and GELU; and the packed weights are a rearrangement of
    w1 and w2 with zero padding: every nonzero 16-byte chunk of w1 and w2
    appears, and the packed byte count is what conv_chain_packed_bytes says."""
    p1, p2 = _chain(2, 211, 48)
    x, w1, _ = sd.random_inputs(p1, "bf16", 86, False)
    _, w2, _ = sd.random_inputs(p2, "bf16", 87, False)
    y, c = run_chain(dev, p1, p2, x, w1, None, w2, None, False, True)
    r, a2, cy = ref.conv_chain(p1, p2, x, w1, None, w2, None, False)
    st = check.check_chain(host(y), r, a2, cy, p1, p2, False)
    assert st["ok"], {k: v for k, v in st.items() if k != "limit"}
    pk = c.pack(to_dev(w1, "bf16", dev), to_dev(w2, "bf16", dev))
    torch.cuda.synchronize()
    assert pk.numel() == c.packed_bytes()
    chunks = pk.cpu().numpy().view(np.uint16).reshape(-1, 8)
    nat = np.concatenate([bits(to_dev(w1, "bf16", dev)).reshape(-1, 8), bits(to_dev(w2, "bf16", dev)).reshape(-1, 8)])
    assert chunks.shape[0] == c.packed_bytes() // 16
    key = lambda a: np.ascontiguousarray(a).view(np.dtype((np.void, 16))).ravel()
    nonzero = chunks[(chunks != 0).any(axis=1)]
    assert np.array_equal(np.sort(key(nonzero)), np.sort(key(nat[(nat != 0).any(axis=1)])))


@pytest.fixture(scope="module")
def chain_workload_oracle():
    """The oracle's batch-32 bf16 frontend (h rounded to bf16 between the
    convs), every output, computed once for both chain kernels."""
    W = sd.workload(3)
    (p1, _, _), (p2, _, _) = W["layers"]
    return W, ref.conv_chain(p1, p2, W["x"], W["w"][0], W["b"][0], W["w"][1], W["b"][1], True)


@pytest.mark.parametrize("packed", [False, True])
def test_chain_workload_full_size(dev, packed, chain_workload_oracle):
    """The batch-32 bf16 frontend at full size, in the launch the benchmark
    times with --fused: every output against the oracle."""
    W, (r, a2, cy) = chain_workload_oracle
    (p1, _, _), (p2, _, _) = W["layers"]
    y, _ = run_chain(dev, p1, p2, W["x"], W["w"][0], W["b"][0], W["w"][1], W["b"][1], True, packed)
    st = check.check_chain(host(y), r, a2, cy, p1, p2, True)
    print("parity:", {k: v for k, v in st.items() if k != "limit"}, flush=True)
    assert st["ok"], {k: v for k, v in st.items() if k != "limit"}
    assert st["n"] == r.size


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("N,L", [(32, 3000), (2, 301)])
def test_chain_integer_h_rounding_bit_exact(dev, N, L, packed):
    """Integer inputs wide enough that the intermediate h needs rounding:
    x, w1, b1 in {-8..8} make conv1's exact sums often larger than 256, so
    they have more than bf16's 8 significant bits and h is their one
    nearest-even rounding (truncating h would change many of them).  w2, b2
    in {-2..2}: conv2's terms are integers whose absolute sum stays below
    2^24 (checked), so its fp32 sums are exact in any order and every bf16
    output has one correct value.  (32, 3000) is the batch-32 frontend shape
    the benchmark times with --fused."""
    p1, p2 = _chain(N, L)
    x, w1, b1 = sd.random_inputs(p1, "bf16", 88, True, kind="int", imax=8)
    _, w2, b2 = sd.random_inputs(p2, "bf16", 89, True, kind="int")
    h = ref.conv_fwd(p1, x, w1, b1, False, want_absdot=False)
    assert np.mean(ref.round_bf16(h) != h) > 0.2          # rounding of h is exercised
    y, _ = run_chain(dev, p1, p2, x, w1, b1, w2, b2, False, packed)
    r, a2, _ = ref.conv_chain(p1, p2, x, w1, b1, w2, b2, False)
    assert float(a2.max()) < 2.0 ** 24                      # conv2's fp32 sums are exact
    assert np.array_equal(bits(y).ravel(), check.round_to_bf16_bits(r).ravel())


def test_chain_empty_batch(dev):
    from convolution_forward_implicit_amd import ConvChain
    p1, p2 = _chain(0, 64)
    c = ConvChain(p1, p2, "bf16", False, False)
    e = lambda s: torch.empty(s, dtype=torch.bfloat16, device=dev)
    y = e(c.y_shape)
    assert c(e(c.x_shape), e(c.w1_shape), None, e(c.w2_shape), None, out=y) is y
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# Backward-data (conv_bwd_data_*): dx against the oracle's input gradient.
# The device sums taps * K terms per element (the rewrite as a forward conv
# adds the zero taps), so the bound's n is that count.
BWD = [
    ("conv1d_s2", sd.conv1d_problem(2, 64, 48, 301, 3, 2, 1)),
    ("grouped2d_s1", sd.problem(2, 4, 16, 8, (1, 13, 11), (1, 3, 3), (1, 1, 1), (0, 1, 1), (1, 1, 1))),
    ("grouped2d_s2_dil", sd.problem(2, 2, 16, 24, (1, 13, 11), (1, 3, 3), (1, 2, 2), (0, 1, 2), (1, 1, 2))),
    ("grouped3d_dil2", sd.problem(1, 8, 32, 32, (6, 9, 9), (3, 3, 3), (1, 1, 1), (2, 2, 2), (2, 2, 2))),
    ("pad_wider_than_filter", sd.conv1d_problem(2, 8, 8, 20, 3, 1, 3)),
    ("odd_channels_s2", sd.conv1d_problem(3, 3, 5, 77, 5, 2, 2)),
    ("stride_gt_filter", sd.problem(2, 1, 16, 8, (1, 17, 19), (1, 2, 2), (1, 3, 3), (0, 0, 1))),
    ("mixed_3d", sd.problem(1, 2, 5, 3, (4, 5, 7), (2, 1, 3), (2, 1, 3), (1, 0, 1), (1, 1, 1))),
    # 1-D strided problems the plan runs as stride phases of dy (no spread copy)
    ("phases_s3_k5", sd.conv1d_problem(2, 16, 8, 60, 5, 3, 2)),
    ("phases_s4_k7_n1_odd", sd.conv1d_problem(1, 8, 16, 50, 7, 4, 3)),
    ("phases_s2_dil3", sd.conv1d_problem(2, 8, 8, 40, 3, 2, 1, 3)),
    ("phases_s3_dil2_n1", sd.conv1d_problem(1, 16, 16, 33, 4, 3, 0, 2)),
]


def _terms(n):
    """A stand-in problem whose reduction length (the bound's n) is n."""
    return {"C": int(n), "filt": (1, 1, 1)}


def _dy(p, dtype, seed, kind):
    rng = np.random.Generator(np.random.PCG64(seed))
    ys = ref.shapes(p)[3]
    if kind == "int":
        return rng.integers(-2, 3, size=ys).astype(np.float32)
    v = rng.uniform(-1.0, 1.0, size=ys).astype(np.float32)
    return sd.round_bf16(v) if dtype == "bf16" else v


def run_bwd_data(dev, p, dtype, dy, w):
    from convolution_forward_implicit_amd import ConvBwdData
    c = ConvBwdData(p, dtype)
    print("case: bwd_data", p, dtype, c.describe(), flush=True)
    dx = c(to_dev(dy, dtype, dev), to_dev(w, dtype, dev))
    torch.cuda.synchronize()
    return dx, c


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,p", BWD, ids=[b[0] for b in BWD])
def test_bwd_data_integer_bit_exact(dev, name, p, dt):
    _, w, _ = sd.random_inputs(p, dt, 91, False, kind="int")
    dy = _dy(p, dt, 92, "int")
    dx, _ = run_bwd_data(dev, p, dt, dy, w)
    r, _ = ref.conv_bwd_data(p, dy, w)
    if dt == "f32":
        assert np.array_equal(host(dx), r)
    else:
        assert np.array_equal(bits(dx).ravel(), check.round_to_bf16_bits(r).ravel())


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,p", BWD, ids=[b[0] for b in BWD])
def test_bwd_data_seeded_float_parity(dev, name, p, dt):
    _, w, _ = sd.random_inputs(p, dt, 93, False)
    dy = _dy(p, dt, 94, "float")
    dx, _ = run_bwd_data(dev, p, dt, dy, w)
    r, a = ref.conv_bwd_data(p, dy, w)
    st = check.check(host(dx), r, a, _terms(p["K"] * np.prod(p["filt"])), dt, False, False)
    print("parity:", {k: st[k] for k in ("ok", "n", "n_fail", "max_ratio", "cosine")}, flush=True)
    assert st["ok"], st


@pytest.mark.parametrize("wid", [4, 5])
def test_bwd_data_grouped_workloads_full_size(dev, wid):
    """The grouped 2-D and dilated 3-D workload shapes at full size: every
    input-gradient element against the oracle."""
    W = sd.workload(wid)
    (p, _, _), = W["layers"]
    dy = _dy(p, "bf16", 95, "float")
    dx, _ = run_bwd_data(dev, p, "bf16", dy, W["w"][0])
    r, a = ref.conv_bwd_data(p, dy, W["w"][0])
    st = check.check(host(dx), r, a, _terms(p["K"] * np.prod(p["filt"])), "bf16", False, False)
    print("parity:", {k: st[k] for k in ("ok", "n", "n_fail", "max_ratio", "cosine")}, flush=True)
    assert st["ok"], st


@pytest.mark.parametrize("wid", [2, 3])
def test_bwd_data_frontend_full_size_sampled(dev, wid):
    """Both layers of the fp32 batch-1 and bf16 batch-32 frontends at full
    size, in the launch the benchmark's backward-data pass times: 4000
    random input-gradient elements plus a stride through the tensor."""
    W = sd.workload(wid)
    dt = W["dtype"]
    for li, (p, _, _) in enumerate(W["layers"]):
        dy = _dy(p, dt, 110 + li, "float")
        dx, _ = run_bwd_data(dev, p, dt, dy, W["w"][li])
        n = int(np.prod(ref.shapes(p)[0]))
        rng = np.random.Generator(np.random.PCG64(112 + li))
        idx = np.unique(np.concatenate([rng.integers(0, n, 4000), np.arange(0, n, n // 97)]))
        r, a = ref.conv_bwd_data_points(p, dy, W["w"][li], idx)
        st = check.check(host(dx).ravel()[idx], r, a, _terms(p["K"] * np.prod(p["filt"])), dt, False, False)
        print("parity:", li, {k: st[k] for k in ("ok", "n", "n_fail", "max_ratio", "cosine")}, flush=True)
        assert st["ok"], (li, st)


def test_bwd_data_empty_batch(dev):
    from convolution_forward_implicit_amd import ConvBwdData
    p = sd.conv1d_problem(0, 8, 8, 20, 3, 2, 1)
    c = ConvBwdData(p, "f32")
    dx = torch.empty(c.dx_shape, dtype=torch.float32, device=dev)
    assert c(torch.empty(c.dy_shape, dtype=torch.float32, device=dev),
             torch.empty(c.w_shape, dtype=torch.float32, device=dev), out=dx) is dx
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# Backward-weight (conv_bwd_weight_*, bf16): dw against the oracle's weight
# gradient; the device sums N*Do*Ho*Wo terms per element (bound's n).
WGRAD = [
    ("conv1d_s2", sd.conv1d_problem(2, 64, 48, 301, 3, 2, 1)),
    ("grouped2d_s1", sd.problem(2, 4, 16, 8, (1, 13, 11), (1, 3, 3), (1, 1, 1), (0, 1, 1), (1, 1, 1))),
    ("grouped2d_s2_dil", sd.problem(2, 2, 16, 24, (1, 13, 11), (1, 3, 3), (1, 2, 2), (0, 1, 2), (1, 1, 2))),
    ("grouped3d_dil2", sd.problem(1, 8, 32, 32, (6, 9, 9), (3, 3, 3), (1, 1, 1), (2, 2, 2), (2, 2, 2))),
    ("wide_channels_k5", sd.conv1d_problem(1, 96, 80, 200, 5, 1, 2)),
    ("ragged_tiles", sd.problem(3, 1, 72, 40, (1, 7, 9), (1, 3, 3), (1, 1, 2), (0, 1, 1), (1, 1, 1))),
    ("pointwise", sd.problem(2, 2, 64, 64, (1, 6, 7), (1, 1, 1))),
    # 32-channel tiles with 3 taps and with 1 tap: waves past the last block
    # read a clamped block whose sums are never stored
    ("kt32_taps3", sd.conv1d_problem(2, 32, 32, 150, 3, 1, 1)),
    ("kt32_taps5_ragged", sd.conv1d_problem(3, 16, 24, 97, 5, 2, 2)),
]


def run_bwd_weight(dev, p, x, dy):
    from convolution_forward_implicit_amd import ConvBwdWeight
    c = ConvBwdWeight(p)
    print("case: bwd_weight", p, c.describe(), flush=True)
    dw = c(to_dev(x, "bf16", dev), to_dev(dy, "bf16", dev))
    torch.cuda.synchronize()
    return dw, c


def _pixels(p):
    return p["N"] * int(np.prod(ref.out_dims(p)))


@pytest.mark.parametrize("name,p", WGRAD, ids=[b[0] for b in WGRAD])
def test_bwd_weight_integer_bit_exact(dev, name, p):
    x, _, _ = sd.random_inputs(p, "bf16", 97, False, kind="int")
    dy = _dy(p, "bf16", 98, "int")
    dw, _ = run_bwd_weight(dev, p, x, dy)
    r, _ = ref.conv_bwd_weight(p, x, dy)
    assert np.array_equal(bits(dw).ravel(), check.round_to_bf16_bits(r).ravel())


@pytest.mark.parametrize("name,p", WGRAD, ids=[b[0] for b in WGRAD])
def test_bwd_weight_seeded_float_parity(dev, name, p):
    x, _, _ = sd.random_inputs(p, "bf16", 99, False)
    dy = _dy(p, "bf16", 100, "float")
    dw, _ = run_bwd_weight(dev, p, x, dy)
    r, a = ref.conv_bwd_weight(p, x, dy)
    st = check.check(host(dw), r, a, _terms(_pixels(p)), "bf16", False, False)
    print("parity:", {k: st[k] for k in ("ok", "n", "n_fail", "max_ratio", "cosine")}, flush=True)
    assert st["ok"], st


@pytest.mark.parametrize("wid", [4, 5])
def test_bwd_weight_grouped_workloads_full_size(dev, wid):
    """The grouped workload shapes at full size: every weight-gradient
    element (each a sum over every output pixel) against the oracle."""
    W = sd.workload(wid)
    (p, _, _), = W["layers"]
    dy = _dy(p, "bf16", 101, "float")
    dw, _ = run_bwd_weight(dev, p, W["x"], dy)
    r, a = ref.conv_bwd_weight(p, W["x"], dy)
    st = check.check(host(dw), r, a, _terms(_pixels(p)), "bf16", False, False)
    print("parity:", {k: st[k] for k in ("ok", "n", "n_fail", "max_ratio", "cosine")}, flush=True)
    assert st["ok"], st


def test_bwd_weight_frontend_full_size_sampled(dev):
    """Both layers of the bf16 batch-32 frontend at full size, in the launch
    the benchmark's backward-weight pass times (layer 2's input a seeded
    U[-1, 1) tensor of its shape): 2000 random weight-gradient elements, each
    a sum over all 96000 or 48000 output pixels."""
    W = sd.workload(3)
    for li, (p, _, _) in enumerate(W["layers"]):
        if li == 0:
            x = W["x"]
        else:
            rng = np.random.Generator(np.random.PCG64(120))
            x = sd.round_bf16(rng.uniform(-1.0, 1.0, size=ref.shapes(p)[0]).astype(np.float32))
        dy = _dy(p, "bf16", 121 + li, "float")
        dw, _ = run_bwd_weight(dev, p, x, dy)
        n = int(np.prod(ref.shapes(p)[1]))
        idx = np.unique(np.random.Generator(np.random.PCG64(123 + li)).integers(0, n, 2000))
        r, a = ref.conv_bwd_weight_points(p, x, dy, idx)
        st = check.check(host(dw).ravel()[idx], r, a, _terms(_pixels(p)), "bf16", False, False)
        print("parity:", li, {k: st[k] for k in ("ok", "n", "n_fail", "max_ratio", "cosine")}, flush=True)
        assert st["ok"], (li, st)


def test_bwd_weight_empty_batch_is_zero_and_repeatable(dev):
    from convolution_forward_implicit_amd import ConvBwdWeight
    p = sd.conv1d_problem(0, 16, 8, 20, 3, 2, 1)
    c = ConvBwdWeight(p)
    dw = torch.full(c.dw_shape, 7.0, dtype=torch.bfloat16, device=dev)
    c(torch.empty(c.x_shape, dtype=torch.bfloat16, device=dev),
      torch.empty(c.dy_shape, dtype=torch.bfloat16, device=dev), out=dw)
    torch.cuda.synchronize()
    assert float(dw.float().abs().max()) == 0.0
    # a real problem twice: bitwise the same (fixed-order reduction)
    q = WGRAD[1][1]
    x, _, _ = sd.random_inputs(q, "bf16", 103, False)
    dy = _dy(q, "bf16", 104, "float")
    a, _ = run_bwd_weight(dev, q, x, dy)
    b, _ = run_bwd_weight(dev, q, x, dy)
    assert torch.equal(a, b)


# --------------------------------------------------------------------------
# Random shapes through both backward passes (another seed than the forward
# selector's): dx in the problem's dtype, and dw (bf16) where the
# backward-weight kernels take the shape (C and K per group multiples of 8).
RANDOM_BWD = _random_problems(n=32, seed=3031)


@pytest.mark.parametrize("k,dt,p", [(i, r[0], r[2]) for i, r in enumerate(RANDOM_BWD)],
                         ids=["b%02d_%s" % (i, r[0]) for i, r in enumerate(RANDOM_BWD)])
def test_backward_passes_on_random_shapes(dev, k, dt, p):
    from convolution_forward_implicit_amd import ConvBwdWeight, ConvError
    _, w, _ = sd.random_inputs(p, dt, 1300 + k, False)
    dy = _dy(p, dt, 1400 + k, "float")
    dx, _ = run_bwd_data(dev, p, dt, dy, w)
    r, a = ref.conv_bwd_data(p, dy, w)
    st = check.check(host(dx), r, a, _terms(p["K"] * np.prod(p["filt"])), dt, False, False)
    print("parity dx:", {q: st[q] for q in ("ok", "n", "n_fail", "max_ratio", "cosine")}, flush=True)
    assert st["ok"], st
    try:
        ConvBwdWeight(p).close()
    except ConvError:
        return
    x, _, _ = sd.random_inputs(p, "bf16", 1500 + k, False)
    dy = _dy(p, "bf16", 1600 + k, "float")
    dw, _ = run_bwd_weight(dev, p, x, dy)
    r, a = ref.conv_bwd_weight(p, x, dy)
    st = check.check(host(dw), r, a, _terms(_pixels(p)), "bf16", False, False)
    print("parity dw:", {q: st[q] for q in ("ok", "n", "n_fail", "max_ratio", "cosine")}, flush=True)
    assert st["ok"], st
