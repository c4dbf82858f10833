"""Pins of the fp64 oracle against facts that do not come from the oracle:
values printed on the pages, closed forms, invariants, library routines and
an independent brute force.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import ref, check
import synthdata as sd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# Independent brute force: explicit zero padding, dilation by inserting zeros
# into the kernel, then a plain window sum per output.  No index arithmetic
# is shared with the oracle's direct formulation.
def brute_force(p, x, w, b=None, gelu=False):
    N, G, C, K = p["N"], p["G"], p["C"], p["K"]
    (Di, Hi, Wi), (Z, Y, X) = p["in"], p["filt"]
    (sd_, sh, sw), (pd, ph, pw), (dd, dh, dw) = p["stride"], p["pad"], p["dil"]
    xp = np.zeros((N, Di + 2 * pd, Hi + 2 * ph, Wi + 2 * pw, G, C))
    xp[:, pd:pd + Di, ph:ph + Hi, pw:pw + Wi] = x
    ez, ey, ex = (Z - 1) * dd + 1, (Y - 1) * dh + 1, (X - 1) * dw + 1
    wd = np.zeros((G, K, ez, ey, ex, C))
    wd[:, :, ::dd, ::dh, ::dw, :] = w
    Do = (xp.shape[1] - ez) // sd_ + 1
    Ho = (xp.shape[2] - ey) // sh + 1
    Wo = (xp.shape[3] - ex) // sw + 1
    y = np.zeros((N, Do, Ho, Wo, G, K))
    for n, od, oh, ow in itertools.product(range(N), range(Do), range(Ho), range(Wo)):
        win = xp[n, od * sd_:od * sd_ + ez, oh * sh:oh * sh + ey, ow * sw:ow * sw + ex]
        for g in range(G):
            y[n, od, oh, ow, g] = np.tensordot(wd[g], win[:, :, :, g, :],
                                               axes=([1, 2, 3, 4], [0, 1, 2, 3]))
    if b is not None:
        y = y + b.reshape(1, 1, 1, 1, G, K)
    if gelu:
        y = ref.gelu(y)
    return y


def rnd(p, seed, has_bias=True):
    return sd.random_inputs(p, "f32", seed, has_bias)


# --------------------------------------------------------------------------
# Output extents
def test_out_dims_of_every_workload():
    expect = {1: [(1, 1, 3000)], 2: [(1, 1, 3000), (1, 1, 1500)],
              3: [(1, 1, 3000), (1, 1, 1500)], 4: [(1, 56, 56)], 5: [(16, 28, 28)]}
    for wid, outs in expect.items():
        assert [ref.out_dims(p) for p, _, _ in sd.layers(wid)] == outs


def test_page_dispatch_shapes_and_useful_flop():
    """The conv1d issue prints the two dispatch grids (L_out x K), their
    isolated times and useful GFLOP/s; the reduction length of the 384-ch
    conv (1152 iterations), its invocation count (576k) and MACs (664 M)."""
    g = json.load(open(os.path.join(GOLDEN, "executorch_conv1d_issue.json")))
    for d in g["dispatches"]:
        p = sd.conv1d_problem(1, d["C"], d["K"], d["L_in"], d["k"], d["s"], 1)
        assert ref.out_dims(p)[2] == d["L_out"]
        assert [ref.out_dims(p)[2], d["K"], 1] == d["grid"]
        rate = ref.useful_flop(p) / (d["ms_isolated"] * 1e-3) / 1e9
        assert abs(rate - d["gflops_printed"]) / d["gflops_printed"] < 0.01
    f = g["fetch_statement"]
    d = g["dispatches"][f["layer"]]
    p = sd.conv1d_problem(1, d["C"], d["K"], d["L_in"], d["k"], d["s"], 1)
    assert check.reduction_length(p, False) == f["iterations_per_invocation"]
    assert ref.out_dims(p)[2] * d["K"] == f["invocations"]
    assert round(ref.useful_flop(p) / 2 / 1e6) == f["macs_printed_millions"]


def test_degenerate_descriptor_rejected():
    p = sd.problem(1, 1, 1, 1, (1, 1, 2), (1, 1, 5))   # window larger than input
    with pytest.raises(ValueError):
        ref.out_dims(p)


# --------------------------------------------------------------------------
# Brute force on an exhaustive tiny grid
GRID = []
for ndim, s, pd, dl, G in itertools.product((1, 2, 3), (1, 2, 3), (0, 1, 2), (1, 2), (1, 3)):
    if ndim == 1:
        p = sd.problem(2, G, 3, 2, (1, 1, 9), (1, 1, 3), (1, 1, s), (0, 0, pd), (1, 1, dl))
    elif ndim == 2:
        p = sd.problem(1, G, 2, 3, (1, 7, 6), (1, 3, 2), (1, s, s), (0, pd, pd), (1, dl, dl))
    else:
        p = sd.problem(1, G, 2, 2, (5, 4, 6), (2, 3, 2), (s, s, s), (pd, pd, pd), (dl, dl, dl))
    try:
        ref.out_dims(p)
    except ValueError:
        continue
    GRID.append(p)


@pytest.mark.parametrize("idx", range(len(GRID)))
def test_oracle_matches_brute_force(idx):
    p = GRID[idx]
    x, w, b = rnd(p, 10 + idx)
    for bias, gelu in ((None, False), (b, True)):
        y = ref.conv_fwd(p, x, w, bias, gelu, want_absdot=False)
        yb = brute_force(p, x.astype(np.float64), w.astype(np.float64),
                         None if bias is None else bias.astype(np.float64), gelu)
        assert y.shape == yb.shape
        assert np.max(np.abs(y - yb)) <= 1e-12 * max(1.0, np.max(np.abs(yb)))


def _torch_conv(p, x, w, b):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    N, G, C, K = p["N"], p["G"], p["C"], p["K"]
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))  # N D H W G C
    xt = xt.reshape(N, *p["in"], G * C).permute(0, 4, 1, 2, 3)          # N GC D H W
    wt = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float64))  # G K Z Y X C
    wt = wt.reshape(G * K, *p["filt"], C).permute(0, 4, 1, 2, 3)        # GK C Z Y X
    bt = None if b is None else torch.from_numpy(np.asarray(b, dtype=np.float64).reshape(-1))
    y = F.conv3d(xt, wt.contiguous(), bt, stride=p["stride"], padding=p["pad"],
                 dilation=p["dil"], groups=G)
    return y.permute(0, 2, 3, 4, 1).reshape(N, *y.shape[2:], G, K).numpy()


@pytest.mark.parametrize("p", [
    sd.conv1d_problem(1, 80, 384, 300, 3, 1, 1),
    sd.conv1d_problem(2, 384, 64, 301, 3, 2, 1),
    sd.problem(2, 4, 16, 8, (1, 13, 11), (1, 3, 3), (1, 2, 1), (0, 1, 2), (1, 1, 2)),
    sd.problem(1, 8, 8, 4, (6, 9, 9), (3, 3, 3), (1, 1, 1), (2, 2, 2), (2, 2, 2)),
    sd.problem(1, 2, 5, 3, (4, 5, 7), (2, 1, 3), (2, 1, 3), (1, 0, 1), (1, 1, 1)),
], ids=["conv1d80", "conv1d_s2", "grouped2d", "grouped3d_dil2", "odd3d"])
def test_oracle_matches_torch_fp64(p):
    x, w, b = rnd(p, 77)
    y = ref.conv_fwd(p, x, w, b, False, want_absdot=False)
    yt = _torch_conv(p, x, w, b)
    assert np.max(np.abs(y - yt)) <= 1e-12 * max(1.0, np.max(np.abs(yt)))


# --------------------------------------------------------------------------
# Invariants
def test_one_dimension_in_any_axis():
    """conv1d == conv2d with H = 1 == conv3d with D = H = 1: the same 1-D
    signal placed along D, H or W gives the same result."""
    L, C, K, k, s, pd, dl = 23, 3, 4, 3, 2, 2, 2
    base = sd.conv1d_problem(2, C, K, L, k, s, pd, dl)
    x, w, b = rnd(base, 5)
    yw = ref.conv_fwd(base, x, w, b, True, want_absdot=False)
    for ax in (0, 1):
        ins, f, st, pp, dd = [1, 1, 1], [1, 1, 1], [1, 1, 1], [0, 0, 0], [1, 1, 1]
        ins[ax], f[ax], st[ax], pp[ax], dd[ax] = L, k, s, pd, dl
        p = sd.problem(2, 1, C, K, ins, f, st, pp, dd)
        xs, ws, _, ys = ref.shapes(p)
        y = ref.conv_fwd(p, x.reshape(xs), w.reshape(ws), b, True, want_absdot=False)
        assert np.array_equal(y.reshape(yw.shape), yw)


def test_grouped_is_independent_convs():
    p = sd.problem(2, 3, 4, 5, (3, 6, 7), (2, 3, 3), (1, 2, 1), (1, 1, 0), (1, 1, 2))
    x, w, b = rnd(p, 6)
    y = ref.conv_fwd(p, x, w, b, False, want_absdot=False)
    for g in range(3):
        q = dict(p, G=1)
        yg = ref.conv_fwd(q, x[..., g:g + 1, :], w[g:g + 1], b[g:g + 1], False, want_absdot=False)
        assert np.array_equal(yg[..., 0, :], y[..., g, :])


@pytest.mark.parametrize("p,t0", [
    (sd.conv1d_problem(2, 4, 6, 17, 5, 2, 3, 2), (0, 0, 3)),
    (sd.problem(1, 2, 3, 3, (1, 9, 8), (1, 3, 3), (1, 1, 2), (0, 1, 2), (1, 2, 1)), (0, 2, 0)),
    (sd.problem(1, 1, 3, 5, (5, 6, 7), (3, 2, 3), (2, 1, 1), (2, 1, 1), (2, 1, 2)), (2, 0, 1)),
])
def test_delta_kernel_shifts_input(p, t0):
    """w[g,k,t,c] = 1 iff c == k mod C and t == t0 (off-centre, so a flipped
    kernel fails) gives y[o,k] = x[o*s - p + t0*d, k mod C], or 0 where that
    position is padding."""
    x, _, _ = rnd(p, 9, has_bias=False)
    G, C, K = p["G"], p["C"], p["K"]
    w = np.zeros(ref.shapes(p)[1])
    for k in range(K):
        w[:, k, t0[0], t0[1], t0[2], k % C] = 1.0
    y = ref.conv_fwd(p, x, w, None, False, want_absdot=False)
    Do, Ho, Wo = ref.out_dims(p)
    exp = np.zeros_like(y)
    for n, od, oh, ow in itertools.product(range(p["N"]), range(Do), range(Ho), range(Wo)):
        pos = [o * s - q + t * d for o, s, q, t, d in
               zip((od, oh, ow), p["stride"], p["pad"], t0, p["dil"])]
        if all(0 <= v < I for v, I in zip(pos, p["in"])):
            for k in range(K):
                exp[n, od, oh, ow, :, k] = x[n, pos[0], pos[1], pos[2], :, k % C]
    assert np.array_equal(y, exp)


def _valid_taps(O, I, F, s, pd, d):
    return np.array([sum(1 for t in range(F) if 0 <= o * s - pd + t * d < I) for o in range(O)])


@pytest.mark.parametrize("wid", [1, 4, 5])
def test_all_ones_counts_valid_taps(wid):
    """All-ones x and w: y[o] = C * prod_d v_d(o_d), with v_d counting the
    taps that land inside the input (checked at the configured shapes, with
    the batch cut to 1)."""
    p = dict(sd.layers(wid)[0][0], N=1)
    xs, ws, _, _ = ref.shapes(p)
    y = ref.conv_fwd(p, np.ones(xs), np.ones(ws), None, False, want_absdot=False)
    O = ref.out_dims(p)
    v = [_valid_taps(O[i], p["in"][i], p["filt"][i], p["stride"][i], p["pad"][i], p["dil"][i])
         for i in range(3)]
    exp = p["C"] * v[0][:, None, None] * v[1][None, :, None] * v[2][None, None, :]
    assert np.array_equal(y[0, :, :, :, :, :], np.broadcast_to(exp[..., None, None], y.shape[1:]))
    if wid == 5:
        assert sorted(set(np.unique(exp))) [-4:] == [256, 384, 576, 864]


def test_pointwise_conv_is_matmul():
    p = sd.problem(3, 2, 7, 5, (2, 3, 4), (1, 1, 1))
    x, w, _ = rnd(p, 11, has_bias=False)
    y = ref.conv_fwd(p, x, w, None, False, want_absdot=False)
    for g in range(2):
        a = x[..., g, :].reshape(-1, 7).astype(np.float64)
        assert np.max(np.abs(y[..., g, :].reshape(-1, 5) - a @ w[g].reshape(5, 7).T.astype(np.float64))) < 1e-13


def test_single_channel_is_numpy_correlate():
    p = sd.conv1d_problem(1, 1, 1, 50, 5, 1, 2)
    x, w, _ = rnd(p, 12, has_bias=False)
    y = ref.conv_fwd(p, x, w, None, False, want_absdot=False).ravel()
    xp = np.pad(x.ravel().astype(np.float64), 2)
    assert np.max(np.abs(y - np.correlate(xp, w.ravel().astype(np.float64), "valid"))) < 1e-13


def test_linear_in_x_and_w():
    p = sd.problem(2, 2, 3, 4, (3, 5, 6), (2, 3, 2), (1, 2, 1), (1, 1, 1), (1, 1, 2))
    x1, w1, _ = (None if v is None else v.astype(np.float64) for v in rnd(p, 13, has_bias=False))
    x2, w2, _ = (None if v is None else v.astype(np.float64) for v in rnd(p, 14, has_bias=False))
    a, c = 0.75, -1.5
    f = lambda xx, ww: ref.conv_fwd(p, xx, ww, None, False, want_absdot=False)
    lhs = f(a * x1 + c * x2, w1)
    assert np.max(np.abs(lhs - (a * f(x1, w1) + c * f(x2, w1)))) < 1e-12
    lhs = f(x1, a * w1 + c * w2)
    assert np.max(np.abs(lhs - (a * f(x1, w1) + c * f(x1, w2)))) < 1e-12


def test_gelu_closed_forms():
    t = np.linspace(-6, 6, 241)
    g = ref.gelu(t)
    assert ref.gelu(0.0) == 0.0
    assert np.max(np.abs((g - ref.gelu(-t)) - t)) < 1e-14           # GELU(t)-GELU(-t) = t
    assert abs(float(ref.gelu(1.0)) - 0.8413447460685429) < 1e-15    # Phi(1)
    assert abs(float(ref.gelu(-1.0)) + 0.15865525393145707) < 1e-15  # -Phi(-1)
    # slope bound used by the tolerance: max GELU' = 1.1289 at t = sqrt(2)
    gp = np.gradient(g, t)
    assert 1.12 < gp.max() < 1.13


def test_oracle_gelu_epilogue_matches_python_gelu():
    p = sd.conv1d_problem(1, 5, 7, 31, 3, 1, 1)
    x, w, b = rnd(p, 15)
    pre = ref.conv_fwd(p, 3 * x, w, b, False, want_absdot=False)
    post = ref.conv_fwd(p, 3 * x, w, b, True, want_absdot=False)
    assert np.max(np.abs(post - ref.gelu(pre))) < 1e-14


def test_points_equal_full_output():
    p = sd.problem(2, 3, 5, 4, (3, 7, 6), (2, 2, 3), (1, 2, 1), (1, 0, 2), (2, 1, 1))
    x, w, b = rnd(p, 16)
    y, ad = ref.conv_fwd(p, x, w, b, True)
    idx = np.random.Generator(np.random.PCG64(3)).integers(0, y.size, 200)
    yp, adp = ref.conv_fwd_points(p, x, w, b, True, idx)
    assert np.array_equal(yp, y.ravel()[idx]) and np.array_equal(adp, ad.ravel()[idx])
    with pytest.raises(ValueError):
        ref.conv_fwd_points(p, x, w, b, True, [y.size])


def test_absdot_is_sum_of_abs_terms():
    p = sd.conv1d_problem(1, 2, 1, 4, 3, 1, 1)
    x = np.array([1.0, -2.0, 3.0, -4.0, 5.0, 6.0, -7.0, 8.0]).reshape(ref.shapes(p)[0])
    w = np.array([1.0, -1.0, 2.0, 0.5, -3.0, 1.0]).reshape(ref.shapes(p)[1])
    b = np.array([[-0.25]])
    y, ad = ref.conv_fwd(p, x, w, b, False)
    # output 0 sees input pixels -1 (padding), 0, 1 with taps 0, 1, 2
    # pixel 0 = (1,-2) * tap1 (2, 0.5); pixel 1 = (3,-4) * tap2 (-3, 1)
    assert y.ravel()[0] == -0.25 + (1 * 2 + -2 * 0.5) + (3 * -3 + -4 * 1)
    assert ad.ravel()[0] == 0.25 + 2 + 1 + 9 + 4


# --------------------------------------------------------------------------
# The tolerance and the bf16 rounding used to grade the device
def test_bound_holds_for_fp32_sums_and_rejects_a_perturbation():
    p = sd.conv1d_problem(1, 384, 8, 40, 3, 2, 1)
    x, w, b = rnd(p, 17)
    y, ad = ref.conv_fwd(p, x, w, b, True)
    # an fp32 evaluation, summed in a different order (reversed taps)
    x32, w32 = x.astype(np.float32), w.astype(np.float32)
    xs = np.pad(x32.reshape(40, 384), ((1, 1), (0, 0)))
    pre = np.zeros((20, 8), np.float32)
    for o in range(20):
        acc = np.zeros(8, np.float32)
        for t in (2, 1, 0):
            acc = acc + (w32.reshape(8, 3, 384)[:, t, :] * xs[2 * o + t][None, :]).sum(1, dtype=np.float32)
        pre[o] = acc + b.reshape(8)
    g32 = (0.5 * pre.astype(np.float64) * np.vectorize(math.erfc)(-pre / math.sqrt(2))).astype(np.float32)
    st = check.check(g32, y, ad, p, "f32", True, True)
    assert st["ok"], st
    bad = g32.astype(np.float64).ravel().copy()
    i = int(np.argmax(np.abs(y)))
    bad[i] += 3 * check.bound(y.ravel()[i:i + 1], ad.ravel()[i:i + 1], p, "f32", True, True)[0]
    assert not check.check(bad, y, ad, p, "f32", True, True)["ok"]


def test_round_to_bf16_bits_ieee_patterns():
    vals = [1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 257.0, 259.0, -1.0, 0.0, 2 ** -133, 2 ** -140,
            4608.0, 1.5 * 2 ** 127, 1 + 2 ** -8 + 2 ** -23]
    exp = [0x3F80, 0x3F80, 0x3F82, 0x4380, 0x4382, 0xBF80, 0x0000, 0x0001, 0x0000,
           0x4590, 0x7F40, 0x3F81]
    got = check.round_to_bf16_bits(np.array(vals))
    assert [int(v) for v in got] == exp
    assert np.array_equal(check.bf16_bits_to_f64(np.array([0x3F80, 0x4382, 0xC000], np.uint16)),
                          [1.0, 260.0, -2.0])
    # agrees with the input generator's own rounding
    r = np.random.Generator(np.random.PCG64(1)).normal(size=1000).astype(np.float32)
    assert np.array_equal(check.bf16_bits_to_f64(check.round_to_bf16_bits(r)),
                          sd.round_bf16(r).astype(np.float64))


def test_workload_generation_is_seeded_and_bf16_exact():
    a, b_ = sd.workload(4), sd.workload(4)
    assert np.array_equal(a["x"], b_["x"]) and np.array_equal(a["w"][0], b_["w"][0])
    assert np.array_equal(sd.round_bf16(a["x"]), a["x"])
    w3 = sd.workload(3)
    assert w3["x"].shape == (32, 1, 1, 3000, 1, 80)
    assert w3["w"][1].shape == (1, 384, 1, 1, 3, 384)
    assert abs(float(np.std(w3["w"][1])) - 1 / math.sqrt(1152)) < 2e-3


# --------------------------------------------------------------------------
# bf16 rounding of exact values and the two-conv chain (fused frontend)
def test_round_bf16_against_bit_patterns_and_hand_ties():
    rng = np.random.Generator(np.random.PCG64(71))
    v = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                        [0.0, -0.0, 1.0, -2.5, 2.0 ** -126, 2.0 ** -130, 65504.0]]).astype(np.float32)
    got = ref.round_bf16(v.astype(np.float64))
    want = check.bf16_bits_to_f64(check.round_to_bf16_bits(v.astype(np.float64)))
    assert np.array_equal(got, want)
    # ties (values between two bf16 neighbours, exactly half way) go to even
    hand = {1 + 2 ** -8: 1.0, 1 + 3 * 2 ** -8: 1 + 2 ** -6, -(1 + 2 ** -8): -1.0,
            2 ** -134: 0.0, 3 * 2 ** -134: 2 ** -132, 1 + 2 ** -8 + 2 ** -40: 1 + 2 ** -7}
    for a, b in hand.items():
        assert ref.round_bf16(np.array([a]))[0] == b, (a, b)
    # a value that float32 would round first (double rounding) is rounded once here
    a = 1 + 2 ** -8 + 2 ** -30      # float32 -> 1 + 2^-8 -> bf16 1.0; exact -> 1 + 2^-7
    assert ref.round_bf16(np.array([a]))[0] == 1 + 2 ** -7


def _chain_problems(N, C1, K1, K2, L):
    p1 = sd.conv1d_problem(N, C1, K1, L, 3, 1, 1)
    p2 = sd.conv1d_problem(N, K1, K2, L, 3, 2, 1)
    return p1, p2


@pytest.mark.parametrize("gelu", [False, True])
def test_chain_delta_filters_closed_form(gelu):
    """conv1 copies input channel k mod C1 (centre tap), conv2 copies channel
    k (centre tap, stride 2): y[n, o, k] = act(round_bf16(act(x[n, 2o, k mod C1])))
    with act = GELU or identity."""
    N, C1, K1, L = 2, 16, 48, 37
    p1, p2 = _chain_problems(N, C1, K1, K1, L)
    rng = np.random.Generator(np.random.PCG64(72))
    x = sd.round_bf16(rng.uniform(-4, 4, ref.shapes(p1)[0]).astype(np.float32))
    w1 = np.zeros(ref.shapes(p1)[1])
    w2 = np.zeros(ref.shapes(p2)[1])
    for k in range(K1):
        w1[0, k, 0, 0, 1, k % C1] = 1.0
        w2[0, k, 0, 0, 1, k] = 1.0
    y, _, _ = ref.conv_chain(p1, p2, x, w1, None, w2, None, gelu)
    act = (lambda t: 0.5 * t * np.vectorize(math.erfc)(-t / math.sqrt(2.0))) if gelu else (lambda t: t)
    xs = x.astype(np.float64).reshape(N, L, C1)
    Lo = ref.out_dims(p2)[2]
    want = np.empty((N, Lo, K1))
    for k in range(K1):
        want[:, :, k] = act(ref.round_bf16(act(xs[:, 0:2 * Lo:2, k % C1])))
    assert np.array_equal(y.reshape(N, Lo, K1), want)


def test_chain_interior_equals_composed_kernel():
    """Away from the borders (where the zero padding of h matters) the chain
    with no activation is one 5-tap, stride-2 conv whose kernel is the
    composition of the two: W[k, s, c] = sum_{t2+t1=s} sum_j w2[k,t2,j] w1[j,t1,c].
    Integer inputs keep every value exact (h fits bf16)."""
    N, C1, K1, K2, L = 2, 5, 7, 6, 40
    p1, p2 = _chain_problems(N, C1, K1, K2, L)
    rng = np.random.Generator(np.random.PCG64(73))
    x = rng.integers(-2, 3, ref.shapes(p1)[0]).astype(np.float64)
    w1 = rng.integers(-1, 2, ref.shapes(p1)[1]).astype(np.float64)
    w2 = rng.integers(-1, 2, ref.shapes(p2)[1]).astype(np.float64)
    y, _, _ = ref.conv_chain(p1, p2, x, w1, None, w2, None, False)
    W1 = w1.reshape(K1, 3, C1)
    W2 = w2.reshape(K2, 3, K1)
    Wc = np.zeros((K2, 5, C1))
    for t2 in range(3):
        for t1 in range(3):
            Wc[:, t2 + t1, :] += W2[:, t2, :] @ W1[:, t1, :]
    xs = x.reshape(N, L, C1)
    Lo = ref.out_dims(p2)[2]
    ys = y.reshape(N, Lo, K2)
    for o in range(1, Lo - 1):          # h positions 2o-1 .. 2o+1 are all inside [1, L-2]
        win = xs[:, 2 * o - 2:2 * o + 3, :]              # x positions 2o-2 .. 2o+2
        want = np.einsum("nsc,ksc->nk", win, Wc)
        assert np.array_equal(ys[:, o, :], want), o


def test_chain_points_equal_full_chain():
    N, C1, K1, K2, L = 2, 16, 24, 8, 29
    p1, p2 = _chain_problems(N, C1, K1, K2, L)
    rng = np.random.Generator(np.random.PCG64(74))
    x = rng.standard_normal(ref.shapes(p1)[0])
    w1 = rng.standard_normal(ref.shapes(p1)[1]) * 0.2
    b1 = rng.standard_normal(ref.shapes(p1)[2]) * 0.1
    w2 = rng.standard_normal(ref.shapes(p2)[1]) * 0.2
    b2 = rng.standard_normal(ref.shapes(p2)[2]) * 0.1
    y, a2, c = ref.conv_chain(p1, p2, x, w1, b1, w2, b2, True)
    idx = np.array([0, 1, 7, 100, y.size - 1], dtype=np.int64)
    yp, a2p, cp = ref.conv_chain_points(p1, p2, x, w1, b1, w2, b2, True, idx)
    assert np.array_equal(yp, y.ravel()[idx])
    assert np.allclose(a2p, a2.ravel()[idx], rtol=1e-13, atol=0)
    assert np.allclose(cp, c.ravel()[idx], rtol=1e-13, atol=0)


def test_chain_bound_accepts_a_float32_chain_and_rejects_a_perturbation():
    """A float32 re-implementation of the chain (float32 sums, bf16-rounded
    h) stays within check_chain's bound; adding 3x the bound fails it."""
    N, C1, K1, K2, L = 1, 16, 32, 16, 33
    p1, p2 = _chain_problems(N, C1, K1, K2, L)
    rng = np.random.Generator(np.random.PCG64(75))
    x = sd.round_bf16(rng.uniform(-1, 1, ref.shapes(p1)[0]).astype(np.float32))
    w1 = sd.round_bf16((rng.standard_normal(ref.shapes(p1)[1]) * 0.1).astype(np.float32))
    b1 = sd.round_bf16((rng.standard_normal(ref.shapes(p1)[2]) * 0.02).astype(np.float32))
    w2 = sd.round_bf16((rng.standard_normal(ref.shapes(p2)[1]) * 0.1).astype(np.float32))
    b2 = sd.round_bf16((rng.standard_normal(ref.shapes(p2)[2]) * 0.02).astype(np.float32))
    y, a2, c = ref.conv_chain(p1, p2, x, w1, b1, w2, b2, True)

    def f32_conv(xx, ww, bb, Cin, Kout, Lin, stride):
        xs = np.zeros((Lin + 2, Cin), np.float32)
        xs[1:-1] = xx.reshape(Lin, Cin)
        Lout = (Lin - 1) // stride + 1
        out = np.zeros((Lout, Kout), np.float32)
        Wt = ww.reshape(Kout, 3, Cin).astype(np.float32)
        for o in range(Lout):
            acc = bb.astype(np.float32).copy()
            for t in range(3):
                acc = acc + (xs[o * stride + t][None, :] * Wt[:, t, :]).sum(axis=1, dtype=np.float32)
            out[o] = acc
        g = 0.5 * out.astype(np.float64) * np.vectorize(math.erfc)(-out.astype(np.float64) / math.sqrt(2.0))
        return g.astype(np.float32)

    h = f32_conv(x, w1, b1, C1, K1, L, 1)
    h = sd.round_bf16(h)
    g = f32_conv(h, w2, b2, K1, K2, L, 2).astype(np.float64).ravel()
    st = check.check_chain(g, y, a2, c, p1, p2, True)
    assert st["ok"], {k: v for k, v in st.items() if k != "limit"}
    for i in (0, g.size // 2, g.size - 1):
        bad = g.copy()
        bad[i] = y.ravel()[i] + 3 * st["limit"][i]
        assert not check.check_chain(bad, y, a2, c, p1, p2, True)["ok"]



# --------------------------------------------------------------------------
# Backward passes (oracle.ref.conv_bwd_data / conv_bwd_weight), pinned to the
# pinned forward sum and to torch's autograd in fp64.
@pytest.mark.parametrize("idx", range(len(GRID)))
def test_backward_passes_are_the_adjoints_of_the_forward_sum(idx):
    """<conv(x, w), dy> = <x, dgrad(dy, w)> = <w, wgrad(x, dy)> for random
    x, w, dy: the two gradients of the bilinear forward map.  Any index, sign
    or stride mistake in either backward loop breaks one of the equalities
    (the forward sum itself is pinned above)."""
    p = GRID[idx]
    xs, ws, _, ys = ref.shapes(p)
    rng = np.random.default_rng(500 + idx)
    x, w, dy = rng.standard_normal(xs), rng.standard_normal(ws), rng.standard_normal(ys)
    y = ref.conv_fwd(p, x, w, None, False, want_absdot=False)
    dx, adx = ref.conv_bwd_data(p, dy, w)
    dw, adw = ref.conv_bwd_weight(p, x, dy)
    lhs = float(np.sum(y * dy))
    scale = float(np.sum(np.abs(y) * np.abs(dy))) + 1.0
    assert abs(lhs - float(np.sum(x * dx))) <= 1e-12 * scale
    assert abs(lhs - float(np.sum(w * dw))) <= 1e-12 * scale
    # and each one against its own brute force: dx[i] = d<y, dy>/dx[i] as the
    # forward of a one-hot x, dw likewise, at a few random elements
    for _ in range(3):
        i = tuple(int(rng.integers(0, s)) for s in xs)
        e = np.zeros(xs); e[i] = 1.0
        assert abs(np.sum(ref.conv_fwd(p, e, w, None, False, want_absdot=False) * dy) - dx[i]) <= 1e-12 * (1 + adx[i])
        j = tuple(int(rng.integers(0, s)) for s in ws)
        e = np.zeros(ws); e[j] = 1.0
        assert abs(np.sum(ref.conv_fwd(p, x, e, None, False, want_absdot=False) * dy) - dw[j]) <= 1e-12 * (1 + adw[j])


@pytest.mark.parametrize("p", [
    sd.conv1d_problem(2, 384, 64, 301, 3, 2, 1),
    sd.problem(2, 4, 16, 8, (1, 13, 11), (1, 3, 3), (1, 2, 1), (0, 1, 2), (1, 1, 2)),
    sd.problem(1, 8, 8, 4, (6, 9, 9), (3, 3, 3), (1, 1, 1), (2, 2, 2), (2, 2, 2)),
    sd.problem(1, 2, 5, 3, (4, 5, 7), (2, 1, 3), (2, 1, 3), (1, 0, 1), (1, 1, 1)),
], ids=["conv1d_s2", "grouped2d", "grouped3d_dil2", "odd3d"])
def test_backward_passes_match_torch_autograd_fp64(p):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    N, G, C, K = p["N"], p["G"], p["C"], p["K"]
    xs, ws, _, ys = ref.shapes(p)
    rng = np.random.default_rng(78)
    x, w, dy = rng.standard_normal(xs), rng.standard_normal(ws), rng.standard_normal(ys)
    xt = torch.from_numpy(x).reshape(N, *p["in"], G * C).permute(0, 4, 1, 2, 3).contiguous().requires_grad_(True)
    wt = torch.from_numpy(w).reshape(G * K, *p["filt"], C).permute(0, 4, 1, 2, 3).contiguous().requires_grad_(True)
    yt = F.conv3d(xt, wt, None, stride=p["stride"], padding=p["pad"], dilation=p["dil"], groups=G)
    dyt = torch.from_numpy(dy).reshape(N, *ys[1:4], G * K).permute(0, 4, 1, 2, 3).contiguous()
    yt.backward(dyt)
    dx_t = xt.grad.permute(0, 2, 3, 4, 1).reshape(xs).numpy()
    dw_t = wt.grad.permute(0, 2, 3, 4, 1).reshape(ws).numpy()
    dx, _ = ref.conv_bwd_data(p, dy, w)
    dw, _ = ref.conv_bwd_weight(p, x, dy)
    assert np.max(np.abs(dx - dx_t)) <= 1e-12 * max(1.0, np.max(np.abs(dx_t)))
    assert np.max(np.abs(dw - dw_t)) <= 1e-12 * max(1.0, np.max(np.abs(dw_t)))


@pytest.mark.parametrize("p,t0", [
    (sd.conv1d_problem(2, 4, 6, 17, 5, 2, 3, 2), (0, 0, 3)),
    (sd.problem(1, 1, 3, 5, (5, 6, 7), (3, 2, 3), (2, 1, 1), (2, 1, 1), (2, 1, 2)), (2, 0, 1)),
])
def test_backward_data_of_a_delta_kernel_scatters_dy(p, t0):
    """w[g,k,t,c] = 1 iff c == k mod C and t == t0: each dy[o,k] lands on
    dx[o*s - p + t0*d, k mod C] (dropped in the padding), summed over the k
    that share a channel -- exact in any dtype."""
    xs, ws, _, ys = ref.shapes(p)
    dy = np.random.default_rng(11).integers(-3, 4, ys).astype(np.float64)
    G, C, K = p["G"], p["C"], p["K"]
    w = np.zeros(ws)
    for k in range(K):
        w[:, k, t0[0], t0[1], t0[2], k % C] = 1.0
    dx, _ = ref.conv_bwd_data(p, dy, w)
    exp = np.zeros(xs)
    Do, Ho, Wo = ref.out_dims(p)
    for n, od, oh, ow in itertools.product(range(p["N"]), range(Do), range(Ho), range(Wo)):
        pos = [o * s - q + t * d for o, s, q, t, d in zip((od, oh, ow), p["stride"], p["pad"], t0, p["dil"])]
        if all(0 <= v < I for v, I in zip(pos, p["in"])):
            for k in range(K):
                exp[n, pos[0], pos[1], pos[2], :, k % C] += dy[n, od, oh, ow, :, k]
    assert np.array_equal(dx, exp)


@pytest.mark.parametrize("wid", [4, 5])
def test_backward_weight_all_ones_counts_valid_outputs(wid):
    """All-ones x and dy: dw[g,k,t,c] = N * prod_d (number of outputs o_d whose
    tap t_d lands inside the input), at the configured grouped shapes (batch
    cut to 1)."""
    p = dict(sd.layers(wid)[0][0], N=1)
    xs, ws, _, ys = ref.shapes(p)
    dw, _ = ref.conv_bwd_weight(p, np.ones(xs), np.ones(ys))
    O = ref.out_dims(p)
    cnt = [np.array([sum(1 for o in range(O[i]) if 0 <= o * p["stride"][i] - p["pad"][i] + t * p["dil"][i] < p["in"][i])
                     for t in range(p["filt"][i])]) for i in range(3)]
    exp = p["N"] * cnt[0][:, None, None] * cnt[1][None, :, None] * cnt[2][None, None, :]
    assert np.array_equal(dw, np.broadcast_to(exp[None, None, :, :, :, None], dw.shape))


def test_backward_points_equal_full_outputs():
    p = sd.problem(2, 3, 4, 5, (3, 5, 6), (2, 3, 2), (1, 2, 2), (1, 1, 0), (1, 1, 2))
    xs, ws, _, ys = ref.shapes(p)
    rng = np.random.default_rng(3)
    x, w, dy = rng.standard_normal(xs), rng.standard_normal(ws), rng.standard_normal(ys)
    dx, adx = ref.conv_bwd_data(p, dy, w)
    dw, adw = ref.conv_bwd_weight(p, x, dy)
    ix = rng.integers(0, dx.size, 200)
    iw = rng.integers(0, dw.size, 200)
    v, a = ref.conv_bwd_data_points(p, dy, w, ix)
    assert np.array_equal(v, dx.ravel()[ix]) and np.array_equal(a, adx.ravel()[ix])
    v, a = ref.conv_bwd_weight_points(p, x, dy, iw)
    assert np.array_equal(v, dw.ravel()[iw]) and np.array_equal(a, adw.ravel()[iw])
