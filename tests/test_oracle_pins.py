"""Pins for the CPU oracle: every oracle function is checked against something
other than itself - the pages' worked examples (tests/golden/), closed forms,
invariants, brute-force enumeration, and PyTorch's CPU routines in float64 for
the cases that reduce to a library call.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from transposed_convolution_epilogues_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def t64(a):
    return None if a is None else torch.tensor(np.asarray(a), dtype=torch.float64)


def rnd(rng, shape, lo=-1.0, hi=1.0):
    return rng.uniform(lo, hi, shape).astype(np.float32)


# --------------------------------------------------------------- sizes
def test_size_formulas_page_examples():
    for c in golden("sizes.json")["cases"]:
        if c["kind"] == "conv":
            got = O.conv_out_len(c["L"], c["k"], c["s"], c["p"], c["d"])
        elif c["kind"] == "convT":
            got = O.convT_out_len(c["L"], c["k"], c["s"], c["p"], c["d"], c["op"])
        else:
            got = O.pool_out_len(c["L"], c["w"])
        assert got == c["out"], c["source"]


def test_size_formulas_match_torch_shapes():
    rng = np.random.default_rng(11)
    for _ in range(200):
        L, k, s, p, d = (int(rng.integers(1, 12)), int(rng.integers(1, 5)), int(rng.integers(1, 4)),
                         int(rng.integers(0, 3)), int(rng.integers(1, 3)))
        x = torch.zeros(1, 1, L, 1, 1, dtype=torch.float64)
        w = torch.zeros(1, 1, k, 1, 1, dtype=torch.float64)
        if L + 2 * p >= d * (k - 1) + 1:
            assert F.conv3d(x, w, stride=(s, 1, 1), padding=(p, 0, 0), dilation=(d, 1, 1)).shape[2] == \
                O.conv_out_len(L, k, s, p, d)
        op = int(rng.integers(0, max(s, d)))
        n_out = O.convT_out_len(L, k, s, p, d, op)
        if n_out > 0:
            y = F.conv_transpose3d(x, w, stride=(s, 1, 1), padding=(p, 0, 0), dilation=(d, 1, 1),
                                   output_padding=(op, 0, 0))
            assert y.shape[2] == n_out
        wp = int(rng.integers(1, 5))
        if L >= wp:
            assert F.avg_pool3d(torch.zeros(1, 1, L, wp, wp), wp).shape[2] == O.pool_out_len(L, wp)


# ------------------------------------------------------------- conv3d
def _rand_conv_case(rng):
    while True:
        wl = W.random_small_workload("conv3d", rng, max_spatial=8)
        if all(v > 0 for v in O.output_shape(wl)):
            return wl


@pytest.mark.parametrize("seed", range(24))
def test_conv3d_matches_torch_float64(seed):
    rng = np.random.default_rng(100 + seed)
    wl = _rand_conv_case(rng)
    inp = W.make_inputs(wl)
    y = O.conv3d(inp.x, inp.w, inp.b, wl.stride, wl.pad, wl.dilation, wl.groups)
    yt = F.conv3d(t64(inp.x), t64(inp.w), t64(inp.b), wl.stride, wl.pad, wl.dilation, wl.groups).numpy()
    assert y.shape == yt.shape
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=1e-12)


def test_conv3d_impulse_response():
    # one 1 at an interior input position: y[n,oc,o] = W[oc, ic - g*Cin_g, k] wherever
    # q = o*s - p + k*d, and bias elsewhere (exact)
    rng = np.random.default_rng(3)
    s, p, d, groups = (2, 1, 1), (1, 2, 0), (1, 2, 1), 2
    x = np.zeros((1, 4, 9, 10, 7), np.float32)
    q = (4, 5, 3)
    ic = 3
    x[0, ic][q] = 1.0
    w = rnd(rng, (6, 2, 3, 2, 3))
    b = rnd(rng, 6)
    y = O.conv3d(x, w, b, s, p, d, groups)
    g_of_ic = ic // 2
    expect = np.broadcast_to(b.astype(np.float64)[None, :, None, None, None], y.shape).copy()
    for oc in range(6):
        if oc // 3 != g_of_ic:
            continue
        for k in itertools.product(range(3), range(2), range(3)):
            num = [q[j] + p[j] - k[j] * d[j] for j in range(3)]
            if all(v % s[j] == 0 and 0 <= v // s[j] < y.shape[2 + j] for j, v in enumerate(num)):
                o = tuple(v // s[j] for j, v in enumerate(num))
                expect[(0, oc) + o] += w[oc, ic - 2 * g_of_ic][k]
    np.testing.assert_array_equal(y, expect)


def test_conv3d_constant_input():
    rng = np.random.default_rng(4)
    x = np.ones((2, 3, 6, 7, 5), np.float32)
    w = rnd(rng, (5, 3, 3, 2, 3))
    b = rnd(rng, 5)
    y = O.conv3d(x, w, b)
    expect = b.astype(np.float64) + w.astype(np.float64).reshape(5, -1).sum(1)
    np.testing.assert_allclose(y, np.broadcast_to(expect[None, :, None, None, None], y.shape), rtol=1e-14,
                               atol=1e-14)


def test_conv3d_kk1_equals_per_slice_conv2d():
    # a (k,k,1) Conv3d on x[N,C,H,W,D] is a Conv2d applied to every depth slice
    # (page l1_p59, the per-depth-slice equivalence and its permute/reshape recipe)
    rng = np.random.default_rng(5)
    N, C, H, Wd, D, Co = 2, 3, 12, 11, 5, 8
    x = rnd(rng, (N, C, H, Wd, D))
    w = rnd(rng, (Co, C, 3, 3, 1))
    y = O.conv3d(x, w, None)
    xp = t64(x).permute(0, 4, 1, 2, 3).reshape(N * D, C, H, Wd)
    y2 = F.conv2d(xp, t64(w).squeeze(-1))
    y2 = y2.view(N, D, Co, H - 2, Wd - 2).permute(0, 2, 3, 4, 1).numpy()
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)


def test_conv3d_linearity():
    rng = np.random.default_rng(6)
    x1, x2 = rnd(rng, (1, 2, 6, 6, 6)), rnd(rng, (1, 2, 6, 6, 6))
    w1, w2 = rnd(rng, (3, 2, 3, 3, 3)), rnd(rng, (3, 2, 3, 3, 3))
    a = lambda x, w: O.conv3d(x, w, None, (1, 2, 1), (1, 0, 2), (2, 1, 1))
    # x1+x2 is rounded to float32, so compare against the exact sum only loosely
    np.testing.assert_allclose(a(x1 + x2, w1), a(x1, w1) + a(x2, w1), atol=1e-6)
    np.testing.assert_allclose(a(x1, w1 + w2), a(x1, w1) + a(x1, w2), atol=1e-6)
    np.testing.assert_allclose(a(2 * x1, w1), 2 * a(x1, w1), rtol=1e-14, atol=1e-14)


def test_conv3d_at_matches_full():
    rng = np.random.default_rng(7)
    x = rnd(rng, (2, 4, 7, 8, 6))
    w = rnd(rng, (6, 2, 3, 2, 3))
    b = rnd(rng, 6)
    kw = dict(stride=(1, 2, 1), pad=(1, 1, 2), dilation=(2, 1, 1), groups=2)
    y = O.conv3d(x, w, b, **kw)
    flat = np.arange(y.size)
    np.testing.assert_array_equal(O.conv3d_at(x, w, flat, b, **kw), y.ravel())


# --------------------------------------------------- conv_transpose3d
def _rand_convT_case(rng):
    while True:
        wl = W.random_small_workload("conv_transpose3d", rng, max_spatial=7)
        if all(v > 0 for v in O.output_shape(wl)):
            return wl


@pytest.mark.parametrize("seed", range(24))
def test_convT_matches_torch_float64(seed):
    rng = np.random.default_rng(200 + seed)
    wl = _rand_convT_case(rng)
    inp = W.make_inputs(wl)
    y = O.conv_transpose3d(inp.x, inp.w, inp.b, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
    yt = F.conv_transpose3d(t64(inp.x), t64(inp.w), t64(inp.b), wl.stride, wl.pad, wl.output_pad, wl.groups,
                            wl.dilation).numpy()
    assert y.shape == yt.shape
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(8))
def test_convT_gather_equals_scatter(seed):
    rng = np.random.default_rng(300 + seed)
    wl = _rand_convT_case(rng)
    inp = W.make_inputs(wl)
    kw = dict(stride=wl.stride, pad=wl.pad, dilation=wl.dilation, output_pad=wl.output_pad, groups=wl.groups)
    y = O.conv_transpose3d(inp.x, inp.w, inp.b, **kw)
    g = O.conv_transpose3d_at(inp.x, inp.w, np.arange(y.size), inp.b, **kw)
    np.testing.assert_allclose(g, y.ravel(), rtol=1e-13, atol=1e-13)


def _taps_1d(L_in, k, s, p, d):
    """(input index, tap) pairs reaching each output index, read off the oracle by
    impulse responses: x = e_i, W = e_k."""
    L_out = O.convT_out_len(L_in, k, s, p, d, 0)
    taps = {o: [] for o in range(L_out)}
    for i in range(L_in):
        for kk in range(k):
            x = np.zeros((1, 1, 1, 1, L_in), np.float32)
            x[0, 0, 0, 0, i] = 1
            w = np.zeros((1, 1, 1, 1, k), np.float32)
            w[0, 0, 0, 0, kk] = 1
            y = O.conv_transpose3d(x, w, None, (1, 1, s), (0, 0, p), (1, 1, d))
            for o in np.nonzero(y[0, 0, 0, 0])[0]:
                taps[int(o)].append([i, kk])
    return L_out, taps


def test_convT_taps_page_l2_p72_worked_example():
    g = golden("convT_taps_p72.json")
    L_out, taps = _taps_1d(g["L_in"], g["k"], g["s"], g["p"], g["d"])
    assert L_out == g["L_out"]
    for o, pairs in g["taps"].items():
        assert sorted(taps[int(o)]) == sorted(pairs)


def test_convT_taps_page_l1_p77_worked_example():
    g = golden("convT_taps_p77.json")
    L_out, taps = _taps_1d(g["L_in"], g["k"], g["s"], g["p"], g["d"])
    assert L_out == g["L_out"]
    for o, pairs in g["taps_prefix"].items():
        assert sorted(taps[int(o)]) == sorted(pairs)
    if g["even_outputs_receive_nothing"]:
        assert all(not taps[o] for o in range(0, L_out, 2))
    assert sum(len(v) for v in taps.values()) == g["valid_pairs"]


def _valid_pairs(L_in, k, s, p, d, L_out):
    return sum(1 for i in range(L_in) for kk in range(k) if 0 <= i * s - p + kk * d < L_out)


def test_convT_valid_pair_counts_by_ones():
    # sum of a 1-D transposed conv of ones with unit taps = number of (i,k) pairs that
    # land inside the output; compared with direct enumeration
    for (L, k, s, p, d) in [(16, 3, 2, 1, 2), (32, 3, 2, 1, 2), (32, 3, 2, 1, 1), (7, 4, 3, 2, 2)]:
        L_out = O.convT_out_len(L, k, s, p, d, 0)
        y = O.conv_transpose3d(np.ones((1, 1, 1, 1, L), np.float32), np.ones((1, 1, 1, 1, k), np.float32),
                               None, (1, 1, s), (0, 0, p), (1, 1, d))
        assert y.sum() == _valid_pairs(L, k, s, p, d, L_out)
    assert _valid_pairs(16, 3, 2, 1, 2, 33) == 46
    assert _valid_pairs(32, 3, 2, 1, 2, 65) == 94


def test_convT_checkerboard_s2_p1_d2():
    # every output with any even coordinate is exactly the bias (page l1_p77, the
    # parity argument: 2*(di + kd) - 1 is always odd)
    rng = np.random.default_rng(8)
    x = rnd(rng, (2, 3, 6, 8, 8))
    w = rnd(rng, (3, 4, 3, 3, 3))
    b = rnd(rng, 4)
    y = O.conv_transpose3d(x, w, b, (2, 2, 2), (1, 1, 1), (2, 2, 2))
    assert y.shape == (2, 4, 13, 17, 17)
    mask = np.zeros(y.shape[2:], bool)
    mask[1::2, 1::2, 1::2] = True
    bb = np.broadcast_to(b.astype(np.float64)[None, :, None, None, None], y.shape)
    assert np.array_equal(y[..., ~mask], bb[..., ~mask])
    assert np.all(y[..., mask] != bb[..., mask])


def test_convT_sublattice_equals_stride1_conv():
    # s2 p1 d2 k3: y[:, :, 1::2, 1::2, 1::2] = conv3d(x, Wf, stride 1, pad 1) with
    # Wf[oc, ic, k] = W[ic, oc, 2 - k]; o = 2i - 1 + 2k is odd, o = 2q + 1 gives i = q + 1 - k
    rng = np.random.default_rng(9)
    x = rnd(rng, (2, 3, 5, 6, 7))
    w = rnd(rng, (3, 4, 3, 3, 3))
    y = O.conv_transpose3d(x, w, None, (2, 2, 2), (1, 1, 1), (2, 2, 2))
    wf = np.ascontiguousarray(w.transpose(1, 0, 2, 3, 4)[:, :, ::-1, ::-1, ::-1])
    yc = O.conv3d(x, wf, None, (1, 1, 1), (1, 1, 1), (1, 1, 1))
    np.testing.assert_allclose(y[:, :, 1::2, 1::2, 1::2], yc, rtol=1e-13, atol=1e-13)


def test_convT_stride1_is_flipped_conv():
    # ConvT(s=1, p, d) = conv(pad d(k-1) - p) with flipped, channel-transposed W
    rng = np.random.default_rng(10)
    for (k, p, d) in [(3, 1, 1), (3, 0, 2), (2, 1, 1), (3, 2, 2)]:
        x = rnd(rng, (1, 2, 5, 6, 4))
        w = rnd(rng, (2, 3, k, k, k))
        y = O.conv_transpose3d(x, w, None, (1, 1, 1), (p,) * 3, (d,) * 3)
        wf = np.ascontiguousarray(w.transpose(1, 0, 2, 3, 4)[:, :, ::-1, ::-1, ::-1])
        q = d * (k - 1) - p
        yc = O.conv3d(x, wf, None, (1, 1, 1), (q,) * 3, (d,) * 3)
        np.testing.assert_allclose(y, yc, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_adjoint_identity(seed):
    # <conv(x; W), y> = <x, convT(y; W)> with the same W, stride, padding, dilation
    # and groups; output_padding chosen so convT(y) has x's shape
    rng = np.random.default_rng(400 + seed)
    groups = int(rng.choice([1, 2]))
    cin, cout = 2 * groups, 3 * groups
    k = tuple(int(a) for a in rng.integers(1, 4, 3))
    s = tuple(int(a) for a in rng.integers(1, 4, 3))
    d = tuple(int(a) for a in rng.integers(1, 3, 3))
    p = tuple(int(a) for a in rng.integers(0, 2, 3))
    S = tuple(int(rng.integers(d[j] * (k[j] - 1) + 1, 11)) for j in range(3))
    x = rnd(rng, (2, cin) + S)
    w = rnd(rng, (cout, cin // groups) + k)
    yshape = O.conv3d_out_shape(x.shape, cout, k, s, p, d)
    yy = rnd(rng, yshape)
    op = tuple(S[j] - O.convT_out_len(yshape[2 + j], k[j], s[j], p[j], d[j], 0) for j in range(3))
    assert all(0 <= op[j] < max(s[j], d[j]) for j in range(3))
    lhs = float((O.conv3d(x, w, None, s, p, d, groups) * yy.astype(np.float64)).sum())
    xt = O.conv_transpose3d(yy, w, None, s, p, d, op, groups)
    assert xt.shape == x.shape
    rhs = float((x.astype(np.float64) * xt).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


# ------------------------------------------------------------ epilogues
def test_avgpool_twice_equals_avgpool4():
    # page l2_p72: AvgPool3d(2) applied twice is one AvgPool3d(4, stride 4), floor mode
    rng = np.random.default_rng(12)
    for S in [(8, 8, 8), (63, 9, 11), (7, 12, 5)]:
        y = rng.uniform(-1, 1, (2, 3) + S)
        a = O.avgpool3d(O.avgpool3d(y, 2), 2)
        b = O.avgpool3d(y, 4)
        assert a.shape == b.shape
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_avgpool_matches_torch_and_drops_tail():
    rng = np.random.default_rng(13)
    y = rng.uniform(-1, 1, (2, 3, 63, 10, 9))
    for w in (2, 3, 4):
        np.testing.assert_allclose(O.avgpool3d(y, w), F.avg_pool3d(torch.tensor(y), w).numpy(), rtol=1e-13,
                                   atol=1e-14)
    # the tail the floor mode drops does not matter (page l2_p72: indices 60, 61, 62)
    y2 = y.copy()
    y2[:, :, 60:63] = 1e6
    assert np.array_equal(O.avgpool3d(y, 4), O.avgpool3d(y2, 4))
    assert O.avgpool3d(y, 4).shape[2] == 15


def test_maxpool_matches_torch():
    rng = np.random.default_rng(14)
    y = rng.uniform(-1, 1, (2, 3, 9, 10, 7))
    for w in (2, 3):
        np.testing.assert_array_equal(O.maxpool3d(y, w), F.max_pool3d(torch.tensor(y), w).numpy())


def test_batchnorm_matches_torch_and_invariants():
    rng = np.random.default_rng(15)
    y = rng.normal(0.3, 2.0, (4, 5, 6, 7, 3))
    gamma = rnd(rng, 5, 0.5, 1.5)
    beta = rnd(rng, 5, -0.5, 0.5)
    z, mu, var = O.batchnorm_train(y, gamma, beta, 1e-5)
    zt = F.batch_norm(torch.tensor(y), None, None, t64(gamma), t64(beta), training=True, eps=1e-5).numpy()
    np.testing.assert_allclose(z, zt, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mu, y.mean(axis=(0, 2, 3, 4)), rtol=1e-13)
    np.testing.assert_allclose(var, y.var(axis=(0, 2, 3, 4)), rtol=1e-12)
    # mean(z) = beta; biased var(z) = gamma^2 var / (var + eps)
    np.testing.assert_allclose(z.mean(axis=(0, 2, 3, 4)), beta, atol=1e-10)
    np.testing.assert_allclose(z.var(axis=(0, 2, 3, 4)), gamma.astype(np.float64) ** 2 * var / (var + 1e-5),
                               rtol=1e-10)
    # gamma = 0 gives beta exactly
    z0, _, _ = O.batchnorm_train(y, np.zeros(5, np.float32), beta)
    assert np.array_equal(z0, np.broadcast_to(beta.astype(np.float64)[None, :, None, None, None], y.shape))


def test_batchnorm_commutes_with_avgpool():
    # BN is a per-channel affine map and average pooling is linear, so
    # avgpool(BN(y)) = BN_affine(avgpool(y)) with the statistics of the unpooled y
    rng = np.random.default_rng(16)
    y = rng.uniform(-1, 1, (3, 2, 9, 8, 10))
    gamma, beta = rnd(rng, 2, 0.5, 1.5), rnd(rng, 2, -0.5, 0.5)
    z, mu, var = O.batchnorm_train(y, gamma, beta)
    a = O.avgpool3d(z, 2)
    pooled = O.avgpool3d(y, 2)
    b = (gamma[None, :, None, None, None] * (pooled - mu[None, :, None, None, None]) /
         np.sqrt(var[None, :, None, None, None] + 1e-5) + beta[None, :, None, None, None])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_logsumexp_page_examples():
    g = golden("lse_examples.json")
    for c in g["cases"]:
        v = np.array(c["values"], np.float64).reshape(1, -1, 1)
        got = O.logsumexp_channels(v)[0, 0, 0]
        assert abs(got - c["expected"]) <= c["tol"], (c, got)


def test_logsumexp_closed_forms_and_bounds():
    rng = np.random.default_rng(17)
    # C equal values v give v + ln C
    for C in (1, 2, 64):
        v = np.full((1, C, 3), -3.25)
        np.testing.assert_allclose(O.logsumexp_channels(v)[0, 0], -3.25 + math.log(C), rtol=1e-15)
    # max_c v <= lse <= max_c v + ln C, and torch agreement
    v = rng.normal(0, 5, (4, 64, 50))
    lse = O.logsumexp_channels(v)[:, 0]
    mx = v.max(axis=1)
    assert np.all(lse >= mx) and np.all(lse <= mx + math.log(64) + 1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(torch.tensor(v), dim=1).numpy(), rtol=1e-14, atol=1e-13)
    # large magnitudes do not overflow
    big = np.array([[[1000.0], [999.0]]])
    np.testing.assert_allclose(O.logsumexp_channels(big)[0, 0, 0], 1000 + math.log1p(math.exp(-1)), rtol=1e-15)


def test_relu():
    v = np.array([-2.0, -0.0, 0.0, 1e-30, 3.5])
    r = O.relu(v)
    assert list(r) == [0.0, 0.0, 0.0, 1e-30, 3.5]


# -------------------------------------------------------- fused modules
def _torch_convT_bn_pool(inp, wl):
    y = F.conv_transpose3d(t64(inp.x), t64(inp.w), t64(inp.b), wl.stride, wl.pad, wl.output_pad, wl.groups,
                           wl.dilation)
    mean = y.mean(dim=(0, 2, 3, 4))
    var = y.var(dim=(0, 2, 3, 4), unbiased=False)
    z = F.batch_norm(y, None, None, t64(inp.gamma), t64(inp.beta), training=True, eps=wl.eps)
    # the module's two AvgPool3d(2) stages when pool == 4
    if wl.pool == 4:
        out = F.avg_pool3d(F.avg_pool3d(z, 2), 2)
    else:
        out = F.avg_pool3d(z, wl.pool)
    return out.numpy(), mean.numpy(), var.numpy()


@pytest.mark.parametrize("case", [
    dict(x_shape=(4, 3, 8, 8, 8), cout=16, pool=4),
    dict(x_shape=(3, 2, 7, 9, 8), cout=5, pool=4, kernel=(3, 2, 3), stride=(2, 3, 2), pad=(1, 0, 1)),
    dict(x_shape=(2, 4, 6, 6, 6), cout=4, pool=2, groups=2, dilation=(2, 1, 1)),
    dict(x_shape=(2, 3, 5, 5, 5), cout=6, pool=3, output_pad=(1, 0, 1)),
])
def test_convT_bn_avgpool_matches_torch_module(case):
    wl = W.CONFIGS["c4"].with_(**case)
    inp = W.make_inputs(wl)
    out, mean, var = O.run_workload(wl, inp)
    ot, mt, vt = _torch_convT_bn_pool(inp, wl)
    assert out.shape == ot.shape
    np.testing.assert_allclose(out, ot, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(mean, mt, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(var, vt, rtol=1e-11)


# --------------------------------------------- eval mode, running statistics
EVAL_CASES = [
    dict(x_shape=(3, 3, 8, 8, 8), cout=16, pool=4),
    dict(x_shape=(2, 2, 7, 9, 8), cout=5, pool=2, kernel=(3, 2, 3), stride=(2, 3, 2), pad=(1, 0, 1)),
    dict(x_shape=(2, 4, 6, 6, 6), cout=4, pool=3, groups=2, dilation=(2, 1, 1), output_pad=(1, 0, 0)),
]


@pytest.mark.parametrize("case", EVAL_CASES)
def test_convT_bn_eval_avgpool_matches_torch_module(case):
    """Eval-mode BatchNorm3d ([p72]'s shipped variant) against PyTorch's
    batch_norm with running statistics, in float64, then the pool."""
    wl = W.CONFIGS["c4"].with_(**case)
    inp = W.make_inputs(wl)
    rm, rv = W.make_running_stats(wl.cout, 7)
    out = O.convT_bn_eval_avgpool(inp.x, inp.w, inp.b, inp.gamma, inp.beta, rm, rv, wl.eps, wl.pool, wl.stride,
                                  wl.pad, wl.dilation, wl.output_pad, wl.groups)
    y = F.conv_transpose3d(t64(inp.x), t64(inp.w), t64(inp.b), wl.stride, wl.pad, wl.output_pad, wl.groups,
                           wl.dilation)
    z = F.batch_norm(y, t64(rm), t64(rv), t64(inp.gamma), t64(inp.beta), training=False, eps=wl.eps)
    ref = F.avg_pool3d(z, wl.pool).numpy()
    assert out.shape == ref.shape
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)


def test_convT_bn_eval_with_batch_statistics_equals_training_mode():
    """Eval mode fed the batch's own mean and biased variance normalises exactly
    as training mode does (up to the float32 cast of the statistics)."""
    wl = W.CONFIGS["c4"].with_(x_shape=(3, 3, 8, 8, 8))
    inp = W.make_inputs(wl)
    out_t, mean, var = O.run_workload(wl, inp)
    out_e = O.convT_bn_eval_avgpool(inp.x, inp.w, inp.b, inp.gamma, inp.beta, mean.astype(np.float32),
                                    var.astype(np.float32), wl.eps, wl.pool, wl.stride, wl.pad, wl.dilation,
                                    wl.output_pad, wl.groups)
    np.testing.assert_allclose(out_e, out_t, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("momentum", [0.1, 0.3])
def test_bn_running_update_matches_torch_module(momentum):
    """One training-mode forward of torch.nn.BatchNorm3d (float64) updates the
    running statistics exactly as the oracle does: the unbiased batch
    variance, blended with the momentum ([p72]'s 0.1)."""
    wl = W.CONFIGS["c4"].with_(x_shape=(2, 3, 6, 7, 5), cout=6)
    inp = W.make_inputs(wl)
    rm, rv = W.make_running_stats(wl.cout, 11)
    _, mean, var = O.run_workload(wl, inp)
    y = F.conv_transpose3d(t64(inp.x), t64(inp.w), t64(inp.b), wl.stride, wl.pad, wl.output_pad, wl.groups,
                           wl.dilation)
    bn = torch.nn.BatchNorm3d(wl.cout, eps=wl.eps, momentum=momentum, dtype=torch.float64)
    with torch.no_grad():
        bn.running_mean.copy_(t64(rm))
        bn.running_var.copy_(t64(rv))
    bn.train()
    bn(y)
    count = y.numel() // wl.cout
    nrm, nrv = O.bn_running_update(rm, rv, mean, var, count, momentum)
    np.testing.assert_allclose(nrm, bn.running_mean.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(nrv, bn.running_var.numpy(), rtol=1e-12, atol=1e-14)


def test_bn_running_update_closed_forms():
    rng = np.random.default_rng(5)
    rm, rv = rng.uniform(-1, 1, 4), rng.uniform(0.5, 2, 4)
    bm, bv = rng.uniform(-1, 1, 4), rng.uniform(0.1, 3, 4)
    a, b = O.bn_running_update(rm, rv, bm, bv, 10, 0.0)   # momentum 0: unchanged
    assert np.array_equal(a, rm) and np.array_equal(b, rv)
    a, b = O.bn_running_update(rm, rv, bm, bv, 10, 1.0)   # momentum 1: the batch's own statistics
    np.testing.assert_allclose(a, bm, rtol=1e-15)
    np.testing.assert_allclose(b, bv * 10 / 9, rtol=1e-15)


def test_convT_bn_avgpool_bias_cancels_and_gamma_zero():
    wl = W.CONFIGS["c4"].with_(x_shape=(3, 3, 8, 8, 8))
    inp = W.make_inputs(wl)
    out, mean, _ = O.run_workload(wl, inp)
    inp0 = W.Inputs(inp.x, inp.w, np.zeros_like(inp.b), inp.gamma, inp.beta)
    out0, mean0, _ = O.run_workload(wl, inp0)
    np.testing.assert_allclose(out, out0, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(mean - mean0, inp.b.astype(np.float64), rtol=1e-10, atol=1e-12)
    inpg = W.Inputs(inp.x, inp.w, inp.b, np.zeros_like(inp.gamma), inp.beta)
    outg, _, _ = O.run_workload(wl, inpg)
    assert np.array_equal(outg, np.broadcast_to(inp.beta.astype(np.float64)[None, :, None, None, None],
                                                outg.shape))


def test_convT_pool_counts_page_l2_p72():
    # with x = 1, W = 1, no bias, one input channel: the ConvT output at a position is
    # its number of valid taps; an interior 4x4x4 window holds 8*81/3 = 216 per input
    # channel (page l2_p72: 648 MAC per pooled output over 3 input channels), so the
    # pooled mean is 648/64 = 10.125 over the page's 3 channels
    g = golden("c4_counts.json")
    L = g["L_in"]
    x = np.ones((1, g["Cin"], L, L, L), np.float32)
    w = np.ones((g["Cin"], 1, 3, 3, 3), np.float32)
    y = O.conv_transpose3d(x, w, None, (2, 2, 2), (1, 1, 1), (1, 1, 1))
    assert y.shape[2:] == (g["convT_len"],) * 3
    pooled = O.avgpool3d(y, 4)
    assert pooled.shape[2:] == (g["pooled_len"],) * 3
    interior = pooled[0, 0, 1:-1, 1:-1, 1:-1]
    assert np.all(interior * g["window_positions"] == g["interior_macs_per_pooled_output"])
    # total valid MACs of the full C4 module: N*Cout*Cin*prod(valid pairs per dim)
    vp = _valid_pairs(L, 3, 2, 1, 1, g["convT_len"])
    assert vp == 3 * L - 2
    assert y.sum() == g["Cin"] * vp ** 3


def _torch_conv_pool_lse_relu(inp, wl):
    y = F.conv3d(t64(inp.x), t64(inp.w), t64(inp.b), wl.stride, wl.pad, wl.dilation, wl.groups)
    m = F.max_pool3d(y, wl.pool)
    return torch.relu(torch.logsumexp(m, dim=1, keepdim=True)).numpy()


@pytest.mark.parametrize("case", [
    dict(x_shape=(2, 4, 8, 8, 8), cout=8),
    dict(x_shape=(1, 3, 9, 7, 10), cout=5, pool=3),
    dict(x_shape=(2, 4, 6, 6, 6), cout=6, groups=2, stride=(1, 2, 1), dilation=(1, 1, 2), pad=(1, 2, 2)),
])
def test_conv_maxpool_lse_relu_matches_torch_module(case):
    wl = W.CONFIGS["c5"].with_(**case)
    inp = W.make_inputs(wl)
    out = O.run_workload(wl, inp)
    ot = _torch_conv_pool_lse_relu(inp, wl)
    assert out.shape == ot.shape
    np.testing.assert_allclose(out, ot, rtol=1e-12, atol=1e-12)
    flat = np.arange(out.size)
    at = O.conv_maxpool_lse_relu_at(inp.x, inp.w, inp.b, flat, wl.pool, wl.stride, wl.pad, wl.dilation,
                                    wl.groups)
    np.testing.assert_allclose(at, out.ravel(), rtol=1e-14, atol=1e-14)


def test_conv_maxpool_lse_relu_bounds():
    # out = max(L, 0) with max_c m_c <= L <= max_c m_c + ln C
    wl = W.CONFIGS["c5"].with_(x_shape=(1, 4, 6, 8, 8), cout=16)
    inp = W.make_inputs(wl)
    out = O.run_workload(wl, inp)
    y = O.conv3d(inp.x, inp.w, inp.b, wl.stride, wl.pad, wl.dilation)
    mx = O.maxpool3d(y, 2).max(axis=1, keepdims=True)
    assert np.all(out >= np.maximum(mx, 0) - 1e-15)
    assert np.all(out <= np.maximum(mx + math.log(16), 0) + 1e-15)
    assert np.all(out >= 0)


# ------------------------------------------------------ workload sizes
def test_workload_output_shapes():
    assert O.output_shape(W.CONFIGS["c1"]) == (1, 8, 8, 8, 8)
    assert O.output_shape(W.CONFIGS["c2"]) == (16, 64, 254, 254, 10)
    # the stated input D=16, H=W=32 and the size formula give 33 x 65 x 65
    assert O.output_shape(W.CONFIGS["c3"]) == (16, 64, 33, 65, 65)
    assert O.output_shape(W.CONFIGS["c4"]) == (64, 16, 15, 15, 15)
    assert O.output_shape(W.CONFIGS["c5"]) == (4, 1, 16, 64, 64)
