"""GPU parity: every entry point of the C ABI against the CPU oracle, on the
same seeded inputs, element by element, at |gpu - ref| <= 1e-4 + 1e-4 |ref|
(fp32 with inputs in [-1, 1]).

Small and medium shapes (several tiles and a ragged tail) are compared in
full; the five workload configurations run at full size in the same launch
configuration the benchmark uses, compared on sampled outputs the oracle
evaluates one by one, plus properties that hold on every output.  Outputs
are poisoned with NaN first, so an unwritten element fails.  Both the
automatic kernel choice and the forced generic kernels are exercised.
"""
import numpy as np
import pytest
import torch

import oracle as O
from transposed_convolution_epilogues_amd import binding as B
from transposed_convolution_epilogues_amd import workloads as W

pytestmark = pytest.mark.gpu

ATOL = 1e-4
RTOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.library()
    yield
    B.set_variant(0)


@pytest.fixture(params=[0, 1], ids=["auto", "generic"])
def variant(request):
    old = B.set_variant(request.param)
    yield request.param
    B.set_variant(old)


@pytest.fixture(params=[0, 1, 3, 5], ids=["swapped_sums", "generic", "matrix_cores", "per_cell"])
def bn_variant(request):
    """Kernel choices of the c4 module: swapped sums (default), generic, output-phase
    classes on the matrix cores (the second algorithm), per-cell."""
    old = B.set_variant(request.param)
    yield request.param
    B.set_variant(old)


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def poisoned(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def assert_close(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= ATOL + RTOL * np.abs(ref))  # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} outside tolerance; first {idx.tolist()} "
                             f"got {got[bad][:5]} ref {ref[bad][:5]}")


def run_gpu(wl, inp, out=None, ws=None, stats=False):
    kw = dict(stride=wl.stride, pad=wl.pad, dilation=wl.dilation, groups=wl.groups)
    x, w, b = dev(inp.x), dev(inp.w), dev(inp.b)
    shape = O.output_shape(wl)
    out = poisoned(shape) if out is None else out
    if wl.op == "conv3d":
        return B.conv3d_fwd(x, w, b, out=out, **kw)
    if wl.op == "conv_transpose3d":
        return B.conv_transpose3d_fwd(x, w, b, output_pad=wl.output_pad, out=out, **kw)
    if wl.op == "convT_bn_avgpool":
        mean = poisoned((wl.cout,))
        var = poisoned((wl.cout,))
        y = B.convT_bn_avgpool(x, w, b, dev(inp.gamma), dev(inp.beta), wl.eps, wl.pool, output_pad=wl.output_pad,
                               out=out, workspace=ws, batch_mean=mean, batch_var=var, **kw)
        return (y, mean, var) if stats else y
    return B.conv_maxpool_lse_relu(x, w, b, wl.pool, out=out, **kw)


def check_full(wl, inp, name):
    ref = O.run_workload(wl, inp)
    if wl.op == "convT_bn_avgpool":
        y, mean, var = run_gpu(wl, inp, stats=True)
        torch.cuda.synchronize()
        assert_close(name + " out", y.cpu().numpy(), ref[0])
        assert_close(name + " mean", mean.cpu().numpy(), ref[1])
        assert_close(name + " var", var.cpu().numpy(), ref[2])
        return y
    y = run_gpu(wl, inp)
    torch.cuda.synchronize()
    assert_close(name, y.cpu().numpy(), ref)
    return y


# ------------------------------------------------------- random small sweep
def _valid(wl):
    try:
        shape = O.output_shape(wl)
    except Exception:
        return False
    return all(v > 0 for v in shape)


def _random_cases(op, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        base = "conv3d" if op in ("conv3d", "conv_maxpool_lse_relu") else "conv_transpose3d"
        wl = W.random_small_workload(base, rng, max_spatial=9)
        if op == "convT_bn_avgpool":
            wl = wl.with_(op=op, pool=int(rng.integers(1, 4)))
        elif op == "conv_maxpool_lse_relu":
            wl = wl.with_(op=op, pool=int(rng.integers(1, 3)))
        if _valid(wl):
            out.append(wl)
    return out


@pytest.mark.parametrize("op", ["conv3d", "conv_transpose3d", "convT_bn_avgpool", "conv_maxpool_lse_relu"])
def test_random_small_shapes(op, variant):
    for i, wl in enumerate(_random_cases(op, 25, {"conv3d": 1, "conv_transpose3d": 2, "convT_bn_avgpool": 3,
                                                  "conv_maxpool_lse_relu": 4}[op])):
        inp = W.make_inputs(wl)
        print(f"[{op} v{variant}] case {i}: {wl}", flush=True)
        check_full(wl, inp, f"{op}#{i}")


# ------------------------------------- transposed conv, per-phase MFMA path
def _phase_cases(n, seed):
    """Random transposed convs that take a phase kernel (the shared-halo one
    or the per-phase one): strides 1..4, kernels 1..5, dilation 1..3, output
    padding, groups 1/2."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        groups = int(rng.choice([1, 2]))
        wl = W.make("phase", "conv_transpose3d",
                    (int(rng.integers(1, 3)), groups * int(rng.integers(4, 13))) +
                    tuple(int(a) for a in rng.integers(1, 10, size=3)),
                    groups * int(rng.integers(8, 41)), tuple(int(a) for a in rng.integers(1, 6, size=3)),
                    tuple(int(a) for a in rng.integers(1, 5, size=3)), tuple(int(a) for a in rng.integers(0, 4, size=3)),
                    tuple(int(a) for a in rng.integers(1, 4, size=3)), (0, 0, 0), groups, bool(rng.integers(0, 2)),
                    seed=int(rng.integers(0, 2**31)))
        wl = wl.with_(output_pad=tuple(int(rng.integers(0, max(si, di))) for si, di in zip(wl.stride, wl.dilation)))
        if not _valid(wl):
            continue
        if B.conv_transpose3d_algo(wl.x_shape, wl.cout, B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation,
                                                                      wl.output_pad, wl.groups)) not in PHASE_ALGOS:
            continue
        out.append(wl)
    return out


PHASE_ALGOS = ("phase_group", "phase")
# variant 0 takes the shared-halo kernel where it applies; variant 6 the
# one-phase-per-workgroup kernel
PHASE_VARIANTS = {"shared_halo": 0, "per_phase": 6}


@pytest.mark.parametrize("pv", list(PHASE_VARIANTS))
def test_convT_phase_random(pv):
    cases = _phase_cases(30, 71)
    old = B.set_variant(PHASE_VARIANTS[pv])
    try:
        seen = set()
        for i, wl in enumerate(cases):
            p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
            algo = B.conv_transpose3d_algo(wl.x_shape, wl.cout, p)
            assert algo in PHASE_ALGOS, algo
            seen.add(algo)
            print(f"[convT phase {pv} {algo}] case {i}: {wl}", flush=True)
            check_full(wl, W.make_inputs(wl), f"convT phase #{i}")
        assert seen == ({"phase"} if pv == "per_phase" else {"phase_group", "phase"}), seen
    finally:
        B.set_variant(old)


PHASE_MEDIUM = {
    # dense phases (every residue has taps), ragged tiles in every dim
    "k3s2p1d1_op1": W.make("pm", "conv_transpose3d", (2, 16, 5, 9, 37), 40, 3, 2, 1, 1, 1, seed=81),
    "k4s2p1": W.make("pm", "conv_transpose3d", (1, 12, 4, 7, 33), 24, 4, 2, 1, seed=82),
    "k3s3p1_op2_groups2": W.make("pm", "conv_transpose3d", (2, 16, 3, 5, 13), 32, 3, 3, 1, 1, 2, groups=2,
                                 bias=True, seed=83),
    "k3s1p1": W.make("pm", "conv_transpose3d", (1, 8, 4, 6, 40), 16, 3, 1, 1, bias=True, seed=84),
    "mixed": W.make("pm", "conv_transpose3d", (1, 10, 5, 6, 20), 72, (3, 2, 5), (2, 1, 3), (1, 0, 2), (1, 2, 1),
                    (1, 0, 0), bias=True, seed=85),
    # the stride-2 dilation-2 module of the transposed-conv workload, reduced
    "k3s2p1d2": W.CONFIGS["c3"].with_(x_shape=(2, 32, 5, 7, 19)),
    # kernel = stride with more than 8 phases and 9-16 input channels per group:
    # one tap per phase, every input channel staged once, 3 or 4 phases per group
    # (dim-2 residues in one 12-, 16- or 8-byte store, or float by float); the
    # first and last take 3 and 2 phase groups per workgroup with two sets of
    # accumulators, one group's stores between the next group's products
    "k3s3_one_tap_groups2": W.make("pm", "conv_transpose3d", (8, 32, 6, 9, 13), 64, 3, 3, 1, 1, 2, groups=2,
                                   bias=True, seed=88),
    "k4s4_one_tap": W.make("pm", "conv_transpose3d", (1, 8, 3, 4, 6), 16, 4, 4, (1, 2, 3), 1, (0, 1, 3),
                           bias=True, seed=89),
    "k322s322_one_tap": W.make("pm", "conv_transpose3d", (1, 10, 4, 5, 7), 24, (3, 2, 2), (3, 2, 2), (1, 0, 1), 1,
                               (2, 1, 0), bias=True, seed=90),
    "k4s4_one_tap_quads": W.make("pm", "conv_transpose3d", (8, 8, 5, 6, 5), 32, 4, 4, (1, 2, 0), 1, (3, 1, 0),
                                 bias=True, seed=91),
    # two full 32-channel blocks on the two-accumulator path
    "k3s3_one_tap_two_blocks": W.make("pm", "conv_transpose3d", (2, 16, 3, 4, 10), 64, 3, 3, 1, 1, (1, 2, 2),
                                      bias=True, seed=92),
}


@pytest.mark.parametrize("pv", list(PHASE_VARIANTS))
@pytest.mark.parametrize("name", list(PHASE_MEDIUM))
def test_convT_phase_medium(name, pv):
    """Both phase kernels on multi-tile shapes; variant 2 makes the stride-2
    dilation-2 case take the shared-halo kernel instead of the sub-lattice
    one, variant 6 the per-phase kernel."""
    wl = PHASE_MEDIUM[name]
    old = B.set_variant(2 if pv == "shared_halo" else 6)
    try:
        algo = B.conv_transpose3d_algo(wl.x_shape, wl.cout, B.make_params(wl.kernel, wl.stride, wl.pad,
                                                                           wl.dilation, wl.output_pad, wl.groups))
        assert algo == ("phase_group" if pv == "shared_halo" else "phase"), algo
        print(f"[convT phase medium {name}] {wl}", flush=True)
        check_full(wl, W.make_inputs(wl), name)
    finally:
        B.set_variant(old)


UNALIGNED_Y = {
    # the residues of dim 2 leave in one 8-, 16- or 12-byte store per lane when y allows it
    "pairs": W.make("pu", "conv_transpose3d", (1, 8, 3, 5, 20), 40, 3, 2, 1, 1, 1, bias=True, seed=86),
    "quads": W.make("pu", "conv_transpose3d", (1, 8, 3, 4, 9), 16, (3, 3, 4), (1, 2, 4), (1, 1, 0), bias=True,
                    seed=87),
    "triples": PHASE_MEDIUM["k3s3p1_op2_groups2"],
    "triples_one_tap": PHASE_MEDIUM["k3s3_one_tap_groups2"],
    "quads_one_tap": PHASE_MEDIUM["k4s4_one_tap_quads"],
}


@pytest.mark.parametrize("name", list(UNALIGNED_Y))
def test_convT_phase_group_unaligned_output(name):
    """y 4 bytes off a 16-byte boundary: the shared-halo kernel falls back to
    single-float stores where its packed stores need 8 or 16 bytes."""
    wl = UNALIGNED_Y[name]
    p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
    assert B.conv_transpose3d_algo(wl.x_shape, wl.cout, p) == "phase_group"
    inp = W.make_inputs(wl)
    ref = O.run_workload(wl, inp)
    flat = torch.full((int(np.prod(ref.shape)) + 1,), float("nan"), dtype=torch.float32, device="cuda")
    y = flat[1:].view(ref.shape)
    assert y.data_ptr() % 16 == 4
    print(f"[convT unaligned y {name}] {wl}", flush=True)
    B.conv_transpose3d_fwd(dev(inp.x), dev(inp.w), dev(inp.b), wl.stride, wl.pad, wl.dilation, wl.output_pad,
                           wl.groups, out=y)
    torch.cuda.synchronize()
    assert torch.isnan(flat[0]).item()  # nothing written before y
    assert_close(f"unaligned y {name}", y.cpu().numpy(), ref)


@pytest.mark.parametrize("pv", list(PHASE_VARIANTS))
@pytest.mark.parametrize("key", list(W.WIDEN))
def test_convT_widen_full_size_sampled(key, pv):
    """The transposed convs `bench.py --widen` times, at full size through
    both phase kernels, on sampled outputs."""
    wl = W.WIDEN[key]
    p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
    old = B.set_variant(PHASE_VARIANTS[pv])
    try:
        assert B.conv_transpose3d_algo(wl.x_shape, wl.cout, p) == ("phase_group" if pv == "shared_halo" else "phase")
        _widen_sampled(key, wl)
    finally:
        B.set_variant(old)


def _widen_sampled(key, wl):
    inp = W.make_inputs(wl)
    print(f"[convT widen {key}] {wl}", flush=True)
    y = run_gpu(wl, inp)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item()
    flat = np.concatenate([_sample(y.numel(), 40_000, 91), np.arange(0, 300), y.numel() - 1 - np.arange(300)])
    got = y.view(-1)[torch.from_numpy(flat).cuda()].cpu().numpy()
    ref = O.conv_transpose3d_at(inp.x, inp.w, flat, inp.b, wl.stride, wl.pad, wl.dilation, wl.output_pad,
                                wl.groups)
    assert_close(f"widen {key} sampled", got, ref)
    y2 = run_gpu(wl, inp)
    assert torch.equal(y, y2)


# ------------------------------ transposed conv, LDS scatter (second algorithm)
def test_convT_scatter_random():
    cases = _random_cases("conv_transpose3d", 20, 12) + _phase_cases(10, 13)  # drawn under the default variant
    old = B.set_variant(4)
    try:
        for i, wl in enumerate(cases):
            p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
            assert B.conv_transpose3d_algo(wl.x_shape, wl.cout, p) == "scatter"
            print(f"[convT scatter] case {i}: {wl}", flush=True)
            check_full(wl, W.make_inputs(wl), f"convT scatter #{i}")
    finally:
        B.set_variant(old)


@pytest.mark.parametrize("name", list(PHASE_MEDIUM) + ["convT_s2p1d2_cout80", "convT_s2p1d2_bias"])
def test_convT_scatter_medium(name):
    wl = PHASE_MEDIUM.get(name) or MEDIUM[name]
    old = B.set_variant(4)
    try:
        print(f"[convT scatter medium {name}] {wl}", flush=True)
        check_full(wl, W.make_inputs(wl), name)
    finally:
        B.set_variant(old)


# ----------------------------------------------- medium shapes (many tiles)
MEDIUM = {
    # the fast paths' shapes, reduced so the oracle finishes in seconds, with ragged tails
    "conv3d_k333": W.CONFIGS["c1"].with_(x_shape=(2, 32, 5, 11, 37), cout=64),
    "conv3d_k333_cin20": W.CONFIGS["c1"].with_(x_shape=(1, 20, 4, 9, 70), cout=40),
    "conv3d_k331_depthlast": W.CONFIGS["c2"].with_(x_shape=(2, 3, 19, 37, 10)),
    "conv3d_k331_depthlast_d7": W.CONFIGS["c2"].with_(x_shape=(1, 3, 9, 40, 7), cout=48),
    "convT_s2p1d2": W.CONFIGS["c3"].with_(x_shape=(2, 32, 5, 7, 19)),
    "convT_s2p1d2_small_c": W.CONFIGS["c3"].with_(x_shape=(1, 12, 4, 6, 9), cout=24),
    "convT_bn_pool": W.CONFIGS["c4"].with_(x_shape=(3, 3, 14, 13, 18)),
    "convT_bn_pool_exact": W.CONFIGS["c4"].with_(x_shape=(2, 3, 16, 16, 16)),
    "conv_pool_lse": W.CONFIGS["c5"].with_(x_shape=(1, 32, 6, 18, 70)),
    "conv_pool_lse_odd": W.CONFIGS["c5"].with_(x_shape=(2, 32, 5, 9, 35), cout=64),
    "conv_pool_lse_cout40_pad0": W.CONFIGS["c5"].with_(x_shape=(1, 16, 6, 10, 12), cout=40, pad=0),
    "conv3d_k333_cout72_pad0": W.CONFIGS["c1"].with_(x_shape=(1, 8, 4, 6, 9), cout=72, pad=0),
    "conv3d_k333_pad2": W.CONFIGS["c1"].with_(x_shape=(1, 9, 3, 5, 33), cout=16, pad=2),
    "convT_s2p1d2_cout80": W.CONFIGS["c3"].with_(x_shape=(1, 8, 3, 5, 6), cout=80),
    "convT_s2p1d2_bias": W.CONFIGS["c3"].with_(x_shape=(2, 5, 3, 4, 33), cout=16, bias=True),
    "convT_s2p1d2_bias_cout72": W.CONFIGS["c3"].with_(x_shape=(3, 6, 3, 3, 5), cout=72, bias=True),
    # enough tiles per (sample, channel) volume that each K-loop unit's share of the bias-only planes is at
    # most 3 plane pairs: the fixed-count form of that pass (c3's own); 8 tiles x 12 units for 64 x 3 pairs
    "convT_s2p1d2_fixed_run": W.CONFIGS["c3"].with_(x_shape=(1, 32, 2, 16, 64)),
    # the same with bias, 40 channels, partial tiles in two dims: 24 workgroups x 6 units for 2 x 40 x 4 pairs
    "convT_s2p1d2_fixed_run_bias": W.CONFIGS["c3"].with_(x_shape=(2, 16, 3, 13, 70), cout=40, bias=True),
    "conv3d_k331_bias_dil": W.CONFIGS["c2"].with_(x_shape=(1, 2, 9, 12, 5), cout=20, dilation=(2, 2, 1),
                                                  bias=True),
    # rows of O1*S2 floats with O1*S2 % 4 == 0 and 64 channels: the float4 store path, with a partial
    # last chunk per row, bias and dilation, and a row shorter than one chunk
    "conv3d_k331_rows_2chunks": W.CONFIGS["c2"].with_(x_shape=(2, 3, 9, 30, 10)),
    "conv3d_k331_rows_bias_dil": W.CONFIGS["c2"].with_(x_shape=(1, 3, 7, 25, 12), dilation=(2, 2, 1), bias=True),
    "conv3d_k331_rows_short": W.CONFIGS["c2"].with_(x_shape=(1, 3, 5, 8, 8)),
    # 8 workgroups (a multiple of 8, so the XCD remap of the workgroup order applies) whose last one
    # has a single output row
    "conv3d_k331_xcd_odd_rows": W.CONFIGS["c2"].with_(x_shape=(1, 3, 17, 40, 10)),
    # 2 samples x 3 row pairs x 4 chunks = 24 workgroups, last chunk partial
    "conv3d_k331_xcd_chunks": W.CONFIGS["c2"].with_(x_shape=(2, 3, 8, 180, 10)),
    # 40 row pairs x 2 chunks = 80 workgroups: the remap into interleaved runs of 10 per XCD
    "conv3d_k331_xcd_runs": W.CONFIGS["c2"].with_(x_shape=(1, 3, 82, 100, 10)),
    # a second, partial block of 64 output channels; one input channel (K = 9, the 8-step
    # instantiation); a (4,4,1) kernel on 2 channels (K = 32, the 16-step instantiation)
    "conv3d_k331_cout80": W.CONFIGS["c2"].with_(x_shape=(1, 3, 7, 20, 8), cout=80),
    "conv3d_k331_cin1": W.CONFIGS["c2"].with_(x_shape=(1, 1, 6, 30, 12)),
    "conv3d_k441_cin2": W.CONFIGS["c2"].with_(x_shape=(1, 2, 9, 21, 6), kernel=(4, 4, 1)),
    "convT_bn_pool_cin1_cout5": W.CONFIGS["c4"].with_(x_shape=(2, 1, 6, 9, 8), cout=5),
}


@pytest.mark.parametrize("name", list(MEDIUM))
def test_medium_shapes(name, variant):
    wl = MEDIUM[name]
    print(f"[medium {name} v{variant}] {wl}", flush=True)
    check_full(wl, W.make_inputs(wl), name)


def test_c1_full():
    wl = W.CONFIGS["c1"]
    check_full(wl, W.make_inputs(wl), "c1")


# ------------------------------------------- full-size workloads (sampled)
def _sample(size, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(rng.integers(0, size, n))


def test_c2_full_size_sampled():
    wl = W.CONFIGS["c2"]
    inp = W.make_inputs(wl)
    y = run_gpu(wl, inp)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item()
    flat = np.concatenate([_sample(y.numel(), 200_000, 21),
                           np.arange(0, 2540 * 3), y.numel() - 1 - np.arange(2540 * 3)])
    got = y.view(-1)[torch.from_numpy(flat).cuda()].cpu().numpy()
    ref = O.conv3d_at(inp.x, inp.w, flat, inp.b, wl.stride, wl.pad, wl.dilation, wl.groups)
    assert_close("c2 sampled", got, ref)
    # the first and the last image in full (both ends of the workgroup order)
    for n in (0, wl.x_shape[0] - 1):
        ref_n = O.conv3d(np.ascontiguousarray(inp.x[n:n + 1]), inp.w, inp.b, wl.stride, wl.pad, wl.dilation,
                         wl.groups)
        assert_close(f"c2 image {n}", y[n:n + 1].cpu().numpy(), ref_n)
    # repeat and compare bit for bit
    y2 = run_gpu(wl, inp)
    assert torch.equal(y, y2)


def test_c3_full_size_every_element():
    """The whole 16x64x33x65x65 output against the oracle's scatter definition."""
    wl = W.CONFIGS["c3"]
    inp = W.make_inputs(wl)
    y = run_gpu(wl, inp)
    torch.cuda.synchronize()
    assert_close("c3 full", y.cpu().numpy(), O.run_workload(wl, inp))


def test_c3_full_size_sampled_and_checkerboard():
    wl = W.CONFIGS["c3"]
    inp = W.make_inputs(wl)
    y = run_gpu(wl, inp)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (16, 64, 33, 65, 65)
    # every output with an even coordinate is exactly zero (no bias)
    odd = torch.zeros(y.shape[2:], dtype=torch.bool, device="cuda")
    odd[1::2, 1::2, 1::2] = True
    assert (y[:, :, ~odd] == 0).all().item()
    assert not torch.isnan(y).any().item()
    assert (y[:, :, odd] != 0).float().mean().item() > 0.999
    # sampled values, weighted towards the odd sub-lattice
    S = y.shape
    rng = np.random.default_rng(31)
    k = 150_000
    n, c = rng.integers(0, S[0], k), rng.integers(0, S[1], k)
    o0, o1, o2 = 2 * rng.integers(0, 16, k) + 1, 2 * rng.integers(0, 32, k) + 1, 2 * rng.integers(0, 32, k) + 1
    flat = np.unique(np.concatenate([(((n * S[1] + c) * S[2] + o0) * S[3] + o1) * S[4] + o2,
                                     _sample(y.numel(), 20_000, 32)]))
    got = y.view(-1)[torch.from_numpy(flat).cuda()].cpu().numpy()
    ref = O.conv_transpose3d_at(inp.x, inp.w, flat, inp.b, wl.stride, wl.pad, wl.dilation, wl.output_pad,
                                wl.groups)
    assert_close("c3 sampled", got, ref)
    y2 = run_gpu(wl, inp)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("v", [0, 5, 3], ids=["swapped_sums", "per_cell", "matrix_cores"])
def test_c4_full_size(v):
    old = B.set_variant(v)
    try:
        wl = W.CONFIGS["c4"]
        p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
        assert B.convT_bn_avgpool_algo(wl.x_shape, wl.cout, p, wl.pool) == {0: "bn_swap", 5: "bn_cells",
                                                                             3: "bn_mfma"}[v]
        inp = W.make_inputs(wl)
        y = check_full(wl, inp, "c4")
        # repeat (the workspace is reused) and compare bit for bit
        y2 = run_gpu(wl, inp)
        assert torch.equal(y, y2)
    finally:
        B.set_variant(old)


@pytest.mark.parametrize("dist", ["unit", "offset4"])
@pytest.mark.parametrize("v", [0, 5, 3], ids=["swapped_sums", "per_cell", "matrix_cores"])
def test_c4_full_size_offset_inputs(v, dist):
    """The module at full size with inputs whose mean is far from zero: U[0,1)
    (the pages' torch.rand) and 4 + U[-1,1].  The batch variance is then a
    difference of large sums, the case that exposes cancellation."""
    wl = W.CONFIGS["c4"]
    inp = W.make_inputs(wl, x_dist=dist)
    old = B.set_variant(v)
    try:
        print(f"[c4 {dist} v{v}]", flush=True)
        check_full(wl, inp, f"c4 {dist} v{v}")
    finally:
        B.set_variant(old)


@pytest.mark.parametrize("dist", ["unit", "offset4"])
def test_c4_generic_offset_inputs(dist):
    wl = W.CONFIGS["c4"].with_(x_shape=(3, 3, 14, 13, 18))
    old = B.set_variant(1)
    try:
        check_full(wl, W.make_inputs(wl, x_dist=dist), f"c4 generic {dist}")
    finally:
        B.set_variant(old)


MFMA_MEDIUM = {
    # the matrix-core phase-class path on ragged boxes, every supported input channel count, Cout <= 16
    "c4_reduced": W.CONFIGS["c4"].with_(x_shape=(3, 3, 14, 13, 18)),
    "cin1_cout5": W.CONFIGS["c4"].with_(x_shape=(2, 1, 6, 9, 8), cout=5),
    "cin2_cout12_bias": W.CONFIGS["c4"].with_(x_shape=(1, 2, 17, 5, 6), cout=12, bias=True),
    "cin4_cout16": W.CONFIGS["c4"].with_(x_shape=(2, 4, 9, 7, 20), cout=16),
    "exact_windows": W.CONFIGS["c4"].with_(x_shape=(2, 3, 16, 16, 16)),
    "several_boxes": W.CONFIGS["c4"].with_(x_shape=(1, 3, 40, 36, 20)),
    "tiny": W.CONFIGS["c4"].with_(x_shape=(1, 3, 3, 3, 4), cout=7),
}


@pytest.mark.parametrize("name", list(MFMA_MEDIUM))
def test_c4_matrix_core_medium(name):
    wl = MFMA_MEDIUM[name]
    old = B.set_variant(3)  # the module's second algorithm where the swapped sums would apply
    try:
        p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
        assert B.convT_bn_avgpool_algo(wl.x_shape, wl.cout, p, wl.pool) == "bn_mfma"
        print(f"[c4 matrix cores {name}] {wl}", flush=True)
        check_full(wl, W.make_inputs(wl), name)
    finally:
        B.set_variant(old)


@pytest.mark.parametrize("v,shape", [(3, (2, 3, 9, 10, 20)), (0, (2, 3, 9, 10, 20)), (0, (64, 3, 32, 32, 32))],
                         ids=["matrix_cores", "swapped_sums", "swapped_sums_full"])
def test_c4_unaligned_input(v, shape):
    """x 4 bytes off a 16-byte boundary: both algorithms stage the input with
    scalar loads instead of 16-byte ones (the swapped sums at full size then
    take their general statistics and pooled kernels)."""
    wl = W.CONFIGS["c4"].with_(x_shape=shape)
    inp = W.make_inputs(wl)
    ref, ref_mean, ref_var = O.run_workload(wl, inp)
    flat = torch.empty(int(np.prod(wl.x_shape)) + 1, dtype=torch.float32, device="cuda")
    x = flat[1:].view(wl.x_shape)
    x.copy_(dev(inp.x))
    assert x.data_ptr() % 16 == 4
    out, mean, var = poisoned(ref.shape), poisoned((wl.cout,)), poisoned((wl.cout,))
    old = B.set_variant(v)
    try:
        p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
        assert B.convT_bn_avgpool_algo(wl.x_shape, wl.cout, p, wl.pool) == {0: "bn_swap", 3: "bn_mfma"}[v]
        print(f"[c4 unaligned v{v}] {shape}", flush=True)
        B.convT_bn_avgpool(x, dev(inp.w), dev(inp.b), dev(inp.gamma), dev(inp.beta), wl.eps, wl.pool, wl.stride,
                           wl.pad, wl.dilation, out=out, batch_mean=mean, batch_var=var)
    finally:
        B.set_variant(old)
    assert_close("c4 unaligned out", out.cpu().numpy(), ref)
    assert_close("c4 unaligned mean", mean.cpu().numpy(), ref_mean)
    assert_close("c4 unaligned var", var.cpu().numpy(), ref_var)


SWAP_MEDIUM = {
    # the swapped-sums path on ragged shapes and every supported channel count
    "c4_reduced": W.CONFIGS["c4"].with_(x_shape=(3, 3, 14, 13, 18)),
    "cin1_cout5": W.CONFIGS["c4"].with_(x_shape=(2, 1, 6, 9, 8), cout=5),
    "cin2_cout32": W.CONFIGS["c4"].with_(x_shape=(2, 2, 5, 7, 11), cout=32),
    "exact_windows": W.CONFIGS["c4"].with_(x_shape=(2, 3, 16, 16, 16)),
    "tiny": W.CONFIGS["c4"].with_(x_shape=(1, 3, 3, 3, 4), cout=7),
    # faces too large for LDS: the boundary Gram matrices read x directly
    "wide_faces": W.CONFIGS["c4"].with_(x_shape=(1, 3, 3, 70, 66), cout=9),
}


@pytest.mark.parametrize("name", list(SWAP_MEDIUM))
def test_c4_swapped_sums_medium(name):
    wl = SWAP_MEDIUM[name]
    old = B.set_variant(0)
    try:
        p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
        assert B.convT_bn_avgpool_algo(wl.x_shape, wl.cout, p, wl.pool) == "bn_swap"
        print(f"[c4 swapped sums {name}] {wl}", flush=True)
        check_full(wl, W.make_inputs(wl), name)
    finally:
        B.set_variant(old)


def test_c5_full_size_every_element():
    """All 4x1x16x64x64 outputs against the oracle's module (conv, max-pool,
    two-pass logsumexp, ReLU in float64)."""
    wl = W.CONFIGS["c5"]
    inp = W.make_inputs(wl)
    y = run_gpu(wl, inp)
    torch.cuda.synchronize()
    assert_close("c5 full", y.cpu().numpy(), O.run_workload(wl, inp))


def test_c5_full_size_sampled():
    wl = W.CONFIGS["c5"]
    inp = W.make_inputs(wl)
    y = run_gpu(wl, inp)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (4, 1, 16, 64, 64)
    assert torch.isfinite(y).all().item() and (y >= 0).all().item()
    flat = np.concatenate([_sample(y.numel(), 3000, 51), np.arange(0, 64), y.numel() - 1 - np.arange(64)])
    got = y.view(-1)[torch.from_numpy(flat).cuda()].cpu().numpy()
    ref = O.conv_maxpool_lse_relu_at(inp.x, inp.w, inp.b, flat, wl.pool, wl.stride, wl.pad, wl.dilation,
                                     wl.groups)
    assert_close("c5 sampled", got, ref)
    y2 = run_gpu(wl, inp)
    assert torch.equal(y, y2)


# ------------------------------------ BatchNorm: eval mode, running statistics
BN_EVAL = {
    "c4_reduced": W.CONFIGS["c4"].with_(x_shape=(3, 3, 14, 13, 18)),
    "c4_cin1_cout5": W.CONFIGS["c4"].with_(x_shape=(2, 1, 6, 9, 8), cout=5),
    "generic_pool2_groups": W.CONFIGS["c4"].with_(x_shape=(2, 4, 5, 6, 7), cout=6, pool=2, groups=2,
                                                  kernel=(3, 2, 3), stride=(2, 1, 2), output_pad=(1, 0, 0)),
}


def _bn_eval_gpu(wl, inp, rm, rv):
    return B.convT_bn_avgpool(dev(inp.x), dev(inp.w), dev(inp.b), dev(inp.gamma), dev(inp.beta), wl.eps, wl.pool,
                              wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups,
                              out=poisoned(O.output_shape(wl)), training=False, running_mean=dev(rm),
                              running_var=dev(rv))


@pytest.mark.parametrize("name", list(BN_EVAL))
def test_bn_eval_mode(name, bn_variant):
    variant = bn_variant
    wl = BN_EVAL[name]
    inp = W.make_inputs(wl)
    rm, rv = W.make_running_stats(wl.cout, 17)
    print(f"[bn eval {name} v{variant}] {wl}", flush=True)
    y = _bn_eval_gpu(wl, inp, rm, rv)
    torch.cuda.synchronize()
    ref = O.convT_bn_eval_avgpool(inp.x, inp.w, inp.b, inp.gamma, inp.beta, rm, rv, wl.eps, wl.pool, wl.stride,
                                  wl.pad, wl.dilation, wl.output_pad, wl.groups)
    assert_close(f"bn eval {name}", y.cpu().numpy(), ref)


def test_bn_eval_mode_c4_full_size():
    wl = W.CONFIGS["c4"]
    inp = W.make_inputs(wl)
    rm, rv = W.make_running_stats(wl.cout, 19)
    y = _bn_eval_gpu(wl, inp, rm, rv)
    torch.cuda.synchronize()
    ref = O.convT_bn_eval_avgpool(inp.x, inp.w, inp.b, inp.gamma, inp.beta, rm, rv, wl.eps, wl.pool, wl.stride,
                                  wl.pad, wl.dilation, wl.output_pad, wl.groups)
    assert_close("bn eval c4", y.cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["c4_reduced", "generic_pool2_groups"])
def test_bn_running_statistics_update(name, bn_variant):
    wl = BN_EVAL[name]
    inp = W.make_inputs(wl)
    rm0, rv0 = W.make_running_stats(wl.cout, 23)
    rm, rv = dev(rm0), dev(rv0)
    kw = dict(stride=wl.stride, pad=wl.pad, dilation=wl.dilation, output_pad=wl.output_pad, groups=wl.groups)
    args = (dev(inp.x), dev(inp.w), dev(inp.b), dev(inp.gamma), dev(inp.beta), wl.eps, wl.pool)
    y = B.convT_bn_avgpool(*args, out=poisoned(O.output_shape(wl)), running_mean=rm, running_var=rv,
                           momentum=0.1, **kw)
    y_plain = B.convT_bn_avgpool(*args, out=poisoned(O.output_shape(wl)), **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y_plain)  # the update does not change the output
    out, mean, var = O.run_workload(wl, inp)
    assert_close(f"bn running out {name}", y.cpu().numpy(), out)
    cshape = O.convT_out_shape(wl.x_shape, wl.cout, wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad)
    count = cshape[0] * cshape[2] * cshape[3] * cshape[4]
    erm, erv = O.bn_running_update(rm0, rv0, mean, var, count, 0.1)
    assert_close(f"running mean {name}", rm.cpu().numpy(), erm)
    assert_close(f"running var {name}", rv.cpu().numpy(), erv)


@pytest.mark.parametrize("dist", ["unit", "offset4"])
def test_bn_eval_and_running_update_offset_inputs(dist, bn_variant):
    """Eval mode and the running-statistics update on inputs with a large mean."""
    wl = BN_EVAL["c4_reduced"]
    inp = W.make_inputs(wl, x_dist=dist)
    rm0, rv0 = W.make_running_stats(wl.cout, 29)
    y = _bn_eval_gpu(wl, inp, rm0, rv0)
    torch.cuda.synchronize()
    ref = O.convT_bn_eval_avgpool(inp.x, inp.w, inp.b, inp.gamma, inp.beta, rm0, rv0, wl.eps, wl.pool, wl.stride,
                                  wl.pad, wl.dilation, wl.output_pad, wl.groups)
    assert_close(f"bn eval {dist}", y.cpu().numpy(), ref)
    rm, rv = dev(rm0), dev(rv0)
    kw = dict(stride=wl.stride, pad=wl.pad, dilation=wl.dilation, output_pad=wl.output_pad, groups=wl.groups)
    y = B.convT_bn_avgpool(dev(inp.x), dev(inp.w), dev(inp.b), dev(inp.gamma), dev(inp.beta), wl.eps, wl.pool,
                           out=poisoned(O.output_shape(wl)), running_mean=rm, running_var=rv, momentum=0.1, **kw)
    torch.cuda.synchronize()
    out, mean, var = O.run_workload(wl, inp)
    assert_close(f"bn running out {dist}", y.cpu().numpy(), out)
    cshape = O.convT_out_shape(wl.x_shape, wl.cout, wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad)
    erm, erv = O.bn_running_update(rm0, rv0, mean, var, cshape[0] * cshape[2] * cshape[3] * cshape[4], 0.1)
    assert_close(f"running mean {dist}", rm.cpu().numpy(), erm)
    assert_close(f"running var {dist}", rv.cpu().numpy(), erv)


# ----------------------------------------------------------- edge cases
EDGE = {
    "conv_1x1x1_single": W.make("e", "conv3d", (1, 1, 1, 1, 1), 1, 1, bias=True, seed=7),
    "conv_kernel_equals_input": W.make("e", "conv3d", (2, 3, 3, 3, 3), 5, 3, seed=8),
    "conv_big_stride": W.make("e", "conv3d", (1, 2, 9, 9, 9), 3, 2, stride=5, pad=2, seed=9),
    "conv_groups_depthwise": W.make("e", "conv3d", (1, 4, 6, 6, 6), 4, 3, pad=1, groups=4, seed=10),
    "convT_1x1x1": W.make("e", "conv_transpose3d", (1, 2, 1, 1, 1), 3, 1, seed=11),
    "convT_outpad_max": W.make("e", "conv_transpose3d", (1, 2, 3, 4, 5), 2, 3, stride=3, pad=1, dilation=2,
                               output_pad=2, seed=12),
    "convT_pad_exceeds_taps": W.make("e", "conv_transpose3d", (1, 2, 6, 6, 6), 2, 3, stride=1, pad=3, seed=13),
    "bn_pool_single_window": W.make("e", "convT_bn_avgpool", (1, 3, 2, 2, 2), 4, 3, stride=2, pad=1, pool=3,
                                    seed=14),
    "bn_pool_pool1": W.make("e", "convT_bn_avgpool", (2, 2, 3, 3, 3), 3, 3, stride=2, pad=1, pool=1, seed=15),
    "lse_single_channel": W.make("e", "conv_maxpool_lse_relu", (1, 2, 4, 4, 4), 1, 3, pad=1, pool=2, seed=16),
    "lse_pool_whole": W.make("e", "conv_maxpool_lse_relu", (1, 3, 4, 4, 4), 6, 3, pad=1, pool=4, seed=17),
    # the stride-2 dilation-2 sub-lattice path on degenerate grids: one input voxel (a 4-plane tile with
    # 3 planes empty, bias-only output around one odd point), a thin grid, and W spanning two tiles with
    # Cout past one 64-channel block
    "convT_s2d2_single_voxel": W.make("e", "conv_transpose3d", (1, 4, 1, 1, 1), 8, 3, stride=2, pad=1,
                                      dilation=2, bias=True, seed=18),
    "convT_s2d2_thin": W.make("e", "conv_transpose3d", (2, 5, 1, 3, 1), 3, 3, stride=2, pad=1, dilation=2,
                              seed=19),
    "convT_s2d2_wide_cout70": W.make("e", "conv_transpose3d", (1, 3, 2, 1, 40), 70, 3, stride=2, pad=1,
                                     dilation=2, bias=True, seed=20),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name, variant):
    wl = EDGE[name]
    check_full(wl, W.make_inputs(wl), name)


def test_lse_all_negative_gives_zero_and_large_values():
    # a strongly negative bias makes every logsumexp negative: ReLU gives exactly 0;
    # a large positive input exercises the max shift
    wl = W.make("e", "conv_maxpool_lse_relu", (1, 4, 4, 6, 6), 8, 3, pad=1, pool=2, seed=18)
    inp = W.make_inputs(wl)
    inp.b[:] = -50.0
    y = run_gpu(wl, inp)
    torch.cuda.synchronize()
    assert (y == 0).all().item()
    inp.b[:] = 80.0
    inp.x[:] = inp.x * 30
    check_full(wl, inp, "lse_large")


def test_c4_module_with_random_bias_and_stats_outputs():
    wl = W.CONFIGS["c4"].with_(x_shape=(2, 3, 10, 12, 9))
    inp = W.make_inputs(wl)
    check_full(wl, inp, "c4 small stats")


def test_nonpositive_eps_and_small_workspace_rejected():
    wl = W.CONFIGS["c4"].with_(x_shape=(1, 3, 8, 8, 8))
    inp = W.make_inputs(wl)
    x, w = dev(inp.x), dev(inp.w)
    with pytest.raises(B.C3DError) as e:
        B.convT_bn_avgpool(x, w, dev(inp.b), dev(inp.gamma), dev(inp.beta), eps=0.0)
    assert e.value.status == 3
    # the binding checks the workspace against the query before calling in
    with pytest.raises(ValueError):
        B.convT_bn_avgpool(x, w, dev(inp.b), dev(inp.gamma), dev(inp.beta),
                           workspace=torch.empty(8, dtype=torch.uint8, device="cuda"))


def test_runs_on_a_side_stream():
    wl = W.CONFIGS["c1"]
    inp = W.make_inputs(wl)
    ref = O.run_workload(wl, inp)
    s = torch.cuda.Stream()
    x, w, b = dev(inp.x), dev(inp.w), dev(inp.b)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = B.conv3d_fwd(x, w, b, wl.stride, wl.pad, out=poisoned(ref.shape), stream=s)
    s.synchronize()
    assert_close("side stream", y.cpu().numpy(), ref)


def test_mfma_probe_matches_its_closed_form():
    """The throughput probe's per-thread sums follow from v_mfma_f32_32x32x2f32's
    operand layout (lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32];
    accumulator v of lane l is D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32]), which
    the conv engines rely on."""
    iters = 3
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    flop = B.probe_mfma_f32(iters, out)
    torch.cuda.synchronize()
    assert flop == 2048 * 4 * iters * 4 * 4096
    lane = np.arange(64)
    a = 1e-3 * lane.astype(np.float64)                 # A value supplied by each lane
    b = 1.0 / (1 + (lane & 7)).astype(np.float64)      # B value supplied by each lane
    A = np.stack([a[np.arange(32) + 32 * k] for k in range(2)], axis=1)   # [32, 2]
    Bm = np.stack([b[np.arange(32) + 32 * k] for k in range(2)], axis=0)  # [2, 32]
    D = iters * (A @ Bm)
    want = np.array([sum(D[8 * (v // 4) + 4 * (l // 32) + v % 4, l % 32] for v in range(16)) * 4 for l in range(64)])
    got = out.view(-1, 256).cpu().numpy()
    np.testing.assert_allclose(got[:, :64], np.broadcast_to(want, (2048, 64)), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(got[:, 64:128], got[:, :64], rtol=0, atol=0)


@pytest.mark.parametrize("valu_per_4", [2, 4, 8, 16])
def test_mfma_valu_probe_keeps_the_mfma_results(valu_per_4):
    """The probe variant with FMAs beside the MFMAs does the same MFMA work
    (same FLOP count, bit-identical sums)."""
    iters = 3
    ref = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    out = torch.full((2048 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flop = B.probe_mfma_f32(iters, ref)
    assert B.probe_mfma_valu_f32(iters, valu_per_4, out) == flop
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
