"""Host-side checks of the C ABI: the library loads and exports every symbol
include/c3d.h declares, the shape queries agree with the oracle's size rules,
and invalid arguments are rejected before anything is launched.  No GPU is
needed: every call here returns during host validation.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from transposed_convolution_epilogues_amd import binding as B
from transposed_convolution_epilogues_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "c3d.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|c3d_status|char\s*\*|const char\s*\*)\s*\**\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_four_entry_points():
    syms = header_symbols()
    for name in ("conv3d_fwd", "conv_transpose3d_fwd", "convT_bn_avgpool", "conv_maxpool_lse_relu"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = B.library()
    syms = header_symbols()
    assert len(syms) >= 10
    for name in syms:
        assert hasattr(lib, name), name
    assert set(B.EXPORTS) == set(syms)


def _p(k=3, s=1, p=0, d=1, op=0, g=1):
    return B.make_params(k, s, p, d, op, g)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_shape_queries_match_oracle(name):
    wl = W.CONFIGS[name]
    p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
    if wl.op == "conv3d":
        got = B.conv3d_out_dims(wl.x_shape, wl.cout, p)
    elif wl.op == "conv_transpose3d":
        got = B.conv_transpose3d_out_dims(wl.x_shape, wl.cout, p)
    elif wl.op == "convT_bn_avgpool":
        got = B.convT_bn_avgpool_out_dims(wl.x_shape, wl.cout, p, wl.pool)
    else:
        got = B.conv_maxpool_lse_relu_out_dims(wl.x_shape, wl.cout, p, wl.pool)
    assert got == O.output_shape(wl)


def test_shape_queries_random_match_oracle():
    rng = np.random.default_rng(5)
    for _ in range(300):
        op = "conv3d" if rng.integers(0, 2) else "conv_transpose3d"
        wl = W.random_small_workload(op, rng)
        p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
        ref = O.output_shape(wl)
        fn = B.conv3d_out_dims if op == "conv3d" else B.conv_transpose3d_out_dims
        if all(v > 0 for v in ref):
            assert fn(wl.x_shape, wl.cout, p) == ref
        else:
            with pytest.raises(B.C3DError) as e:
                fn(wl.x_shape, wl.cout, p)
            assert e.value.status == 2


def _call_conv(lib, x=1, w=1, y=1, shape=(1, 4, 8, 8, 8), cout=8, params=None, bias=None, fn="conv3d_fwd"):
    params = params or _p(3, 1, 1)
    vp = ctypes.c_void_p
    # fake non-null aligned device addresses: these calls must fail validation
    # before any pointer is dereferenced or any kernel is launched
    ptr = lambda v: None if v is None else vp(4096 * v)
    return getattr(lib, fn)(ptr(x), B._shape5(shape), ptr(w), cout, ctypes.byref(params),
                            ptr(bias) if bias is not None else None, ptr(y), None)


def test_errors_are_reported_before_launch():
    lib = B.library()
    assert _call_conv(lib, x=None) == 1
    assert _call_conv(lib, w=None) == 1
    assert _call_conv(lib, y=None) == 1
    assert _call_conv(lib, shape=(1, 4, 0, 8, 8)) == 2
    assert _call_conv(lib, shape=(0, 4, 8, 8, 8)) == 2  # empty batch: rejected, nothing launched
    assert _call_conv(lib, shape=(1, 0, 8, 8, 8)) == 2
    assert _call_conv(lib, shape=(1, (1 << 30) + 4, 1, 1, 1), params=_p(1, 1, 0)) == 2  # Cin above 2^30
    assert _call_conv(lib, shape=(1, 6, 8, 8, 8), params=_p(3, 1, 1, 1, 0, 4)) == 2  # Cin % groups
    assert _call_conv(lib, cout=6, params=_p(3, 1, 1, 1, 0, 4), shape=(1, 8, 8, 8, 8)) == 2  # Cout % groups
    assert _call_conv(lib, shape=(1, 4, 2, 8, 8), params=_p(3, 1, 0)) == 2  # empty output
    assert _call_conv(lib, params=_p(0, 1, 1)) == 3
    assert _call_conv(lib, params=_p(3, 0, 1)) == 3
    assert _call_conv(lib, params=_p(3, 1, -1)) == 3
    assert _call_conv(lib, params=_p(3, 1, 1, 0)) == 3
    assert _call_conv(lib, params=_p(3, 1, 1, 1, 1)) == 3  # output_pad on a direct conv
    assert _call_conv(lib, params=_p(3, 1, 1, 1, 0, 0)) == 3
    # output_pad must be < max(stride, dilation) for the transposed conv
    assert _call_conv(lib, fn="conv_transpose3d_fwd", params=_p(3, 2, 1, 1, 2)) == 3
    assert _call_conv(lib, fn="conv_transpose3d_fwd", params=_p(3, 2, 1, 3, 2), x=None) == 1
    # misaligned pointer
    vp = ctypes.c_void_p
    assert lib.conv3d_fwd(vp(4098), B._shape5((1, 4, 8, 8, 8)), vp(4096), 8, ctypes.byref(_p(3, 1, 1)), None,
                          vp(8192), None) == 7


def test_fused_op_errors_are_reported_before_launch():
    lib = B.library()
    vp = ctypes.c_void_p
    p = _p(3, 2, 1)
    xs = B._shape5((2, 3, 8, 8, 8))
    ws_need = lib.convT_bn_avgpool_workspace_bytes(xs, 16, ctypes.byref(p), 4)
    assert ws_need > 0
    ok = dict(x=vp(4096), w=vp(8192), b=None, g=vp(12288), be=vp(16384), y=vp(20480), ws=vp(24576))

    def call(eps=1e-5, pool=4, ws_bytes=ws_need, **kw):
        a = dict(ok, **kw)
        return lib.convT_bn_avgpool(a["x"], xs, a["w"], 16, ctypes.byref(p), a["b"], a["g"], a["be"], eps, pool,
                                    a["y"], a["ws"], ws_bytes, None, None, None)

    assert call(g=None) == 1
    assert call(be=None) == 1
    assert call(eps=0.0) == 3
    assert call(eps=float("nan")) == 3
    assert call(pool=0) == 3
    assert call(pool=16) == 2  # ConvT output 15 < pool
    assert call(ws=None) == 4
    assert call(ws_bytes=8) == 4  # the query covers every kernel choice; any path needs more than this
    assert call(ws=vp(24580)) == 7  # workspace must be 8-byte aligned
    pc = _p(3, 1, 1)
    assert lib.conv_maxpool_lse_relu(vp(4096), B._shape5((1, 4, 8, 8, 8)), vp(8192), 8, ctypes.byref(pc), None,
                                     0, vp(12288), None) == 3
    assert lib.conv_maxpool_lse_relu(vp(4096), B._shape5((1, 4, 1, 8, 8)), vp(8192), 8, ctypes.byref(pc), None,
                                     2, vp(12288), None) == 2


def test_bn_running_stats_and_eval_errors_are_reported_before_launch():
    lib = B.library()
    vp = ctypes.c_void_p
    p = _p(3, 2, 1)
    xs = B._shape5((2, 3, 8, 8, 8))
    ws_need = lib.convT_bn_avgpool_workspace_bytes(xs, 16, ctypes.byref(p), 4)
    ok = dict(x=vp(4096), w=vp(8192), b=None, g=vp(12288), be=vp(16384), y=vp(20480), ws=vp(24576),
              rm=vp(28672), rv=vp(32768))

    def call(training=1, momentum=0.1, eps=1e-5, shape=xs, params=p, **kw):
        a = dict(ok, **kw)
        return lib.convT_bn_avgpool_ex(a["x"], shape, a["w"], 16, ctypes.byref(params), a["b"], a["g"], a["be"],
                                       eps, 4 if shape is xs else 1, training, momentum, a["rm"], a["rv"], a["y"],
                                       a["ws"], ws_need, None, None, None)

    assert call(training=0, rm=None, rv=None) == 1       # eval mode needs the running statistics
    assert call(training=0, rv=None) == 1
    assert call(rm=None) == 1                             # both or neither
    assert call(momentum=1.5) == 3
    assert call(momentum=-0.1) == 3
    assert call(momentum=float("nan")) == 3
    assert call(training=0, eps=0.0) == 3
    assert call(training=0, g=None) == 1
    assert call(training=0, rm=vp(28674)) == 7            # misaligned running mean
    assert call(ws=None) == 4                             # training still needs the workspace
    # one element per channel: no unbiased variance for the running update
    assert call(shape=B._shape5((1, 3, 1, 1, 1)), params=_p(1, 1, 0)) == 2


def test_status_strings():
    lib = B.library()
    for code in range(8):
        assert lib.c3d_status_str(code)
    assert lib.c3d_status_str(99) == b"unknown status"


def test_binding_rejects_cpu_tensors():
    import torch

    x = torch.zeros(1, 4, 8, 8, 8)
    w = torch.zeros(8, 4, 3, 3, 3)
    with pytest.raises(TypeError):
        B.conv3d_fwd(x, w, None, 1, 1, out=torch.zeros(1, 8, 8, 8, 8))


# ------------------------------------------- binding validation before launch
LAUNCHES = ("conv3d_fwd", "conv_transpose3d_fwd", "convT_bn_avgpool", "convT_bn_avgpool_ex",
            "conv_maxpool_lse_relu", "c3d_probe_mfma_f32", "c3d_probe_mfma_valu_f32")


class _NoLaunch:
    """The real library for host-only queries; every entry point that would
    launch a kernel fails the test instead."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        if name in LAUNCHES:
            def launched(*a, **k):
                raise AssertionError(f"{name} was called: validation should have failed first")
            return launched
        return getattr(self._lib, name)


@pytest.fixture
def no_launch(monkeypatch):
    monkeypatch.setattr(B, "_LIB", _NoLaunch(B.library()))
    yield
    monkeypatch.setattr(B, "_LIB", None)


def _z(*shape):
    import torch
    return torch.zeros(*shape)


def _conv_ok():
    # conv3d / conv_maxpool_lse_relu: x[1,4,8,8,8], w[8,4,3,3,3], pad 1
    return dict(x=_z(1, 4, 8, 8, 8), w=_z(8, 4, 3, 3, 3), bias=_z(8))


CONV_BAD = {
    "x_not_5d": dict(x=_z(4, 8, 8, 8)),
    "w_not_5d": dict(w=_z(8, 4, 3, 3)),
    "w_channels": dict(w=_z(8, 3, 3, 3, 3)),
    "w_channels_groups": dict(w=_z(8, 4, 3, 3, 3), groups=2),
    "groups_zero": dict(groups=0),
    "bias_length": dict(bias=_z(7)),
    "bias_2d": dict(bias=_z(8, 1)),
    "out_shape": dict(out=_z(1, 8, 8, 8, 7)),
}


@pytest.mark.parametrize("case", list(CONV_BAD))
def test_conv3d_binding_rejects_mis_shaped_tensors(case, no_launch):
    a = dict(_conv_ok(), groups=1, out=None)
    a.update(CONV_BAD[case])
    with pytest.raises(ValueError):
        B.conv3d_fwd(a["x"], a["w"], a["bias"], 1, 1, 1, a["groups"], out=a["out"])


LSE_BAD = dict(CONV_BAD, out_shape=dict(out=_z(1, 8, 4, 4, 4)))


@pytest.mark.parametrize("case", list(LSE_BAD))
def test_conv_maxpool_lse_relu_binding_rejects_mis_shaped_tensors(case, no_launch):
    a = dict(_conv_ok(), groups=1, out=None)
    a.update(LSE_BAD[case])
    with pytest.raises(ValueError):
        B.conv_maxpool_lse_relu(a["x"], a["w"], a["bias"], 2, 1, 1, 1, a["groups"], out=a["out"])


def _convT_ok():
    # x[2,8,4,4,4], w[8,16,3,3,3], s2 p1 -> y[2,16,7,7,7]
    return dict(x=_z(2, 8, 4, 4, 4), w=_z(8, 16, 3, 3, 3), bias=_z(16))


CONVT_BAD = {
    "x_not_5d": dict(x=_z(2, 8, 4, 4)),
    "w_in_channels": dict(w=_z(4, 16, 3, 3, 3)),
    "bias_length": dict(bias=_z(8)),
    "bias_length_groups": dict(bias=_z(16), groups=2),  # Cout = 16 * 2 = 32
    "out_shape": dict(out=_z(2, 16, 7, 7, 8)),
}


@pytest.mark.parametrize("case", list(CONVT_BAD))
def test_conv_transpose3d_binding_rejects_mis_shaped_tensors(case, no_launch):
    a = dict(_convT_ok(), groups=1, out=None)
    a.update(CONVT_BAD[case])
    with pytest.raises(ValueError):
        B.conv_transpose3d_fwd(a["x"], a["w"], a["bias"], 2, 1, 1, 0, a["groups"], out=a["out"])


def _bn_ok():
    # the module's geometry at a small size: x[2,3,8,8,8], w[3,16,3,3,3] -> t[2,16,15,15,15] -> y[2,16,3,3,3]
    return dict(x=_z(2, 3, 8, 8, 8), w=_z(3, 16, 3, 3, 3), conv_bias=_z(16), gamma=_z(16), beta=_z(16),
                out=None, workspace=None, batch_mean=None, batch_var=None, running_mean=None, running_var=None,
                training=True)


BN_BAD = {
    "w_in_channels": dict(w=_z(4, 16, 3, 3, 3)),
    "conv_bias_length": dict(conv_bias=_z(15)),
    "gamma_length": dict(gamma=_z(17)),
    "beta_length": dict(beta=_z(8)),
    "gamma_missing": dict(gamma=None),
    "batch_mean_length": dict(batch_mean=_z(15)),
    "batch_var_length": dict(batch_var=_z(1)),
    "running_mean_length": dict(running_mean=_z(15), running_var=_z(16)),
    "running_var_length": dict(running_mean=_z(16), running_var=_z(32)),
    "running_mean_alone": dict(running_mean=_z(16)),
    "eval_without_running": dict(training=False),
    "out_shape": dict(out=_z(2, 16, 3, 3, 4)),
    "workspace_small": dict(workspace=_z(1)),
}


@pytest.mark.parametrize("case", list(BN_BAD))
def test_convT_bn_avgpool_binding_rejects_mis_shaped_tensors(case, no_launch):
    a = _bn_ok()
    a.update(BN_BAD[case])
    with pytest.raises(ValueError):
        B.convT_bn_avgpool(a["x"], a["w"], a["conv_bias"], a["gamma"], a["beta"], 1e-5, 4, 2, 1,
                           out=a["out"], workspace=a["workspace"], batch_mean=a["batch_mean"],
                           batch_var=a["batch_var"], training=a["training"], running_mean=a["running_mean"],
                           running_var=a["running_var"])


def test_well_shaped_host_tensors_stop_at_the_device_check(no_launch):
    """Correct shapes reach the device check, which rejects host tensors
    (TypeError) before any launch."""
    c = _conv_ok()
    with pytest.raises(TypeError):
        B.conv3d_fwd(c["x"], c["w"], c["bias"], 1, 1, out=_z(1, 8, 8, 8, 8))
    with pytest.raises(TypeError):
        B.conv_maxpool_lse_relu(c["x"], c["w"], c["bias"], 2, 1, 1, out=_z(1, 1, 4, 4, 4))
    t = _convT_ok()
    with pytest.raises(TypeError):
        B.conv_transpose3d_fwd(t["x"], t["w"], t["bias"], 2, 1, out=_z(2, 16, 7, 7, 7))
    a = _bn_ok()
    with pytest.raises(TypeError):
        B.convT_bn_avgpool(a["x"], a["w"], a["conv_bias"], a["gamma"], a["beta"], 1e-5, 4, 2, 1,
                           out=_z(2, 16, 3, 3, 3), workspace=_z(1 << 16), batch_mean=_z(16), batch_var=_z(16),
                           running_mean=_z(16), running_var=_z(16))
    with pytest.raises(TypeError):
        B.probe_mfma_f32(10, _z(1 << 19))
    with pytest.raises(TypeError):
        B.probe_mfma_valu_f32(10, 4, _z(1 << 19))


def test_variant_override_is_per_thread():
    """c3d_set_variant changes only the calling thread's kernel choice."""
    import threading

    params = B.make_params((3, 3, 1), 1, 0, 1, 0, 1)
    xs, cout = (16, 3, 256, 256, 10), 64
    old = B.set_variant(1)
    try:
        assert B.conv3d_algo(xs, cout, params) == "direct"
        seen = {}

        def other():
            seen["algo"] = B.conv3d_algo(xs, cout, params)
            seen["old"] = B.set_variant(2)

        th = threading.Thread(target=other)
        th.start()
        th.join()
        assert seen == {"algo": "k1last", "old": 0}
        assert B.conv3d_algo(xs, cout, params) == "direct"  # the other thread's setting did not leak here
    finally:
        B.set_variant(old)


# ----------------------------------------------------------- kernel choice
ALGO_CASES = [
    # (op, x_shape, cout, kernel, stride, pad, dilation, output_pad, groups, variant, expected)
    ("conv3d", (16, 3, 256, 256, 10), 64, (3, 3, 1), 1, 0, 1, 0, 1, 0, "k1last"),       # c2
    ("conv3d", (1, 4, 8, 8, 8), 8, 3, 1, 1, 1, 0, 1, 0, "direct"),                      # c1: below 2^19 MAC
    ("conv3d", (1, 4, 8, 8, 16), 8, 3, 1, 1, 1, 0, 1, 0, "mfma333"),                    # 884,736 MAC
    ("conv3d", (1, 2, 8, 8, 8), 8, 3, 1, 1, 1, 0, 1, 0, "direct"),                      # too few channels
    ("conv3d", (1, 8, 8, 8, 8), 8, 3, 2, 1, 1, 0, 1, 0, "direct"),                      # strided
    ("conv3d", (16, 3, 256, 256, 10), 64, (3, 3, 1), 1, 0, 1, 0, 1, 1, "direct"),       # forced generic
    ("conv_transpose3d", (16, 32, 16, 32, 32), 64, 3, 2, 1, 2, 0, 1, 0, "sublattice"),  # c3
    ("conv_transpose3d", (16, 32, 16, 32, 32), 64, 3, 2, 1, 2, 0, 1, 2, "phase_group"), # c3, general path
    ("conv_transpose3d", (16, 32, 16, 32, 32), 64, 3, 2, 1, 2, 0, 1, 6, "phase"),       # one phase per workgroup
    ("conv_transpose3d", (1, 8, 4, 4, 4), 1025, 3, 2, 1, 2, 0, 1, 0, "phase_group"),    # 33 channel blocks
    ("conv_transpose3d", (16, 32, 16, 32, 32), 64, 3, 2, 1, 2, 0, 1, 1, "direct"),
    ("conv_transpose3d", (2, 16, 8, 8, 8), 32, 3, 2, 1, 1, 1, 1, 0, "phase_group"),     # dense phases
    ("conv_transpose3d", (2, 16, 8, 8, 8), 32, 3, 2, 1, 1, 1, 1, 6, "phase"),
    ("conv_transpose3d", (2, 16, 8, 8, 8), 32, 4, 2, 1, 1, 0, 1, 0, "phase_group"),
    ("conv_transpose3d", (2, 16, 8, 8, 8), 32, 3, 3, 1, 1, 2, 2, 0, "phase_group"),     # s3, groups
    ("conv_transpose3d", (2, 16, 8, 8, 8), 32, 3, 1, 1, 1, 0, 1, 0, "phase_group"),     # stride 1
    ("conv_transpose3d", (2, 16, 8, 8, 8), 32, (5, 5, 3), 2, (2, 2, 1), 1, 0, 1, 0, "phase"),  # 75 taps > 64
    ("conv_transpose3d", (2, 16, 8, 8, 8), 32, 3, 5, 1, 1, 0, 1, 0, "direct"),          # stride > 4
    ("conv_transpose3d", (2, 16, 8, 8, 8), 32, 7, 2, 1, 1, 0, 1, 0, "direct"),          # 4 taps per residue
    ("conv_transpose3d", (2, 16, 8, 8, 8), 32, 3, 1, 1, 2, 0, 1, 0, "direct"),          # offsets span 4
    ("conv_transpose3d", (2, 3, 8, 8, 8), 32, 3, 2, 1, 1, 0, 1, 0, "direct"),           # Cin/groups < 4
    ("conv_transpose3d", (2, 16, 8, 8, 8), 4, 3, 2, 1, 1, 0, 1, 0, "direct"),           # Cout/groups < 8
    ("conv_transpose3d", (16, 32, 16, 32, 32), 64, 3, 2, 1, 2, 0, 1, 4, "scatter"),     # variant 4
    ("conv_transpose3d", (2, 3, 8, 8, 8), 4, 3, 5, 1, 1, 0, 1, 4, "scatter"),
    ("conv3d", (16, 3, 256, 256, 10), 64, (3, 3, 1), 1, 0, 1, 0, 1, 4, "k1last"),       # conv unaffected
    ("conv3d", (1, 3, 7, 20, 8), 80, (3, 3, 1), 1, 0, 1, 0, 1, 0, "k1last"),            # two channel blocks
    ("conv3d", (1, 2, 9, 21, 6), 64, (4, 4, 1), 1, 0, 1, 0, 1, 0, "k1last"),            # K = 32
    ("conv3d", (1, 4, 9, 21, 6), 64, (3, 3, 1), 1, 0, 1, 0, 1, 0, "direct"),            # K = 36 > 32
    ("conv3d", (1, 3, 9, 21, 6), 8, (3, 3, 1), 1, 0, 1, 0, 1, 0, "direct"),             # Cout < 16
    ("conv3d", (1, 3, 9, 21, 6), 64, (3, 3, 1), 1, 1, 1, 0, 1, 0, "direct"),            # padding
]


@pytest.mark.parametrize("case", ALGO_CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(ALGO_CASES)])
def test_kernel_choice(case):
    op, xs, cout, k, s, p, d, op_, g, variant, expected = case
    params = B.make_params(k, s, p, d, op_, g)
    old = B.set_variant(variant)
    try:
        got = (B.conv3d_algo if op == "conv3d" else B.conv_transpose3d_algo)(xs, cout, params)
    finally:
        B.set_variant(old)
    assert got == expected


BN_ALGO_CASES = [
    # (x_shape, cout, kernel, stride, pad, pool, variant, expected)
    ((64, 3, 32, 32, 32), 16, 3, 2, 1, 4, 0, "bn_swap"),    # c4: swapped sums
    ((64, 3, 32, 32, 32), 16, 3, 2, 1, 4, 4, "bn_swap"),
    ((64, 3, 32, 32, 32), 16, 3, 2, 1, 4, 3, "bn_mfma"),    # the module's second algorithm
    ((64, 3, 32, 32, 32), 16, 3, 2, 1, 4, 2, "bn_mfma"),
    ((64, 3, 32, 32, 32), 16, 3, 2, 1, 4, 5, "bn_cells"),   # per-cell fp32 kernel on request
    ((64, 3, 32, 32, 32), 16, 3, 2, 1, 4, 1, "direct"),
    ((2, 4, 8, 8, 8), 16, 3, 2, 1, 4, 3, "bn_mfma"),       # Cin 4: outside the swapped-sums path
    ((2, 3, 8, 8, 8), 40, 3, 2, 1, 4, 3, "bn_cells"),      # Cout 40: outside both
    ((2, 3, 8, 8, 8), 17, 3, 2, 1, 4, 0, "bn_swap"),       # Cout 17: two N tiles on the swapped sums
    ((2, 3, 8, 8, 8), 17, 3, 2, 1, 4, 3, "bn_cells"),      # outside the phase-class kernel (Cout > 16)
    ((2, 4, 8, 8, 8), 16, 3, 2, 1, 4, 0, "bn_mfma"),       # Cin 4: default outside the swapped sums
    ((2, 5, 8, 8, 8), 16, 3, 2, 1, 4, 0, "direct"),        # Cin 5
    ((2, 3, 8, 8, 8), 16, 3, 2, 1, 2, 3, "direct"),        # pool 2
    ((2, 3, 8, 8, 8), 16, 3, 1, 1, 4, 0, "direct"),        # stride 1
]


@pytest.mark.parametrize("case", BN_ALGO_CASES, ids=[f"bn-{i}" for i in range(len(BN_ALGO_CASES))])
def test_bn_kernel_choice(case):
    xs, cout, k, s, p, pool, variant, expected = case
    old = B.set_variant(variant)
    try:
        got = B.convT_bn_avgpool_algo(xs, cout, B.make_params(k, s, p), pool)
    finally:
        B.set_variant(old)
    assert got == expected


def test_kernel_choice_rejects_invalid_arguments():
    with pytest.raises(B.C3DError):
        B.conv_transpose3d_algo((1, 4, 4, 4, 4), 8, B.make_params(3, 2, 1, 1, 2))  # output_pad >= stride
    lib = B.library()
    xs = (ctypes.c_int64 * 5)(1, 4, 4, 4, 4)
    assert lib.c3d_conv3d_algo(xs, 8, ctypes.byref(B.make_params(3)), None) == 1  # C3D_ERR_NULL


def _code(name):
    return next(k for k, v in B.STATUS.items() if v == name)


def test_mfma_probe_rejects_bad_arguments_before_launching():
    lib = B.library()
    flop = ctypes.c_int64(0)
    assert lib.c3d_probe_mfma_f32(10, None, 1 << 20, ctypes.byref(flop), None) == 1  # C3D_ERR_NULL
    fake = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    assert lib.c3d_probe_mfma_f32(0, fake, 1 << 20, ctypes.byref(flop), None) == _code("C3D_ERR_PARAM")
    assert lib.c3d_probe_mfma_f32(10, fake, 1000, ctypes.byref(flop), None) == _code("C3D_ERR_PARAM")
    assert lib.c3d_probe_mfma_f32(10, ctypes.c_void_p(4098), 1 << 20, ctypes.byref(flop), None) == \
        _code("C3D_ERR_ALIGN")


def test_mfma_valu_probe_rejects_bad_arguments_before_launching():
    lib = B.library()
    flop = ctypes.c_int64(0)
    fake = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    assert lib.c3d_probe_mfma_valu_f32(10, 4, None, 1 << 20, ctypes.byref(flop), None) == 1  # C3D_ERR_NULL
    for bad in (0, 1, 3, 5, 32, -4):
        assert lib.c3d_probe_mfma_valu_f32(10, bad, fake, 1 << 20, ctypes.byref(flop), None) == \
            _code("C3D_ERR_PARAM"), bad
    assert lib.c3d_probe_mfma_valu_f32(0, 4, fake, 1 << 20, ctypes.byref(flop), None) == _code("C3D_ERR_PARAM")
    assert lib.c3d_probe_mfma_valu_f32(10, 4, fake, 1000, ctypes.byref(flop), None) == _code("C3D_ERR_PARAM")
    assert lib.c3d_probe_mfma_valu_f32(10, 4, ctypes.c_void_p(4098), 1 << 20, ctypes.byref(flop), None) == \
        _code("C3D_ERR_ALIGN")


def test_noalloc_refuses_more_than_its_scratch_before_any_hip_call():
    """convT_bn_avgpool_noalloc checks the partials its kernels need against
    its static scratch before it touches the GPU (no GPU is needed here)."""
    wl = W.CONFIGS["c4"].with_(x_shape=(4096, 3, 32, 32, 32))  # about 16 MiB of partials
    p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
    assert B.convT_bn_avgpool_workspace_bytes(wl.x_shape, wl.cout, p, wl.pool) > B.NOALLOC_SCRATCH_BYTES
    lib = B.library()
    vp = ctypes.c_void_p
    st = lib.convT_bn_avgpool_noalloc(vp(4096), B._shape5(wl.x_shape), vp(8192), wl.cout, ctypes.byref(p), None,
                                      vp(12288), vp(16384), 1e-5, 4, vp(20480), None, None, None)
    assert st == 8  # C3D_ERR_SCRATCH_LIMIT
    assert b"static scratch" in lib.c3d_status_str(8)
    # invalid geometry is still reported as such
    st = lib.convT_bn_avgpool_noalloc(vp(4096), B._shape5((1, 3, 1, 1, 1)), vp(8192), wl.cout, ctypes.byref(p),
                                      None, vp(12288), vp(16384), 1e-5, 4, vp(20480), None, None, None)
    assert st == 2
