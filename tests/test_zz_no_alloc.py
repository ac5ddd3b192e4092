"""The entry point that allocates nothing (convT_bn_avgpool_noalloc) against
the allocating convT_bn_avgpool: same output and batch statistics, to the
parity bar |a - b| <= 1e-4 + 1e-4 |b|, on two calls in a row, the second
with a smaller input (the static scratch keeps the first call's partials, so
the second must read only what it wrote itself).
"""
import numpy as np
import pytest
import torch

from transposed_convolution_epilogues_amd import binding as B
from transposed_convolution_epilogues_amd import workloads as W

pytestmark = pytest.mark.gpu

ATOL = 1e-4
RTOL = 1e-4


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def close(name, got, ref):
    got = got.detach().cpu().numpy().astype(np.float64)
    ref = ref.detach().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    bad = ~(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))
    assert not bad.any(), f"{name}: {int(bad.sum())}/{bad.size} outside tolerance"


def _one(wl):
    inp = W.make_inputs(wl)
    x, w, b, gm, bt = dev(inp.x), dev(inp.w), dev(inp.b), dev(inp.gamma), dev(inp.beta)
    kw = dict(stride=wl.stride, pad=wl.pad, dilation=wl.dilation, output_pad=wl.output_pad, groups=wl.groups)
    p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
    shape = B.convT_bn_avgpool_out_dims(wl.x_shape, wl.cout, p, wl.pool)
    nan = lambda s: torch.full(s, float("nan"), device="cuda")
    ref, rm, rv = nan(shape), nan((wl.cout,)), nan((wl.cout,))
    B.convT_bn_avgpool(x, w, b, gm, bt, wl.eps, wl.pool, out=ref, batch_mean=rm, batch_var=rv, **kw)
    got, gmn, gvr = nan(shape), nan((wl.cout,)), nan((wl.cout,))
    B.convT_bn_avgpool_noalloc(x, w, b, gm, bt, got, wl.eps, wl.pool, batch_mean=gmn, batch_var=gvr, **kw)
    torch.cuda.synchronize()
    close("out", got, ref)
    close("batch_mean", gmn, rm)
    close("batch_var", gvr, rv)


def test_noalloc_matches_allocating_entry_point_on_two_calls():
    c4 = W.CONFIGS["c4"]
    print("noalloc: c4 full size", c4.x_shape, flush=True)
    _one(c4)
    small = c4.with_(x_shape=(3, 3, 9, 13, 11))
    print("noalloc: smaller second call", small.x_shape, flush=True)
    _one(small)
