"""Python access to the CPU oracle (``c3d_oracle.c``).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package.  It marshals numpy arrays into the C
oracle; every computation happens in the C file, in float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c3d_oracle.c")
LIB = os.path.join(HERE, "libc3d_oracle.so")


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, portable ISA)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-Wno-unknown-pragmas", "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _Params(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32 * 3), ("s", ctypes.c_int32 * 3),
                ("p", ctypes.c_int32 * 3), ("d", ctypes.c_int32 * 3),
                ("op", ctypes.c_int32 * 3), ("groups", ctypes.c_int32)]


_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.c_void_p
_f64p = ctypes.c_void_p


def load(path: str = LIB):
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
        build(SRC, path)
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(_Params)
    i64 = ctypes.c_int64
    sig = {
        "oracle_num_threads": ([], ctypes.c_int),
        "oracle_conv_out_len": ([i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32], i64),
        "oracle_convT_out_len": ([i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32], i64),
        "oracle_pool_out_len": ([i64, ctypes.c_int32], i64),
        "oracle_conv3d": ([_f32p, _i64p, _f32p, i64, P, _f32p, _f64p], None),
        "oracle_conv3d_rows": ([_f32p, _i64p, _f32p, i64, P, _f32p, i64, i64, _f64p], None),
        "oracle_conv3d_at": ([_f32p, _i64p, _f32p, i64, P, _f32p, _i64p, i64, _f64p], None),
        "oracle_conv_transpose3d": ([_f32p, _i64p, _f32p, i64, P, _f32p, _f64p], None),
        "oracle_conv_transpose3d_at": ([_f32p, _i64p, _f32p, i64, P, _f32p, _i64p, i64, _f64p], None),
        "oracle_batchnorm_train": ([_f64p, i64, i64, i64, _f32p, _f32p, ctypes.c_double, _f64p, _f64p], None),
        "oracle_avgpool3d": ([_f64p, i64, _i64p, ctypes.c_int32, _f64p], None),
        "oracle_maxpool3d": ([_f64p, i64, _i64p, ctypes.c_int32, _f64p], None),
        "oracle_logsumexp_channels": ([_f64p, i64, i64, i64, _f64p], None),
        "oracle_relu": ([_f64p, i64], None),
        "oracle_convT_bn_avgpool": ([_f32p, _i64p, _f32p, i64, P, _f32p, _f32p, _f32p, ctypes.c_double,
                                     ctypes.c_int32, _f64p, _f64p, _f64p], None),
        "oracle_convT_bn_eval_avgpool": ([_f32p, _i64p, _f32p, i64, P, _f32p, _f32p, _f32p, _f32p, _f32p,
                                          ctypes.c_double, ctypes.c_int32, _f64p], None),
        "oracle_bn_running_update": ([i64, ctypes.c_double, i64, _f64p, _f64p, _f64p, _f64p], None),
        "oracle_conv_maxpool_lse_relu": ([_f32p, _i64p, _f32p, i64, P, _f32p, ctypes.c_int32, _f64p], None),
        "oracle_conv_maxpool_lse_relu_at": ([_f32p, _i64p, _f32p, i64, P, _f32p, ctypes.c_int32, _i64p,
                                             i64, _f64p], None),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


def _params(k, s, p, d, op=(0, 0, 0), groups=1) -> _Params:
    t = _Params()
    for name, v in (("k", k), ("s", s), ("p", p), ("d", d), ("op", op)):
        arr = getattr(t, name)
        for j in range(3):
            arr[j] = int(v[j])
    t.groups = int(groups)
    return t


def _f32(a: Optional[np.ndarray]):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data


def _shape(xs: Sequence[int]):
    return (ctypes.c_int64 * 5)(*[int(v) for v in xs])


def _idx(flat):
    flat = np.ascontiguousarray(flat, dtype=np.int64)
    return flat, flat.ctypes.data_as(_i64p)


# ---------------------------------------------------------------- sizes
def conv_out_len(L, k, s, p, d) -> int:
    return int(lib().oracle_conv_out_len(L, k, s, p, d))


def convT_out_len(L, k, s, p, d, op=0) -> int:
    return int(lib().oracle_convT_out_len(L, k, s, p, d, op))


def pool_out_len(L, w) -> int:
    return int(lib().oracle_pool_out_len(L, w))


def conv3d_out_shape(x_shape, cout, k, s, p, d):
    return (x_shape[0], cout) + tuple(conv_out_len(x_shape[2 + j], k[j], s[j], p[j], d[j]) for j in range(3))


def convT_out_shape(x_shape, cout, k, s, p, d, op=(0, 0, 0)):
    return (x_shape[0], cout) + tuple(convT_out_len(x_shape[2 + j], k[j], s[j], p[j], d[j], op[j])
                                      for j in range(3))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ------------------------------------------------------------ conv ops
def conv3d(x, w, bias=None, stride=(1, 1, 1), pad=(0, 0, 0), dilation=(1, 1, 1), groups=1):
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(bias)
    k = w.shape[2:]
    cout = w.shape[0]
    ys = conv3d_out_shape(x.shape, cout, k, stride, pad, dilation)
    y = np.empty(ys, np.float64)
    if y.size:
        lib().oracle_conv3d(xp, _shape(x.shape), wp, cout, _params(k, stride, pad, dilation, groups=groups),
                            bp, y.ctypes.data)
    return y


def conv3d_at(x, w, flat, bias=None, stride=(1, 1, 1), pad=(0, 0, 0), dilation=(1, 1, 1), groups=1):
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(bias)
    flat, fp = _idx(flat)
    out = np.empty(flat.shape, np.float64)
    lib().oracle_conv3d_at(xp, _shape(x.shape), wp, w.shape[0],
                           _params(w.shape[2:], stride, pad, dilation, groups=groups), bp, fp, flat.size,
                           out.ctypes.data)
    return out


def conv_transpose3d(x, w, bias=None, stride=(1, 1, 1), pad=(0, 0, 0), dilation=(1, 1, 1),
                     output_pad=(0, 0, 0), groups=1):
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(bias)
    k = w.shape[2:]
    cout = w.shape[1] * groups
    ys = convT_out_shape(x.shape, cout, k, stride, pad, dilation, output_pad)
    y = np.empty(ys, np.float64)
    if y.size:
        lib().oracle_conv_transpose3d(xp, _shape(x.shape), wp, cout,
                                      _params(k, stride, pad, dilation, output_pad, groups), bp, y.ctypes.data)
    return y


def conv_transpose3d_at(x, w, flat, bias=None, stride=(1, 1, 1), pad=(0, 0, 0), dilation=(1, 1, 1),
                        output_pad=(0, 0, 0), groups=1):
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(bias)
    flat, fp = _idx(flat)
    out = np.empty(flat.shape, np.float64)
    lib().oracle_conv_transpose3d_at(xp, _shape(x.shape), wp, w.shape[1] * groups,
                                     _params(w.shape[2:], stride, pad, dilation, output_pad, groups), bp, fp,
                                     flat.size, out.ctypes.data)
    return out


# ------------------------------------------------------------ epilogues
def batchnorm_train(y, gamma=None, beta=None, eps=1e-5):
    """Returns (z, mean, biased_var) for y[N, C, ...] (float64)."""
    z = np.array(y, dtype=np.float64, order="C", copy=True)
    N, C = z.shape[:2]
    plane = int(np.prod(z.shape[2:]))
    g, gp = _f32(gamma)
    b, bp = _f32(beta)
    mean = np.empty(C, np.float64)
    var = np.empty(C, np.float64)
    lib().oracle_batchnorm_train(z.ctypes.data, N, C, plane, gp, bp, float(eps), mean.ctypes.data,
                                 var.ctypes.data)
    return z, mean, var


def _pool(fn, y, w):
    y = np.ascontiguousarray(y, dtype=np.float64)
    S = y.shape[-3:]
    lead = y.shape[:-3]
    P = tuple(pool_out_len(S[j], w) for j in range(3))
    out = np.empty(lead + P, np.float64)
    if out.size:
        fn(y.ctypes.data, int(np.prod(lead)), _shape(tuple(S) + (0, 0)), int(w), out.ctypes.data)
    return out


def avgpool3d(y, w):
    return _pool(lib().oracle_avgpool3d, y, w)


def maxpool3d(y, w):
    return _pool(lib().oracle_maxpool3d, y, w)


def logsumexp_channels(y):
    y = np.ascontiguousarray(y, dtype=np.float64)
    N, C = y.shape[:2]
    plane = int(np.prod(y.shape[2:]))
    out = np.empty((N, 1) + y.shape[2:], np.float64)
    lib().oracle_logsumexp_channels(y.ctypes.data, N, C, plane, out.ctypes.data)
    return out


def relu(y):
    z = np.array(y, dtype=np.float64, order="C", copy=True)
    lib().oracle_relu(z.ctypes.data, z.size)
    return z


# ------------------------------------------------------- fused modules
def convT_bn_avgpool(x, w, bias, gamma, beta, eps=1e-5, pool=4, stride=(2, 2, 2), pad=(1, 1, 1),
                     dilation=(1, 1, 1), output_pad=(0, 0, 0), groups=1):
    """Returns (out, batch_mean, batch_var_biased)."""
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(bias)
    g, gp = _f32(gamma)
    be, bep = _f32(beta)
    k = w.shape[2:]
    cout = w.shape[1] * groups
    ys = convT_out_shape(x.shape, cout, k, stride, pad, dilation, output_pad)
    P = tuple(pool_out_len(ys[2 + j], pool) for j in range(3))
    out = np.empty((x.shape[0], cout) + P, np.float64)
    mean = np.empty(cout, np.float64)
    var = np.empty(cout, np.float64)
    lib().oracle_convT_bn_avgpool(xp, _shape(x.shape), wp, cout,
                                  _params(k, stride, pad, dilation, output_pad, groups), bp, gp, bep,
                                  float(eps), int(pool), out.ctypes.data, mean.ctypes.data, var.ctypes.data)
    return out, mean, var


def convT_bn_eval_avgpool(x, w, bias, gamma, beta, running_mean, running_var, eps=1e-5, pool=4,
                          stride=(2, 2, 2), pad=(1, 1, 1), dilation=(1, 1, 1), output_pad=(0, 0, 0), groups=1):
    """The ConvT -> BatchNorm3d -> AvgPool module with BN in eval mode ([p72]):
    BN normalises with the running statistics.  Returns out (float64)."""
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(bias)
    g, gp = _f32(gamma)
    be, bep = _f32(beta)
    rm, rmp = _f32(running_mean)
    rv, rvp = _f32(running_var)
    k = w.shape[2:]
    cout = w.shape[1] * groups
    ys = convT_out_shape(x.shape, cout, k, stride, pad, dilation, output_pad)
    P = tuple(pool_out_len(ys[2 + j], pool) for j in range(3))
    out = np.empty((x.shape[0], cout) + P, np.float64)
    lib().oracle_convT_bn_eval_avgpool(xp, _shape(x.shape), wp, cout,
                                       _params(k, stride, pad, dilation, output_pad, groups), bp, gp, bep, rmp, rvp,
                                       float(eps), int(pool), out.ctypes.data)
    return out


def bn_running_update(running_mean, running_var, batch_mean, batch_var_biased, count, momentum=0.1):
    """Running statistics after one training-mode forward ([p72]'s momentum;
    the running variance tracks the unbiased batch variance).  Returns new
    (running_mean, running_var) in float64."""
    bm = np.ascontiguousarray(batch_mean, np.float64)
    bv = np.ascontiguousarray(batch_var_biased, np.float64)
    rm = np.array(running_mean, np.float64)
    rv = np.array(running_var, np.float64)
    lib().oracle_bn_running_update(len(rm), float(momentum), int(count), bm.ctypes.data, bv.ctypes.data,
                                   rm.ctypes.data, rv.ctypes.data)
    return rm, rv


def conv_maxpool_lse_relu(x, w, bias, pool=2, stride=(1, 1, 1), pad=(1, 1, 1), dilation=(1, 1, 1), groups=1):
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(bias)
    k = w.shape[2:]
    cout = w.shape[0]
    ys = conv3d_out_shape(x.shape, cout, k, stride, pad, dilation)
    P = tuple(pool_out_len(ys[2 + j], pool) for j in range(3))
    out = np.empty((x.shape[0], 1) + P, np.float64)
    if out.size:
        lib().oracle_conv_maxpool_lse_relu(xp, _shape(x.shape), wp, cout,
                                           _params(k, stride, pad, dilation, groups=groups), bp, int(pool),
                                           out.ctypes.data)
    return out


def conv_maxpool_lse_relu_at(x, w, bias, flat, pool=2, stride=(1, 1, 1), pad=(1, 1, 1), dilation=(1, 1, 1),
                             groups=1):
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(bias)
    flat, fp = _idx(flat)
    out = np.empty(flat.shape, np.float64)
    lib().oracle_conv_maxpool_lse_relu_at(xp, _shape(x.shape), wp, w.shape[0],
                                          _params(w.shape[2:], stride, pad, dilation, groups=groups), bp,
                                          int(pool), fp, flat.size, out.ctypes.data)
    return out


# --------------------------------------------------- workload helpers
def run_workload(wl, inp):
    """Full oracle result for a workload (see transposed_convolution_epilogues_amd.workloads)."""
    kw = dict(stride=wl.stride, pad=wl.pad, dilation=wl.dilation)
    if wl.op == "conv3d":
        return conv3d(inp.x, inp.w, inp.b, groups=wl.groups, **kw)
    if wl.op == "conv_transpose3d":
        return conv_transpose3d(inp.x, inp.w, inp.b, output_pad=wl.output_pad, groups=wl.groups, **kw)
    if wl.op == "convT_bn_avgpool":
        return convT_bn_avgpool(inp.x, inp.w, inp.b, inp.gamma, inp.beta, wl.eps, wl.pool,
                                output_pad=wl.output_pad, groups=wl.groups, **kw)
    if wl.op == "conv_maxpool_lse_relu":
        return conv_maxpool_lse_relu(inp.x, inp.w, inp.b, wl.pool, groups=wl.groups, **kw)
    raise ValueError(wl.op)


def output_shape(wl):
    """Output shape of a workload by the oracle's size rules."""
    if wl.op == "conv3d":
        return conv3d_out_shape(wl.x_shape, wl.cout, wl.kernel, wl.stride, wl.pad, wl.dilation)
    if wl.op == "conv_transpose3d":
        return convT_out_shape(wl.x_shape, wl.cout, wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad)
    if wl.op == "convT_bn_avgpool":
        ys = convT_out_shape(wl.x_shape, wl.cout, wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad)
        return ys[:2] + tuple(pool_out_len(ys[2 + j], wl.pool) for j in range(3))
    ys = conv3d_out_shape(wl.x_shape, wl.cout, wl.kernel, wl.stride, wl.pad, wl.dilation)
    return (ys[0], 1) + tuple(pool_out_len(ys[2 + j], wl.pool) for j in range(3))
