"""Seeded synthetic inputs for the five workloads, shared by the CPU oracle tests
and the HIP path.

This module only draws random tensors and records the module hyper-parameters
of each workload; it holds none of the method's arithmetic (no output-size
formula, no convolution, no pooling).

Workloads (each page is a POPCORNBENCH transcript titled "Kimi-K2.6 <id>"):

* ``c1`` - small Conv3d NCDHW, 4->8 channels, 8^3, kernel 3, stride 1, pad 1,
  bias.  Not on the pages; the smallest end-to-end case.
* ``c2`` - Conv3d with a (3,3,1) kernel on a depth-last ``x[N,C,H,W,D]``,
  16 x 3 x 256 x 256 x 10 -> 64 channels, stride 1, pad 0, no bias
  (page l1_p59, problem statement).
* ``c3`` - ConvTranspose3d 32->64, kernel 3, stride 2, pad 1, dilation 2, no
  bias, on x[16,32,16,32,32] (page l1_p77, problem statement).
* ``c4`` - ConvTranspose3d(3->16, k3, s2, p1, bias) -> BatchNorm3d with batch
  statistics -> AvgPool3d(2) -> AvgPool3d(2) on x[64,3,32,32,32]
  (page l2_p72, problem statement).
* ``c5`` - Conv3d(32->64, k3, s1, p1, bias) -> MaxPool3d(2) -> logsumexp over
  channels -> ReLU on x[4,32,32,128,128] (page l2_p43, problem statement).

Distributions: x ~ U[-1, 1]; weight and bias ~ U(-1/sqrt(fan_in), 1/sqrt(fan_in))
with fan_in = weight.shape[1] * kD * kH * kW (PyTorch's default initialiser
for conv modules); gamma ~ U[0.5, 1.5]; beta ~ U[-0.5, 0.5].  Draws are made in
float64 with ``numpy.random.default_rng(seed)`` in the order x, W, b, gamma,
beta and cast to float32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

Triple = Tuple[int, int, int]


def _t(v) -> Triple:
    if isinstance(v, int):
        return (v, v, v)
    v = tuple(int(a) for a in v)
    assert len(v) == 3
    return v  # type: ignore[return-value]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Hyper-parameters of one module instance plus its input shape."""

    name: str
    op: str  # conv3d | conv_transpose3d | convT_bn_avgpool | conv_maxpool_lse_relu
    x_shape: Tuple[int, int, int, int, int]
    cout: int
    kernel: Triple
    stride: Triple = (1, 1, 1)
    pad: Triple = (0, 0, 0)
    dilation: Triple = (1, 1, 1)
    output_pad: Triple = (0, 0, 0)
    groups: int = 1
    bias: bool = True
    pool: int = 0  # window = stride of the pooling epilogue (0: none)
    eps: float = 1e-5
    seed: int = 0
    description: str = ""

    @property
    def transposed(self) -> bool:
        return self.op in ("conv_transpose3d", "convT_bn_avgpool")

    @property
    def weight_shape(self) -> Tuple[int, ...]:
        cin = self.x_shape[1]
        if self.transposed:
            return (cin, self.cout // self.groups) + tuple(self.kernel)
        return (self.cout, cin // self.groups) + tuple(self.kernel)

    def with_(self, **kw) -> "Workload":
        for key in ("kernel", "stride", "pad", "dilation", "output_pad"):
            if key in kw:
                kw[key] = _t(kw[key])
        return dataclasses.replace(self, **kw)


def make(name, op, x_shape, cout, kernel, stride=1, pad=0, dilation=1,
         output_pad=0, groups=1, bias=True, pool=0, eps=1e-5, seed=0,
         description="") -> Workload:
    return Workload(name=name, op=op, x_shape=tuple(int(a) for a in x_shape),
                    cout=int(cout), kernel=_t(kernel), stride=_t(stride),
                    pad=_t(pad), dilation=_t(dilation),
                    output_pad=_t(output_pad), groups=int(groups),
                    bias=bool(bias), pool=int(pool), eps=float(eps),
                    seed=int(seed), description=description)


CONFIGS = {
    "c1": make("c1", "conv3d", (1, 4, 8, 8, 8), 8, 3, 1, 1, 1, bias=True,
               seed=1, description="Conv3d 4->8, 8^3, k3 s1 p1, bias"),
    "c2": make("c2", "conv3d", (16, 3, 256, 256, 10), 64, (3, 3, 1), 1, 0, 1,
               bias=False, seed=2,
               description="Conv3d (3,3,1) kernel on depth-last x[16,3,256,256,10], no bias"),
    "c3": make("c3", "conv_transpose3d", (16, 32, 16, 32, 32), 64, 3, 2, 1, 2,
               bias=False, seed=3,
               description="ConvTranspose3d 32->64 k3 s2 p1 d2 on x[16,32,16,32,32], no bias"),
    "c4": make("c4", "convT_bn_avgpool", (64, 3, 32, 32, 32), 16, 3, 2, 1, 1,
               bias=True, pool=4, eps=1e-5, seed=4,
               description="ConvTranspose3d 3->16 k3 s2 p1 + BatchNorm3d (batch stats) + AvgPool3d(2) twice"),
    "c5": make("c5", "conv_maxpool_lse_relu", (4, 32, 32, 128, 128), 64, 3, 1, 1, 1,
               bias=True, pool=2, seed=5,
               description="Conv3d 32->64 k3 s1 p1 + MaxPool3d(2) + logsumexp(dim=1) + ReLU"),
}


# Transposed convs beyond the five configurations, for the per-output-phase
# MFMA path (timed by `bench.py --widen`; reduced copies are parity cases).
WIDEN = {
    "t1": make("t1", "conv_transpose3d", (16, 32, 16, 32, 32), 64, 3, 2, 1, 1, 1, bias=True, seed=101,
               description="ConvTranspose3d 32->64 k3 s2 p1 output_padding 1 (x2 upsampling) on "
                           "x[16,32,16,32,32] -> [16,64,32,64,64]"),
    "t2": make("t2", "conv_transpose3d", (8, 64, 16, 32, 32), 32, 4, 2, 1, bias=True, seed=102,
               description="ConvTranspose3d 64->32 k4 s2 p1 on x[8,64,16,32,32] -> [8,32,32,64,64]"),
    "t3": make("t3", "conv_transpose3d", (8, 32, 8, 16, 16), 64, 3, 3, 1, 1, 2, groups=2, bias=True, seed=103,
               description="ConvTranspose3d 32->64 groups 2 k3 s3 p1 output_padding 2 on x[8,32,8,16,16] "
                           "-> [8,64,24,48,48]"),
}


@dataclasses.dataclass
class Inputs:
    x: np.ndarray
    w: np.ndarray
    b: Optional[np.ndarray]
    gamma: Optional[np.ndarray]
    beta: Optional[np.ndarray]


def _uniform(rng: np.random.Generator, lo: float, hi: float, shape) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def make_inputs(wl: Workload, seed: Optional[int] = None,
                x_dist: str = "uniform") -> Inputs:
    """Draw x, W, b, gamma, beta (in that order) for a workload.

    ``x_dist`` may be ``"uniform"`` (U[-1,1], the default), ``"unit"``
    (U[0,1), the distribution of ``torch.rand`` that the pages' harness draws
    inputs from), ``"offset4"`` (4 + U[-1,1], a mean well away from zero) or
    ``"ones"`` / ``"zeros"`` for structured test inputs; the parameter draws
    are unchanged.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    if x_dist == "uniform":
        x = _uniform(rng, -1.0, 1.0, wl.x_shape)
    elif x_dist == "unit":
        x = _uniform(rng, 0.0, 1.0, wl.x_shape)
    elif x_dist == "offset4":
        x = (_uniform(rng, -1.0, 1.0, wl.x_shape).astype(np.float64) + 4.0).astype(np.float32)
    elif x_dist == "ones":
        x = np.ones(wl.x_shape, np.float32)
    elif x_dist == "zeros":
        x = np.zeros(wl.x_shape, np.float32)
    else:
        raise ValueError(x_dist)
    ws = wl.weight_shape
    fan_in = ws[1] * ws[2] * ws[3] * ws[4]
    bound = 1.0 / math.sqrt(fan_in)
    w = _uniform(rng, -bound, bound, ws)
    b = _uniform(rng, -bound, bound, (wl.cout,)) if wl.bias else None
    gamma = beta = None
    if wl.op == "convT_bn_avgpool":
        gamma = _uniform(rng, 0.5, 1.5, (wl.cout,))
        beta = _uniform(rng, -0.5, 0.5, (wl.cout,))
    return Inputs(x=x, w=w, b=b, gamma=gamma, beta=beta)


def make_running_stats(cout: int, seed: int) -> Tuple[np.ndarray, np.ndarray]:
    """BatchNorm running statistics for eval-mode tests: mean ~ U[-0.25, 0.25],
    variance ~ U[0.5, 2.0], drawn in float64 with their own seed and cast to
    float32."""
    rng = np.random.default_rng(seed)
    rm = _uniform(rng, -0.25, 0.25, (cout,))
    rv = _uniform(rng, 0.5, 2.0, (cout,))
    return rm, rv


def random_small_workload(op: str, rng: np.random.Generator, max_spatial: int = 9,
                          allow_groups: bool = True) -> Workload:
    """A random small module for sweep tests: stride 1..3, pad 0..2,
    dilation 1..2, groups 1/2/4, odd and even sizes, bias on/off."""
    groups = int(rng.choice([1, 2, 4])) if allow_groups else 1
    cin = groups * int(rng.integers(1, 4))
    cout = groups * int(rng.integers(1, 4))
    k = tuple(int(a) for a in rng.integers(1, 4, size=3))
    s = tuple(int(a) for a in rng.integers(1, 4, size=3))
    d = tuple(int(a) for a in rng.integers(1, 3, size=3))
    p = tuple(int(a) for a in rng.integers(0, 3, size=3))
    sp = tuple(int(a) for a in rng.integers(1, max_spatial + 1, size=3))
    n = int(rng.integers(1, 3))
    bias = bool(rng.integers(0, 2))
    opad = (0, 0, 0)
    if op == "conv_transpose3d":
        opad = tuple(int(rng.integers(0, max(si, di))) for si, di in zip(s, d))
    # Some draws give an empty output; callers reject those with their own
    # output-size rule.
    return make("rand", op, (n, cin) + sp, cout, k, s, p, d, opad, groups, bias,
                seed=int(rng.integers(0, 2**31)))
