"""ctypes binding of the C ABI in include/c3d.h (argument marshalling only).

Each function takes PyTorch tensors that already live on the GPU, checks that
they are contiguous float32 device tensors, and passes raw device pointers,
shapes and the current HIP stream to libc3d.so.  Every step of the
computation runs in the library's HIP kernels; there is no CPU or PyTorch
fallback, and a missing library is an error.  Output and workspace tensors
are allocated with PyTorch when the caller does not pass them (memory only).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libc3d.so")

C3D_OK = 0
STATUS = {0: "C3D_OK", 1: "C3D_ERR_NULL", 2: "C3D_ERR_SHAPE", 3: "C3D_ERR_PARAM", 4: "C3D_ERR_WORKSPACE",
          5: "C3D_ERR_UNSUPPORTED", 6: "C3D_ERR_HIP", 7: "C3D_ERR_ALIGN", 8: "C3D_ERR_SCRATCH_LIMIT"}
NOALLOC_SCRATCH_BYTES = 4 << 20  # C3D_NOALLOC_SCRATCH_BYTES

EXPORTS = ("c3d_conv3d_out_dims", "c3d_conv_transpose3d_out_dims", "c3d_convT_bn_avgpool_out_dims",
           "c3d_conv_maxpool_lse_relu_out_dims", "conv3d_fwd", "conv_transpose3d_fwd",
           "convT_bn_avgpool_workspace_bytes", "convT_bn_avgpool", "convT_bn_avgpool_ex", "convT_bn_avgpool_noalloc",
           "conv_maxpool_lse_relu",
           "c3d_status_str",
           "c3d_set_variant", "c3d_conv3d_algo", "c3d_conv_transpose3d_algo", "c3d_convT_bn_avgpool_algo",
           "c3d_probe_mfma_f32", "c3d_probe_mfma_valu_f32")

ALGO = {0: "direct", 1: "k1last", 2: "mfma333", 3: "sublattice", 4: "phase", 5: "bn_cells", 6: "bn_swap",
        7: "scatter", 8: "bn_mfma", 9: "phase_group"}


class C3DError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_lib().c3d_status_str(status).decode()})")


class ConvParams(ctypes.Structure):
    """Mirror of c3d_conv_params."""
    _fields_ = [("kernel", ctypes.c_int32 * 3), ("stride", ctypes.c_int32 * 3), ("pad", ctypes.c_int32 * 3),
                ("dilation", ctypes.c_int32 * 3), ("output_pad", ctypes.c_int32 * 3), ("groups", ctypes.c_int32)]


Int3 = Union[int, Sequence[int]]


def _t3(v: Int3) -> Tuple[int, int, int]:
    if isinstance(v, int):
        return (v, v, v)
    v = tuple(int(a) for a in v)
    if len(v) != 3:
        raise ValueError("expected an int or a 3-sequence")
    return v  # type: ignore[return-value]


def make_params(kernel: Int3, stride: Int3 = 1, pad: Int3 = 0, dilation: Int3 = 1, output_pad: Int3 = 0,
                groups: int = 1) -> ConvParams:
    p = ConvParams()
    for name, v in (("kernel", kernel), ("stride", stride), ("pad", pad), ("dilation", dilation),
                    ("output_pad", output_pad)):
        arr = getattr(p, name)
        for j, a in enumerate(_t3(v)):
            arr[j] = a
    p.groups = int(groups)
    return p


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library {LIB_PATH} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    i64p = ctypes.POINTER(ctypes.c_int64)
    P = ctypes.POINTER(ConvParams)
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.c3d_conv3d_out_dims.argtypes = [i64p, i64, P, i64p]
    lib.c3d_conv_transpose3d_out_dims.argtypes = [i64p, i64, P, i64p]
    lib.c3d_convT_bn_avgpool_out_dims.argtypes = [i64p, i64, P, ctypes.c_int32, i64p]
    lib.c3d_conv_maxpool_lse_relu_out_dims.argtypes = [i64p, i64, P, ctypes.c_int32, i64p]
    lib.conv3d_fwd.argtypes = [vp, i64p, vp, i64, P, vp, vp, vp]
    lib.conv_transpose3d_fwd.argtypes = [vp, i64p, vp, i64, P, vp, vp, vp]
    lib.convT_bn_avgpool_workspace_bytes.argtypes = [i64p, i64, P, ctypes.c_int32]
    lib.convT_bn_avgpool_workspace_bytes.restype = ctypes.c_size_t
    lib.convT_bn_avgpool.argtypes = [vp, i64p, vp, i64, P, vp, vp, vp, ctypes.c_float, ctypes.c_int32, vp, vp,
                                     ctypes.c_size_t, vp, vp, vp]
    lib.convT_bn_avgpool_ex.argtypes = [vp, i64p, vp, i64, P, vp, vp, vp, ctypes.c_float, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_float, vp, vp, vp, vp, ctypes.c_size_t, vp, vp, vp]
    lib.conv_maxpool_lse_relu.argtypes = [vp, i64p, vp, i64, P, vp, ctypes.c_int32, vp, vp]
    lib.convT_bn_avgpool_noalloc.argtypes = [vp, i64p, vp, i64, P, vp, vp, vp, ctypes.c_float, ctypes.c_int32, vp,
                                             vp, vp, vp]
    lib.c3d_status_str.argtypes = [ctypes.c_int]  # c3d_status is an int-sized enum
    lib.c3d_status_str.restype = ctypes.c_char_p
    lib.c3d_set_variant.argtypes = [ctypes.c_int]
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.c3d_conv3d_algo.argtypes = [i64p, i64, P, i32p]
    lib.c3d_conv_transpose3d_algo.argtypes = [i64p, i64, P, i32p]
    lib.c3d_convT_bn_avgpool_algo.argtypes = [i64p, i64, P, ctypes.c_int32, i32p]
    lib.c3d_probe_mfma_f32.argtypes = [i64, ctypes.c_void_p, i64, i64p, ctypes.c_void_p]
    lib.c3d_probe_mfma_valu_f32.argtypes = [i64, ctypes.c_int32, ctypes.c_void_p, i64, i64p, ctypes.c_void_p]
    for name in ("c3d_conv3d_out_dims", "c3d_conv_transpose3d_out_dims", "c3d_convT_bn_avgpool_out_dims",
                 "c3d_conv_maxpool_lse_relu_out_dims", "conv3d_fwd", "conv_transpose3d_fwd",
                 "convT_bn_avgpool", "convT_bn_avgpool_ex", "conv_maxpool_lse_relu", "c3d_set_variant",
                 "c3d_conv3d_algo",
                 "c3d_conv_transpose3d_algo", "c3d_convT_bn_avgpool_algo", "c3d_probe_mfma_f32",
                 "c3d_probe_mfma_valu_f32", "convT_bn_avgpool_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _LIB = lib
    return lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def _shape5(shape) -> ctypes.Array:
    if len(shape) != 5:
        raise ValueError("expected a 5-D shape [N, C, S0, S1, S2]")
    return (ctypes.c_int64 * 5)(*[int(v) for v in shape])


# ---------------------------------------------------------------- validation
# The C ABI takes raw device pointers and cannot see how large a buffer is, so
# a tensor of the wrong shape would turn into an out-of-bounds device access.
# Every wrapper below therefore checks, before anything is launched:
#   1. shapes: x and w are 5-D, the weight's channel dim matches x, every
#      per-channel vector holds exactly Cout elements, `out` has the shape the
#      C shape query returns, the workspace holds at least the queried bytes
#      (ValueError);
#   2. then every tensor is float32 (the workspace: any dtype), on the GPU
#      (TypeError), on x's device and contiguous (ValueError).
# Shapes are checked first, so a mis-shaped call fails the same way with or
# without a GPU.


def _tensor(t, name: str, required: bool = True) -> Optional[torch.Tensor]:
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    return t


def _rank5(t: torch.Tensor, name: str):
    if t.dim() != 5:
        raise ValueError(f"{name} must be 5-D, got shape {tuple(t.shape)}")


def _vec(t: Optional[torch.Tensor], name: str, n: int):
    if t is not None and (t.dim() != 1 or int(t.shape[0]) != n):
        raise ValueError(f"{name} must have shape ({n},), got {tuple(t.shape)}")


def _out(out: Optional[torch.Tensor], shape, like: torch.Tensor) -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    out = _tensor(out, "out")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    return out


def _placed(x: torch.Tensor, **tensors):
    """Device checks (after the shape checks): float32, on the GPU, on x's
    device, contiguous.  Returns the raw pointers by name (None stays None)."""
    ptrs = {}
    for name, t in (("x", x),) + tuple(tensors.items()):
        if t is None:
            ptrs[name] = None
            continue
        if t.dtype != torch.float32 or t.device.type != "cuda":
            raise TypeError(f"{name} must be a float32 tensor on the GPU (got {t.dtype} on {t.device})")
        if t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        ptrs[name] = ctypes.c_void_p(t.data_ptr())
    return ptrs


def _workspace(ws: torch.Tensor, need: int):
    ws = _tensor(ws, "workspace")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, the call needs {need}")
    return ws


def _workspace_ptr(ws: torch.Tensor, x: torch.Tensor):
    if ws.device.type != "cuda":
        raise TypeError(f"workspace must be on the GPU (got {ws.device})")
    if ws.device != x.device:
        raise ValueError(f"workspace is on {ws.device}, x on {x.device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if ws.data_ptr() % 8:
        raise ValueError("workspace must be 8-byte aligned")
    return ctypes.c_void_p(ws.data_ptr())


def _conv_operands(x, w, groups: int, transposed: bool) -> int:
    """Checks x and w against each other; returns Cout."""
    x = _tensor(x, "x")
    w = _tensor(w, "w")
    _rank5(x, "x")
    _rank5(w, "w")
    groups = int(groups)
    if groups < 1:
        raise ValueError(f"groups must be >= 1, got {groups}")
    if transposed:
        # [Cin, Cout/groups, k0, k1, k2]
        if int(w.shape[0]) != int(x.shape[1]):
            raise ValueError(f"w.shape[0] = {int(w.shape[0])} must equal x's {int(x.shape[1])} input channels")
        return int(w.shape[1]) * groups
    # [Cout, Cin/groups, k0, k1, k2]
    if int(w.shape[1]) * groups != int(x.shape[1]):
        raise ValueError(f"w.shape[1] * groups = {int(w.shape[1]) * groups} must equal x's {int(x.shape[1])} "
                         "input channels")
    return int(w.shape[0])


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(st: int, where: str):
    if st != C3D_OK:
        raise C3DError(st, where)


def probe_mfma_f32(iters: int, out: torch.Tensor, stream=None) -> int:
    """Launch the matrix-core throughput probe on the stream; returns the
    launch's FLOP count (time it with events on the same stream)."""
    flop = ctypes.c_int64(0)
    out = _tensor(out, "out")
    if out.dtype != torch.float32 or out.device.type != "cuda" or not out.is_contiguous():
        raise TypeError("out must be a contiguous float32 tensor on the GPU")
    _check(_lib().c3d_probe_mfma_f32(int(iters), ctypes.c_void_p(out.data_ptr()), int(out.numel()),
                                     ctypes.byref(flop), _stream(stream)), "c3d_probe_mfma_f32")
    return int(flop.value)


def probe_mfma_valu_f32(iters: int, valu_per_4: int, out: torch.Tensor, stream=None) -> int:
    """Launch the probe with valu_per_4 independent FMAs after every 4 MFMAs
    of a wave; returns the launch's MFMA FLOP count."""
    flop = ctypes.c_int64(0)
    out = _tensor(out, "out")
    if out.dtype != torch.float32 or out.device.type != "cuda" or not out.is_contiguous():
        raise TypeError("out must be a contiguous float32 tensor on the GPU")
    _check(_lib().c3d_probe_mfma_valu_f32(int(iters), int(valu_per_4), ctypes.c_void_p(out.data_ptr()),
                                          int(out.numel()), ctypes.byref(flop), _stream(stream)),
           "c3d_probe_mfma_valu_f32")
    return int(flop.value)


def set_variant(variant: int) -> int:
    """0 = automatic kernel choice, 1 = force the generic direct kernels,
    2 = skip the shape-specialised kernels (general MFMA paths where they apply),
    3 = automatic, but convT_bn_avgpool's second algorithm (the output-phase classes on
        the matrix cores) where the swapped sums would apply,
    4 = automatic, but conv_transpose3d_fwd scatters into an LDS output tile,
    5 = automatic, but convT_bn_avgpool runs its one-thread-per-cell fp32 kernel,
    6 = automatic, but conv_transpose3d_fwd runs one output phase per workgroup
        (the per-phase kernel) wherever it applies.
    The setting is the calling thread's own (the library keeps it thread-local)."""
    return int(_lib().c3d_set_variant(int(variant)))


def conv3d_algo(x_shape, cout: int, params: ConvParams) -> str:
    """Name of the kernel conv3d_fwd would run for these arguments (host-only query)."""
    v = ctypes.c_int32(-1)
    _check(_lib().c3d_conv3d_algo(_shape5(x_shape), int(cout), ctypes.byref(params), ctypes.byref(v)),
           "c3d_conv3d_algo")
    return ALGO[v.value]


def convT_bn_avgpool_algo(x_shape, cout: int, params: ConvParams, pool: int) -> str:
    """Name of the kernel convT_bn_avgpool(_ex) would run for these arguments (host-only query)."""
    v = ctypes.c_int32(-1)
    _check(_lib().c3d_convT_bn_avgpool_algo(_shape5(x_shape), int(cout), ctypes.byref(params), int(pool),
                                            ctypes.byref(v)), "c3d_convT_bn_avgpool_algo")
    return ALGO[v.value]


def conv_transpose3d_algo(x_shape, cout: int, params: ConvParams) -> str:
    """Name of the kernel conv_transpose3d_fwd would run for these arguments (host-only query)."""
    v = ctypes.c_int32(-1)
    _check(_lib().c3d_conv_transpose3d_algo(_shape5(x_shape), int(cout), ctypes.byref(params), ctypes.byref(v)),
           "c3d_conv_transpose3d_algo")
    return ALGO[v.value]


def conv3d_out_dims(x_shape, cout: int, params: ConvParams) -> Tuple[int, ...]:
    ys = (ctypes.c_int64 * 5)()
    _check(_lib().c3d_conv3d_out_dims(_shape5(x_shape), int(cout), ctypes.byref(params), ys),
           "c3d_conv3d_out_dims")
    return tuple(int(v) for v in ys)


def conv_transpose3d_out_dims(x_shape, cout: int, params: ConvParams) -> Tuple[int, ...]:
    ys = (ctypes.c_int64 * 5)()
    _check(_lib().c3d_conv_transpose3d_out_dims(_shape5(x_shape), int(cout), ctypes.byref(params), ys),
           "c3d_conv_transpose3d_out_dims")
    return tuple(int(v) for v in ys)


def convT_bn_avgpool_out_dims(x_shape, cout: int, params: ConvParams, pool: int) -> Tuple[int, ...]:
    ys = (ctypes.c_int64 * 5)()
    _check(_lib().c3d_convT_bn_avgpool_out_dims(_shape5(x_shape), int(cout), ctypes.byref(params), int(pool), ys),
           "c3d_convT_bn_avgpool_out_dims")
    return tuple(int(v) for v in ys)


def conv_maxpool_lse_relu_out_dims(x_shape, cout: int, params: ConvParams, pool: int) -> Tuple[int, ...]:
    ys = (ctypes.c_int64 * 5)()
    _check(_lib().c3d_conv_maxpool_lse_relu_out_dims(_shape5(x_shape), int(cout), ctypes.byref(params),
                                                      int(pool), ys), "c3d_conv_maxpool_lse_relu_out_dims")
    return tuple(int(v) for v in ys)


def conv3d_fwd(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, stride: Int3 = 1,
               pad: Int3 = 0, dilation: Int3 = 1, groups: int = 1, out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """y = conv3d(x, w, bias); w is [Cout, Cin/groups, k0, k1, k2]."""
    cout = _conv_operands(x, w, groups, transposed=False)
    params = make_params(tuple(w.shape[2:]), stride, pad, dilation, 0, groups)
    ys = conv3d_out_dims(x.shape, cout, params)
    _vec(_tensor(bias, "bias", False), "bias", cout)
    out = _out(out, ys, x)
    ptr = _placed(x, w=w, bias=bias, out=out)
    _check(_lib().conv3d_fwd(ptr["x"], _shape5(x.shape), ptr["w"], cout, ctypes.byref(params), ptr["bias"],
                             ptr["out"], _stream(stream)), "conv3d_fwd")
    return out


def conv_transpose3d_fwd(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, stride: Int3 = 1,
                         pad: Int3 = 0, dilation: Int3 = 1, output_pad: Int3 = 0, groups: int = 1,
                         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = conv_transpose3d(x, w, bias); w is [Cin, Cout/groups, k0, k1, k2]."""
    cout = _conv_operands(x, w, groups, transposed=True)
    params = make_params(tuple(w.shape[2:]), stride, pad, dilation, output_pad, groups)
    ys = conv_transpose3d_out_dims(x.shape, cout, params)
    _vec(_tensor(bias, "bias", False), "bias", cout)
    out = _out(out, ys, x)
    ptr = _placed(x, w=w, bias=bias, out=out)
    _check(_lib().conv_transpose3d_fwd(ptr["x"], _shape5(x.shape), ptr["w"], cout, ctypes.byref(params),
                                       ptr["bias"], ptr["out"], _stream(stream)), "conv_transpose3d_fwd")
    return out


def convT_bn_avgpool_workspace_bytes(x_shape, cout: int, params: ConvParams, pool: int) -> int:
    return int(_lib().convT_bn_avgpool_workspace_bytes(_shape5(x_shape), int(cout), ctypes.byref(params),
                                                       int(pool)))


def convT_bn_avgpool(x: torch.Tensor, w: torch.Tensor, conv_bias: Optional[torch.Tensor], gamma: torch.Tensor,
                     beta: torch.Tensor, eps: float = 1e-5, pool: int = 4, stride: Int3 = 2, pad: Int3 = 1,
                     dilation: Int3 = 1, output_pad: Int3 = 0, groups: int = 1,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     batch_mean: Optional[torch.Tensor] = None, batch_var: Optional[torch.Tensor] = None,
                     stream=None, training: bool = True, momentum: float = 0.1,
                     running_mean: Optional[torch.Tensor] = None,
                     running_var: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ConvTranspose3d -> BatchNorm3d -> AvgPool3d(pool).  Training mode
    normalises with the batch statistics and, when running_mean/running_var
    are given, updates them in place; eval mode (training=False) normalises
    with them."""
    cout = _conv_operands(x, w, groups, transposed=True)
    params = make_params(tuple(w.shape[2:]), stride, pad, dilation, output_pad, groups)
    ys = convT_bn_avgpool_out_dims(x.shape, cout, params, pool)
    vecs = dict(conv_bias=_tensor(conv_bias, "conv_bias", False), gamma=_tensor(gamma, "gamma"),
                beta=_tensor(beta, "beta"), batch_mean=_tensor(batch_mean, "batch_mean", False),
                batch_var=_tensor(batch_var, "batch_var", False),
                running_mean=_tensor(running_mean, "running_mean", False),
                running_var=_tensor(running_var, "running_var", False))
    for name, t in vecs.items():
        _vec(t, name, cout)
    if (running_mean is None) != (running_var is None):
        raise ValueError("running_mean and running_var go together")
    if not training and running_mean is None:
        raise ValueError("eval mode (training=False) needs running_mean and running_var")
    out = _out(out, ys, x)
    if training:
        nbytes = convT_bn_avgpool_workspace_bytes(x.shape, cout, params, pool)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 8), dtype=torch.uint8, device=x.device)
        workspace = _workspace(workspace, nbytes)
    ptr = _placed(x, w=w, out=out, **vecs)
    if training:
        ws_ptr, ws_bytes = _workspace_ptr(workspace, x), workspace.numel() * workspace.element_size()
    else:
        ws_ptr, ws_bytes = None, 0
    head = (ptr["x"], _shape5(x.shape), ptr["w"], cout, ctypes.byref(params), ptr["conv_bias"], ptr["gamma"],
            ptr["beta"], float(eps), int(pool))
    tail = (ws_ptr, ws_bytes, ptr["batch_mean"], ptr["batch_var"], _stream(stream))
    if training and running_mean is None:
        _check(_lib().convT_bn_avgpool(*head, ptr["out"], *tail), "convT_bn_avgpool")
    else:
        _check(_lib().convT_bn_avgpool_ex(*head, int(bool(training)), float(momentum), ptr["running_mean"],
                                          ptr["running_var"], ptr["out"], *tail), "convT_bn_avgpool_ex")
    return out


def convT_bn_avgpool_noalloc(x: torch.Tensor, w: torch.Tensor, conv_bias: Optional[torch.Tensor],
                             gamma: torch.Tensor, beta: torch.Tensor, out: torch.Tensor, eps: float = 1e-5,
                             pool: int = 4, stride: Int3 = 2, pad: Int3 = 1, dilation: Int3 = 1,
                             output_pad: Int3 = 0, groups: int = 1, batch_mean: Optional[torch.Tensor] = None,
                             batch_var: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """convT_bn_avgpool (training mode, batch statistics) through the entry
    point that allocates nothing: its partials go to the library's static
    per-GPU scratch, and the caller passes `out`.  Calls that overlap on one
    GPU share that scratch and race."""
    cout = _conv_operands(x, w, groups, transposed=True)
    params = make_params(tuple(w.shape[2:]), stride, pad, dilation, output_pad, groups)
    ys = convT_bn_avgpool_out_dims(x.shape, cout, params, pool)
    vecs = dict(conv_bias=_tensor(conv_bias, "conv_bias", False), gamma=_tensor(gamma, "gamma"),
                beta=_tensor(beta, "beta"), batch_mean=_tensor(batch_mean, "batch_mean", False),
                batch_var=_tensor(batch_var, "batch_var", False))
    for name, t in vecs.items():
        _vec(t, name, cout)
    out = _tensor(out, "out")
    out = _out(out, ys, x)
    ptr = _placed(x, w=w, out=out, **vecs)
    _check(_lib().convT_bn_avgpool_noalloc(ptr["x"], _shape5(x.shape), ptr["w"], cout, ctypes.byref(params),
                                           ptr["conv_bias"], ptr["gamma"], ptr["beta"], float(eps), int(pool),
                                           ptr["out"], ptr["batch_mean"], ptr["batch_var"], _stream(stream)),
           "convT_bn_avgpool_noalloc")
    return out


def conv_maxpool_lse_relu(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, pool: int = 2,
                          stride: Int3 = 1, pad: Int3 = 1, dilation: Int3 = 1, groups: int = 1,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Conv3d -> MaxPool3d(pool) -> logsumexp over channels (keepdim) -> ReLU."""
    cout = _conv_operands(x, w, groups, transposed=False)
    params = make_params(tuple(w.shape[2:]), stride, pad, dilation, 0, groups)
    ys = conv_maxpool_lse_relu_out_dims(x.shape, cout, params, pool)
    _vec(_tensor(bias, "bias", False), "bias", cout)
    out = _out(out, ys, x)
    ptr = _placed(x, w=w, bias=bias, out=out)
    _check(_lib().conv_maxpool_lse_relu(ptr["x"], _shape5(x.shape), ptr["w"], cout, ctypes.byref(params),
                                        ptr["bias"], int(pool), ptr["out"], _stream(stream)),
           "conv_maxpool_lse_relu")
    return out
