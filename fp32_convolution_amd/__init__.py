"""fp32_convolution_amd: Python binding of libfconv (fused fp32 convolutions, MI355X / gfx950).

Argument marshalling only: every function checks dtype, device and layout,
then calls the C ABI of ``libfconv.so`` (declared in ``include/fconv.h``) with
raw device pointers and torch's current HIP stream.  All arithmetic runs in
the library's HIP kernels.  There is no fallback: if the library is missing,
importing this package raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfconv.so")

FCONV_OK = 0
FCONV_EINVAL = -1
FCONV_EUNSUPPORTED = -2
FCONV_EHIP = -3
FCONV_ESCRATCH = -4
NOALLOC_MAX_PARTIALS = 1 << 18

ALGO_AUTO = 0
ALGO_DIRECT_MFMA = 1
ALGO_DIRECT_SIMPLE = 2
ALGO_BOXSUM = 3

POOL_AVG = 0
POOL_MAX = 1
RELU = 1
CEIL_MODE = 2

DWSEP_AUTO = 0
DWSEP_SEPARABLE = 1
DWSEP_DENSE = 2

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libfconv.so not found at {LIB_PATH}; build it first with `python fp32_convolution_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i64p = ctypes.POINTER(ctypes.c_int64)
_SIGS = {
    "fconv2d_pool_sigmoid_sum": ([_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _vp], ctypes.c_int),
    "fconv2d_pool_sigmoid_sum_algo": (
        [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, ctypes.c_int, _vp, _vp], ctypes.c_int),
    "fconv2d_pool_map": (
        [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, ctypes.c_int, _vp, _vp], ctypes.c_int),
    "fconv2d_pool_debug_map": ([_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _vp], ctypes.c_int),
    "fconv2d_pool_sigmoid_sum_det": (
        [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, ctypes.c_int, _vp, ctypes.c_size_t, _vp, _vp],
        ctypes.c_int),
    "fconv2d_pool_sigmoid_sum_det_noalloc": (
        [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, ctypes.c_int, _vp, _vp], ctypes.c_int),
    "fconv2d_pool_sigmoid_sum_det_workspace": (
        [_i64, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "fconv2d_pool_out_size": ([_i64, _i64, _i64, _i64, _i64p, _i64p], ctypes.c_int),
    "fconv2d_pool_sigmoid_sum_ex": (
        [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp],
        ctypes.c_int),
    "fconv2d_pool_map_ex": (
        [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp],
        ctypes.c_int),
    "fconv2d_pool_out_size_ex": ([_i64, _i64, _i64, _i64, ctypes.c_int, _i64p, _i64p], ctypes.c_int),
    "fconv2d_pool_sigmoid_sum_det_ex": (
        [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp,
         ctypes.c_size_t, _vp, _vp], ctypes.c_int),
    "fconv2d_pool_sigmoid_sum_det_workspace_ex": (
        [_i64, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
         ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "fconv2d_select_algo": ([_i64, _i64, _i64, _i64], ctypes.c_int),
    "dwsep_conv1d": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp], ctypes.c_int),
    "dwsep_conv1d_out_len": ([_i64, _i64, _i64], ctypes.c_int64),
    "dwsep_conv1d_ex": (
        [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _vp], ctypes.c_int),
    "dwsep_conv1d_out_len_ex": ([_i64, _i64, _i64, _i64, _i64], ctypes.c_int64),
    "dwsep_conv1d_algo": (
        [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, ctypes.c_int, _vp, _vp], ctypes.c_int),
    "fconv_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "fconv_version": ([], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class FconvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.fconv_strerror(status).decode()} ({status})")


def _check(rc: int, what: str) -> None:
    if rc != FCONV_OK:
        raise FconvError(rc, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_f32(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# torch's current stream on a device as a raw handle: the private accessor
# skips building a Stream object (a few microseconds a call, which is most
# of a small call's cost); the public one is the fallback.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _call(t, fn, *args):
    """Calls fn(*args, stream) with t's device current (switching only when
    another one is) and that device's current torch stream."""
    idx = t.get_device()
    st = ctypes.c_void_p(_raw_stream(idx) if _raw_stream is not None else torch.cuda.current_stream(idx).cuda_stream)
    if idx == torch.cuda.current_device():
        return fn(*args, st)
    with torch.cuda.device(idx):
        return fn(*args, st)


def version() -> int:
    return lib.fconv_version()


def _pool_flags(relu: bool, ceil_mode: bool) -> int:
    return (RELU if relu else 0) | (CEIL_MODE if ceil_mode else 0)


def conv2d_out_size(H: int, W: int, K: int, pool: int, ceil_mode: bool = False):
    ph, pw = ctypes.c_int64(), ctypes.c_int64()
    if ceil_mode:
        _check(lib.fconv2d_pool_out_size_ex(H, W, K, pool, CEIL_MODE, ctypes.byref(ph), ctypes.byref(pw)),
               "fconv2d_pool_out_size_ex")
    else:
        _check(lib.fconv2d_pool_out_size(H, W, K, pool, ctypes.byref(ph), ctypes.byref(pw)), "fconv2d_pool_out_size")
    return ph.value, pw.value


def conv2d_select_algo(Cin: int, Cout: int, K: int, pool: int) -> int:
    return lib.fconv2d_select_algo(Cin, Cout, K, pool)


def _conv2d_args(x, w, b):
    _dev_f32(x, "x")
    _dev_f32(w, "w")
    if b is not None:
        _dev_f32(b, "bias")
    if x.dim() != 4 or w.dim() != 4 or w.shape[2] != w.shape[3] or w.shape[1] != x.shape[1]:
        raise ValueError(f"expected x[B,Cin,H,W] and w[Cout,Cin,K,K], got {tuple(x.shape)} and {tuple(w.shape)}")
    if b is not None and tuple(b.shape) != (w.shape[0],):
        raise ValueError(f"bias must be [Cout]={w.shape[0]}, got {tuple(b.shape)}")
    d = x.get_device()
    if w.get_device() != d or (b is not None and b.get_device() != d):
        raise ValueError("x, w and bias must be on the same device")


def conv2d_pool_sigmoid_sum(x, w, b, pool: int, out=None, algo: int = ALGO_AUTO, pool_mode: int = POOL_AVG,
                            relu: bool = False, ceil_mode: bool = False):
    """Conv2d(stride 1, no pad) -> [ReLU] -> AvgPool2d or MaxPool2d(pool, floor or ceil) -> sigmoid -> sum
    over (C,H,W): out[B].  The defaults are the plain chain (average pool, no ReLU, floor).  The sum's
    partials take scratch the library keeps per stream (else from its stream-ordered pool); repeated calls give identical bits."""
    _conv2d_args(x, w, b)
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    if out is None:
        out = torch.empty(B, dtype=torch.float32, device=x.device)
    else:
        _dev_f32(out, "out")
        if tuple(out.shape) != (B,) or out.get_device() != x.get_device():
            raise ValueError("out must be [B] on x's device")
    flags = _pool_flags(relu, ceil_mode)
    if pool_mode == POOL_AVG and flags == 0:
        rc = _call(x, lib.fconv2d_pool_sigmoid_sum_algo, _ptr(x), B, Cin, H, W, _ptr(w), Cout, K, _ptr(b), pool, algo,
                   _ptr(out))
    else:
        rc = _call(x, lib.fconv2d_pool_sigmoid_sum_ex, _ptr(x), B, Cin, H, W, _ptr(w), Cout, K, _ptr(b), pool,
                   pool_mode, flags, algo, _ptr(out))
    _check(rc, "fconv2d_pool_sigmoid_sum")
    return out


def conv2d_det_workspace_bytes(B, Cin, H, W, Cout, K, pool, algo: int = ALGO_AUTO, pool_mode: int = POOL_AVG,
                               relu: bool = False, ceil_mode: bool = False) -> int:
    n = ctypes.c_size_t()
    flags = _pool_flags(relu, ceil_mode)
    if pool_mode == POOL_AVG and flags == 0:
        _check(lib.fconv2d_pool_sigmoid_sum_det_workspace(B, Cin, H, W, Cout, K, pool, algo, ctypes.byref(n)),
               "fconv2d_pool_sigmoid_sum_det_workspace")
    else:
        _check(lib.fconv2d_pool_sigmoid_sum_det_workspace_ex(B, Cin, H, W, Cout, K, pool, pool_mode, flags, algo,
                                                             ctypes.byref(n)),
               "fconv2d_pool_sigmoid_sum_det_workspace_ex")
    return n.value


def conv2d_pool_sigmoid_sum_det(x, w, b, pool: int, out=None, algo: int = ALGO_AUTO, workspace=None,
                                pool_mode: int = POOL_AVG, relu: bool = False, ceil_mode: bool = False):
    """conv2d_pool_sigmoid_sum with a caller-owned workspace for its partial sums (same kernels, same
    fixed-order reduction, same bits).

    workspace: a device tensor of at least conv2d_det_workspace_bytes() bytes,
    or None to allocate one here.
    """
    _conv2d_args(x, w, b)
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    if out is None:
        out = torch.empty(B, dtype=torch.float32, device=x.device)
    else:
        _dev_f32(out, "out")
        if tuple(out.shape) != (B,) or out.get_device() != x.get_device():
            raise ValueError("out must be [B] on x's device")
    need = conv2d_det_workspace_bytes(B, Cin, H, W, Cout, K, pool, algo, pool_mode, relu, ceil_mode)
    if workspace is None:
        workspace = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=x.device)
    if not workspace.is_cuda or workspace.get_device() != x.get_device() or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on x's device")
    nbytes = workspace.numel() * workspace.element_size()
    flags = _pool_flags(relu, ceil_mode)
    if pool_mode == POOL_AVG and flags == 0:
        rc = _call(x, lib.fconv2d_pool_sigmoid_sum_det, _ptr(x), B, Cin, H, W, _ptr(w), Cout, K, _ptr(b), pool, algo,
                   _ptr(workspace), nbytes, _ptr(out))
    else:
        rc = _call(x, lib.fconv2d_pool_sigmoid_sum_det_ex, _ptr(x), B, Cin, H, W, _ptr(w), Cout, K, _ptr(b), pool,
                   pool_mode, flags, algo, _ptr(workspace), nbytes, _ptr(out))
    _check(rc, "fconv2d_pool_sigmoid_sum_det")
    return out


def conv2d_pool_sigmoid_sum_det_noalloc(x, w, b, pool: int, out, algo: int = ALGO_AUTO):
    """conv2d_pool_sigmoid_sum_det with its partials in the library's fixed per-GPU array: no
    allocation anywhere in the call (`out` must be given).  Calls that overlap in time on one GPU
    race; see include/fconv.h."""
    _conv2d_args(x, w, b)
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    _dev_f32(out, "out")
    if tuple(out.shape) != (B,) or out.get_device() != x.get_device():
        raise ValueError("out must be [B] on x's device")
    rc = _call(x, lib.fconv2d_pool_sigmoid_sum_det_noalloc, _ptr(x), B, Cin, H, W, _ptr(w), Cout, K, _ptr(b), pool,
               algo, _ptr(out))
    _check(rc, "fconv2d_pool_sigmoid_sum_det_noalloc")
    return out


def conv2d_pool_map(x, w, b, pool: int, out=None, algo: int = ALGO_AUTO, pool_mode: int = POOL_AVG,
                    relu: bool = False, ceil_mode: bool = False):
    """Pre-sigmoid pooled map [B,Cout,PH,PW] of the same fused computation."""
    _conv2d_args(x, w, b)
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    PH, PW = conv2d_out_size(H, W, K, pool, ceil_mode)
    if out is None:
        out = torch.empty((B, Cout, PH, PW), dtype=torch.float32, device=x.device)
    else:
        _dev_f32(out, "out")
        if tuple(out.shape) != (B, Cout, PH, PW) or out.get_device() != x.get_device():
            raise ValueError("out must be [B,Cout,PH,PW] on x's device")
    flags = _pool_flags(relu, ceil_mode)
    if pool_mode == POOL_AVG and flags == 0:
        rc = _call(x, lib.fconv2d_pool_map, _ptr(x), B, Cin, H, W, _ptr(w), Cout, K, _ptr(b), pool, algo, _ptr(out))
    else:
        rc = _call(x, lib.fconv2d_pool_map_ex, _ptr(x), B, Cin, H, W, _ptr(w), Cout, K, _ptr(b), pool, pool_mode,
                   flags, algo, _ptr(out))
    _check(rc, "fconv2d_pool_map")
    return out


def dwsep_out_len(T: int, K: int, pad: int, stride: int = 1, dilation: int = 1) -> int:
    return int(lib.dwsep_conv1d_out_len_ex(T, K, pad, stride, dilation))


def dwsep_conv1d(x, w_dw, w_pw, b_pw, pad: int, out=None, stride: int = 1, dilation: int = 1,
                 algo: int = DWSEP_AUTO):
    """Depthwise Conv1d(K, pad, stride, dilation) -> pointwise 1x1 Conv1d + bias: y[B,O,Tout].

    w_dw may be [C,K] or PyTorch's [C,1,K]; w_pw [O,C] or [O,C,1].
    """
    _dev_f32(x, "x")
    _dev_f32(w_dw, "w_dw")
    _dev_f32(w_pw, "w_pw")
    if b_pw is not None:
        _dev_f32(b_pw, "b_pw")
    if w_dw.dim() == 3 and w_dw.shape[1] == 1:
        w_dw = w_dw.view(w_dw.shape[0], w_dw.shape[2])
    if w_pw.dim() == 3 and w_pw.shape[2] == 1:
        w_pw = w_pw.view(w_pw.shape[0], w_pw.shape[1])
    if x.dim() != 3 or w_dw.dim() != 2 or w_pw.dim() != 2 or w_dw.shape[0] != x.shape[1] or \
            w_pw.shape[1] != x.shape[1]:
        raise ValueError(f"expected x[B,C,T], w_dw[C,K], w_pw[O,C]; got {tuple(x.shape)}, "
                         f"{tuple(w_dw.shape)}, {tuple(w_pw.shape)}")
    B, C, T = x.shape
    K = w_dw.shape[1]
    O = w_pw.shape[0]
    if b_pw is not None and tuple(b_pw.shape) != (O,):
        raise ValueError(f"b_pw must be [O]={O}")
    d = x.get_device()
    for t in (w_dw, w_pw, b_pw, out):
        if t is not None and t.get_device() != d:
            raise ValueError("all tensors must be on x's device")
    Tout = dwsep_out_len(T, K, pad, stride, dilation)
    if Tout < 1:
        raise FconvError(FCONV_EINVAL, "dwsep_conv1d")
    if out is None:
        out = torch.empty((B, O, Tout), dtype=torch.float32, device=x.device)
    else:
        _dev_f32(out, "out")
        if tuple(out.shape) != (B, O, Tout):
            raise ValueError(f"out must be [B,O,Tout]=({B},{O},{Tout})")
    rc = _call(x, lib.dwsep_conv1d_algo, _ptr(x), B, C, T, _ptr(w_dw), K, _ptr(w_pw), O, _ptr(b_pw), pad, stride,
               dilation, algo, _ptr(out))
    _check(rc, "dwsep_conv1d")
    return out
