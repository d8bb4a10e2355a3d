"""Fused fp32 convolutions for AMD MI355X (gfx950): a thin ctypes binding over
``libconvfuse.so``.

The binding only marshals arguments: it checks that tensors are contiguous fp32 on the
current GPU, allocates outputs with torch, and passes raw device pointers and the current
HIP stream to the C ABI declared in ``include/convfuse.h``.  Every arithmetic step runs in
the library's HIP kernels; there is no fallback path, and a missing or unloadable library
raises.
"""
from __future__ import annotations

import ctypes
import threading

from . import _build

__all__ = [
    "conv3d_mish_tanh", "conv3d_div_maxpool_gap_bias_sum", "conv3d_div_maxpool", "dwsep_conv2d",
    "conv3d_bias", "mish_tanh", "div_maxpool_gap_bias_sum", "depthwise_conv2d",
    "pointwise_conv2d", "dwsep_conv2d_split_bf16", "conv3d_mish_tanh_split_bf16",
    "conv3d_div_maxpool_gap_bias_sum_split_bf16", "conv_out_len", "out_dims_conv3d",
    "out_dims_conv2d", "build_id", "last_kernel", "measure_mfma",
    "ConvFuseError", "lib", "library_path", "EXPORTED_SYMBOLS",
]

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_DEVICE = 0, 1, 2, 3, 4
_ERR_NAMES = {ERR_NULL: "NULL", ERR_SHAPE: "SHAPE", ERR_UNSUPPORTED: "UNSUPPORTED",
              ERR_DEVICE: "DEVICE"}

EXPORTED_SYMBOLS = (
    "conv3d_mish_tanh", "conv3d_div_maxpool_gap_bias_sum", "conv3d_div_maxpool", "dwsep_conv2d",
    "conv3d_bias", "mish_tanh", "div_maxpool_gap_bias_sum", "depthwise_conv2d",
    "pointwise_conv2d", "dwsep_conv2d_split_bf16", "conv3d_mish_tanh_split_bf16",
    "conv3d_div_maxpool_gap_bias_sum_split_bf16",
    "convfuse_conv_out_len", "convfuse_out_dims_conv3d", "convfuse_out_dims_conv2d",
    "convfuse_build_id", "convfuse_last_kernel", "convfuse_last_error", "convfuse_abi_version",
    "convfuse_measure_mfma",
)

_lib = None
_lock = threading.Lock()
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class ConvFuseError(RuntimeError):
    def __init__(self, code, message):
        super().__init__("convfuse error %s (%d): %s" % (_ERR_NAMES.get(code, "?"), code, message))
        self.code = code


def library_path():
    return _build.LIB


def lib():
    """The loaded libconvfuse.so (built in-tree first if it does not exist yet).  Raises if
    the binary was compiled from other sources than the ones in this tree."""
    global _lib
    with _lock:
        if _lib is None:
            if not _build.LIB.exists():
                _build.build()
            L = ctypes.CDLL(str(_build.LIB))
            L.convfuse_build_id.restype = ctypes.c_char_p
            built, want = L.convfuse_build_id().decode(), _build.source_sha()
            if built != want:
                raise RuntimeError(
                    "%s was built from sources %s, but the tree holds %s: rebuild it "
                    "(python -m implicit_gemm_convolution_conv3d_amd._build)"
                    % (_build.LIB, built, want))
            L.conv3d_mish_tanh.argtypes = [_vp] * 4 + [_i64] * 9 + [_vp]
            L.conv3d_div_maxpool_gap_bias_sum.argtypes = (
                [_vp] * 3 + [ctypes.c_float, _i64, _vp, _vp] + [_i64] * 7 + [_vp])
            L.conv3d_div_maxpool.argtypes = (
                [_vp] * 3 + [ctypes.c_float, _i64, _vp] + [_i64] * 7 + [_vp])
            L.dwsep_conv2d.argtypes = [_vp] * 6 + [_i64] * 9 + [_vp]
            L.dwsep_conv2d_split_bf16.argtypes = [_vp] * 6 + [_i64] * 9 + [_vp]
            L.conv3d_mish_tanh_split_bf16.argtypes = [_vp] * 4 + [_i64] * 9 + [_vp]
            L.conv3d_div_maxpool_gap_bias_sum_split_bf16.argtypes = (
                [_vp] * 3 + [ctypes.c_float, _i64, _vp, _vp] + [_i64] * 7 + [_vp])
            L.conv3d_bias.argtypes = [_vp] * 4 + [_i64] * 9 + [_vp]
            L.mish_tanh.argtypes = [_vp, _vp, _i64, _vp]
            L.div_maxpool_gap_bias_sum.argtypes = (
                [_vp, ctypes.c_float, _i64, _vp, _vp] + [_i64] * 5 + [_vp])
            L.depthwise_conv2d.argtypes = [_vp] * 4 + [_i64] * 8 + [_vp]
            L.pointwise_conv2d.argtypes = [_vp] * 4 + [_i64] * 5 + [_vp]
            L.convfuse_conv_out_len.argtypes = [_i64] * 5 + [ctypes.POINTER(_i64)]
            L.convfuse_out_dims_conv3d.argtypes = [_i64] * 6 + [ctypes.POINTER(_i64)] * 3
            L.convfuse_out_dims_conv2d.argtypes = [_i64] * 6 + [ctypes.POINTER(_i64)] * 2
            L.convfuse_measure_mfma.argtypes = [_vp, _i64, _i64, _vp]
            L.convfuse_last_error.restype = ctypes.c_char_p
            L.convfuse_last_kernel.restype = ctypes.c_char_p
            L.convfuse_abi_version.restype = ctypes.c_int
            for name in ("conv3d_mish_tanh", "conv3d_div_maxpool_gap_bias_sum", "dwsep_conv2d",
                         "convfuse_conv_out_len"):
                getattr(L, name).restype = ctypes.c_int
            _lib = L
    return _lib


def _check(rc):
    if rc != OK:
        raise ConvFuseError(rc, lib().convfuse_last_error().decode(errors="replace"))


def measure_mfma(iters, workgroups, out):
    """Diagnostic fp32 matrix-core issue loop (see convfuse_measure_mfma); out: 1-element
    float32 CUDA tensor."""
    import torch
    with torch.cuda.device(out.device):
        _check(lib().convfuse_measure_mfma(_ptr(out, "out", (1,)), iters, workgroups,
                                           _stream(out)))
    return out


def conv_out_len(n, k, stride=1, pad=0, dilation=1):
    out = _i64()
    _check(lib().convfuse_conv_out_len(n, k, stride, pad, dilation, ctypes.byref(out)))
    return out.value


def out_dims_conv3d(D, H, W, k, stride=1, pad=0):
    """(OD, OH, OW) of a Conv3d (convfuse_out_dims_conv3d)."""
    o = [_i64() for _ in range(3)]
    _check(lib().convfuse_out_dims_conv3d(D, H, W, k, stride, pad, *map(ctypes.byref, o)))
    return tuple(v.value for v in o)


def out_dims_conv2d(H, W, K, stride=1, pad=0, dilation=1):
    """(Ho, Wo) of the depthwise step of a depthwise-separable Conv2d
    (convfuse_out_dims_conv2d)."""
    o = [_i64() for _ in range(2)]
    _check(lib().convfuse_out_dims_conv2d(H, W, K, stride, pad, dilation, *map(ctypes.byref, o)))
    return tuple(v.value for v in o)


def last_kernel():
    """Name of the last kernel this thread launched through the library."""
    return lib().convfuse_last_kernel().decode()


def build_id():
    """Source hash the loaded library was compiled from (convfuse_build_id)."""
    return lib().convfuse_build_id().decode()


def _ptr(t, name, shape=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32 (got %s)" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t.data_ptr() or None


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def conv3d_mish_tanh_split_bf16(x, w, b=None, stride=1, padding=0, out=None):
    """conv3d_mish_tanh with the implicit GEMM as a three-term bf16 split of fp32 (opt-in)."""
    return conv3d_mish_tanh(x, w, b, stride, padding, out, _entry="conv3d_mish_tanh_split_bf16")


def conv3d_mish_tanh(x, w, b=None, stride=1, padding=0, out=None, _entry="conv3d_mish_tanh"):
    """y = tanh(mish(conv3d(x, w) + b)); x [N,Cin,D,H,W], w [Cout,Cin,k,k,k], b [Cout]."""
    import torch
    N, C, D, H, W = x.shape
    O, C2, k = w.shape[0], w.shape[1], w.shape[2]
    if C2 != C or tuple(w.shape[2:]) != (k, k, k):
        raise ValueError("weight %s does not match input %s" % (tuple(w.shape), tuple(x.shape)))
    if b is not None and tuple(b.shape) != (O,):
        raise ValueError("bias must have shape (%d,)" % O)
    shp = (N, O) + out_dims_conv3d(D, H, W, k, stride, padding)
    if out is None:
        out = torch.empty(shp, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(getattr(lib(), _entry)(_ptr(x, "x"), _ptr(w, "w"), _ptr(b, "b"),
                                      _ptr(out, "out", shp), N, C, D, H, W, O, k, stride,
                                      padding, _stream(x)))
    return out


def conv3d_div_maxpool_gap_bias_sum_split_bf16(x, w, conv_b, divisor, pool, bias, out=None):
    """conv3d_div_maxpool_gap_bias_sum with the Conv3d as a three-term bf16 split (opt-in)."""
    return conv3d_div_maxpool_gap_bias_sum(x, w, conv_b, divisor, pool, bias, out,
                                           _entry="conv3d_div_maxpool_gap_bias_sum_split_bf16")


def conv3d_div_maxpool_gap_bias_sum(x, w, conv_b, divisor, pool, bias, out=None,
                                    _entry="conv3d_div_maxpool_gap_bias_sum"):
    """out[n] = sum_c(mean(maxpool((conv3d(x,w)+conv_b)/divisor)) + bias[c]); out [N]."""
    import torch
    N, C, D, H, W = x.shape
    O, C2, k = w.shape[0], w.shape[1], w.shape[2]
    if C2 != C or tuple(w.shape[2:]) != (k, k, k):
        raise ValueError("weight %s does not match input %s" % (tuple(w.shape), tuple(x.shape)))
    if conv_b is not None and tuple(conv_b.shape) != (O,):
        raise ValueError("conv_b must have shape (%d,)" % O)
    if bias.numel() != O:
        raise ValueError("bias must have %d elements" % O)
    if out is None:
        out = torch.empty((N,), dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(getattr(lib(), _entry)(
            _ptr(x, "x"), _ptr(w, "w"), _ptr(conv_b, "conv_b"), float(divisor), pool,
            _ptr(bias, "bias"), _ptr(out, "out", (N,)), N, C, D, H, W, O, k, _stream(x)))
    return out


def conv3d_div_maxpool(x, w, conv_b, divisor, pool, out=None):
    """y = maxpool_pool((conv3d(x,w)+conv_b)/divisor); y [N, Cout, PD, PH, PW]."""
    import torch
    N, C, D, H, W = x.shape
    O, C2, k = w.shape[0], w.shape[1], w.shape[2]
    if C2 != C or tuple(w.shape[2:]) != (k, k, k):
        raise ValueError("weight %s does not match input %s" % (tuple(w.shape), tuple(x.shape)))
    if conv_b is not None and tuple(conv_b.shape) != (O,):
        raise ValueError("conv_b must have shape (%d,)" % O)
    shp = (N, O) + tuple(conv_out_len(conv_out_len(s, k), pool, pool) for s in (D, H, W))
    if out is None:
        out = torch.empty(shp, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().conv3d_div_maxpool(
            _ptr(x, "x"), _ptr(w, "w"), _ptr(conv_b, "conv_b"), float(divisor), pool,
            _ptr(out, "out", shp), N, C, D, H, W, O, k, _stream(x)))
    return out


def dwsep_conv2d_split_bf16(x, dw_w, dw_b, pw_w, pw_b, stride=1, padding=1, dilation=1,
                            out=None):
    """dwsep_conv2d with the pointwise GEMM as a three-term bf16 split of fp32 (opt-in)."""
    return dwsep_conv2d(x, dw_w, dw_b, pw_w, pw_b, stride, padding, dilation, out,
                        _entry="dwsep_conv2d_split_bf16")


def dwsep_conv2d(x, dw_w, dw_b, pw_w, pw_b, stride=1, padding=1, dilation=1, out=None,
                 _entry="dwsep_conv2d"):
    """y = pointwise(depthwise(x)); x [N,Cin,H,W], dw_w [Cin,1,K,K], pw_w [Cout,Cin,1,1]."""
    import torch
    N, C, H, W = x.shape
    K = dw_w.shape[-1]
    O = pw_w.shape[0]
    if tuple(dw_w.shape) != (C, 1, K, K) or tuple(pw_w.shape) != (O, C, 1, 1):
        raise ValueError("weights %s / %s do not match input %s"
                         % (tuple(dw_w.shape), tuple(pw_w.shape), tuple(x.shape)))
    if dw_b is not None and tuple(dw_b.shape) != (C,):
        raise ValueError("dw_b must have shape (%d,)" % C)
    if pw_b is not None and tuple(pw_b.shape) != (O,):
        raise ValueError("pw_b must have shape (%d,)" % O)
    shp = (N, O) + out_dims_conv2d(H, W, K, stride, padding, dilation)
    if out is None:
        out = torch.empty(shp, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(getattr(lib(), _entry)(_ptr(x, "x"), _ptr(dw_w, "dw_w"), _ptr(dw_b, "dw_b"),
                                  _ptr(pw_w, "pw_w"), _ptr(pw_b, "pw_b"), _ptr(out, "out", shp),
                                  N, C, H, W, O, K, stride, padding, dilation, _stream(x)))
    return out


# ----------------------------------------------------------------- unfused path steps
def conv3d_bias(x, w, b=None, stride=1, padding=0, out=None):
    """y = conv3d(x, w) + b (the unfused path's convolution); y [N, Cout, OD, OH, OW]."""
    import torch
    N, C, D, H, W = x.shape
    O, C2, k = w.shape[0], w.shape[1], w.shape[2]
    if C2 != C or tuple(w.shape[2:]) != (k, k, k):
        raise ValueError("weight %s does not match input %s" % (tuple(w.shape), tuple(x.shape)))
    if b is not None and tuple(b.shape) != (O,):
        raise ValueError("bias must have shape (%d,)" % O)
    shp = (N, O) + out_dims_conv3d(D, H, W, k, stride, padding)
    if out is None:
        out = torch.empty(shp, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().conv3d_bias(_ptr(x, "x"), _ptr(w, "w"), _ptr(b, "b"), _ptr(out, "out", shp),
                                 N, C, D, H, W, O, k, stride, padding, _stream(x)))
    return out


def mish_tanh(v, out=None):
    """y = tanh(mish(v)) elementwise (out may be v)."""
    import torch
    if out is None:
        out = torch.empty_like(v)
    with torch.cuda.device(v.device):
        _check(lib().mish_tanh(_ptr(v, "v"), _ptr(out, "out", tuple(v.shape)), v.numel(),
                               _stream(v)))
    return out


def div_maxpool_gap_bias_sum(conv, divisor, pool, bias, out=None):
    """out[n] = sum_c(mean(maxpool(conv/divisor)) + bias[c]) from a stored conv output."""
    import torch
    N, C, OD, OH, OW = conv.shape
    if bias.numel() != C:
        raise ValueError("bias must have %d elements" % C)
    if out is None:
        out = torch.empty((N,), dtype=torch.float32, device=conv.device)
    with torch.cuda.device(conv.device):
        _check(lib().div_maxpool_gap_bias_sum(_ptr(conv, "conv"), float(divisor), pool,
                                              _ptr(bias, "bias"), _ptr(out, "out", (N,)),
                                              N, C, OD, OH, OW, _stream(conv)))
    return out


def depthwise_conv2d(x, dw_w, dw_b=None, stride=1, padding=1, dilation=1, out=None):
    """y = depthwise conv of x (+ dw_b); y [N, C, Ho, Wo]."""
    import torch
    N, C, H, W = x.shape
    K = dw_w.shape[-1]
    if tuple(dw_w.shape) != (C, 1, K, K):
        raise ValueError("dw_w %s does not match input %s" % (tuple(dw_w.shape), tuple(x.shape)))
    shp = (N, C) + out_dims_conv2d(H, W, K, stride, padding, dilation)
    if out is None:
        out = torch.empty(shp, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().depthwise_conv2d(_ptr(x, "x"), _ptr(dw_w, "dw_w"), _ptr(dw_b, "dw_b"),
                                      _ptr(out, "out", shp), N, C, H, W, K, stride, padding,
                                      dilation, _stream(x)))
    return out


def pointwise_conv2d(x, pw_w, pw_b=None, out=None):
    """y = 1x1 conv of x (+ pw_b); x [N, Cin, H, W] -> y [N, Cout, H, W]."""
    import torch
    N, C, H, W = x.shape
    O = pw_w.shape[0]
    if tuple(pw_w.shape) != (O, C, 1, 1):
        raise ValueError("pw_w %s does not match input %s" % (tuple(pw_w.shape), tuple(x.shape)))
    shp = (N, O, H, W)
    if out is None:
        out = torch.empty(shp, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().pointwise_conv2d(_ptr(x, "x"), _ptr(pw_w, "pw_w"), _ptr(pw_b, "pw_b"),
                                      _ptr(out, "out", shp), N, C, H, W, O, _stream(x)))
    return out
