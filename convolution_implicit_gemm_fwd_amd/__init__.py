"""MI355X-native 2-D convolution forward as an implicit GEMM.

NHWC input, OHWI weight, fp32 bias and fp32 NHWC output; bf16 (or fp32)
inputs; hand-written HIP kernels for gfx950 behind the C ABI of
include/convimg.h.  ``abi`` is the ctypes binding of that ABI (same names);
``conv2d_nhwc`` below wraps it for torch tensors, using torch only for device
memory and the current stream; ``conv2d_bwd_data_nhwc`` and
``conv2d_bwd_weight_nhwc`` do the same for the gradients with respect to the
input (stride 1) and to the weights, and ``conv2d_nchw`` for NCHW / OIHW
tensors with an fp32 or bf16 output.

Importing the package loads nothing; the HIP library is loaded on first use
and its absence is an error (there is no fallback path).
"""
from __future__ import annotations

from . import abi
from .abi import (CONVIMG_BF16, CONVIMG_FP32, LibraryMissing, conv2d_bwd_data,
                  conv2d_bwd_data_weights, conv2d_bwd_weight, conv2d_bwd_weight_workspace,
                  conv2d_fwd, conv2d_fwd_autotune, conv2d_fwd_autotune_clear, conv2d_fwd_force,
                  conv2d_fwd_nchw, conv2d_fwd_nchw_workspace, conv2d_fwd_num_tiles, conv2d_fwd_out_dim,
                  conv2d_fwd_plan, conv2d_fwd_status, conv2d_fwd_test_spin_limit, conv2d_release,
                  conv2d_strerror)

__all__ = ["abi", "conv2d_nhwc", "conv2d_bwd_data_nhwc", "conv2d_bwd_weight_nhwc",
           "conv2d_bwd_data", "conv2d_bwd_data_weights", "conv2d_bwd_weight",
           "conv2d_bwd_weight_workspace", "conv2d_fwd", "conv2d_fwd_autotune",
           "conv2d_fwd_autotune_clear", "conv2d_fwd_nchw", "conv2d_fwd_nchw_workspace", "conv2d_nchw",
           "conv2d_fwd_out_dim", "conv2d_fwd_plan", "conv2d_strerror", "conv2d_fwd_force",
           "conv2d_fwd_num_tiles", "conv2d_fwd_status", "conv2d_fwd_test_spin_limit", "conv2d_release", "CONVIMG_BF16", "CONVIMG_FP32", "LibraryMissing"]


def _stream_of(stream, device):
    """(raw stream pointer, whether it is torch's current stream on device)."""
    import torch

    cur = torch.cuda.current_stream(device).cuda_stream
    if stream is None:
        return cur, True
    return stream, stream == cur


def _keep_for_stream(tensors, stream, device):
    """Buffers allocated here on torch's current stream but used by work on
    another stream: tell the caching allocator, so that it does not hand
    their memory out again until that stream has run the work."""
    import torch

    ext = torch.cuda.ExternalStream(stream, device=device)
    for t in tensors:
        if t is not None:
            t.record_stream(ext)


def _dtype_of(a, b, what):
    import torch

    if a.dtype == torch.bfloat16 and b.dtype == torch.bfloat16:
        return CONVIMG_BF16
    if a.dtype == torch.float32 and b.dtype == torch.float32:
        return CONVIMG_FP32
    raise TypeError("%s must both be bfloat16 or both float32" % what)


def conv2d_nhwc(x, w, bias=None, stride=1, pad=0, dilation=1, out=None, stream=None):
    """out[N,OH,OW,OC] (fp32) = conv2d(x[N,H,W,IC], w[OC,KH,KW,IC]) + bias[OC].

    x and w: contiguous CUDA (HIP) tensors, both bfloat16 or both float32.
    bias: contiguous float32 [OC] or None.  out: optional preallocated
    float32 [N,OH,OW,OC].  Runs on ``stream`` (default: torch's current
    stream of x's device) and returns without waiting.
    """
    import torch

    dtype = _dtype_of(x, w, "x and w")
    if not (x.is_cuda and w.is_cuda):
        raise ValueError("x and w must be device tensors")
    if x.dim() != 4 or w.dim() != 4 or x.shape[3] != w.shape[3]:
        raise ValueError("x must be [N,H,W,IC] and w [OC,KH,KW,IC]")
    if not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x and w must be contiguous (NHWC / OHWI)")
    N, H, W, IC = x.shape
    OC, KH, KW, _ = w.shape
    if bias is not None:
        if bias.dtype != torch.float32 or not bias.is_cuda or bias.numel() != OC \
                or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous float32 device tensor of OC values")
    OH = conv2d_fwd_out_dim(H, KH, stride, pad, dilation)
    OW = conv2d_fwd_out_dim(W, KW, stride, pad, dilation)
    if OH <= 0 or OW <= 0:
        raise ValueError("no output pixel for this shape")
    fresh = []
    if out is None:
        out = torch.empty((N, OH, OW, OC), dtype=torch.float32, device=x.device)
        fresh.append(out)
    elif (tuple(out.shape) != (N, OH, OW, OC) or out.dtype != torch.float32
          or not out.is_contiguous() or not out.is_cuda):
        raise ValueError("out must be a contiguous float32 [N,OH,OW,OC] device tensor")
    stream, current = _stream_of(stream, x.device)
    with torch.cuda.device(x.device):
        rc = conv2d_fwd(x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else None,
                        N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out.data_ptr(),
                        stream)
    if rc != 0:
        raise RuntimeError("conv2d_fwd failed: %s (status %d)" % (conv2d_strerror(rc), rc))
    if not current:
        _keep_for_stream(fresh, stream, x.device)
    return out


def conv2d_bwd_data_nhwc(dy, w, H, W, stride=1, pad=0, dilation=1, dx=None, wt=None,
                         stream=None):
    """dx[N,H,W,IC] (fp32): gradient of conv2d_nhwc's output with respect to x.

    dy: contiguous [N,OH,OW,OC] device tensor (the output gradient), w: the
    forward weights [OC,KH,KW,IC]; both bfloat16 or both float32.  H, W,
    stride, pad, dilation: the forward problem (any stride, window and padding).
    wt: optional workspace of w's numel and dtype that receives the flipped,
    transposed weights [IC,KH,KW,OC]; dx: optional preallocated output.  Runs
    on ``stream`` (default: torch's current stream) without waiting.
    """
    import torch

    dtype = _dtype_of(dy, w, "dy and w")
    if not (dy.is_cuda and w.is_cuda):
        raise ValueError("dy and w must be device tensors")
    if dy.dim() != 4 or w.dim() != 4 or dy.shape[3] != w.shape[0]:
        raise ValueError("dy must be [N,OH,OW,OC] and w [OC,KH,KW,IC]")
    if not (dy.is_contiguous() and w.is_contiguous()):
        raise ValueError("dy and w must be contiguous (NHWC / OHWI)")
    N, OH, OW, OC = dy.shape
    _, KH, KW, IC = w.shape
    if (conv2d_fwd_out_dim(H, KH, stride, pad, dilation) != OH
            or conv2d_fwd_out_dim(W, KW, stride, pad, dilation) != OW):
        raise ValueError("dy's extent is not the forward output extent of H x W")
    fresh = []
    if wt is None:
        wt = torch.empty(w.numel(), dtype=w.dtype, device=w.device)
        fresh.append(wt)
    elif (wt.numel() != w.numel() or wt.dtype != w.dtype or not wt.is_contiguous()
          or not wt.is_cuda):
        raise ValueError("wt must be a contiguous device tensor of w's size and dtype")
    if dx is None:
        dx = torch.empty((N, H, W, IC), dtype=torch.float32, device=dy.device)
        fresh.append(dx)
    elif (tuple(dx.shape) != (N, H, W, IC) or dx.dtype != torch.float32
          or not dx.is_contiguous() or not dx.is_cuda):
        raise ValueError("dx must be a contiguous float32 [N,H,W,IC] device tensor")
    stream, current = _stream_of(stream, dy.device)
    with torch.cuda.device(dy.device):
        rc = conv2d_bwd_data(dy.data_ptr(), w.data_ptr(), N, H, W, IC, OC, KH, KW, stride, pad,
                             dilation, dtype, wt.data_ptr(), dx.data_ptr(), stream)
    if rc != 0:
        raise RuntimeError("conv2d_bwd_data failed: %s (status %d)" % (conv2d_strerror(rc), rc))
    if not current:
        _keep_for_stream(fresh, stream, dy.device)
    return dx


def conv2d_bwd_weight_nhwc(x, dy, KH, KW, stride=1, pad=0, dilation=1, dw=None, ws=None,
                           stream=None):
    """dw[OC,KH,KW,IC] (fp32): gradient of conv2d_nhwc's output with respect to w.

    x: contiguous [N,H,W,IC] device tensor, dy: contiguous [N,OH,OW,OC] (the
    output gradient), both bfloat16 or both float32 (fp32 storage: the fp32
    kernel); KH, KW, stride, pad, dilation: the
    forward problem.  ws: optional uint8 device workspace of at least
    ``conv2d_bwd_weight_workspace`` bytes (allocated here when needed and not
    given); dw: optional preallocated output.  Runs on ``stream`` (default:
    torch's current stream) without waiting.
    """
    import torch

    if x.dtype != dy.dtype or x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("the weight backward takes x and dy both bfloat16 or both float32")
    dtype = CONVIMG_BF16 if x.dtype == torch.bfloat16 else CONVIMG_FP32
    if not (x.is_cuda and dy.is_cuda):
        raise ValueError("x and dy must be device tensors")
    if x.dim() != 4 or dy.dim() != 4 or x.shape[0] != dy.shape[0]:
        raise ValueError("x must be [N,H,W,IC] and dy [N,OH,OW,OC]")
    if not (x.is_contiguous() and dy.is_contiguous()):
        raise ValueError("x and dy must be contiguous (NHWC)")
    N, H, W, IC = x.shape
    _, OH, OW, OC = dy.shape
    if (conv2d_fwd_out_dim(H, KH, stride, pad, dilation) != OH
            or conv2d_fwd_out_dim(W, KW, stride, pad, dilation) != OW):
        raise ValueError("dy's extent is not the forward output extent of H x W")
    with torch.cuda.device(x.device):
        rc, need = conv2d_bwd_weight_workspace(N, H, W, IC, OC, KH, KW, stride, pad, dilation,
                                               dtype)
        if rc != 0:
            raise RuntimeError("conv2d_bwd_weight_workspace failed: %s (status %d)"
                               % (conv2d_strerror(rc), rc))
        fresh = []
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
            fresh.append(ws)
        if dw is None:
            dw = torch.empty((OC, KH, KW, IC), dtype=torch.float32, device=x.device)
            fresh.append(dw)
        elif (tuple(dw.shape) != (OC, KH, KW, IC) or dw.dtype != torch.float32
              or not dw.is_contiguous() or not dw.is_cuda):
            raise ValueError("dw must be a contiguous float32 [OC,KH,KW,IC] device tensor")
        stream, current = _stream_of(stream, x.device)
        ws_ptr = ws.data_ptr() if ws is not None else None
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
        rc = conv2d_bwd_weight(x.data_ptr(), dy.data_ptr(), N, H, W, IC, OC, KH, KW, stride, pad,
                               dilation, dtype, dw.data_ptr(), ws_ptr, ws_bytes, stream)
    if rc != 0:
        raise RuntimeError("conv2d_bwd_weight failed: %s (status %d)" % (conv2d_strerror(rc), rc))
    if not current:
        _keep_for_stream(fresh, stream, x.device)
    return dw


def conv2d_nchw(x, w, bias=None, stride=1, pad=0, dilation=1, out_dtype=None, out=None, ws=None,
                stream=None):
    """out[N,OC,OH,OW] = conv2d(x[N,IC,H,W], w[OC,IC,KH,KW]) + bias[OC], NCHW.

    x and w: contiguous device tensors, both bfloat16 or both float32.
    out_dtype: torch.float32 (default) or torch.bfloat16 (the fp32 result
    rounded to nearest even).  ws: optional uint8 workspace of at least
    ``conv2d_fwd_nchw_workspace`` bytes (allocated here when not given).
    Runs on ``stream`` (default: torch's current stream) without waiting.
    """
    import torch

    dtype = _dtype_of(x, w, "x and w")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if not (x.is_cuda and w.is_cuda):
        raise ValueError("x and w must be device tensors")
    if x.dim() != 4 or w.dim() != 4 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [N,IC,H,W] and w [OC,IC,KH,KW]")
    if not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x and w must be contiguous (NCHW / OIHW)")
    N, IC, H, W = x.shape
    OC, _, KH, KW = w.shape
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_cuda
                             or bias.numel() != OC or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 device tensor of OC values")
    OH = conv2d_fwd_out_dim(H, KH, stride, pad, dilation)
    OW = conv2d_fwd_out_dim(W, KW, stride, pad, dilation)
    if OH <= 0 or OW <= 0:
        raise ValueError("no output pixel for this shape")
    with torch.cuda.device(x.device):
        rc, need = conv2d_fwd_nchw_workspace(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype)
        if rc != 0:
            raise RuntimeError("conv2d_fwd_nchw_workspace failed: %s (status %d)"
                               % (conv2d_strerror(rc), rc))
        fresh = []
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
            fresh.append(ws)
        if out is None:
            out = torch.empty((N, OC, OH, OW), dtype=out_dtype, device=x.device)
            fresh.append(out)
        elif (tuple(out.shape) != (N, OC, OH, OW) or out.dtype != out_dtype
              or not out.is_contiguous() or not out.is_cuda):
            raise ValueError("out must be a contiguous [N,OC,OH,OW] device tensor of out_dtype")
        stream, current = _stream_of(stream, x.device)
        od = CONVIMG_BF16 if out_dtype == torch.bfloat16 else CONVIMG_FP32
        rc = conv2d_fwd_nchw(x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else None,
                             N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, od, out.data_ptr(),
                             ws.data_ptr(), ws.numel(), stream)
    if rc != 0:
        raise RuntimeError("conv2d_fwd_nchw failed: %s (status %d)" % (conv2d_strerror(rc), rc))
    if not current:
        _keep_for_stream(fresh, stream, x.device)
    return out
