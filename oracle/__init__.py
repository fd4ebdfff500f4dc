"""CPU oracle for 2-D convolution forward (NHWC input, OHWI weight) and its
two backward passes (gradients with respect to the input and the weights).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library and its binding never import it, and it imports nothing of theirs.

The arithmetic lives in ``conv_ref.c`` (plain C, fp64, OpenMP over output
pixels); this module only marshals numpy arrays to it.  What it computes and
which passage of the pages each part follows is stated in that file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "conv_ref.c")
SO = os.path.join(HERE, "libconvref.so")
GCC_FLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Werror"]


def compile_source(src: str, so: str) -> str:
    """Compile an oracle source file into a shared library with plain gcc."""
    tmp = so + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, so)
    return so


def build(force: bool = True) -> str:
    """Build ``libconvref.so`` next to its source (always, unless force=False
    and it already exists)."""
    global _default
    if force or not os.path.exists(SO):
        compile_source(SRC, SO)
        _default = None
    return SO


def _dptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _as_f64(a, ndim, name):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if a.ndim != ndim:
        raise ValueError("%s must have %d dims, got %s" % (name, ndim, a.shape))
    return a


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, so_path: str = SO):
        lib = ctypes.CDLL(so_path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.c_int
        lib.oracle_out_dim.argtypes = [ip] * 5
        lib.oracle_out_dim.restype = ip
        lib.oracle_conv2d_fwd.argtypes = [dp, dp, dp] + [ip] * 10 + [dp, dp]
        lib.oracle_conv2d_fwd.restype = ip
        lib.oracle_conv2d_fwd_pixels.argtypes = (
            [dp, dp, dp] + [ip] * 10
            + [ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, dp, dp])
        lib.oracle_conv2d_fwd_pixels.restype = ip
        lib.oracle_conv2d_bwd_data.argtypes = [dp, dp] + [ip] * 10 + [dp, dp]
        lib.oracle_conv2d_bwd_data.restype = ip
        lib.oracle_conv2d_bwd_weight.argtypes = [dp, dp] + [ip] * 10 + [dp, dp]
        lib.oracle_conv2d_bwd_weight.restype = ip
        lib.oracle_set_threads.argtypes = [ip]
        lib.oracle_set_threads.restype = ip
        self.lib = lib
        self.path = so_path

    def out_dim(self, size: int, k: int, stride: int, pad: int, dilation: int) -> int:
        """Output extent along one axis (-1 when no window fits)."""
        return self.lib.oracle_out_dim(size, k, stride, pad, dilation)

    def set_threads(self, n: int) -> int:
        """Set the OpenMP thread count (n <= 0 keeps it); returns the count in use."""
        return self.lib.oracle_set_threads(int(n))

    def _shapes(self, x, w, bias, stride, pad, dilation):
        x = _as_f64(x, 4, "x")
        w = _as_f64(w, 4, "w")
        N, H, W, IC = x.shape
        OC, KH, KW, IC2 = w.shape
        if IC2 != IC:
            raise ValueError("channel mismatch: x has %d, w has %d" % (IC, IC2))
        b = None if bias is None else _as_f64(bias, 1, "bias")
        if b is not None and b.shape[0] != OC:
            raise ValueError("bias must have OC entries")
        OH = self.out_dim(H, KH, stride, pad, dilation)
        OW = self.out_dim(W, KW, stride, pad, dilation)
        if OH <= 0 or OW <= 0:
            raise ValueError("no output: OH=%d OW=%d" % (OH, OW))
        return x, w, b, (N, H, W, IC, OC, KH, KW, OH, OW)

    def conv2d_fwd(self, x, w, bias=None, stride=1, pad=0, dilation=1):
        """Full forward convolution in fp64.

        x: [N][H][W][IC], w: [OC][KH][KW][IC], bias: [OC] or None.
        Returns (y, S), both float64 [N][OH][OW][OC]; S = sum |x*w| per output.
        """
        x, w, b, (N, H, W, IC, OC, KH, KW, OH, OW) = self._shapes(x, w, bias, stride, pad, dilation)
        y = np.empty((N, OH, OW, OC), np.float64)
        S = np.empty((N, OH, OW, OC), np.float64)
        rc = self.lib.oracle_conv2d_fwd(_dptr(x), _dptr(w), _dptr(b), N, H, W, IC, OC, KH, KW,
                                        stride, pad, dilation, _dptr(y), _dptr(S))
        if rc != 0:
            raise ValueError("oracle rejected the shape")
        return y, S

    def conv2d_fwd_pixels(self, x, w, bias, stride, pad, dilation, pixels):
        """Forward convolution at selected output pixels only.

        pixels: flat indices (n*OH + oh)*OW + ow.  Returns (y, S), float64
        [len(pixels)][OC].
        """
        x, w, b, (N, H, W, IC, OC, KH, KW, OH, OW) = self._shapes(x, w, bias, stride, pad, dilation)
        pix = np.ascontiguousarray(np.asarray(pixels, dtype=np.int64))
        y = np.empty((pix.shape[0], OC), np.float64)
        S = np.empty((pix.shape[0], OC), np.float64)
        rc = self.lib.oracle_conv2d_fwd_pixels(
            _dptr(x), _dptr(w), _dptr(b), N, H, W, IC, OC, KH, KW, stride, pad, dilation,
            pix.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), pix.shape[0], _dptr(y), _dptr(S))
        if rc != 0:
            raise ValueError("oracle rejected the shape or a pixel index")
        return y, S

    def conv2d_bwd_data(self, dy, w, H, W, stride=1, pad=0, dilation=1):
        """Gradient of the forward convolution with respect to its input.

        dy: [N][OH][OW][OC] (OH, OW the forward extents of H, W), w:
        [OC][KH][KW][IC].  Returns (dx, S), float64 [N][H][W][IC]; S = sum
        |dy*w| over the terms of each element.
        """
        dy = _as_f64(dy, 4, "dy")
        w = _as_f64(w, 4, "w")
        N, OH, OW, OC = dy.shape
        OC2, KH, KW, IC = w.shape
        if OC2 != OC:
            raise ValueError("channel mismatch: dy has %d, w has %d" % (OC, OC2))
        if (self.out_dim(H, KH, stride, pad, dilation), self.out_dim(W, KW, stride, pad, dilation)) != (OH, OW):
            raise ValueError("dy extent does not match the forward output of H, W")
        dx = np.empty((N, H, W, IC), np.float64)
        S = np.empty((N, H, W, IC), np.float64)
        rc = self.lib.oracle_conv2d_bwd_data(_dptr(dy), _dptr(w), N, H, W, IC, OC, KH, KW,
                                             stride, pad, dilation, _dptr(dx), _dptr(S))
        if rc != 0:
            raise ValueError("oracle rejected the shape")
        return dx, S

    def conv2d_bwd_weight(self, x, dy, KH, KW, stride=1, pad=0, dilation=1):
        """Gradient of the forward convolution with respect to its weights.

        x: [N][H][W][IC], dy: [N][OH][OW][OC] (OH, OW the forward extents).
        Returns (dw, S), float64 [OC][KH][KW][IC]; S = sum |dy*x| over the
        terms of each element.
        """
        x = _as_f64(x, 4, "x")
        dy = _as_f64(dy, 4, "dy")
        N, H, W, IC = x.shape
        N2, OH, OW, OC = dy.shape
        if N2 != N:
            raise ValueError("batch mismatch: x has %d, dy has %d" % (N, N2))
        if (self.out_dim(H, KH, stride, pad, dilation), self.out_dim(W, KW, stride, pad, dilation)) != (OH, OW):
            raise ValueError("dy extent does not match the forward output of H, W")
        dw = np.empty((OC, KH, KW, IC), np.float64)
        S = np.empty((OC, KH, KW, IC), np.float64)
        rc = self.lib.oracle_conv2d_bwd_weight(_dptr(x), _dptr(dy), N, H, W, IC, OC, KH, KW,
                                               stride, pad, dilation, _dptr(dw), _dptr(S))
        if rc != 0:
            raise ValueError("oracle rejected the shape")
        return dw, S


_default = None


def get() -> Oracle:
    """The oracle built from ``conv_ref.c`` (built first if nothing is)."""
    global _default
    if _default is None:
        if not os.path.exists(SO):
            build()
        _default = Oracle(SO)
    return _default


def out_dim(size, k, stride, pad, dilation):
    return get().out_dim(size, k, stride, pad, dilation)


def set_threads(n):
    return get().set_threads(n)


def conv2d_fwd(x, w, bias=None, stride=1, pad=0, dilation=1):
    return get().conv2d_fwd(x, w, bias, stride, pad, dilation)


def conv2d_fwd_pixels(x, w, bias, stride, pad, dilation, pixels):
    return get().conv2d_fwd_pixels(x, w, bias, stride, pad, dilation, pixels)


def conv2d_bwd_data(dy, w, H, W, stride=1, pad=0, dilation=1):
    return get().conv2d_bwd_data(dy, w, H, W, stride, pad, dilation)


def conv2d_bwd_weight(x, dy, KH, KW, stride=1, pad=0, dilation=1):
    return get().conv2d_bwd_weight(x, dy, KH, KW, stride, pad, dilation)
