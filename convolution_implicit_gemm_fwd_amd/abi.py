"""ctypes binding of libconvimg's C ABI (include/convimg.h), same names.

Argument marshalling only: every step of the convolution runs in the HIP
library.  Loading fails loudly when the library has not been built; there is
no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libconvimg.so")

CONVIMG_BF16 = 0
CONVIMG_FP32 = 1

CONVIMG_OK = 0
CONVIMG_ERR_NULL = 1
CONVIMG_ERR_SHAPE = 2
CONVIMG_ERR_DTYPE = 3
CONVIMG_ERR_RANGE = 4
CONVIMG_ERR_ALIAS = 5
CONVIMG_ERR_ALLOC = 6
CONVIMG_ERR_LAUNCH = 7
CONVIMG_ERR_DEVICE = 8
CONVIMG_ERR_TIMEOUT = 9
CONVIMG_ERR_UNSUPPORTED = 10
CONVIMG_ERR_WORKSPACE = 11
CONVIMG_ERR_SCRATCH = 12

CONVIMG_LOADER_TAP = 0
CONVIMG_LOADER_VEC8 = 1
CONVIMG_LOADER_SCALAR = 2
CONVIMG_LOADER_FP32 = 3

CONVIMG_KIND_REGS = 0
CONVIMG_KIND_PIPE = 1
CONVIMG_KIND_PATCH = 2
CONVIMG_KIND_STRIP = 3
CONVIMG_KIND_WINDOW = 4
CONVIMG_KIND_RESIDENT = 5
CONVIMG_KIND_IMAGE = 6

# Every symbol include/convimg.h declares.
EXPORTS = ("conv2d_fwd", "conv2d_fwd_out_dim", "conv2d_fwd_plan", "conv2d_strerror",
           "conv2d_fwd_force", "conv2d_fwd_num_tiles", "conv2d_fwd_tile_kind", "conv2d_fwd_status",
           "conv2d_release", "conv2d_bwd_data", "conv2d_bwd_data_weights", "conv2d_bwd_weight",
           "conv2d_bwd_weight_workspace", "conv2d_fwd_autotune", "conv2d_fwd_autotune_clear",
           "conv2d_fwd_nchw", "conv2d_fwd_nchw_workspace", "conv2d_fwd_test_spin_limit",
           "conv2d_fwd_noalloc")


class convimg_plan(ctypes.Structure):
    _fields_ = [("OH", ctypes.c_int), ("OW", ctypes.c_int), ("M", ctypes.c_longlong),
                ("Ngemm", ctypes.c_int), ("K", ctypes.c_int), ("tile_id", ctypes.c_int),
                ("BM", ctypes.c_int), ("BN", ctypes.c_int), ("BK", ctypes.c_int),
                ("loader", ctypes.c_int), ("splits", ctypes.c_int), ("tiles_m", ctypes.c_int),
                ("tiles_n", ctypes.c_int), ("ktiles", ctypes.c_int), ("grid", ctypes.c_int),
                ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class LibraryMissing(RuntimeError):
    pass


_lib = None


def load(path: str = LIB_PATH):
    """Load libconvimg.so (once).  Raises LibraryMissing if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LibraryMissing(
            "libconvimg.so is not built (%s); build it with "
            "`python -m convolution_implicit_gemm_fwd_amd.build`" % path)
    lib = ctypes.CDLL(path)
    i, vp = ctypes.c_int, ctypes.c_void_p
    lib.conv2d_fwd.argtypes = [vp, vp, vp] + [i] * 11 + [vp, vp]
    lib.conv2d_fwd.restype = i
    lib.conv2d_fwd_noalloc.argtypes = [vp, vp, vp] + [i] * 11 + [vp, vp]
    lib.conv2d_fwd_noalloc.restype = i
    lib.conv2d_fwd_out_dim.argtypes = [i] * 5
    lib.conv2d_fwd_out_dim.restype = i
    lib.conv2d_fwd_plan.argtypes = [i] * 12 + [ctypes.POINTER(convimg_plan)]
    lib.conv2d_fwd_plan.restype = i
    lib.conv2d_strerror.argtypes = [i]
    lib.conv2d_strerror.restype = ctypes.c_char_p
    lib.conv2d_fwd_force.argtypes = [i, i, i]
    lib.conv2d_fwd_force.restype = i
    lib.conv2d_fwd_num_tiles.argtypes = []
    lib.conv2d_fwd_num_tiles.restype = i
    lib.conv2d_fwd_tile_kind.argtypes = [i]
    lib.conv2d_fwd_tile_kind.restype = i
    lib.conv2d_fwd_status.argtypes = [vp]
    lib.conv2d_fwd_status.restype = i
    lib.conv2d_fwd_test_spin_limit.argtypes = [i]
    lib.conv2d_fwd_test_spin_limit.restype = i
    lib.conv2d_release.argtypes = []
    lib.conv2d_release.restype = None
    lib.conv2d_bwd_data.argtypes = [vp, vp] + [i] * 11 + [vp, vp, vp]
    lib.conv2d_bwd_data.restype = i
    lib.conv2d_bwd_data_weights.argtypes = [vp] + [i] * 5 + [vp, vp]
    lib.conv2d_bwd_data_weights.restype = i
    lib.conv2d_bwd_weight.argtypes = [vp, vp] + [i] * 11 + [vp, vp, ctypes.c_size_t, vp]
    lib.conv2d_bwd_weight.restype = i
    lib.conv2d_bwd_weight_workspace.argtypes = [i] * 11 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.conv2d_bwd_weight_workspace.restype = i
    ip, fp = ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float)
    lib.conv2d_fwd_autotune.argtypes = [vp, vp, vp] + [i] * 11 + [vp, vp, ip, ip, fp, fp]
    lib.conv2d_fwd_autotune.restype = i
    lib.conv2d_fwd_autotune_clear.argtypes = []
    lib.conv2d_fwd_autotune_clear.restype = None
    lib.conv2d_fwd_nchw.argtypes = [vp, vp, vp] + [i] * 12 + [vp, vp, ctypes.c_size_t, vp]
    lib.conv2d_fwd_nchw.restype = i
    lib.conv2d_fwd_nchw_workspace.argtypes = [i] * 11 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.conv2d_fwd_nchw_workspace.restype = i
    _lib = lib
    return lib


def conv2d_fwd(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out, stream):
    """Raw C call: pointers are integers (device addresses), returns a status."""
    return load().conv2d_fwd(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation,
                             dtype, out, stream)


def conv2d_fwd_noalloc(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out, stream):
    """Raw C call of the entry point that allocates nothing (same arguments
    as conv2d_fwd), returns a status."""
    return load().conv2d_fwd_noalloc(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation,
                                     dtype, out, stream)


def conv2d_bwd_data(dy, w, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, wt, dx, stream):
    """Raw C call of the data backward (device addresses as integers), returns a status."""
    return load().conv2d_bwd_data(dy, w, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype,
                                  wt, dx, stream)


def conv2d_bwd_data_weights(w, OC, KH, KW, IC, dtype, wt, stream):
    """Raw C call of the data backward's weight transform, returns a status."""
    return load().conv2d_bwd_data_weights(w, OC, KH, KW, IC, dtype, wt, stream)


def conv2d_bwd_weight(x, dy, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, dw, ws, ws_bytes,
                      stream):
    """Raw C call of the weight backward (device addresses as integers), returns a status."""
    return load().conv2d_bwd_weight(x, dy, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, dw,
                                    ws, ws_bytes, stream)


def conv2d_bwd_weight_workspace(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype):
    """Returns (status, workspace bytes the weight backward needs on the current device)."""
    b = ctypes.c_size_t(0)
    rc = load().conv2d_bwd_weight_workspace(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype,
                                            ctypes.byref(b))
    return rc, b.value


def conv2d_fwd_autotune(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out,
                        stream):
    """Raw C call of the autotuner.  Returns (status, tile, splits, us_best, us_default)."""
    t, sp = ctypes.c_int(-1), ctypes.c_int(-1)
    ub, ud = ctypes.c_float(0.0), ctypes.c_float(0.0)
    rc = load().conv2d_fwd_autotune(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype,
                                    out, stream, ctypes.byref(t), ctypes.byref(sp), ctypes.byref(ub),
                                    ctypes.byref(ud))
    return rc, t.value, sp.value, ub.value, ud.value


def conv2d_fwd_autotune_clear():
    load().conv2d_fwd_autotune_clear()


def conv2d_fwd_nchw(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out_dtype, out,
                    ws, ws_bytes, stream):
    """Raw C call of the NCHW entry point, returns a status."""
    return load().conv2d_fwd_nchw(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype,
                                  out_dtype, out, ws, ws_bytes, stream)


def conv2d_fwd_nchw_workspace(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype):
    """Returns (status, workspace bytes of conv2d_fwd_nchw)."""
    b = ctypes.c_size_t(0)
    rc = load().conv2d_fwd_nchw_workspace(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype,
                                          ctypes.byref(b))
    return rc, b.value


def conv2d_fwd_out_dim(size, k, stride, pad, dilation):
    return load().conv2d_fwd_out_dim(size, k, stride, pad, dilation)


def conv2d_fwd_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, num_cus):
    """Returns (status, plan dict or None)."""
    p = convimg_plan()
    rc = load().conv2d_fwd_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, num_cus,
                                ctypes.byref(p))
    return rc, (p.as_dict() if rc == CONVIMG_OK else None)


def conv2d_strerror(status):
    return load().conv2d_strerror(status).decode()


def conv2d_fwd_force(tile_id=-1, splits=-1, loader=-1):
    return load().conv2d_fwd_force(tile_id, splits, loader)


def conv2d_fwd_num_tiles():
    return load().conv2d_fwd_num_tiles()


def conv2d_fwd_tile_kind(tile_id):
    return load().conv2d_fwd_tile_kind(tile_id)


def conv2d_fwd_status(stream):
    return load().conv2d_fwd_status(stream)


def conv2d_fwd_test_spin_limit(iterations):
    """Test knob: split-K wait bound in sleep iterations (< 1: default).
    Returns the previous bound."""
    return load().conv2d_fwd_test_spin_limit(iterations)


def conv2d_release():
    load().conv2d_release()
