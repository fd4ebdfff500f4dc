"""Helpers for the GPU parity tests: upload seeded inputs, call the HIP
library through its C ABI, compare with the oracle.

Tolerance (per element): |y_gpu - y_oracle| <= 1e-3 * S + 1e-5, where S is
the oracle's sum of |x*w| over the same terms; any non-finite value fails.
The GPU's summation order differs from the oracle's; fp32 recursive
summation of K exact bf16 products errs by at most about K * 2^-24 * S
(2.7e-4 * S at K = 4608), inside the bound.

The output buffer is pre-filled with NaN (an element the kernel never
writes fails), and a guard region after it holds a sentinel that must
survive (a write past the end fails).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from convolution_implicit_gemm_fwd_amd import abi
from convolution_implicit_gemm_fwd_amd.workloads import BF16, FP32, Workload, make_inputs

import oracle

GUARD = 4096
SENTINEL = 1234.5
RTOL = 1e-3
ATOL = 1e-5


def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp, misalign=False):
    """x, w, bias device tensors holding the workload's stored bytes."""
    def up(a, is_bf16):
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if is_bf16 else a))
        if is_bf16:
            t = t.view(torch.bfloat16)
        if not misalign:
            return t.cuda()
        flat = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        flat[1:].copy_(t.reshape(-1))
        return flat[1:].view(t.shape)        # starts one element past a 16-byte boundary
    is_bf16 = inp.x_store.dtype == np.uint16
    x = up(inp.x_store, is_bf16)
    w = up(inp.w_store, is_bf16)
    b = torch.from_numpy(inp.bias).cuda()
    return x, w, b


def run_hip(wl: Workload, x, w, b, dtype, use_bias=True, stream=None, out=None):
    """Call conv2d_fwd through the C ABI; returns (out_full, guard_ok_fn)."""
    OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
    OW = abi.conv2d_fwd_out_dim(wl.W, wl.KW, wl.stride, wl.pad, wl.dilation)
    assert OH > 0 and OW > 0
    n_out = wl.N * OH * OW * wl.OC
    if out is None:
        out = torch.full((n_out + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
        out[n_out:] = SENTINEL
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = abi.conv2d_fwd(x.data_ptr(), w.data_ptr(), b.data_ptr() if use_bias else None,
                        wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride, wl.pad,
                        wl.dilation, dtype, out.data_ptr(), s)
    assert rc == 0, "conv2d_fwd: %s" % abi.conv2d_strerror(rc)
    return out, (OH, OW, n_out)


def fetch(out, dims, wl):
    OH, OW, n_out = dims
    torch.cuda.synchronize()
    host = out.cpu().numpy()
    assert (host[n_out:] == SENTINEL).all(), "write past the end of out"
    return host[:n_out].reshape(wl.N, OH, OW, wl.OC)


def check(y, yref, S, what=""):
    y = np.asarray(y, np.float64)
    assert y.shape == yref.shape, "%s: shape %s vs oracle %s" % (what, y.shape, yref.shape)
    finite = np.isfinite(y)
    assert finite.all(), "%s: %d non-finite outputs (first at %s)" % (
        what, (~finite).sum(), np.argwhere(~finite)[0])
    err = np.abs(y - yref)
    tol = RTOL * S + ATOL
    ratio = err / tol
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert (err <= tol).all(), "%s: %d outside tolerance, worst %s err %.3g tol %.3g" % (
        what, (err > tol).sum(), worst, err[worst], tol[worst])
    return float(ratio.max())


def oracle_full(inp, wl, use_bias=True):
    return oracle.conv2d_fwd(inp.x32, inp.w32, inp.bias if use_bias else None,
                             wl.stride, wl.pad, wl.dilation)


def parity(wl: Workload, seed=0, dtype=None, use_bias=True, misalign=False, round_bf16=True,
           force=(-1, -1, -1), ref=None):
    """Run one problem on the GPU and compare all outputs with the oracle."""
    dtype = wl.dtype if dtype is None else dtype
    inp = make_inputs(wl, seed=seed, round_bf16=round_bf16, dtype=dtype)
    x, w, b = to_device(inp, misalign=misalign)
    abi.conv2d_fwd_force(*force)
    try:
        out, dims = run_hip(wl, x, w, b, dtype, use_bias)
        y = fetch(out, dims, wl)
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    if ref is None:
        ref = oracle_full(inp, wl, use_bias)
    yref, S = ref
    return check(y, yref, S, "%s dtype=%d force=%s" % (wl, dtype, force)), y, ref


def shape(N, H, W, IC, OC, KH, KW, s, p, d, dtype=BF16, name="case"):
    return Workload(name, N, IC, H, W, OC, KH, KW, s, p, d, dtype,
                    ("normal", 0.0, 1.0), ("normal", 0.0, 1.0 / np.sqrt(IC * KH * KW)),
                    ("normal", 0.0, 0.1))
