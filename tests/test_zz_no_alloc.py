"""conv2d_fwd_noalloc: the entry point that allocates nothing, against
conv2d_fwd.

It runs the same plans and kernels as conv2d_fwd with its split-K
semaphores in a fixed device array instead of the library's pool, so its
output must equal conv2d_fwd's bit for bit and the oracle's within the
forward tolerance.  Two calls in a row, the second on a smaller problem (the
shared array keeps the first call's contents), with split-K forced so that
the scratch array is used, and once on an automatic plan that needs none.
"""
import numpy as np
import pytest
import torch

from convolution_implicit_gemm_fwd_amd import abi
from convolution_implicit_gemm_fwd_amd.workloads import BF16, WORKLOADS, make_inputs

from gpu_harness import GUARD, SENTINEL, check, log, need_gpu, oracle_full, shape, to_device

pytestmark = pytest.mark.gpu

SPLITK = (11, 4, -1)      # pipelined 128x64 tile, 4 splits


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    abi.conv2d_fwd_force(-1, -1, -1)
    yield
    abi.conv2d_fwd_force(-1, -1, -1)


def _call(fn, wl, x, w, b):
    OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
    OW = abi.conv2d_fwd_out_dim(wl.W, wl.KW, wl.stride, wl.pad, wl.dilation)
    n_out = wl.N * OH * OW * wl.OC
    out = torch.full((n_out + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    out[n_out:] = SENTINEL
    rc = fn(x.data_ptr(), w.data_ptr(), b.data_ptr(), wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH,
            wl.KW, wl.stride, wl.pad, wl.dilation, BF16, out.data_ptr(),
            torch.cuda.current_stream().cuda_stream)
    assert rc == 0, abi.conv2d_strerror(rc)
    torch.cuda.synchronize()
    host = out.cpu().numpy()
    assert (host[n_out:] == SENTINEL).all(), "write past the end of out"
    return host[:n_out].reshape(wl.N, OH, OW, wl.OC)


def _compare(wl, force, seed):
    inp = make_inputs(wl, seed=seed)
    x, w, b = to_device(inp)
    abi.conv2d_fwd_force(*force)
    try:
        rc, plan = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride,
                                       wl.pad, wl.dilation, BF16, 0)
        log("noalloc %s force %s plan %s" % (wl.name, force, plan))
        y_na = _call(abi.conv2d_fwd_noalloc, wl, x, w, b)
        y_ref = _call(abi.conv2d_fwd, wl, x, w, b)
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    assert np.array_equal(y_na, y_ref), "conv2d_fwd_noalloc differs from conv2d_fwd"
    yref, S = oracle_full(inp, wl)
    check(y_na, yref, S, "noalloc %s" % wl.name)
    return plan


def test_noalloc_matches_conv2d_fwd_twice_second_smaller():
    big = WORKLOADS["largek"]                                   # 100 tiles x 4 splits
    small = shape(2, 9, 9, 128, 96, 3, 3, 1, 1, 1, name="small split-K")
    p1 = _compare(big, SPLITK, seed=0)
    p2 = _compare(small, SPLITK, seed=1)
    assert p1["splits"] > 1 and p2["splits"] > 1
    assert p2["tiles_m"] * p2["tiles_n"] < p1["tiles_m"] * p1["tiles_n"]
    assert abi.conv2d_fwd_status(torch.cuda.current_stream().cuda_stream) == 0


def test_noalloc_automatic_plan():
    wl = WORKLOADS["resnet3x3"].scaled(N=2)
    _compare(wl, (-1, -1, -1), seed=2)
