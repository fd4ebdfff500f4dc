"""GPU parity of the weight backward (conv2d_bwd_weight) against the fp64
oracle's definition of the weight gradient, element by element with
|err| <= 1e-3*S + 1e-5 (S: the oracle's sum of |dy*x| over each element's
terms).

The kernels sum each pixel range's products in MFMA accumulators (one add
per 32 pixels; the row-window kernel then adds its four pixel quarters),
then the ranges in a fixed order, so the fp32 rounding grows with (pixels
per range)/32 + ranges + 32 additions, a few hundred at most here: far
inside the bound.

dw is pre-filled with NaN (an element never written fails) and followed by
a sentinel guard; the workspace gets a guard after the bytes the library
asks for.  Covered: the ResNet-style layer at full size (several pixel
ranges), the 512-channel layer (one range per tile), the 7x7 stride-2 stem
(IC = 3: element-wise gather), a dilated layer, channel tails, strides,
dilations, non-square windows, OC off the vector width, misaligned x,
fewer pixels than one step, the row-window kernel's unit layouts (short
rows, rows cut into segments, unequal segments left to the transpose-read
kernel); repeatability through the workspace and in
place (ranges adding into dw in turn), the in-place wait forced to time
out; the workspace-size error; the torch wrapper.  The named layers run at
full size.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_fwd_amd as cig
from convolution_implicit_gemm_fwd_amd import abi
from convolution_implicit_gemm_fwd_amd.workloads import BF16, FP32, WORKLOADS, make_wgrad_inputs

import oracle
from gpu_harness import GUARD, SENTINEL, check, log, need_gpu, shape

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def upload(a, misalign=False):
    if a.dtype == np.float32:
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16))).view(torch.bfloat16)
    if not misalign:
        return t.cuda()
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    flat[1:].copy_(t.reshape(-1))
    return flat[1:].view(t.shape)


def run_wgrad(wl, inp, misalign=False, ws_extra=0, misalign_dy=False, dtype=BF16):
    x, dy = upload(inp.x_store, misalign), upload(inp.w_store, misalign_dy)
    K = wl.KH * wl.KW * wl.IC
    n_dw = wl.OC * K
    dw = torch.full((n_dw + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    dw[n_dw:] = SENTINEL
    rc, need = abi.conv2d_bwd_weight_workspace(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW,
                                               wl.stride, wl.pad, wl.dilation, dtype)
    assert rc == 0, abi.conv2d_strerror(rc)
    ws = torch.full((need + 4096 + ws_extra,), 0x5A, dtype=torch.uint8, device="cuda")
    log("wgrad %s dtype %d workspace %d bytes" % (wl, dtype, need))
    rc = abi.conv2d_bwd_weight(x.data_ptr(), dy.data_ptr(), wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH,
                               wl.KW, wl.stride, wl.pad, wl.dilation, dtype, dw.data_ptr(),
                               ws.data_ptr() if need else None, need,
                               torch.cuda.current_stream().cuda_stream)
    assert rc == 0, abi.conv2d_strerror(rc)
    torch.cuda.synchronize()
    host = dw.cpu().numpy()
    assert (host[n_dw:] == SENTINEL).all(), "write past the end of dw"
    assert (ws[need:].cpu().numpy() == 0x5A).all(), "write past the workspace it asked for"
    return host[:n_dw].reshape(wl.OC, wl.KH, wl.KW, wl.IC), need


def wgrad_parity(wl, seed=0, misalign=False, misalign_dy=False, dtype=BF16):
    OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
    OW = abi.conv2d_fwd_out_dim(wl.W, wl.KW, wl.stride, wl.pad, wl.dilation)
    inp = make_wgrad_inputs(wl, OH, OW, seed=seed, dtype=dtype)
    y, need = run_wgrad(wl, inp, misalign, misalign_dy=misalign_dy, dtype=dtype)
    yref, S = oracle.conv2d_bwd_weight(inp.x32, inp.w32, wl.KH, wl.KW, wl.stride, wl.pad,
                                       wl.dilation)
    ratio = check(y, yref, S, "wgrad %s" % (wl,))
    log("wgrad %s worst err/tol %.3g (workspace %d)" % (wl.name, ratio, need))
    return y, need


# the four named bf16 layers at full size, planned as bench.py --op wgrad runs them
FULL = [WORKLOADS["resnet3x3"], WORKLOADS["largek"], WORKLOADS["stem7x7"], WORKLOADS["dilated"]]

SMALL = [
    shape(2, 13, 11, 24, 40, 3, 3, 1, 1, 1, name="IC 24 OC 40 tails"),
    shape(2, 15, 17, 16, 50, 3, 3, 2, 1, 1, name="stride 2, OC 50 (element-wise dy)"),
    shape(1, 20, 20, 64, 64, 3, 3, 1, 2, 2, name="dilation 2"),
    shape(3, 10, 10, 64, 96, 1, 1, 1, 0, 1, name="1x1"),
    shape(2, 12, 14, 32, 48, 3, 5, 1, 2, 1, name="3x5 window"),
    shape(2, 30, 30, 3, 64, 7, 7, 2, 3, 1, name="IC 3 7x7 stride 2"),
    shape(1, 9, 9, 5, 7, 3, 3, 1, 1, 1, name="IC 5 OC 7"),
    shape(1, 4, 5, 8, 8, 3, 3, 1, 1, 1, name="fewer pixels than a step"),
    shape(1, 3, 3, 8, 8, 3, 3, 1, 0, 1, name="single output pixel"),
    shape(4, 28, 28, 128, 128, 3, 3, 1, 1, 1, name="128 channels, several ranges"),
    # the row-window kernel's unit layouts: several short rows a step, rows
    # cut into equal segments (one and two a step, a step's segments from two
    # rows, OC off the tile), unequal segments (the transpose-read kernel)
    shape(3, 9, 7, 64, 64, 3, 3, 1, 1, 1, name="rows of 7: eighteen a step"),
    shape(1, 6, 100, 64, 64, 3, 3, 1, 1, 1, name="rows of 100: two segments of 50"),
    shape(2, 7, 80, 64, 72, 3, 3, 1, 1, 1, name="rows of 80: segments across rows, OC 72"),
    shape(1, 5, 127, 64, 64, 3, 3, 1, 1, 1, name="rows of 127: unequal segments"),
]
# planned with four pixel ranges per tile by both kernels (the most that add
# into dw in turn): the row-window kernel with 16-byte aligned x, the
# general kernel with x one element off
IN_PLACE = shape(1, 24, 48, 64, 128, 3, 3, 1, 1, 1, name="four ranges in place")


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_wgrad_full_size(wl):
    wgrad_parity(wl)


# fp32 storage: the fp32 kernel (64 x 64 tiles, fp32 products and sums),
# values as drawn (not bf16-rounded); one pixel range a tile (dw written
# directly) and several (the workspace and the ordered sum), channel tails,
# strides, dilations, windows, and layers of the named shapes at N = 2
F32 = [
    shape(1, 8, 8, 16, 16, 3, 3, 1, 1, 1, dtype=FP32, name="fp32 tiny"),
    shape(1, 9, 9, 5, 7, 3, 3, 1, 1, 1, dtype=FP32, name="fp32 IC 5 OC 7"),
    shape(2, 13, 11, 24, 40, 3, 3, 1, 1, 1, dtype=FP32, name="fp32 IC 24 OC 40"),
    shape(2, 15, 17, 16, 50, 3, 3, 2, 1, 1, dtype=FP32, name="fp32 stride 2, OC 50"),
    shape(1, 20, 20, 64, 64, 3, 3, 1, 2, 2, dtype=FP32, name="fp32 dilation 2"),
    shape(3, 10, 10, 64, 96, 1, 1, 1, 0, 1, dtype=FP32, name="fp32 1x1"),
    shape(2, 12, 14, 32, 48, 3, 5, 1, 2, 1, dtype=FP32, name="fp32 3x5 window"),
    shape(2, 30, 30, 3, 64, 7, 7, 2, 3, 1, dtype=FP32, name="fp32 IC 3 7x7 stride 2"),
    shape(1, 3, 3, 8, 8, 3, 3, 1, 0, 1, dtype=FP32, name="fp32 single output pixel"),
    WORKLOADS["resnet3x3"].scaled(N=2, dtype=FP32, name="fp32 resnet3x3 N=2"),
    WORKLOADS["largek"].scaled(N=2, dtype=FP32, name="fp32 largek N=2"),
]


@pytest.mark.parametrize("wl", F32, ids=lambda w: w.name)
def test_wgrad_fp32_storage(wl):
    wgrad_parity(wl, dtype=FP32)


def test_wgrad_fp32_repeatable():
    """The fp32 path's ranges through the workspace are added in a fixed
    order: two calls give the same bits."""
    wl = F32[-2]
    OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
    OW = abi.conv2d_fwd_out_dim(wl.W, wl.KW, wl.stride, wl.pad, wl.dilation)
    inp = make_wgrad_inputs(wl, OH, OW, seed=3, dtype=FP32)
    y1, need = run_wgrad(wl, inp, dtype=FP32)
    y2, _ = run_wgrad(wl, inp, dtype=FP32)
    assert need > 0, "expected several ranges through the workspace"
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_wgrad_shapes(wl):
    wgrad_parity(wl)


def test_wgrad_misaligned_x():
    wgrad_parity(shape(2, 10, 10, 64, 64, 3, 3, 1, 1, 1, name="misaligned x"), misalign=True)


def test_wgrad_misaligned_dy():
    """dy one element off a 16-byte boundary: the element-wise dy gather with
    the 16-byte x gather."""
    wgrad_parity(shape(2, 11, 9, 32, 64, 3, 3, 1, 1, 1, name="misaligned dy"), misalign_dy=True)
    wgrad_parity(shape(1, 12, 12, 24, 48, 3, 3, 2, 1, 1, name="misaligned x and dy"), misalign=True,
                 misalign_dy=True)


def test_wgrad_repeatable():
    wl = WORKLOADS["resnet3x3"].scaled(N=2)
    OH, OW = wl.H, wl.W
    inp = make_wgrad_inputs(wl, OH, OW, seed=5)
    a, need = run_wgrad(wl, inp)
    b, _ = run_wgrad(wl, inp)
    assert need > 0, "this shape should use several pixel ranges"
    assert np.array_equal(a, b), "two calls gave different bits"


def test_wgrad_in_place_ranges_repeatable():
    """Four pixel ranges a tile add into dw in turn (no workspace): the same
    bits on every call, and the status stays clean."""
    wl = IN_PLACE
    inp = make_wgrad_inputs(wl, 24, 48, seed=4)
    a, need = run_wgrad(wl, inp)
    b, _ = run_wgrad(wl, inp)
    assert need == 0, "four ranges should add in place"
    assert np.array_equal(a, b), "two calls gave different bits"
    assert abi.conv2d_fwd_status(torch.cuda.current_stream().cuda_stream) == abi.CONVIMG_OK


@pytest.mark.parametrize("misalign", [False, True], ids=["row-window kernel", "misaligned x: general kernel"])
def test_wgrad_four_ranges_in_place(misalign):
    """Four pixel ranges per tile, the most that add in place: no
    workspace, parity with the oracle, through either kernel."""
    y, need = wgrad_parity(IN_PLACE, seed=2, misalign=misalign)
    assert need == 0, "four ranges should add in place"


def test_wgrad_in_place_timeout_poisons_and_resets():
    """The in-place turn wait forced to give up from the host (a
    one-iteration bound): a range that gives up writes NaN over its part of
    dw, conv2d_fwd_status reports the timeout and resets the semaphores, and
    the next call with the normal bound is correct.  (Whether a range gives up
    depends on timing; either outcome is checked.)"""
    wl = IN_PLACE
    inp = make_wgrad_inputs(wl, 24, 48, seed=0)
    yref, S = oracle.conv2d_bwd_weight(inp.x32, inp.w32, wl.KH, wl.KW, wl.stride, wl.pad,
                                       wl.dilation)
    sptr = torch.cuda.current_stream().cuda_stream
    prev = abi.conv2d_fwd_test_spin_limit(1)
    try:
        y, _ = run_wgrad(wl, inp)
        abi.conv2d_fwd_test_spin_limit(prev)
        status = abi.conv2d_fwd_status(sptr)
        log("forced wgrad timeout: status %d, NaN values %d" % (status, int(np.isnan(y).sum())))
        if status == abi.CONVIMG_OK:
            check(y, yref, S, "no range gave up")
        else:
            assert status == abi.CONVIMG_ERR_TIMEOUT
            assert np.isnan(y).any(), "a range gave up but dw shows no poisoned part"
        assert abi.conv2d_fwd_status(sptr) == abi.CONVIMG_OK
        y, _ = run_wgrad(wl, inp)
    finally:
        abi.conv2d_fwd_test_spin_limit(0)
    assert abi.conv2d_fwd_status(sptr) == abi.CONVIMG_OK
    check(y, yref, S, "after the reset")


def test_wgrad_workspace_too_small():
    wl = WORKLOADS["resnet3x3"].scaled(N=2)
    rc, need = abi.conv2d_bwd_weight_workspace(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW,
                                               wl.stride, wl.pad, wl.dilation, BF16)
    assert rc == 0 and need > 0
    x = torch.zeros((wl.N, wl.H, wl.W, wl.IC), dtype=torch.bfloat16, device="cuda")
    dy = torch.zeros((wl.N, wl.H, wl.W, wl.OC), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((wl.OC, 3, 3, wl.IC), dtype=torch.float32, device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), dy.data_ptr(), wl.N, wl.H, wl.W, wl.IC, wl.OC, 3, 3, 1, 1, 1, BF16,
            dw.data_ptr())
    assert abi.conv2d_bwd_weight(*args, ws.data_ptr(), need - 1, s) == abi.CONVIMG_ERR_WORKSPACE
    assert abi.conv2d_bwd_weight(*args, None, need, s) == abi.CONVIMG_ERR_NULL
    assert abi.conv2d_bwd_weight(*args, x.data_ptr(), need, s) == abi.CONVIMG_ERR_ALIAS


def test_wgrad_torch_wrapper():
    wl = shape(2, 14, 14, 48, 80, 3, 3, 1, 1, 1)
    inp = make_wgrad_inputs(wl, 14, 14, seed=3)
    x, dy = upload(inp.x_store), upload(inp.w_store)
    dw = cig.conv2d_bwd_weight_nhwc(x, dy, 3, 3, stride=1, pad=1)
    torch.cuda.synchronize()
    yref, S = oracle.conv2d_bwd_weight(inp.x32, inp.w32, 3, 3, 1, 1, 1)
    check(dw.cpu().numpy(), yref, S, "wrapper")
