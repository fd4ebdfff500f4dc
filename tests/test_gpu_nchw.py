"""GPU parity of the NCHW entry point (conv2d_fwd_nchw) against the fp64
oracle, whose NHWC result is permuted to NCHW here.

Two routes: the resident kernel's NCHW variant (bf16 input, 3x3 resident
plans, W % 8 == 0: reads NCHW x and writes NCHW out itself, so the
workspace's x and result regions stay untouched), and the permutes around
conv2d_fwd (every other problem).  The workspace is pre-filled with a byte
pattern to tell them apart.

fp32 output: |err| <= 1e-3*S + 1e-5, as for conv2d_fwd.  bf16 output: the
fp32 result rounded to nearest even adds at most 2^-8 of its magnitude, so
|err| <= (1e-3*S + 1e-5)*(1 + 2^-8) + 2^-8*|y_oracle|.  The output is
pre-filled with NaN and followed by a sentinel guard.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_fwd_amd as cig
from convolution_implicit_gemm_fwd_amd import abi
from convolution_implicit_gemm_fwd_amd.workloads import BF16, FP32, WORKLOADS, make_inputs

from gpu_harness import GUARD, check, log, need_gpu, oracle_full, shape

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    abi.conv2d_fwd_force(-1, -1, -1)


def dev(a, is_bf16):
    a = np.ascontiguousarray(a)
    if is_bf16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def nchw_parity(wl, out_bf16=False, dtype=None, use_bias=True, fused=None):
    """fused: None (either route), True / False (the route that must run)."""
    dtype = wl.dtype if dtype is None else dtype
    inp = make_inputs(wl, seed=6, dtype=dtype)
    is_bf16 = dtype == BF16
    x = dev(inp.x_store.transpose(0, 3, 1, 2), is_bf16)          # NCHW
    w = dev(inp.w_store.transpose(0, 3, 1, 2), is_bf16)          # OIHW
    b = torch.from_numpy(inp.bias).cuda()
    OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
    OW = abi.conv2d_fwd_out_dim(wl.W, wl.KW, wl.stride, wl.pad, wl.dilation)
    n_out = wl.N * wl.OC * OH * OW
    rc, need = abi.conv2d_fwd_nchw_workspace(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW,
                                             wl.stride, wl.pad, wl.dilation, dtype)
    assert rc == 0
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    odt = torch.bfloat16 if out_bf16 else torch.float32
    out = torch.full((n_out + GUARD,), float("nan"), dtype=odt, device="cuda")
    out[n_out:] = 7.0
    log("nchw %s out %s" % (wl, odt))
    rc = abi.conv2d_fwd_nchw(x.data_ptr(), w.data_ptr(), b.data_ptr() if use_bias else None,
                             wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride, wl.pad,
                             wl.dilation, dtype, BF16 if out_bf16 else FP32, out.data_ptr(),
                             ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, abi.conv2d_strerror(rc)
    torch.cuda.synchronize()
    nx = wl.N * wl.IC * wl.H * wl.W * (2 if is_bf16 else 4)
    if fused is not None:
        untouched = bool((ws[:nx] == 0xA5).all().item())
        assert untouched == fused, "expected the %s route" % ("fused" if fused else "permute")
    host = out.float().cpu().numpy()
    assert (host[n_out:] == 7.0).all(), "write past the end of out"
    y = host[:n_out].reshape(wl.N, wl.OC, OH, OW)
    yref, S = oracle_full(inp, wl, use_bias)
    yref, S = yref.transpose(0, 3, 1, 2), S.transpose(0, 3, 1, 2)
    if not out_bf16:
        return check(y, yref, S, "nchw %s" % (wl,))
    assert np.isfinite(y).all()
    err = np.abs(y.astype(np.float64) - yref)
    tol = (1e-3 * S + 1e-5) * (1 + U) + U * np.abs(yref)
    assert (err <= tol).all(), "bf16 out: %d outside, worst %.3g" % ((err > tol).sum(), (err / tol).max())
    return float((err / tol).max())


CASES = [WORKLOADS["resnet3x3"], WORKLOADS["stem7x7"].scaled(N=2, name="stem7x7 N=2"),
         WORKLOADS["dilated"].scaled(N=1, H=40, W=40, name="dilated 40x40"),
         WORKLOADS["largek"].scaled(N=2, name="largek N=2"),
         shape(2, 13, 11, 24, 40, 3, 3, 2, 1, 1, name="IC 24 OC 40 stride 2"),
         shape(3, 9, 9, 70, 65, 1, 1, 1, 0, 1, name="1x1, 70 -> 65")]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_nchw_fp32_out(wl):
    nchw_parity(wl)


@pytest.mark.parametrize("wl", CASES[:3] + CASES[4:5], ids=lambda w: w.name)
def test_nchw_bf16_out(wl):
    nchw_parity(wl, out_bf16=True)


FUSED = [WORKLOADS["resnet3x3"].scaled(N=2, name="resnet3x3 N=2"),
         shape(6, 28, 40, 64, 64, 3, 3, 1, 1, 1, name="ranges of 26-27 px across images"),
         shape(20, 32, 32, 32, 64, 3, 3, 1, 1, 1, name="IC 32, ranges of 80 px across images"),
         shape(3, 7, 8, 64, 64, 3, 3, 1, 0, 1, name="OH*OW 30, one pixel a range"),
         shape(4, 20, 24, 16, 40, 3, 3, 1, 1, 1, name="IC 16 OC 40"),
         shape(2, 9, 24, 32, 72, 3, 3, 2, 1, 1, name="IC 32 stride 2, OC 72"),
         shape(1, 6, 8, 128, 64, 3, 3, 1, 1, 2, name="IC 128 dilation 2")]


@pytest.mark.parametrize("out_bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("wl", FUSED, ids=lambda w: w.name)
def test_nchw_fused_route(wl, out_bf16):
    """The resident kernel's NCHW variant: parity, and the workspace's x
    region untouched (no input permute ran)."""
    nchw_parity(wl, out_bf16=out_bf16, fused=True)


def test_nchw_route_choice():
    """Problems the NCHW variant does not serve take the permutes: W % 8 != 0
    on a resident plan, a non-resident plan, fp32 storage."""
    nchw_parity(shape(2, 14, 14, 64, 64, 3, 3, 1, 1, 1, name="W 14"), fused=False)
    nchw_parity(WORKLOADS["largek"].scaled(N=1, name="largek N=1"), fused=False)
    nchw_parity(WORKLOADS["tiny"], dtype=FP32, fused=False)
    nchw_parity(WORKLOADS["resnet3x3"], fused=True)
    nchw_parity(shape(3, 12, 16, 64, 64, 3, 3, 1, 1, 1, name="null bias"), use_bias=False, fused=True)


def test_nchw_fp32_storage_and_null_bias():
    nchw_parity(WORKLOADS["tiny"], dtype=FP32, use_bias=False)
    nchw_parity(shape(2, 10, 12, 12, 20, 3, 3, 1, 1, 1, name="fp32 12->20"), dtype=FP32,
                out_bf16=True)


def test_nchw_torch_wrapper_matches_nhwc_path():
    """The wrapper's fp32 result equals conv2d_nhwc's, permuted: both run the
    same plan on the same values, so the bits agree."""
    wl = shape(2, 14, 14, 32, 48, 3, 3, 1, 1, 1)
    inp = make_inputs(wl, seed=8)
    x_nhwc, w_ohwi = dev(inp.x_store, True), dev(inp.w_store, True)
    b = torch.from_numpy(inp.bias).cuda()
    y_nhwc = cig.conv2d_nhwc(x_nhwc, w_ohwi, b, stride=1, pad=1)
    y_nchw = cig.conv2d_nchw(x_nhwc.permute(0, 3, 1, 2).contiguous(),
                             w_ohwi.permute(0, 3, 1, 2).contiguous(), b, stride=1, pad=1)
    y16 = cig.conv2d_nchw(x_nhwc.permute(0, 3, 1, 2).contiguous(),
                          w_ohwi.permute(0, 3, 1, 2).contiguous(), b, stride=1, pad=1,
                          out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y_nchw, y_nhwc.permute(0, 3, 1, 2))
    assert torch.equal(y16, y_nhwc.permute(0, 3, 1, 2).to(torch.bfloat16))   # torch rounds to nearest even too
