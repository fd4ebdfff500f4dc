"""The torch wrappers on a stream other than torch's current one.

A wrapper that allocates a buffer (its output, or a workspace it frees on
return) on torch's current stream and queues the kernels on another stream
must keep the caching allocator from handing that memory out again before
the other stream has run the kernels.  Each case holds the side stream back
with a sleep kernel, calls the wrapper there, then allocates buffers of the
same sizes on the current stream: none may get the wrapper's memory while
the side stream is still behind, and the result must match the oracle.
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_fwd_amd as cim
from convolution_implicit_gemm_fwd_amd import abi
from convolution_implicit_gemm_fwd_amd.workloads import (BF16, WORKLOADS, make_grad_inputs,
                                                         make_inputs, make_wgrad_inputs)

import oracle
from gpu_harness import check, log, need_gpu

pytestmark = pytest.mark.gpu

SLEEP_CYCLES = 50_000_000      # holds the side stream back for tens of milliseconds


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a.view(np.int16))).view(torch.bfloat16).cuda()


class _Recorder:
    """Wraps torch.empty and remembers (address, bytes) of what it returns."""

    def __init__(self):
        self.blocks = []
        self.real = torch.empty

    def __call__(self, *args, **kwargs):
        t = self.real(*args, **kwargs)
        if t.is_cuda:
            self.blocks.append((t.data_ptr(), t.numel() * t.element_size()))
        return t


def _run_on_side_stream(monkeypatch, call):
    """call(stream_ptr) on a held-back side stream; returns its result after
    checking that same-size allocations on the current stream do not reuse
    the wrapper's buffers meanwhile."""
    side = torch.cuda.Stream()
    rec = _Recorder()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        torch.cuda._sleep(SLEEP_CYCLES)
    monkeypatch.setattr(torch, "empty", rec)
    try:
        result = call(side.cuda_stream)
    finally:
        monkeypatch.setattr(torch, "empty", rec.real)
    assert rec.blocks, "the wrapper allocated nothing"
    taken = {p for p, _ in rec.blocks}
    probes = []
    for _, nbytes in rec.blocks:
        t = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        t.fill_(0xFF)
        probes.append(t)
    reused = [t.data_ptr() for t in probes if t.data_ptr() in taken]
    assert not side.query(), "the side stream finished before the check (sleep too short)"
    assert not reused, "memory still in use on the side stream was handed out again"
    torch.cuda.synchronize()
    return result


def test_forward_wrapper(monkeypatch):
    wl = WORKLOADS["resnet3x3"].scaled(N=2, H=20, W=20)
    inp = make_inputs(wl, seed=1)
    x, w, b = _bf16(inp.x_store), _bf16(inp.w_store), torch.from_numpy(inp.bias).cuda()
    y = _run_on_side_stream(monkeypatch, lambda s: cim.conv2d_nhwc(x, w, b, stride=1, pad=1,
                                                                   stream=s))
    yref, S = oracle.conv2d_fwd(inp.x32, inp.w32, inp.bias, 1, 1, 1)
    check(y.cpu().numpy(), yref, S, "conv2d_nhwc on a side stream")


def test_data_backward_wrapper(monkeypatch):
    wl = WORKLOADS["resnet3x3"].scaled(N=2, H=16, W=16)
    inp = make_grad_inputs(wl, 16, 16, seed=2)
    dy, w = _bf16(inp.x_store), _bf16(inp.w_store)
    dx = _run_on_side_stream(monkeypatch, lambda s: cim.conv2d_bwd_data_nhwc(
        dy, w, 16, 16, stride=1, pad=1, dilation=1, stream=s))
    yref, S = oracle.conv2d_bwd_data(inp.x32, inp.w32, 16, 16, 1, 1, 1)
    check(dx.cpu().numpy(), yref, S, "conv2d_bwd_data_nhwc on a side stream")


def test_weight_backward_wrapper(monkeypatch):
    wl = WORKLOADS["resnet3x3"].scaled(N=2, H=20, W=20)
    inp = make_wgrad_inputs(wl, 20, 20, seed=3)
    x, dy = _bf16(inp.x_store), _bf16(inp.w_store)
    dw = _run_on_side_stream(monkeypatch, lambda s: cim.conv2d_bwd_weight_nhwc(
        x, dy, 3, 3, stride=1, pad=1, dilation=1, stream=s))
    yref, S = oracle.conv2d_bwd_weight(inp.x32, inp.w32, 3, 3, 1, 1, 1)
    check(dw.cpu().numpy(), yref, S, "conv2d_bwd_weight_nhwc on a side stream")


def test_nchw_wrapper(monkeypatch):
    wl = WORKLOADS["resnet3x3"].scaled(N=2, H=18, W=18)
    inp = make_inputs(wl, seed=4)
    x = _bf16(inp.x_store).permute(0, 3, 1, 2).contiguous()
    w = _bf16(inp.w_store).permute(0, 3, 1, 2).contiguous()
    b = torch.from_numpy(inp.bias).cuda()
    y = _run_on_side_stream(monkeypatch, lambda s: cim.conv2d_nchw(x, w, b, stride=1, pad=1,
                                                                   stream=s))
    yref, S = oracle.conv2d_fwd(inp.x32, inp.w32, inp.bias, 1, 1, 1)
    check(y.permute(0, 2, 3, 1).cpu().numpy(), yref, S, "conv2d_nchw on a side stream")
