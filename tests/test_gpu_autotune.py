"""GPU tests of the run-time tile selection (conv2d_fwd_autotune).

For each problem: the autotuner runs every candidate plan on the caller's
buffers, records the fastest, and leaves that plan's output in `out`, which
must match the fp64 oracle to the usual bound (|err| <= 1e-3*S + 1e-5); the
planner then reports the recorded tile, conv2d_fwd (which now runs it) must
match the oracle again, and clearing the table restores the static plan.
The time reported for the choice is never above the static plan's (the
static plan is one of the candidates).
"""
import numpy as np
import pytest
import torch

from convolution_implicit_gemm_fwd_amd import abi
from convolution_implicit_gemm_fwd_amd.workloads import WORKLOADS, make_inputs

from gpu_harness import GUARD, SENTINEL, check, fetch, log, need_gpu, oracle_full, shape, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    abi.conv2d_fwd_force(-1, -1, -1)
    abi.conv2d_fwd_autotune_clear()
    yield
    abi.conv2d_fwd_autotune_clear()


CASES = [WORKLOADS["resnet3x3"].scaled(N=4, name="resnet3x3 N=4"),
         WORKLOADS["largek"].scaled(N=2, name="largek N=2"),
         WORKLOADS["dilated"].scaled(N=1, H=48, W=48, name="dilated 48x48"),
         WORKLOADS["stem7x7"].scaled(N=2, H=64, W=64, name="stem 64x64"),
         shape(2, 17, 13, 40, 72, 3, 3, 2, 1, 1, name="stride 2, IC 40, OC 72"),
         WORKLOADS["tiny"]]


def plan_of(wl):
    rc, p = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride, wl.pad,
                                wl.dilation, wl.dtype, 0)
    assert rc == 0
    return p


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_autotune_choice_and_parity(wl):
    inp = make_inputs(wl, seed=4)
    x, w, b = to_device(inp)
    ref = oracle_full(inp, wl)
    static = plan_of(wl)
    OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
    OW = abi.conv2d_fwd_out_dim(wl.W, wl.KW, wl.stride, wl.pad, wl.dilation)
    n_out = wl.N * OH * OW * wl.OC
    out = torch.full((n_out + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    out[n_out:] = SENTINEL
    s = torch.cuda.current_stream().cuda_stream
    log("autotune %s (static tile %d splits %d)" % (wl, static["tile_id"], static["splits"]))
    rc, tile, splits, us_best, us_default = abi.conv2d_fwd_autotune(
        x.data_ptr(), w.data_ptr(), b.data_ptr(), wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW,
        wl.stride, wl.pad, wl.dilation, wl.dtype, out.data_ptr(), s)
    assert rc == 0, abi.conv2d_strerror(rc)
    log("autotune %s -> tile %d splits %d: %.2f us (static %.2f us)"
        % (wl.name, tile, splits, us_best, us_default))
    assert 0 < us_best <= us_default
    y = fetch(out, (OH, OW, n_out), wl)
    check(y, ref[0], ref[1], "autotuned output %s" % wl)
    tuned = plan_of(wl)
    assert tuned["tile_id"] == tile
    # conv2d_fwd now runs the recorded plan
    out2 = torch.full((n_out + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    out2[n_out:] = SENTINEL
    rc = abi.conv2d_fwd(x.data_ptr(), w.data_ptr(), b.data_ptr(), wl.N, wl.H, wl.W, wl.IC, wl.OC,
                        wl.KH, wl.KW, wl.stride, wl.pad, wl.dilation, wl.dtype, out2.data_ptr(), s)
    assert rc == 0
    check(fetch(out2, (OH, OW, n_out), wl), ref[0], ref[1], "conv2d_fwd after autotune %s" % wl)
    assert abi.conv2d_fwd_status(s) == 0
    abi.conv2d_fwd_autotune_clear()
    again = plan_of(wl)
    assert (again["tile_id"], again["splits"]) == (static["tile_id"], static["splits"])
