"""GPU parity of the data backward (conv2d_bwd_data) against the
fp64 oracle's definition of the input gradient, element by element with the
forward's bound |err| <= 1e-3*S + 1e-5 (S: the oracle's sum of |dy*w| over
each element's terms).

The flipped, transposed weights the call leaves in its workspace are checked
bit-exactly against a numpy index permutation of w (a pure data movement).
dx is pre-filled with NaN (an element never written fails) and followed by a
sentinel guard (a write past the end fails).  Covered: the three stride-1
named layers (ResNet-style, 512-channel, dilated) at full size, IC != OC with
channel tails, 1x1, 5x5, edge paddings (0 and dilation*(K-1)), IC = 3 with a
7x7 window, fp32 storage, and the torch wrapper; the weight transform alone
on non-square windows, channel tails and misaligned buffers (element path);
and the fallback route for the problems the stride-1 mapping does not
serve (strides 2 to 4, dilations with stride, non-square windows, padding
beyond dilation*(K-1), a ResNet-style stride-2 layer, the stem layer at
full size: the kernel by phases of the stride; fp32 storage, OC % 8 != 0
and misaligned buffers: the element-wise kernel).
"""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_fwd_amd as cig
from convolution_implicit_gemm_fwd_amd import abi
from convolution_implicit_gemm_fwd_amd.workloads import BF16, FP32, WORKLOADS, make_grad_inputs

import oracle
from gpu_harness import GUARD, SENTINEL, check, log, need_gpu, shape

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    abi.conv2d_fwd_force(-1, -1, -1)


def upload(a, misalign=False):
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16))).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    if not misalign:
        return t.cuda()
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    flat[1:].copy_(t.reshape(-1))
    return flat[1:].view(t.shape)          # one element past a 16-byte boundary


def bwd_parity(wl, dtype=None, seed=0, misalign=False):
    dtype = wl.dtype if dtype is None else dtype
    OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
    OW = abi.conv2d_fwd_out_dim(wl.W, wl.KW, wl.stride, wl.pad, wl.dilation)
    assert OH > 0 and OW > 0
    inp = make_grad_inputs(wl, OH, OW, seed=seed, dtype=dtype)
    dy, w = upload(inp.x_store, misalign), upload(inp.w_store, misalign)
    n_w = w.numel()
    wt_buf = torch.empty(n_w + (1 if misalign else 0), dtype=w.dtype, device="cuda")
    wt = wt_buf[1:] if misalign else wt_buf
    # a pattern no transform writes everywhere: wt must come back either
    # untouched (the GEMM flipped the weights in LDS itself) or transformed
    wt.view(torch.int16).fill_(0x7F81)
    n_dx = wl.N * wl.H * wl.W * wl.IC
    off = 1 if misalign else 0                 # dx 4-byte but not 16-byte aligned
    dx_buf = torch.full((n_dx + GUARD + off,), float("nan"), dtype=torch.float32, device="cuda")
    dx = dx_buf[off:]
    dx[n_dx:] = SENTINEL
    log("dgrad %s dtype=%d" % (wl, dtype))
    rc = abi.conv2d_bwd_data(dy.data_ptr(), w.data_ptr(), wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH,
                             wl.KW, wl.stride, wl.pad, wl.dilation, dtype, wt.data_ptr(), dx.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert rc == 0, abi.conv2d_strerror(rc)
    torch.cuda.synchronize()
    host = dx.cpu().numpy()
    assert (host[n_dx:] == SENTINEL).all(), "write past the end of dx"
    y = host[:n_dx].reshape(wl.N, wl.H, wl.W, wl.IC)
    # the workspace: untouched where the GEMM flips the weights in LDS (the
    # resident kernel at 64 -> 64 channels), else w[oc][kh][kw][ic] ->
    # wt[ic][KH-1-kh][KW-1-kw][oc], bit for bit
    want = np.ascontiguousarray(inp.w_store[:, ::-1, ::-1, :].transpose(3, 1, 2, 0))
    raw = wt.view(torch.int16).cpu().numpy()
    untouched = bool((raw == 0x7F81).all())
    if not untouched:
        got = raw.view(np.uint16) if dtype == BF16 else wt.cpu().numpy()
        assert np.array_equal(got.reshape(want.shape), want), "flipped weights differ"
    log("dgrad %s: %s" % (wl.name, "weights flipped in LDS" if untouched else "weights transformed into wt"))
    yref, S = oracle.conv2d_bwd_data(inp.x32, inp.w32, wl.H, wl.W, wl.stride, wl.pad, wl.dilation)
    ratio = check(y, yref, S, "dgrad %s" % (wl,))
    log("dgrad %s worst err/tol %.3g" % (wl.name, ratio))
    return y, yref, untouched


# the stride-1 named layers at full size, planned as bench.py --op dgrad runs them
FULL = [WORKLOADS["resnet3x3"], WORKLOADS["largek"], WORKLOADS["dilated"]]

SMALL = [
    shape(2, 13, 11, 24, 40, 3, 3, 1, 1, 1, name="IC 24 OC 40 tails"),
    shape(2, 9, 17, 40, 24, 3, 3, 1, 1, 1, name="IC 40 OC 24 tails"),
    shape(3, 10, 10, 64, 96, 1, 1, 1, 0, 1, name="1x1"),
    shape(2, 12, 12, 32, 48, 5, 5, 1, 2, 1, name="5x5 pad 2"),
    shape(2, 12, 12, 32, 48, 5, 5, 1, 0, 1, name="5x5 pad 0 (full pad after mapping)"),
    shape(2, 11, 11, 64, 64, 3, 3, 1, 2, 1, name="pad = K-1 (no pad after mapping)"),
    shape(1, 20, 20, 64, 64, 3, 3, 1, 0, 2, name="dilation 2 pad 0"),
    shape(1, 21, 19, 16, 72, 3, 3, 1, 6, 3, name="dilation 3 full pad"),
    shape(2, 30, 30, 3, 64, 7, 7, 1, 3, 1, name="IC 3 7x7"),
    shape(1, 8, 8, 1, 1, 3, 3, 1, 1, 1, name="IC 1 OC 1"),
    shape(1, 3, 3, 8, 8, 3, 3, 1, 0, 1, name="single output pixel"),
]


def test_dgrad_weights_flipped_in_lds():
    """The GEMM flips and transposes the forward weights in LDS itself (one
    launch, wt left as it was): the resident kernel at 64 -> 64 channels
    (full size, and a small image), the image kernel per 64-channel chunk
    (the 512-channel layer, 128 -> 192 channels, 64 -> 256 on 7x7 maps)."""
    for wl in (WORKLOADS["resnet3x3"], shape(2, 16, 16, 64, 64, 3, 3, 1, 1, 1, name="64 -> 64 small"),
               WORKLOADS["largek"], shape(4, 14, 14, 128, 192, 3, 3, 1, 1, 1, name="image 128 -> 192"),
               shape(2, 7, 7, 64, 256, 3, 3, 1, 1, 1, name="image 64 -> 256 7x7")):
        _, _, untouched = bwd_parity(wl, seed=3)
        assert untouched, "%s: expected the in-LDS flip, got the transform into wt" % wl.name


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_dgrad_full_size(wl):
    bwd_parity(wl)


# the fallback route: every problem the stride-1 mapping does not serve
GENERAL = [
    shape(2, 15, 17, 24, 40, 3, 3, 2, 1, 1, name="stride 2, channel tails"),
    shape(2, 30, 30, 3, 64, 7, 7, 2, 3, 1, name="stride 2 7x7 IC 3"),
    shape(2, 12, 14, 32, 48, 3, 5, 1, 2, 1, name="3x5 window"),
    shape(1, 9, 9, 16, 16, 3, 3, 1, 3, 1, name="pad 3 > dilation*(K-1)"),
    shape(1, 20, 22, 16, 24, 3, 3, 3, 2, 2, name="stride 3 dilation 2"),
    shape(3, 10, 10, 64, 96, 1, 1, 2, 0, 1, name="1x1 stride 2"),
    shape(2, 13, 11, 24, 40, 3, 3, 2, 1, 1, dtype=FP32, name="fp32 stride 2"),
    shape(1, 5, 5, 8, 8, 5, 3, 2, 2, 1, dtype=FP32, name="fp32 5x3 stride 2"),
    shape(1, 11, 9, 16, 12, 3, 3, 2, 1, 1, name="stride 2 OC 12 (element-wise kernel)"),
    shape(1, 14, 15, 72, 136, 3, 3, 2, 1, 1, name="stride 2, two channel blocks each side"),
    shape(1, 9, 9, 8, 8, 2, 2, 4, 0, 1, name="stride 4 > window: phases no tap reaches"),
    shape(1, 10, 10, 16, 8, 3, 3, 2, 2, 2, name="stride 2 dilation 2"),
    shape(2, 12, 12, 8, 16, 3, 3, 2, 0, 3, name="stride 2 dilation 3"),
    shape(4, 56, 56, 128, 128, 3, 3, 2, 1, 1, name="ResNet-style stride-2 layer, N=4"),
    WORKLOADS["stem7x7"],
]


@pytest.mark.parametrize("wl", GENERAL, ids=lambda w: w.name)
def test_dgrad_general_kernel(wl):
    """Strides above 1, non-square windows and padding beyond dilation*(K-1)
    take the fallback route (dx from its definition; wt untouched)."""
    _, _, untouched = bwd_parity(wl)
    assert untouched, "the fallback route does not use wt"


def test_dgrad_general_misaligned():
    """dy, w and dx off 16-byte alignment at stride 2: the element-wise
    kernel (the kernel by phases needs 16-byte runs of dy)."""
    _, _, untouched = bwd_parity(shape(2, 13, 12, 24, 40, 3, 3, 2, 1, 1), misalign=True)
    assert untouched


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_dgrad_shapes(wl):
    bwd_parity(wl)


@pytest.mark.parametrize("wl", SMALL[:3] + SMALL[6:7], ids=lambda w: w.name)
def test_dgrad_fp32_storage(wl):
    bwd_parity(wl, dtype=FP32)


def test_dgrad_torch_wrapper():
    wl = shape(2, 14, 14, 48, 80, 3, 3, 1, 1, 1)
    inp = make_grad_inputs(wl, 14, 14, seed=3)
    dy, w = upload(inp.x_store), upload(inp.w_store)
    dx = cig.conv2d_bwd_data_nhwc(dy, w, 14, 14, stride=1, pad=1)
    torch.cuda.synchronize()
    yref, S = oracle.conv2d_bwd_data(inp.x32, inp.w32, 14, 14, 1, 1, 1)
    check(dx.cpu().numpy(), yref, S, "wrapper")
    # stride 2 (the fallback route): dy of the 7 x 7 forward output
    dy2 = inp.x_store[:, ::2, ::2].copy()
    dx2 = cig.conv2d_bwd_data_nhwc(upload(dy2), w, 14, 14, stride=2, pad=1)
    torch.cuda.synchronize()
    yref2, S2 = oracle.conv2d_bwd_data(inp.x32[:, ::2, ::2], inp.w32, 14, 14, 2, 1, 1)
    check(dx2.cpu().numpy(), yref2, S2, "wrapper stride 2")


@pytest.mark.parametrize("OC,KH,KW,IC,dtype,misalign", [
    (512, 3, 3, 512, BF16, False),      # 16-byte loads and stores
    (8, 1, 1, 8, BF16, False),          # one partial tile
    (64, 3, 3, 32, FP32, False),        # fp32, 16-byte loads and stores
    (40, 3, 5, 24, BF16, False),        # non-square window
    (70, 2, 3, 45, BF16, False),        # channel counts off the vector: element path
    (64, 3, 3, 64, BF16, True),         # misaligned w and wt: element path
    (36, 5, 1, 20, FP32, False),
    (33, 3, 3, 7, FP32, True),
])
def test_weight_transform_alone(OC, KH, KW, IC, dtype, misalign):
    rng = np.random.default_rng(7)
    n = OC * KH * KW * IC
    if dtype == BF16:
        host = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)   # any bit pattern moves
        dev_t, pad_val = torch.int16, 0x7F7F
    else:
        host = rng.standard_normal(n).astype(np.float32)
        dev_t, pad_val = torch.float32, 1234.5
    off = 1 if misalign else 0
    src = torch.full((n + off,), pad_val, dtype=dev_t, device="cuda")
    src[off:] = torch.from_numpy(host.view(np.int16) if dtype == BF16 else host).cuda()
    dst = torch.full((n + off + GUARD,), pad_val, dtype=dev_t, device="cuda")
    rc = abi.conv2d_bwd_data_weights(src[off:].data_ptr(), OC, KH, KW, IC, dtype,
                                     dst[off:].data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, abi.conv2d_strerror(rc)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    got = got.view(np.uint16) if dtype == BF16 else got
    pad = np.uint16(pad_val) if dtype == BF16 else np.float32(pad_val)
    assert (got[:off] == pad).all() and (got[off + n:] == pad).all(), "write outside wt"
    want = host.reshape(OC, KH, KW, IC)[:, ::-1, ::-1, :].transpose(3, 1, 2, 0)
    assert np.array_equal(got[off:off + n].reshape(IC, KH, KW, OC), want)


def test_dgrad_misaligned_buffers():
    """dy, w, the workspace and dx one element off their 16-byte boundaries:
    the transform's element path and the forward's element-wise gather and
    4-byte stores."""
    bwd_parity(shape(2, 10, 10, 64, 64, 3, 3, 1, 1, 1, name="misaligned 64ch"), misalign=True)
    bwd_parity(shape(1, 9, 12, 16, 40, 3, 3, 1, 2, 2, name="misaligned dilated"), misalign=True)
