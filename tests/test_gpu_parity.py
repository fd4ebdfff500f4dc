"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every comparison is element by element with |err| <= 1e-3*S + 1e-5 (see
gpu_harness.py), on seeded synthetic inputs.  Covered:
  * the five named workloads at full size, all outputs, in the launch
    configuration the benchmark times (automatic plan);
  * fp32 storage (unrounded and bf16-exact values);
  * NULL bias; misaligned buffers (forces the element-wise gather);
  * a seeded sweep of small shapes over every mask (M, N, K tails; IC that
    is and is not a multiple of 8 or 64; stride, padding, dilation);
  * every tile x loader x split-K factor on forced plans;
  * degenerate shapes (1x1, a window covering the input, stride larger than
    the window, outputs that see only padding, IC = 1, OC = 1);
  * split-K determinism and concurrent streams;
  * the largest output the int32 indexing allows, on sampled pixels.
"""
import numpy as np
import pytest
import torch

from convolution_implicit_gemm_fwd_amd import abi
from convolution_implicit_gemm_fwd_amd.workloads import (BF16, FP32, WORKLOAD_ORDER, WORKLOADS,
                                                         make_inputs)

import oracle
from gpu_harness import (GUARD, SENTINEL, check, fetch, log, need_gpu, oracle_full, parity,
                         run_hip, shape, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    abi.conv2d_fwd_force(-1, -1, -1)
    yield
    abi.conv2d_fwd_force(-1, -1, -1)


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_named_workload_full_parity(name):
    wl = WORKLOADS[name]
    rc, plan = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride,
                                   wl.pad, wl.dilation, wl.dtype, 0)
    log("workload %s plan %s" % (name, plan))
    ratio, y, _ = parity(wl)
    log("workload %s worst err/tol %.3g" % (name, ratio))


def test_tiny_fp32_unrounded():
    """fp32 storage of values that are not bf16-representable: the fp32 path
    multiplies in fp32, so the same tolerance holds."""
    parity(WORKLOADS["tiny"], round_bf16=False, dtype=FP32)


def test_tiny_both_storages_agree():
    wl = WORKLOADS["tiny"]
    _, y32, ref = parity(wl, dtype=FP32)
    _, y16, _ = parity(wl, dtype=BF16, ref=ref)
    check(y16, y32.astype(np.float64), ref[1], "bf16 vs fp32 storage")


def test_null_bias():
    wl = WORKLOADS["stem7x7"].scaled(N=2)
    parity(wl, use_bias=False)
    wl = shape(2, 11, 9, 64, 70, 3, 3, 1, 1, 1)
    parity(wl, use_bias=False)


def test_misaligned_buffers():
    for wl in (shape(2, 10, 10, 64, 64, 3, 3, 1, 1, 1), shape(1, 9, 12, 16, 40, 3, 3, 2, 1, 1)):
        _, p = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride,
                                   wl.pad, wl.dilation, BF16, 0)
        parity(wl, misalign=True)


def sweep_shapes(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        N = int(rng.integers(1, 4))
        H, W = int(rng.integers(1, 24)), int(rng.integers(1, 24))
        IC = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 24, 40, 64, 128, 192]))
        OC = int(rng.choice([1, 3, 16, 17, 33, 64, 65, 100, 128, 129, 200]))
        KH, KW = int(rng.choice([1, 2, 3, 5, 7])), int(rng.choice([1, 2, 3, 5, 7]))
        s, p, d = int(rng.integers(1, 4)), int(rng.integers(0, 4)), int(rng.integers(1, 4))
        if d * (KH - 1) + 1 > H + 2 * p or d * (KW - 1) + 1 > W + 2 * p:
            continue
        out.append(shape(N, H, W, IC, OC, KH, KW, s, p, d, name="sweep%d" % len(out)))
    return out


@pytest.mark.parametrize("chunk", range(4))
def test_random_shape_sweep(chunk):
    for i, wl in enumerate(sweep_shapes(100, seed=2024)[chunk * 25:(chunk + 1) * 25]):
        log("sweep %d: %s" % (chunk * 25 + i, wl))
        parity(wl, seed=i)


FORCE_SHAPES = [
    shape(2, 9, 9, 128, 96, 3, 3, 1, 1, 1, name="force-a"),    # M 162, OC tail, 18 K tiles
    shape(1, 13, 7, 64, 130, 3, 2, 2, 2, 2, name="force-b"),   # dilated, non-square kernel
]


@pytest.mark.parametrize("wl", FORCE_SHAPES, ids=lambda w: w.name)
def test_forced_variants(wl):
    inp = make_inputs(wl, seed=5)
    ref = oracle_full(inp, wl)
    for tile in range(abi.conv2d_fwd_num_tiles()):
        for loader in (abi.CONVIMG_LOADER_TAP, abi.CONVIMG_LOADER_VEC8, abi.CONVIMG_LOADER_SCALAR):
            for splits in (1, 2, 3, 5, 8):
                log("forced %s tile=%d loader=%d splits=%d" % (wl.name, tile, loader, splits))
                parity(wl, seed=5, force=(tile, splits, loader), ref=ref)


WINDOW_SHAPES = [
    shape(2, 40, 36, 3, 64, 7, 7, 2, 3, 1, name="stem-like"),
    shape(1, 17, 300, 3, 16, 7, 7, 2, 3, 1, name="rows of 2 units"),   # OW 150; x ends mid-chunk
    shape(2, 20, 22, 3, 70, 3, 3, 2, 1, 1, name="3x3 s2, OC tail"),
    shape(1, 15, 15, 4, 64, 5, 5, 1, 2, 1, name="IC 4 s1"),
    shape(1, 19, 18, 2, 33, 5, 3, 1, 3, 2, name="IC 2 dilated"),
    shape(2, 9, 10, 1, 64, 7, 7, 2, 3, 1, name="IC 1 s2"),
    shape(1, 12, 14, 6, 129, 3, 5, 2, 0, 1, name="IC 6 no pad, 3 slices"),
    shape(3, 5, 6, 3, 8, 3, 3, 2, 4, 1, name="padding beyond window"),
]


@pytest.mark.parametrize("wl", WINDOW_SHAPES, ids=lambda w: w.name)
def test_window_kernel(wl):
    """Few-channel layers take the window kernel; parity with the oracle,
    masked rows and channels, rows split into several units."""
    rc, plan = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride,
                                   wl.pad, wl.dilation, BF16, 0)
    assert abi.conv2d_fwd_tile_kind(plan["tile_id"]) == abi.CONVIMG_KIND_WINDOW, plan
    log("window %s plan %s" % (wl.name, plan))
    parity(wl, seed=7)


RESIDENT_SHAPES = [
    shape(2, 14, 14, 64, 64, 3, 3, 1, 1, 1, name="resnet-like"),
    shape(8, 5, 6, 32, 64, 3, 3, 1, 1, 1, name="ranges over several images"),
    shape(1, 9, 40, 16, 40, 3, 3, 1, 1, 1, name="IC 16, OC tail"),
    shape(2, 9, 9, 128, 100, 3, 3, 1, 1, 1, name="IC 128, two slices"),
    shape(2, 17, 15, 64, 64, 3, 3, 2, 1, 1, name="stride 2"),
    shape(1, 16, 16, 32, 64, 3, 3, 1, 2, 2, name="dilation 2"),
    shape(3, 8, 7, 64, 8, 3, 3, 1, 0, 1, name="no padding, OC 8"),
    shape(1, 3, 3, 64, 64, 3, 3, 1, 3, 1, name="padding beyond window"),
    shape(2, 9, 9, 32, 50, 3, 3, 1, 1, 1, name="OC 50, dword stores"),
]


@pytest.mark.parametrize("wl", RESIDENT_SHAPES, ids=lambda w: w.name)
def test_resident_kernel(wl):
    """Forced onto the kernel with weights and input rows resident in LDS:
    parity with the oracle for ranges crossing rows and images, channel
    tails and several 64-channel slices, strides, dilation and padding."""
    (t,) = [t for t in range(abi.conv2d_fwd_num_tiles())
            if abi.conv2d_fwd_tile_kind(t) == abi.CONVIMG_KIND_RESIDENT]
    abi.conv2d_fwd_force(t, -1, -1)
    try:
        rc, plan = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride,
                                       wl.pad, wl.dilation, BF16, 0)
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    assert plan["tile_id"] == t, plan
    log("resident %s plan %s" % (wl.name, plan))
    parity(wl, seed=11, force=(t, -1, -1))


IMAGE_SHAPES = [
    shape(2, 14, 14, 128, 64, 3, 3, 1, 1, 1, name="largek-like, 2 chunks"),
    shape(3, 7, 7, 256, 100, 3, 3, 1, 1, 1, name="7x7, 4 chunks, OC tail"),
    shape(2, 13, 13, 64, 32, 3, 3, 2, 1, 1, name="stride 2"),
    shape(1, 12, 12, 128, 64, 3, 3, 1, 2, 2, name="dilation 2"),
    shape(2, 16, 16, 64, 32, 3, 3, 1, 0, 1, name="no padding, 7 blocks"),
    shape(5, 4, 4, 64, 64, 3, 3, 1, 1, 1, name="one block per image"),
    shape(1, 9, 11, 192, 40, 3, 3, 1, 1, 1, name="3 chunks, odd sizes"),
    shape(2, 10, 10, 64, 50, 3, 3, 1, 1, 1, name="OC 50, dword stores"),
]


@pytest.mark.parametrize("wl", IMAGE_SHAPES, ids=lambda w: w.name)
def test_image_kernel(wl):
    """Forced onto the kernel with one image x 32 channels per workgroup:
    parity with the oracle over chunk counts, channel tails, strides,
    dilation, padding and the block counts (one wave group idle)."""
    (t,) = [t for t in range(abi.conv2d_fwd_num_tiles())
            if abi.conv2d_fwd_tile_kind(t) == abi.CONVIMG_KIND_IMAGE]
    abi.conv2d_fwd_force(t, -1, -1)
    try:
        rc, plan = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride,
                                       wl.pad, wl.dilation, BF16, 0)
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    assert plan["tile_id"] == t, plan
    log("image %s plan %s" % (wl.name, plan))
    parity(wl, seed=13, force=(t, -1, -1))


DEGENERATE = [
    shape(3, 7, 5, 8, 9, 1, 1, 1, 0, 1, name="1x1"),
    shape(2, 6, 6, 16, 16, 1, 1, 2, 0, 1, name="1x1 stride 2"),
    shape(2, 5, 5, 8, 8, 5, 5, 1, 0, 1, name="window = input"),
    shape(1, 11, 11, 8, 8, 3, 3, 5, 0, 1, name="stride > window"),
    shape(1, 4, 4, 8, 12, 3, 3, 1, 4, 1, name="padding beyond window"),   # border outputs = bias
    shape(2, 9, 9, 1, 5, 3, 3, 1, 1, 1, name="IC 1"),
    shape(2, 9, 9, 64, 1, 3, 3, 1, 1, 1, name="OC 1"),
    shape(1, 20, 20, 8, 8, 3, 3, 1, 9, 9, name="dilation 9"),
    shape(1, 1, 1, 64, 64, 1, 1, 1, 0, 1, name="single pixel"),
    shape(1, 1, 30, 16, 16, 1, 7, 1, 0, 1, name="one row"),
]


@pytest.mark.parametrize("wl", DEGENERATE, ids=lambda w: w.name)
def test_degenerate_shapes(wl):
    parity(wl)


def test_padding_only_outputs_equal_bias():
    """Outputs whose window lies entirely in the padding are exactly the bias."""
    wl = shape(1, 4, 4, 8, 12, 3, 3, 1, 4, 1)
    _, y, _ = parity(wl)
    inp = make_inputs(wl, seed=0)
    assert np.array_equal(y[0, 0, 0], inp.bias)


# The large-K workload's own plan is the image kernel (no split-K); these
# tests force the pipelined 128x64 tile with split-K on it.
SPLITK_FORCE = (11, 4, -1)


def forced_splits(wl):
    abi.conv2d_fwd_force(*SPLITK_FORCE)
    try:
        rc, plan = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride,
                                       wl.pad, wl.dilation, BF16, 0)
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    return plan["splits"]


def test_splitk_deterministic():
    wl = WORKLOADS["largek"]
    assert forced_splits(wl) > 1
    inp = make_inputs(wl, seed=0)
    x, w, b = to_device(inp)
    first = None
    abi.conv2d_fwd_force(*SPLITK_FORCE)
    try:
        for rep in range(10):
            out, dims = run_hip(wl, x, w, b, wl.dtype)
            y = fetch(out, dims, wl)
            if first is None:
                first = y.copy()
            else:
                assert np.array_equal(y, first), "split-K result changed on repeat %d" % rep
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    assert abi.conv2d_fwd_status(torch.cuda.current_stream().cuda_stream) == 0
    yref, S = oracle_full(inp, wl)
    check(first, yref, S, "largek")


def test_splitk_concurrent_streams():
    """Two split-K problems on two streams at once (separate semaphores)."""
    # grids of 56 and 144 workgroups: both fit on the chip at once
    wls = [shape(4, 14, 14, 256, 256, 3, 3, 1, 1, 1, name="s256"),
           shape(2, 14, 14, 512, 512, 3, 3, 1, 1, 1, name="s512")]
    assert all(forced_splits(wl) > 1 for wl in wls)
    ins = [make_inputs(wl, seed=3) for wl in wls]
    devs = [to_device(i) for i in ins]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    abi.conv2d_fwd_force(*SPLITK_FORCE)
    try:
        _splitk_streams_run(wls, devs, streams, outs)
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    for st in streams:
        assert abi.conv2d_fwd_status(st.cuda_stream) == 0
    for wl, inp, (out, dims) in zip(wls, ins, outs):
        y = fetch(out, dims, wl)
        yref, S = oracle_full(inp, wl)
        check(y, yref, S, wl.name)


def _splitk_streams_run(wls, devs, streams, outs):
    for rep in range(3):
        bufs = []
        for wl in wls:
            OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
            n_out = wl.N * OH * OH * wl.OC
            buf = torch.full((n_out + GUARD,), float("nan"), device="cuda")
            buf[n_out:] = SENTINEL
            bufs.append(buf)
        torch.cuda.synchronize()            # prefills done before the other streams start
        outs[:] = [run_hip(wl, x, w, b, BF16, stream=st.cuda_stream, out=buf)
                   for wl, (x, w, b), st, buf in zip(wls, devs, streams, bufs)]
        torch.cuda.synchronize()


def test_largest_int32_output_sampled():
    """N*OH*OW*OC just under 2^31: the last flat output index is near the
    int32 limit.  Checked on sampled pixels (including the last one and the
    pixels around 2^30 and 2^31 flat elements) with the oracle's per-pixel
    entry."""
    wl = shape(1, 2048, 2048, 64, 511, 3, 3, 1, 1, 1, name="int32-edge")
    M = 2048 * 2048
    assert M * 511 < 2 ** 31
    inp = make_inputs(wl, seed=9)
    x, w, b = to_device(inp)
    out = torch.empty((M * 511,), dtype=torch.float32, device="cuda")
    out.fill_(float("nan"))
    OH = abi.conv2d_fwd_out_dim(2048, 3, 1, 1, 1)
    rc = abi.conv2d_fwd(x.data_ptr(), w.data_ptr(), b.data_ptr(), 1, 2048, 2048, 64, 511, 3, 3,
                        1, 1, 1, BF16, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0 and OH == 2048
    rng = np.random.default_rng(1)
    pix = np.unique(np.concatenate([
        [0, 2047, M - 2048, M - 1, (2 ** 30) // 511, (2 ** 30) // 511 + 1, M - 1 - 2049],
        rng.integers(0, M, 200)]))
    rows = out.view(M, 511)[torch.from_numpy(pix).cuda()].cpu().numpy()
    yref, S = oracle.conv2d_fwd_pixels(inp.x32, inp.w32, inp.bias, 1, 1, 1, pix)
    check(rows, yref, S, "int32 edge")
    del out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("OC", [160, 158], ids=["OC160-16B-stores", "OC158-dword-stores"])
@pytest.mark.parametrize("tile_kind", [abi.CONVIMG_KIND_REGS, abi.CONVIMG_KIND_PIPE])
def test_output_between_2_and_4_gib_sampled(OC, tile_kind):
    """An output of 2..4 GiB on the single-split kernels.  Masked lanes (the
    last 64-channel tile is partly past OC) store to the out-of-range buffer
    offset 2^31, which lies inside such an output: the library must take the
    64-bit store path there.  Checked on sampled pixels, always including
    those around flat element 2^29 (byte offset 2^31) and the last one."""
    N, H, W, IC = 64, 256, 256, 8
    wl = shape(N, H, W, IC, OC, 3, 3, 1, 1, 1, name="2-4 GiB out")
    M = N * H * W
    assert 2 ** 31 < M * OC * 4 < 2 ** 32
    tile = [t for t in range(abi.conv2d_fwd_num_tiles())
            if abi.conv2d_fwd_tile_kind(t) == tile_kind and t in (0, 4)][0]   # 128x64 tiles
    inp = make_inputs(wl, seed=17)
    x, w, b = to_device(inp)
    out = torch.full((M * OC,), float("nan"), dtype=torch.float32, device="cuda")
    abi.conv2d_fwd_force(tile, 1, abi.CONVIMG_LOADER_VEC8)
    try:
        rc, plan = abi.conv2d_fwd_plan(N, H, W, IC, OC, 3, 3, 1, 1, 1, BF16, 0)
        assert plan["tile_id"] == tile and plan["splits"] == 1, plan
        log("2-4 GiB OC=%d plan %s" % (OC, plan))
        rc = abi.conv2d_fwd(x.data_ptr(), w.data_ptr(), b.data_ptr(), N, H, W, IC, OC, 3, 3,
                            1, 1, 1, BF16, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert rc == 0, abi.conv2d_strerror(rc)
        torch.cuda.synchronize()
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    hot = (2 ** 29) // OC
    rng = np.random.default_rng(3)
    pix = np.unique(np.concatenate([[0, hot - 1, hot, hot + 1, M - 1], rng.integers(0, M, 100)]))
    rows = out.view(M, OC)[torch.from_numpy(pix).cuda()].cpu().numpy()
    yref, S = oracle.conv2d_fwd_pixels(inp.x32, inp.w32, inp.bias, 1, 1, 1, pix)
    check(rows, yref, S, "2-4 GiB output OC=%d" % OC)
    del out
    torch.cuda.empty_cache()


def test_splitk_timeout_poisons_and_resets():
    """The split-K wait forced to give up from the host (a one-iteration
    bound): a split that gives up writes NaN over its tile instead of adding
    its partial, conv2d_fwd_status reports the timeout and resets the
    semaphores, and the next call with the normal bound is correct.  (Whether
    a split gives up depends on timing; either outcome is checked.)"""
    wl = WORKLOADS["largek"]
    inp = make_inputs(wl, seed=0)
    x, w, b = to_device(inp)
    sptr = torch.cuda.current_stream().cuda_stream
    yref, S = oracle_full(inp, wl)
    abi.conv2d_fwd_force(*SPLITK_FORCE)
    prev = abi.conv2d_fwd_test_spin_limit(1)
    try:
        out, dims = run_hip(wl, x, w, b, wl.dtype)
        torch.cuda.synchronize()
        abi.conv2d_fwd_test_spin_limit(prev)
        status = abi.conv2d_fwd_status(sptr)
        OH, OW, n_out = dims
        y = out[:n_out].cpu().numpy()
        log("forced timeout: status %d, NaN outputs %d" % (status, int(np.isnan(y).sum())))
        if status == abi.CONVIMG_OK:
            check(y.reshape(wl.N, OH, OW, wl.OC), yref, S, "no split gave up")
        else:
            assert status == abi.CONVIMG_ERR_TIMEOUT
            assert np.isnan(y).any(), "a split gave up but out shows no poisoned tile"
        assert abi.conv2d_fwd_status(sptr) == abi.CONVIMG_OK
        out, dims = run_hip(wl, x, w, b, wl.dtype)
        y = fetch(out, dims, wl)
    finally:
        abi.conv2d_fwd_test_spin_limit(0)
        abi.conv2d_fwd_force(-1, -1, -1)
    assert abi.conv2d_fwd_status(sptr) == abi.CONVIMG_OK
    check(y, yref, S, "after the reset")
