"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libconvimg.so loads and exports every function include/convimg.h declares;
* the output extent agrees with the hand-counted table;
* the plan for each named workload has the expected loader, tile and split;
* every argument error is reported with its code before any device work.
"""
import os
import re

import pytest

from convolution_implicit_gemm_fwd_amd import abi
from convolution_implicit_gemm_fwd_amd.workloads import BF16, WORKLOADS, Workload

from pins import read_table

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convimg.h")


@pytest.fixture(scope="module")
def lib():
    return abi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(abi.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), "libconvimg.so does not export %s" % n


def test_out_dim_table(lib):
    for size, k, s, p, d, want in read_table("out_dims.txt"):
        assert abi.conv2d_fwd_out_dim(int(size), int(k), int(s), int(p), int(d)) == int(want)
    assert abi.conv2d_fwd_out_dim(5, 3, 0, 1, 1) == -1
    assert abi.conv2d_fwd_out_dim(5, 3, 1, -1, 1) == -1
    assert abi.conv2d_fwd_out_dim(5, 3, 1, 1, 0) == -1


def test_strerror(lib):
    for code in range(12):
        msg = abi.conv2d_strerror(code)
        assert msg and msg != "unknown status"
    assert abi.conv2d_strerror(1234) == "unknown status"


def plan_of(wl, num_cus=256, dtype=None):
    rc, p = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride, wl.pad,
                                wl.dilation, wl.dtype if dtype is None else dtype, num_cus)
    assert rc == abi.CONVIMG_OK, abi.conv2d_strerror(rc)
    return p


def test_plans_of_named_workloads(lib):
    abi.conv2d_fwd_force(-1, -1, -1)
    p = plan_of(WORKLOADS["tiny"])
    assert p["loader"] == abi.CONVIMG_LOADER_FP32 and (p["OH"], p["OW"]) == (8, 8)
    assert p["M"] == 64 and p["K"] == 144 and p["splits"] == 1
    p = plan_of(WORKLOADS["tiny"], dtype=abi.CONVIMG_BF16)
    assert p["loader"] == abi.CONVIMG_LOADER_VEC8            # IC = 16
    p = plan_of(WORKLOADS["resnet3x3"])
    assert p["loader"] == abi.CONVIMG_LOADER_TAP and p["M"] == 50176 and p["K"] == 576
    assert p["splits"] == 1 and p["grid"] == p["tiles_m"] * p["tiles_n"]
    p = plan_of(WORKLOADS["largek"])
    assert p["loader"] == abi.CONVIMG_LOADER_TAP and p["K"] == 4608
    # 14x14 images: the image kernel, one workgroup per image and 32 channels
    assert abi.conv2d_fwd_tile_kind(p["tile_id"]) == abi.CONVIMG_KIND_IMAGE
    assert p["splits"] == 1 and p["grid"] == 16 * 16
    # the pipelined 128x64 tile on it: long K with few tiles must split
    abi.conv2d_fwd_force(11, -1, -1)
    try:
        p = plan_of(WORKLOADS["largek"])
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    assert p["splits"] > 1, "long K with few tiles must split"
    tiles = p["tiles_m"] * p["tiles_n"]
    assert p["grid"] == (tiles + 7) // 8 * 8 * p["splits"]      # slots per split padded to 8
    p = plan_of(WORKLOADS["stem7x7"])
    assert p["loader"] == abi.CONVIMG_LOADER_SCALAR and (p["OH"], p["OW"]) == (112, 112)
    # 3 channels: the window kernel (7 kernel rows of 21 <= 32 k values each)
    assert abi.conv2d_fwd_tile_kind(p["tile_id"]) == abi.CONVIMG_KIND_WINDOW
    assert p["K"] == 147 and p["ktiles"] == 7 and p["BK"] == 32
    # up to two workgroups per CU, each walking whole 112-pixel output rows
    assert p["grid"] == p["tiles_m"] * p["tiles_n"] <= 2 * 256 and p["BM"] == 112
    p = plan_of(WORKLOADS["dilated"])
    assert p["loader"] == abi.CONVIMG_LOADER_TAP and (p["OH"], p["OW"]) == (128, 128)
    # 512 tiles of 128x128: two workgroups per CU
    assert p["BM"] == 128 and p["BN"] == 128 and p["grid"] == 512 and p["splits"] == 1


def test_tile_kinds(lib):
    kinds = [abi.conv2d_fwd_tile_kind(t) for t in range(abi.conv2d_fwd_num_tiles())]
    assert set(kinds) == {abi.CONVIMG_KIND_REGS, abi.CONVIMG_KIND_PIPE, abi.CONVIMG_KIND_PATCH,
                          abi.CONVIMG_KIND_STRIP, abi.CONVIMG_KIND_WINDOW, abi.CONVIMG_KIND_RESIDENT,
                          abi.CONVIMG_KIND_IMAGE}
    assert abi.conv2d_fwd_tile_kind(-1) == -1
    assert abi.conv2d_fwd_tile_kind(abi.conv2d_fwd_num_tiles()) == -1


def strip_tiles():
    return [t for t in range(abi.conv2d_fwd_num_tiles())
            if abi.conv2d_fwd_tile_kind(t) == abi.CONVIMG_KIND_STRIP]


def test_strip_plans(lib):
    """A forced strip entry selects the strip kernel where the weight slice
    and the patch fit in LDS, with one workgroup per CU per 64 channels and
    strips that cover M; elsewhere the pipelined kernel."""
    try:
        for t in strip_tiles():
            abi.conv2d_fwd_force(t, -1, -1)
            for name, num_cus in (("resnet3x3", 256), ("resnet3x3", 80), ("dilated", 256)):
                wl = WORKLOADS[name]
                p = plan_of(wl, num_cus=num_cus)
                if name == "dilated":
                    # 64 x 1152 bf16 weights plus the patch do not fit next to each other
                    assert abi.conv2d_fwd_tile_kind(p["tile_id"]) != abi.CONVIMG_KIND_STRIP
                    continue
                assert abi.conv2d_fwd_tile_kind(p["tile_id"]) == abi.CONVIMG_KIND_STRIP
                assert p["splits"] == 1 and p["BN"] == 64 and p["threads"] == 768
                assert p["tiles_n"] == 1 and p["grid"] == p["tiles_m"] <= num_cus
                if num_cus == 256:      # 196 pixels per strip: one chunk of at most BM
                    assert p["BM"] >= -(-p["M"] // p["tiles_m"])
                assert p["lds_bytes"] <= 160 * 1024
            # weights too large for LDS (64 x 9 x 192 bf16), and the element-wise
            # loader: never the strip kernel
            for wl in (WORKLOADS["stem7x7"], WORKLOADS["resnet3x3"].scaled(IC=192)):
                assert abi.conv2d_fwd_tile_kind(plan_of(wl)["tile_id"]) != abi.CONVIMG_KIND_STRIP
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)


def shape(N, H, W, IC, OC, KH, KW, s, p, d):
    dist = ("normal", 0.0, 1.0)
    return Workload("case", N, IC, H, W, OC, KH, KW, s, p, d, BF16, dist, dist, dist)


def resident_tile():
    (t,) = [t for t in range(abi.conv2d_fwd_num_tiles())
            if abi.conv2d_fwd_tile_kind(t) == abi.CONVIMG_KIND_RESIDENT]
    return t


def test_resident_plans(lib):
    """The resident entry holds the 64-channel weight slice and the input rows
    of one CU's share of the pixels in LDS: one 8-wave workgroup per CU per 64
    channels where they fit; elsewhere the pipelined kernel."""
    t = resident_tile()
    try:
        abi.conv2d_fwd_force(t, -1, -1)
        p = plan_of(WORKLOADS["resnet3x3"])
        assert p["tile_id"] == t and p["threads"] == 512 and p["splits"] == 1
        assert p["grid"] == p["tiles_m"] * p["tiles_n"] == 256
        # 64 records of 576 bf16 + 16 bytes; 196 pixels span at most 4 output
        # rows, so 6 input rows of 56 pixels of 144 bytes; one zero record;
        # a store scratch of 32 pixels x 36 floats per wave
        assert p["lds_bytes"] == 64 * 1168 + (6 * 56 * 144 + 1023) // 1024 * 1024 + 144 + 8 * 32 * 36 * 4
        # two 64-channel slices: half the CUs per slice
        wl = shape(2, 20, 20, 32, 100, 3, 3, 1, 1, 1)
        p = plan_of(wl)
        assert p["tile_id"] == t and p["tiles_n"] == 2 and p["tiles_m"] == 128
        for wl in (WORKLOADS["largek"],                           # weights do not fit
                   shape(1, 9, 9, 48, 64, 3, 3, 1, 1, 1),          # IC not 16, 32, 64 or 128
                   shape(1, 9, 9, 64, 64, 5, 5, 1, 2, 1)):         # not 3x3
            assert abi.conv2d_fwd_tile_kind(plan_of(wl)["tile_id"]) == abi.CONVIMG_KIND_PIPE
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)


def test_image_plans(lib):
    """The image entry: one workgroup per image and 32 output channels over
    all of K; two buffer sets of (padded image, 9 x 32 weight records) in LDS;
    elsewhere the pipelined kernel."""
    (t,) = [t for t in range(abi.conv2d_fwd_num_tiles())
            if abi.conv2d_fwd_tile_kind(t) == abi.CONVIMG_KIND_IMAGE]
    try:
        abi.conv2d_fwd_force(t, -1, -1)
        p = plan_of(WORKLOADS["largek"])
        assert p["tile_id"] == t and p["threads"] == 512 and p["splits"] == 1
        assert p["grid"] == 16 * (512 // 32) and p["BM"] == 7 * 32 and p["BN"] == 32
        # padded 16x16 image of 144-byte records with a 224-byte gap per row
        # (row stride 158 units of 16 bytes = 9 * 14 mod 16), 288 weight records, twice
        assert p["lds_bytes"] == 2 * (16 * (16 * 144 + 224) + 288 * 144) == 160 * 1024
        for wl in (WORKLOADS["resnet3x3"],                         # 56x56: 98 blocks of 32 pixels
                   shape(2, 14, 14, 96, 64, 3, 3, 1, 1, 1),         # IC not a multiple of 64
                   shape(2, 14, 14, 64, 64, 5, 5, 1, 2, 1)):        # not 3x3
            assert abi.conv2d_fwd_tile_kind(plan_of(wl)["tile_id"]) == abi.CONVIMG_KIND_PIPE
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)


def test_forced_plans(lib):
    wl = WORKLOADS["largek"]
    try:
        for t in range(abi.conv2d_fwd_num_tiles()):
            assert abi.conv2d_fwd_force(t, 3, abi.CONVIMG_LOADER_VEC8) == 0
            p = plan_of(wl)
            if abi.conv2d_fwd_tile_kind(t) == abi.CONVIMG_KIND_IMAGE:
                assert p["tile_id"] == t and p["splits"] == 1     # 14x14 images fit
                continue
            if abi.conv2d_fwd_tile_kind(t) in (abi.CONVIMG_KIND_STRIP, abi.CONVIMG_KIND_WINDOW,
                                               abi.CONVIMG_KIND_RESIDENT):
                # 64 x 4608 bf16 weights do not fit in LDS, and 512 channels are
                # far more than a window holds: the pipelined kernel instead
                assert abi.conv2d_fwd_tile_kind(p["tile_id"]) == abi.CONVIMG_KIND_PIPE
                continue
            if p["tile_id"] != t:
                # LDS-patch tiles take the tap-aligned loader only and do not split
                abi.conv2d_fwd_force(t, 3, abi.CONVIMG_LOADER_TAP)
                p = plan_of(wl)
                assert p["tile_id"] == t and p["splits"] == 1
                assert p["loader"] == abi.CONVIMG_LOADER_TAP
                continue
            # the forced split may be lowered so every workgroup stays resident
            assert 1 <= p["splits"] <= 3
            slots = (p["tiles_m"] * p["tiles_n"] + 7) // 8 * 8 if p["splits"] > 1 else 0
            assert p["splits"] == 1 or p["grid"] == slots * p["splits"]
            assert p["loader"] == abi.CONVIMG_LOADER_VEC8
        # a vector loader is not honoured where the channels do not allow it
        abi.conv2d_fwd_force(-1, -1, abi.CONVIMG_LOADER_TAP)
        assert plan_of(WORKLOADS["stem7x7"])["loader"] == abi.CONVIMG_LOADER_SCALAR
        # splits of the pipelined kernel are clipped to the K tiles (tiny in
        # bf16: one tile, 3 K tiles)
        abi.conv2d_fwd_force(11, 50, -1)
        assert plan_of(WORKLOADS["tiny"], dtype=abi.CONVIMG_BF16)["splits"] == 3
        abi.conv2d_fwd_force(-1, 50, -1)
        # ... and to what stays resident at once: 1568 tiles leave no room
        assert plan_of(WORKLOADS["stem7x7"])["splits"] == 1
        assert abi.conv2d_fwd_force(abi.conv2d_fwd_num_tiles(), -1, -1) == abi.CONVIMG_ERR_SHAPE
        assert abi.conv2d_fwd_force(-1, -1, 3) == abi.CONVIMG_ERR_SHAPE
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)


BASE = dict(N=2, H=8, W=8, IC=16, OC=16, KH=3, KW=3, stride=1, pad=1, dilation=1, dtype=0)


def call(**kw):
    a = dict(BASE, x=0x1000000, w=0x2000000, bias=None, out=0x3000000, stream=None)
    a.update(kw)
    return abi.conv2d_fwd(a["x"], a["w"], a["bias"], a["N"], a["H"], a["W"], a["IC"], a["OC"],
                          a["KH"], a["KW"], a["stride"], a["pad"], a["dilation"], a["dtype"],
                          a["out"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), abi.CONVIMG_ERR_NULL),
    (dict(w=None), abi.CONVIMG_ERR_NULL),
    (dict(out=None), abi.CONVIMG_ERR_NULL),
    (dict(N=0), abi.CONVIMG_ERR_SHAPE),
    (dict(IC=-1), abi.CONVIMG_ERR_SHAPE),
    (dict(KW=0), abi.CONVIMG_ERR_SHAPE),
    (dict(stride=0), abi.CONVIMG_ERR_SHAPE),
    (dict(pad=-1), abi.CONVIMG_ERR_SHAPE),
    (dict(dilation=0), abi.CONVIMG_ERR_SHAPE),
    (dict(H=2, pad=0), abi.CONVIMG_ERR_SHAPE),                 # window larger than input
    (dict(dtype=2), abi.CONVIMG_ERR_DTYPE),
    (dict(N=1 << 12, H=1 << 10, W=1 << 10), abi.CONVIMG_ERR_RANGE),
    (dict(IC=1 << 16, OC=1 << 14), abi.CONVIMG_ERR_RANGE),
    (dict(out=0x1000000 + 64), abi.CONVIMG_ERR_ALIAS),          # out inside x
    (dict(bias=0x3000000 + 16), abi.CONVIMG_ERR_ALIAS),         # bias inside out
])
def test_argument_errors_before_any_device_work(lib, kw, code):
    assert call(**kw) == code


def test_plan_null(lib):
    assert lib.conv2d_fwd_plan(1, 8, 8, 16, 16, 3, 3, 1, 1, 1, 0, 256, None) == abi.CONVIMG_ERR_NULL


def call_bwd(**kw):
    a = dict(BASE, dy=0x1000000, w=0x2000000, wt=0x4000000, dx=0x3000000, stream=None)
    a.update(kw)
    return abi.conv2d_bwd_data(a["dy"], a["w"], a["N"], a["H"], a["W"], a["IC"], a["OC"],
                               a["KH"], a["KW"], a["stride"], a["pad"], a["dilation"], a["dtype"],
                               a["wt"], a["dx"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dy=None), abi.CONVIMG_ERR_NULL),
    (dict(w=None), abi.CONVIMG_ERR_NULL),
    (dict(wt=None), abi.CONVIMG_ERR_NULL),
    (dict(dx=None), abi.CONVIMG_ERR_NULL),
    (dict(N=0), abi.CONVIMG_ERR_SHAPE),
    (dict(H=2, pad=0), abi.CONVIMG_ERR_SHAPE),
    (dict(dtype=2), abi.CONVIMG_ERR_DTYPE),
    # the fallback route's problems (stride 2, KH != KW, pad beyond
    # dilation*(KH-1)) check the same overlaps before any device work
    (dict(stride=2, dx=0x1000000 + 64), abi.CONVIMG_ERR_ALIAS),
    (dict(KW=5, pad=2, dx=0x2000000 - 64), abi.CONVIMG_ERR_ALIAS),
    (dict(pad=3, dx=0x1000000 - 64), abi.CONVIMG_ERR_ALIAS),
    (dict(N=1 << 12, H=1 << 10, W=1 << 10), abi.CONVIMG_ERR_RANGE),
    # 90000 taps: more transform workgroups along one grid axis than HIP allows
    (dict(N=1, H=300, W=300, IC=1, OC=1, KH=300, KW=300, pad=0), abi.CONVIMG_ERR_RANGE),
    (dict(dx=0x1000000 + 64), abi.CONVIMG_ERR_ALIAS),          # dx inside dy
    (dict(wt=0x2000000 + 2), abi.CONVIMG_ERR_ALIAS),           # wt overlaps w
    (dict(wt=0x3000000 + 32), abi.CONVIMG_ERR_ALIAS),          # wt inside dx
])
def test_bwd_data_errors_before_any_device_work(lib, kw, code):
    assert call_bwd(**kw) == code


def test_bwd_data_accepts_the_edge_pads(lib):
    """pad = dilation*(KH-1) maps to pad 0 and pad 0 to full padding: both are
    planned (checked through the forward plans they map to)."""
    for pad, dil in ((2, 1), (0, 1), (4, 2), (0, 3)):
        rc, fwd = abi.conv2d_fwd_plan(2, 9, 9, 24, 40, 3, 3, 1, pad, dil, 0, 256)
        assert rc == abi.CONVIMG_OK
        rc, p = abi.conv2d_fwd_plan(2, fwd["OH"], fwd["OW"], 40, 24, 3, 3, 1,
                                    dil * 2 - pad, dil, 0, 256)
        assert rc == abi.CONVIMG_OK and (p["OH"], p["OW"]) == (9, 9)


@pytest.mark.parametrize("kw,code", [
    (dict(w=None), abi.CONVIMG_ERR_NULL),
    (dict(wt=None), abi.CONVIMG_ERR_NULL),
    (dict(OC=0), abi.CONVIMG_ERR_SHAPE),
    (dict(KW=-1), abi.CONVIMG_ERR_SHAPE),
    (dict(dtype=5), abi.CONVIMG_ERR_DTYPE),
    (dict(OC=1 << 16, IC=1 << 16), abi.CONVIMG_ERR_RANGE),
    (dict(OC=1, IC=1, KH=300, KW=300), abi.CONVIMG_ERR_RANGE),
    (dict(wt=0x2000000 + 16 * 9 * 16 * 2 - 2), abi.CONVIMG_ERR_ALIAS),   # last element of w
])
def test_bwd_data_weights_errors_before_any_device_work(lib, kw, code):
    a = dict(w=0x2000000, OC=16, KH=3, KW=3, IC=16, dtype=0, wt=0x4000000, stream=None)
    a.update(kw)
    assert abi.conv2d_bwd_data_weights(a["w"], a["OC"], a["KH"], a["KW"], a["IC"], a["dtype"],
                                       a["wt"], a["stream"]) == code



def call_wgt(**kw):
    a = dict(BASE, x=0x1000000, dy=0x2000000, dw=0x3000000, ws=0x5000000, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return abi.conv2d_bwd_weight(a["x"], a["dy"], a["N"], a["H"], a["W"], a["IC"], a["OC"], a["KH"],
                                 a["KW"], a["stride"], a["pad"], a["dilation"], a["dtype"], a["dw"],
                                 a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), abi.CONVIMG_ERR_NULL),
    (dict(dy=None), abi.CONVIMG_ERR_NULL),
    (dict(dw=None), abi.CONVIMG_ERR_NULL),
    (dict(N=0), abi.CONVIMG_ERR_SHAPE),
    (dict(H=2, pad=0), abi.CONVIMG_ERR_SHAPE),
    (dict(stride=0), abi.CONVIMG_ERR_SHAPE),
    (dict(dtype=2), abi.CONVIMG_ERR_DTYPE),
    (dict(N=1 << 12, H=1 << 10, W=1 << 10), abi.CONVIMG_ERR_RANGE),
    (dict(dw=0x1000000 + 64), abi.CONVIMG_ERR_ALIAS),          # dw inside x
    (dict(dw=0x2000000 - 16), abi.CONVIMG_ERR_ALIAS),          # dw runs into dy
])
def test_bwd_weight_errors_before_any_device_work(lib, kw, code):
    assert call_wgt(**kw) == code


def test_bwd_weight_workspace_argument_errors(lib):
    assert lib.conv2d_bwd_weight_workspace(2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 0, None) \
        == abi.CONVIMG_ERR_NULL
    # fp32 storage passes the argument checks (its plan then needs the
    # device's CU count: OK on a GPU host, the device error here)
    assert abi.conv2d_bwd_weight_workspace(2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 1)[0] \
        in (abi.CONVIMG_OK, abi.CONVIMG_ERR_DEVICE)
    assert abi.conv2d_bwd_weight_workspace(2, 8, 8, 16, 16, 3, 3, 0, 1, 1, 0)[0] \
        == abi.CONVIMG_ERR_SHAPE



def test_autotune_argument_errors_before_any_device_work(lib):
    a = dict(BASE, x=0x1000000, w=0x2000000, bias=None, out=0x3000000, stream=None)
    args = lambda **kw: dict(a, **kw)
    def call(d):
        return abi.conv2d_fwd_autotune(d["x"], d["w"], d["bias"], d["N"], d["H"], d["W"], d["IC"],
                                       d["OC"], d["KH"], d["KW"], d["stride"], d["pad"],
                                       d["dilation"], d["dtype"], d["out"], d["stream"])[0]
    assert call(args(x=None)) == abi.CONVIMG_ERR_NULL
    assert call(args(out=None)) == abi.CONVIMG_ERR_NULL
    assert call(args(N=0)) == abi.CONVIMG_ERR_SHAPE
    assert call(args(dtype=7)) == abi.CONVIMG_ERR_DTYPE
    abi.conv2d_fwd_autotune_clear()         # callable without a device



def test_nchw_argument_errors_before_any_device_work(lib):
    a = dict(BASE, x=0x1000000, w=0x2000000, bias=None, out=0x3000000, ws=0x6000000,
             ws_bytes=1 << 30, out_dtype=1, stream=None)
    def call(**kw):
        d = dict(a, **kw)
        return abi.conv2d_fwd_nchw(d["x"], d["w"], d["bias"], d["N"], d["H"], d["W"], d["IC"],
                                   d["OC"], d["KH"], d["KW"], d["stride"], d["pad"], d["dilation"],
                                   d["dtype"], d["out_dtype"], d["out"], d["ws"], d["ws_bytes"],
                                   d["stream"])
    assert call(x=None) == abi.CONVIMG_ERR_NULL
    assert call(ws=None) == abi.CONVIMG_ERR_NULL
    assert call(N=0) == abi.CONVIMG_ERR_SHAPE
    assert call(dtype=9) == abi.CONVIMG_ERR_DTYPE
    assert call(out_dtype=5) == abi.CONVIMG_ERR_DTYPE
    rc, need = abi.conv2d_fwd_nchw_workspace(2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 0)
    # x copy (4096 B), w copy (4608 B, ending on a 256-byte boundary), fp32 out (8192 B)
    assert rc == 0 and need == 4096 + 4608 + 8192
    rc, need3 = abi.conv2d_fwd_nchw_workspace(2, 8, 8, 16, 17, 3, 3, 1, 1, 1, 0)
    # w copy of 17 rows (4896 B) rounds up to 5120 before the fp32 out (8704 B)
    assert rc == 0 and need3 == 4096 + 5120 + 8704
    assert call(ws_bytes=need - 1) == abi.CONVIMG_ERR_WORKSPACE
    assert call(out=0x6000000 + 64) == abi.CONVIMG_ERR_ALIAS        # out inside ws
    assert call(ws=0x1000000 + 64) == abi.CONVIMG_ERR_ALIAS         # ws overlaps x
    assert lib.conv2d_fwd_nchw_workspace(2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 0, None) \
        == abi.CONVIMG_ERR_NULL


def test_plan_cache_is_per_thread_and_consistent(lib):
    """The planner keeps a small per-thread cache of recent plans: plans made
    concurrently from many threads (ctypes releases the GIL) for an
    interleaved mix of more shapes than the cache holds equal the plans made
    one by one, and the forced-tile knob bypasses stale entries."""
    import random
    import threading
    rng = random.Random(5)
    shapes = []
    while len(shapes) < 24:
        s = (rng.randint(1, 16), rng.randint(5, 60), rng.randint(5, 60), rng.choice([3, 16, 64, 128, 256]),
             rng.choice([32, 64, 96, 512]), 3, 3, rng.randint(1, 2), 1, rng.randint(1, 2), 0, 256)
        if abi.conv2d_fwd_plan(*s)[0] == 0:
            shapes.append(s)
    want = {s: abi.conv2d_fwd_plan(*s)[1] for s in shapes}
    bad = []

    def worker(seed):
        r = random.Random(seed)
        for _ in range(300):
            s = r.choice(shapes)
            rc, p = abi.conv2d_fwd_plan(*s)
            if rc != 0 or p != want[s]:
                bad.append((s, p))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:2]
    s = shapes[0]
    try:
        assert abi.conv2d_fwd_force(11, -1, -1) == 0
        forced = abi.conv2d_fwd_plan(*s)[1]
        assert forced["tile_id"] in (11, 0)          # 11, or the element-wise fallback
    finally:
        abi.conv2d_fwd_force(-1, -1, -1)
    assert abi.conv2d_fwd_plan(*s)[1] == want[s]
