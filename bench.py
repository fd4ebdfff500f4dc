"""Benchmark: conv2d forward (implicit GEMM, bf16 MFMA) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--op fwd|dgrad]

A step is one conv2d_fwd call (the whole hot path: im2col gather, bf16 MFMA,
fused bias, fp32 store) over the workload's batch, with every input already
resident in device memory.  The default workload is the ResNet-style 3x3
layer (N=16, 56x56, 64 -> 64 channels).  Prints ONE JSON line.

--op wgrad times conv2d_bwd_weight (the gradient with respect to the
weights): a step is the implicit-GEMM kernel plus, when the pixels are split
into ranges, the ordered sum of the ranges; the roofline object prices the
whole call.

--op dgrad times conv2d_bwd_data instead (the gradient with respect to the
input): at stride 1 a step is the forward implicit GEMM it maps to, whose
kernel flips and transposes the weights in LDS where it can (one launch),
else the separate weight transform plus that GEMM (the roofline object then
prices the GEMM kernel alone, timed in its own loop on the same buffers);
other problems (the stem's stride 2) take the fallback route (the kernel
by phases of the stride), one launch.

--nchw f32|bf16 times conv2d_fwd_nchw on NCHW / OIHW copies of the same
inputs (fp32 or bf16 NCHW output).

The default run (the ResNet-style forward) also times the other named
forward configurations -- the large-K layer, the RGB stem and the dilated
layer -- after its own measurement, 3 windows each, and reports them under
other_configs (--no-others skips them); `value` is the main workload's.

Timing: 11 windows (--windows) of K back-to-back calls on one stream, each
between two HIP events recorded on that stream and synchronised on both
sides; before each window's start event a sleep kernel holds the stream
while the host queues the K calls, so the events time the GPU running the
calls back to back (the host's own cost to queue a call is reported as
host_ms_to_queue_a_step).  The value is the median window's time per call;
min and max are reported too.  A cold-cache figure (single calls after
writing a 1 GiB scrub buffer) is reported beside it.  TFLOP/s = 2*M*OC*K /
time with the real K = IC*KH*KW.  The roofline object prices the kernel against HBM
bandwidth or dense bf16 MFMA peak, whichever bounds it at the workload's
arithmetic intensity.  The CPU baseline is the fp64 oracle timed on this
host's cores on the same inputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv2d fwd TFLOP/s (2·M·N·K/s) + % of bf16 MFMA peak, 1×MI355X"
METRIC_WGRAD = "conv2d bwd-weight TFLOP/s (2·N·OH·OW·OC·KH·KW·IC/s) + % of bf16 MFMA peak, 1×MI355X"
METRIC_DGRAD = "conv2d bwd-data TFLOP/s (2·N·H·W·IC·OC·KH·KW/s) + % of bf16 MFMA peak, 1×MI355X"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
MACHINE_BALANCE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte

# HBM traffic per launch measured with rocprofv3 (FETCH_SIZE then WRITE_SIZE,
# each scaled by what the counter reads for a plain copy of known size, see
# --copy-calibration), keyed by workload, with the tile the plan ran and the
# hash of that kernel family's sources.  Reported only while the plan and
# the sources are unchanged; otherwise traffic is null.
TRAFFIC = {
    # profiles/igemm_resident_resnet3x3.md: 7.162 MB read + 12.845 MB written
    "resnet3x3": {"bytes": 20007329, "tile": 33, "kernel": "4cb778c4babd73af"},
    # profiles/igemm_image_largek.md: 25.638 MB read + 6.423 MB written
    "largek": {"bytes": 32060100, "tile": 34, "kernel": "b5fa9f7b6da1e3fe"},
    # profiles/igemm_window_stem7x7.md: 5.283 MB read + 51.380 MB written
    "stem7x7": {"bytes": 56662923, "tile": 32, "kernel": "cc44bd8bb5fdb554"},
    # profiles/igemm_pipe_dilated.md: 19.915 MB read + 33.554 MB written
    "dilated": {"bytes": 53469028, "tile": 15, "kernel": "97d2b4355ecb97cc"},
    # data backward: one launch, the GEMM kernel flipping the weights in LDS
    # (--op dgrad); profiles/dgrad_resident_resnet3x3.md, dgrad_image_largek.md
    "dgrad:resnet3x3": {"bytes": 20009376, "tile": 33, "kernel": "4cb778c4babd73af"},
    "dgrad:largek": {"bytes": 32051800, "tile": 34, "kernel": "b5fa9f7b6da1e3fe"},
    # NCHW entry point with bf16 out: one launch of the resident kernel's
    # NCHW variant (--nchw bf16); profiles/nchw_resident_resnet3x3.md
    "nchw_bf16:resnet3x3": {"bytes": 13725142, "tile": 33, "kernel": "4cb778c4babd73af"},
    # weight backward: the whole call (igemm_wgrad_row_bf16, + wgrad_reduce
    # where the ranges go through the workspace), as the --op wgrad roofline
    # times it; profiles/igemm_wgrad_*.md
    "wgrad:resnet3x3": {"bytes": 36188457, "tile": -2, "kernel": "cfddd831a25cdc45"},
    "wgrad:largek": {"bytes": 44526942, "tile": -2, "kernel": "cfddd831a25cdc45"},
    "wgrad:dilated": {"bytes": 68870308, "tile": -2, "kernel": "cfddd831a25cdc45"},
}

# Sources each kernel family is compiled from (besides igemm_common.hpp).
KIND_SOURCES = {
    -2: ("igemm_wgrad.hpp", "igemm_pipe.hpp", "conv2d_wgrad.hip"),   # weight backward
    -3: ("igemm_dgrad.hpp",),                    # data backward, fallback route
    -1: ("igemm_regs.hpp",),                     # fp32 storage
    0: ("igemm_regs.hpp",),                      # CONVIMG_KIND_REGS
    1: ("igemm_pipe.hpp",),                      # CONVIMG_KIND_PIPE
    2: ("igemm_patch.hpp", "igemm_pipe.hpp"),    # CONVIMG_KIND_PATCH
    3: ("igemm_strip.hpp", "igemm_pipe.hpp"),    # CONVIMG_KIND_STRIP
    4: ("igemm_window.hpp", "igemm_pipe.hpp"),   # CONVIMG_KIND_WINDOW
    5: ("igemm_resident.hpp", "igemm_pipe.hpp"), # CONVIMG_KIND_RESIDENT
    6: ("igemm_image.hpp", "igemm_pipe.hpp"),    # CONVIMG_KIND_IMAGE
}


def kernel_sources_hash(kind):
    """Hash of the sources of one kernel family (see KIND_SOURCES)."""
    import hashlib
    csrc = os.path.join(ROOT, "convolution_implicit_gemm_fwd_amd", "csrc")
    h = hashlib.sha256()
    for name in ("igemm_common.hpp",) + KIND_SOURCES[kind]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="resnet3x3")
    ap.add_argument("--op", choices=("fwd", "dgrad", "wgrad"), default="fwd")
    ap.add_argument("--nchw", choices=("f32", "bf16"), default=None,
                    help="(--op fwd) time conv2d_fwd_nchw on NCHW/OIHW copies of the inputs, "
                         "with an fp32 or bf16 NCHW output (permutes included)")
    ap.add_argument("--autotune", action="store_true",
                    help="(--op fwd) let conv2d_fwd_autotune pick the plan on these inputs first")
    ap.add_argument("--windows", type=int, default=11,
                    help="timing windows of --steps calls each; the line reports their median")
    ap.add_argument("--cold", action=argparse.BooleanOptionalAction, default=True,
                    help="also time single calls after scrubbing the caches (1 GiB write)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="bound on the CPU-baseline sample (0 disables it)")
    ap.add_argument("--force", default=None,
                    help="tile,splits,loader to force instead of the automatic plan (-1 = auto)")
    ap.add_argument("--storage", choices=("bf16", "fp32"), default=None,
                    help="store x and w (dy) in this type instead of the workload's own "
                         "(fp32: the fp32 kernels, products and sums in fp32)")
    ap.add_argument("--others", action=argparse.BooleanOptionalAction, default=True,
                    help="(default forward run) also time the other named forward configurations "
                         "after the main measurement and report them under other_configs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


def copy_calibration(mib):
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "copies": 5}), flush=True)


def cpu_baseline(inp, wl, flops, seconds, op="fwd"):
    """The fp64 oracle on this host: whole-workload passes until `seconds`."""
    import oracle
    o = oracle.get()
    threads = o.set_threads(0)
    runs, t0 = 0, time.perf_counter()
    while True:
        if op == "fwd":
            o.conv2d_fwd(inp.x32, inp.w32, inp.bias, wl.stride, wl.pad, wl.dilation)
        elif op == "wgrad":
            o.conv2d_bwd_weight(inp.x32, inp.w32, wl.KH, wl.KW, wl.stride, wl.pad, wl.dilation)
        else:
            o.conv2d_bwd_data(inp.x32, inp.w32, wl.H, wl.W, wl.stride, wl.pad, wl.dilation)
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds or runs >= 100:
            break
    per = el / runs
    return {"value": round(flops / per / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d full pass(es) of the %s workload's %s (fp64 direct 7-loop, also "
                      "summing |x*w|), %.2f s each" % (runs, wl.name, op, per)}


def dist_text(dist):
    if dist[0] == "normal":
        return "N(%g, sd %g)" % (dist[1], dist[2])
    if dist[0] == "uniform":
        return "U(%g, %g)" % (dist[1], dist[2])
    return dist[0]


def sleep_cycles_per_us():
    """Rate of the counter torch.cuda._sleep spins on, in cycles per us
    (measured once with events around a sleep of known length)."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cycles = 2_000_000
    torch.cuda._sleep(cycles // 10)          # first call: module load
    e0.record()
    torch.cuda._sleep(cycles)
    e1.record()
    torch.cuda.synchronize()
    return cycles / max(e0.elapsed_time(e1) * 1e3, 1.0)


def timed(fn, call_args, steps, warmup, stream, windows=11):
    """Time `steps` back-to-back calls of fn(*call_args) in each of `windows`
    windows.  A window: synchronise; hold the stream with a sleep kernel long
    enough for the host to queue every call of the window; record a start
    event on the stream; the `steps` calls; a stop event; synchronise.  The
    events then bracket the GPU running exactly `steps` calls back to back,
    whatever the host's own cost per call, which is reported separately.
    Returns (median ms per call over the windows, min, max, host ms per
    call to queue one call)."""
    import statistics
    import torch
    rc = fn(*call_args)
    assert rc == 0, rc
    for _ in range(warmup):
        fn(*call_args)
    torch.cuda.synchronize()
    rate = sleep_cycles_per_us()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per, host = [], []
    hold_us = 200.0 + 15.0 * steps
    for _ in range(windows):
        torch.cuda.synchronize()
        torch.cuda._sleep(int(hold_us * rate))      # on the current stream (= `stream`)
        start.record(stream)
        t0 = time.perf_counter()
        for _ in range(steps):
            fn(*call_args)
        t1 = time.perf_counter()
        stop.record(stream)
        torch.cuda.synchronize()
        per.append(start.elapsed_time(stop) / steps)
        host.append((t1 - t0) * 1e3 / steps)
    return statistics.median(per), min(per), max(per), statistics.median(host)


def timed_cold(fn, call_args, stream, launches=11, scrub_mib=1024):
    """Single calls timed with events after writing a scrub buffer larger
    than every cache (L2 and the 256 MB MALL): the inputs come from HBM.
    Returns (median us, min us)."""
    import statistics
    import torch
    scrub = torch.empty(scrub_mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    us = []
    for i in range(launches):
        scrub.fill_(float(i))
        e0.record(stream)
        fn(*call_args)
        e1.record(stream)
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3)
    del scrub
    return statistics.median(us), min(us)


def time_other_forward(names, steps, warmup, windows, stream):
    """The other named forward configurations, each on its own seeded
    inputs with its automatic plan, timed like the main line (fewer
    windows): {name: {us_per_call, tflops, mfma_peak_frac, roofline}}.
    Reported beside the main line, outside its timed region."""
    import numpy as np
    import torch
    from convolution_implicit_gemm_fwd_amd import abi
    from convolution_implicit_gemm_fwd_amd.workloads import BF16, WORKLOADS, make_inputs
    lib = abi.load()
    sptr = stream.cuda_stream
    res = {}
    for name in names:
        wl = WORKLOADS[name]
        OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
        OW = abi.conv2d_fwd_out_dim(wl.W, wl.KW, wl.stride, wl.pad, wl.dilation)
        M, K = wl.N * OH * OW, wl.IC * wl.KH * wl.KW
        inp = make_inputs(wl, seed=0)

        def up(a):
            t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a))
            return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).cuda()

        x, w, b = up(inp.x_store), up(inp.w_store), torch.from_numpy(inp.bias).cuda()
        out = torch.empty((wl.N, OH, OW, wl.OC), dtype=torch.float32, device="cuda")
        args = ((x.data_ptr(), w.data_ptr(), b.data_ptr(), wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW,
                 wl.stride, wl.pad, wl.dilation, wl.dtype, out.data_ptr(), sptr))
        ms = timed(lib.conv2d_fwd, args, steps, warmup, stream, windows)[0]
        esz = 2 if wl.dtype == BF16 else 4
        flops = 2 * M * wl.OC * K
        alg = (wl.N * wl.H * wl.W * wl.IC + wl.OC * K) * esz + wl.OC * 4 + M * wl.OC * 4
        tfl = flops / (ms * 1e-3) / 1e12
        if flops / alg < MACHINE_BALANCE:
            gbs = alg / (ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4)}
        else:
            roof = {"bound": "mfma", "achieved": round(tfl, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tfl / PEAK_BF16_TFLOPS, 4)}
        rc, plan = abi.conv2d_fwd_plan(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride, wl.pad,
                                       wl.dilation, wl.dtype, 0)
        res[name] = {"us_per_call": round(ms * 1e3, 3), "tflops": round(tfl, 2),
                     "mfma_peak_frac": round(tfl / PEAK_BF16_TFLOPS, 4), "roofline": roof,
                     "tile_id": plan["tile_id"] if rc == 0 else None,
                     "steps": steps, "windows": windows}
        del x, w, b, out
    return res


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build runs on a single MI355X "
              "(--gpus %d is not supported)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from convolution_implicit_gemm_fwd_amd import abi
    from convolution_implicit_gemm_fwd_amd.workloads import (BF16, WORKLOADS, make_grad_inputs,
                                                             make_inputs, make_wgrad_inputs)

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    lib = abi.load()                # fails loudly if the HIP library is not built
    wl = WORKLOADS[args.workload]
    if args.storage and (BF16 if args.storage == "bf16" else 1) != wl.dtype:
        wl = wl.scaled(dtype=BF16 if args.storage == "bf16" else 1,
                       name="%s, %s storage" % (wl.name, args.storage))
    dgrad = args.op == "dgrad"
    wgrad = args.op == "wgrad"
    OH = abi.conv2d_fwd_out_dim(wl.H, wl.KH, wl.stride, wl.pad, wl.dilation)
    OW = abi.conv2d_fwd_out_dim(wl.W, wl.KW, wl.stride, wl.pad, wl.dilation)
    M, K = wl.N * OH * OW, wl.IC * wl.KH * wl.KW
    inp = (make_grad_inputs(wl, OH, OW, seed=0, dtype=wl.dtype) if dgrad
           else make_wgrad_inputs(wl, OH, OW, seed=0, dtype=wl.dtype) if wgrad
           else make_inputs(wl, seed=0))

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).cuda()

    x, w, b = up(inp.x_store), up(inp.w_store), torch.from_numpy(inp.bias).cuda()
    if args.force:
        abi.conv2d_fwd_force(*[int(v) for v in args.force.split(",")])
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    esz = 2 if wl.dtype == BF16 else 4
    if wgrad:
        # x holds x, w holds dy [N,OH,OW,OC]
        out = torch.empty((wl.OC, wl.KH, wl.KW, wl.IC), dtype=torch.float32, device="cuda")
        rc, need = abi.conv2d_bwd_weight_workspace(wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW,
                                                   wl.stride, wl.pad, wl.dilation, wl.dtype)
        assert rc == 0, abi.conv2d_strerror(rc)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        gemm = (wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride, wl.pad, wl.dilation)
        call_args = ((x.data_ptr(), w.data_ptr()) + gemm
                     + (wl.dtype, out.data_ptr(), ws.data_ptr(), need, sptr))
        fn = lib.conv2d_bwd_weight
        alg_bytes = (wl.N * wl.H * wl.W * wl.IC + M * wl.OC) * esz + wl.OC * K * 4
    elif not dgrad:
        out = torch.empty((wl.N, OH, OW, wl.OC), dtype=torch.float32, device="cuda")
        gemm = (wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW, wl.stride, wl.pad, wl.dilation)
        call_args = ((x.data_ptr(), w.data_ptr(), b.data_ptr()) + gemm
                     + (wl.dtype, out.data_ptr(), sptr))
        fn = lib.conv2d_fwd
        alg_bytes = (wl.N * wl.H * wl.W * wl.IC + wl.OC * K) * esz + wl.OC * 4 + M * wl.OC * 4
    else:
        # x holds dy [N,OH,OW,OC]; the data backward maps to a forward
        # convolution of dy with the flipped, transposed weights
        out = torch.empty((wl.N, wl.H, wl.W, wl.IC), dtype=torch.float32, device="cuda")
        # a byte pattern that no transform leaves: tells the one-launch path
        # (wt untouched) from the transform + GEMM path
        wt = torch.full(w.shape, 0x7F81, dtype=torch.int16, device="cuda").view(w.dtype)
        call_args = (x.data_ptr(), w.data_ptr(), wl.N, wl.H, wl.W, wl.IC, wl.OC, wl.KH, wl.KW,
                     wl.stride, wl.pad, wl.dilation, wl.dtype, wt.data_ptr(), out.data_ptr(), sptr)
        fn = lib.conv2d_bwd_data
        gemm = (wl.N, OH, OW, wl.OC, wl.IC, wl.KH, wl.KW, 1,
                wl.dilation * (wl.KH - 1) - wl.pad, wl.dilation)
        alg_bytes = (M * wl.OC + wl.OC * K) * esz + wl.N * wl.H * wl.W * wl.IC * 4
    if args.nchw and args.op == "fwd":
        # NCHW / OIHW copies of the same values; the call permutes them in
        # its workspace, runs the same implicit GEMM and permutes the result
        xn = x.permute(0, 3, 1, 2).contiguous()
        wn = w.permute(0, 3, 1, 2).contiguous()
        rc, need = abi.conv2d_fwd_nchw_workspace(*gemm, wl.dtype)
        assert rc == 0, abi.conv2d_strerror(rc)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        od = BF16 if args.nchw == "bf16" else 1
        out = torch.empty(wl.N * wl.OC * OH * OW,
                          dtype=torch.bfloat16 if od == BF16 else torch.float32, device="cuda")
        call_args = ((xn.data_ptr(), wn.data_ptr(), b.data_ptr()) + gemm
                     + (wl.dtype, od, out.data_ptr(), ws.data_ptr(), need, sptr))
        fn = lib.conv2d_fwd_nchw
        if od == BF16:
            alg_bytes -= M * wl.OC * 2
    tuned = None
    if args.autotune and args.op == "fwd":
        rc, t_tile, t_splits, t_best, t_default = abi.conv2d_fwd_autotune(*call_args)
        assert rc == 0, abi.conv2d_strerror(rc)
        tuned = {"tile_id": t_tile, "splits": t_splits, "us_best": round(t_best, 3),
                 "us_static": round(t_default, 3)}
    # the data backward's fallback route (stride > 1, KH != KW, pad beyond
    # dilation*(KH-1)) maps to no forward problem
    general = dgrad and (wl.stride != 1 or wl.KH != wl.KW or wl.pad > wl.dilation * (wl.KH - 1))
    if general:
        plan = {"tile_id": -3, "BM": 64, "BN": 64, "BK": 64, "loader": -1, "splits": None, "grid": None}
    else:
        rc, plan = abi.conv2d_fwd_plan(*gemm, wl.dtype, 0)
        assert rc == 0, abi.conv2d_strerror(rc)
    if wgrad:
        # the weight backward has its own kernel; report its workspace instead
        plan = {"tile_id": -2, "BM": 64, "BN": 192 if wl.dtype == BF16 else 64, "BK": 64, "loader": -1, "splits": None,
                "grid": None, "workspace_bytes": need}

    ms_step, ms_min, ms_max, host_ms = timed(fn, call_args, args.steps, args.warmup, stream,
                                             args.windows)
    assert abi.conv2d_fwd_status(sptr) == 0
    one_launch = dgrad and bool((wt.view(torch.int16) == 0x7F81).all().item())
    if dgrad and not one_launch:
        # the implicit-GEMM kernel alone, on the weights the steps left in wt
        gemm_args = (x.data_ptr(), wt.data_ptr(), None) + gemm + (wl.dtype, out.data_ptr(), sptr)
        ms_gemm = timed(lib.conv2d_fwd, gemm_args, args.steps, args.warmup, stream, args.windows)[0]
        assert abi.conv2d_fwd_status(sptr) == 0
    else:
        ms_gemm = ms_step
    cold = None
    if args.cold:
        cold_med, cold_min = timed_cold(fn, call_args, stream)
        cold = {"median_us": round(cold_med, 3), "min_us": round(cold_min, 3), "launches": 11,
                "scrub_bytes": 1 << 30}

    flops = 2 * M * wl.OC * K          # = 2*N*H*W*IC*OC*KH*KW for the stride-1 data backward
    tflops = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (ms_gemm * 1e-3) / 1e12
    ai = flops / alg_bytes
    peak_flops = PEAK_BF16_TFLOPS if wl.dtype == BF16 else PEAK_FP32_MFMA_TFLOPS
    # the balance point of the arithmetic the path runs (fp32 storage: the
    # fp32 MFMA peak)
    if ai < peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = alg_bytes / (ms_gemm * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(gemm_tflops / peak_flops, 4)}
    kind = (abi.conv2d_fwd_tile_kind(plan["tile_id"]) if plan["tile_id"] >= 0
            else -2 if wgrad else -3 if general else -1)
    ksrc = kernel_sources_hash(kind)
    t = TRAFFIC.get("nchw_%s:%s" % (args.nchw, wl.name) if args.nchw
                    else wl.name if args.op == "fwd" else args.op + ":" + wl.name)
    roof["traffic"] = (t["bytes"] if t and t["tile"] == plan["tile_id"] and t["kernel"] == ksrc
                       else None)

    line = {
        "metric": METRIC_DGRAD if dgrad else METRIC_WGRAD if wgrad else METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == BF16 else "f32",
        "data": ("synthetic (seeded; x %s, dy N(0, sd 1); %s)" % (
                     dist_text(wl.x_dist), "bf16-rounded" if wl.dtype == BF16 else "fp32 as drawn")
                 if wgrad else
                 "synthetic (seeded; %s %s, w %s%s; bf16-rounded)" % (
                     "dy" if dgrad else "x", dist_text(wl.x_dist), dist_text(wl.w_dist),
                     "" if dgrad else ", bias " + dist_text(wl.bias_dist))),
        "config": {"workload": wl.name + (" data backward" if dgrad else " weight backward"
                                          if wgrad else " NCHW, %s out" % args.nchw
                                          if args.nchw else ""), "N": wl.N,
                   "H": wl.H, "W": wl.W, "IC": wl.IC,
                   "OC": wl.OC, "KH": wl.KH, "KW": wl.KW, "stride": wl.stride, "pad": wl.pad,
                   "dilation": wl.dilation, "M": M, "K": K,
                   "plan": {k: plan[k] for k in ("tile_id", "BM", "BN", "BK", "loader",
                                                 "splits", "grid", "workspace_bytes")
                            if k in plan}},
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "windows": {"count": args.windows, "steps_each": args.steps,
                    "median_ms_per_step": round(ms_step, 6), "min_ms_per_step": round(ms_min, 6),
                    "max_ms_per_step": round(ms_max, 6)},
        "host_ms_to_queue_a_step": round(host_ms, 6),
        "kernel_sources": ksrc,
    }
    if dgrad:
        line["gemm_ms"] = round(ms_gemm, 6)
        line["dgrad_launches"] = 1 if one_launch else 2
    if cold is not None:
        line["cold_single_call"] = cold
    if tuned is not None:
        line["autotune"] = tuned
    if args.others and args.op == "fwd" and not args.nchw and not args.force and not args.autotune \
            and not args.storage and args.workload == "resnet3x3":
        line["other_configs"] = time_other_forward(("largek", "stem7x7", "dilated"), min(args.steps, 500),
                                                   min(args.warmup, 50), 3, stream)
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(inp, wl, flops, args.cpu_seconds, args.op)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
