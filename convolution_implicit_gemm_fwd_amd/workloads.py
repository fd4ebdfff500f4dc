"""Named convolution workloads and their seeded synthetic inputs.

This module holds shapes and random-number recipes only; it contains none of
the convolution's arithmetic, so both the HIP path's tests and the oracle may
take their inputs from it.  Everything is numpy on the host; nothing here
touches a GPU.

Inputs are drawn in float32 with ``numpy.random.default_rng(seed)`` in the
order x, w, bias.  Tensors the workload stores as bf16 are rounded to bf16
with round-to-nearest-even, so the GPU path and the oracle see identical
values.  A normal distribution's second parameter is its standard deviation
(weights use fan-in scaling 1/sqrt(K)).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

BF16 = 0   # dtype code for bf16 storage of x and w
FP32 = 1   # dtype code for fp32 storage of x and w


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    IC: int
    H: int
    W: int
    OC: int
    KH: int
    KW: int
    stride: int
    pad: int
    dilation: int
    dtype: int          # BF16 or FP32 storage of x and w
    x_dist: tuple       # ("uniform", lo, hi) or ("normal", mean, std)
    w_dist: tuple
    bias_dist: tuple    # as above, or ("zeros",)

    def scaled(self, **changes) -> "Workload":
        return dataclasses.replace(self, **changes)


def _std(k):
    return 1.0 / np.sqrt(k)


WORKLOADS = {
    # tiny 3x3: the oracle finishes in milliseconds; x and w stored as fp32
    "tiny": Workload("tiny", 1, 16, 8, 8, 16, 3, 3, 1, 1, 1, FP32,
                     ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0),
                     ("uniform", -0.1, 0.1)),
    # ResNet-style 3x3 layer, 56x56, 64 -> 64 channels
    "resnet3x3": Workload("resnet3x3", 16, 64, 56, 56, 64, 3, 3, 1, 1, 1, BF16,
                          ("normal", 0.0, 1.0), ("normal", 0.0, _std(576)),
                          ("normal", 0.0, 0.01)),
    # deep layer, 14x14, 512 -> 512 channels: long K, few output tiles
    "largek": Workload("largek", 16, 512, 14, 14, 512, 3, 3, 1, 1, 1, BF16,
                       ("normal", 0.0, 1.0), ("normal", 0.0, _std(4608)),
                       ("normal", 0.0, 0.01)),
    # 7x7 stride-2 stem on RGB input: IC = 3, K = 147
    "stem7x7": Workload("stem7x7", 16, 3, 224, 224, 64, 7, 7, 2, 3, 1, BF16,
                        ("uniform", 0.0, 1.0), ("normal", 0.0, _std(147)),
                        ("zeros",)),
    # dilated 3x3 on a 128x128 map, 128 -> 128 channels
    "dilated": Workload("dilated", 4, 128, 128, 128, 128, 3, 3, 1, 2, 2, BF16,
                        ("normal", 0.0, 1.0), ("normal", 0.0, _std(1152)),
                        ("normal", 0.0, 0.01)),
}

# Order in which the workloads are listed everywhere (tiny first).
WORKLOAD_ORDER = ("tiny", "resnet3x3", "largek", "stem7x7", "dilated")


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs must be finite (the generators only draw finite values).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _draw(rng, dist, shape):
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape).astype(np.float32)
    if kind == "normal":
        return rng.normal(dist[1], dist[2], size=shape).astype(np.float32)
    if kind == "zeros":
        return np.zeros(shape, np.float32)
    raise ValueError("unknown distribution %r" % (dist,))


@dataclasses.dataclass
class Inputs:
    """Host-side inputs of one workload.

    x32/w32 hold the values as float32 (bf16-exact when ``rounded``);
    x_store/w_store hold the bytes the GPU receives (uint16 bf16 bits for
    BF16 storage, float32 for FP32 storage).
    """
    workload: Workload
    x32: np.ndarray
    w32: np.ndarray
    bias: np.ndarray
    x_store: np.ndarray
    w_store: np.ndarray
    rounded: bool

    def sha256(self) -> dict:
        return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
                for k, v in (("x", self.x_store), ("w", self.w_store), ("bias", self.bias))}


def make_inputs(wl: Workload, seed: int = 0, round_bf16: bool = True,
                dtype: int | None = None) -> Inputs:
    """Draw x [N,H,W,IC], w [OC,KH,KW,IC], bias [OC] for a workload.

    ``round_bf16`` rounds x and w to bf16 values even when they are stored as
    fp32 (then bf16 and fp32 storage of the same draw hold equal values).
    ``dtype`` overrides the workload's storage type.
    """
    dtype = wl.dtype if dtype is None else dtype
    rng = np.random.default_rng(seed)
    x = _draw(rng, wl.x_dist, (wl.N, wl.H, wl.W, wl.IC))
    w = _draw(rng, wl.w_dist, (wl.OC, wl.KH, wl.KW, wl.IC))
    b = _draw(rng, wl.bias_dist, (wl.OC,))
    if dtype == BF16 and not round_bf16:
        raise ValueError("bf16 storage needs bf16-rounded values")
    if round_bf16:
        xb, wb = round_to_bf16_bits(x), round_to_bf16_bits(w)
        x, w = bf16_bits_to_f32(xb), bf16_bits_to_f32(wb)
    if dtype == BF16:
        x_store, w_store = xb, wb
    else:
        x_store, w_store = x, w
    return Inputs(wl, x, w, b, x_store, w_store, round_bf16)


def make_grad_inputs(wl: Workload, OH: int, OW: int, seed: int = 0,
                     dtype: int | None = None) -> Inputs:
    """Draw the data-backward inputs of a workload: dy [N,OH,OW,OC] from the
    workload's x distribution, then w [OC,KH,KW,IC] as in ``make_inputs``.

    OH, OW: the forward output extent, given by the caller (this module
    computes nothing of the convolution).  The result's x32/x_store hold dy;
    bias is drawn but unused.  Values are bf16-rounded.
    """
    dtype = wl.dtype if dtype is None else dtype
    rng = np.random.default_rng(seed)
    dy = round_to_bf16_bits(_draw(rng, wl.x_dist, (wl.N, OH, OW, wl.OC)))
    w = round_to_bf16_bits(_draw(rng, wl.w_dist, (wl.OC, wl.KH, wl.KW, wl.IC)))
    b = _draw(rng, wl.bias_dist, (wl.OC,))
    dy32, w32 = bf16_bits_to_f32(dy), bf16_bits_to_f32(w)
    if dtype == BF16:
        return Inputs(wl, dy32, w32, b, dy, w, True)
    return Inputs(wl, dy32, w32, b, dy32, w32, True)


def make_wgrad_inputs(wl: Workload, OH: int, OW: int, seed: int = 0,
                      dtype: int | None = None) -> Inputs:
    """Draw the weight-backward inputs of a workload: x [N,H,W,IC] from the
    workload's x distribution, then dy [N,OH,OW,OC] from N(0, 1); for bf16
    storage (the default) both bf16-rounded and stored as bf16, for fp32
    storage (``dtype`` FP32) both kept and stored as drawn in float32.

    OH, OW: the forward output extent, given by the caller.  The result's
    x32/x_store hold x and its w32/w_store hold dy; bias is unused (zeros).
    """
    dtype = BF16 if dtype is None else dtype
    rng = np.random.default_rng(seed)
    x = _draw(rng, wl.x_dist, (wl.N, wl.H, wl.W, wl.IC))
    dy = _draw(rng, ("normal", 0.0, 1.0), (wl.N, OH, OW, wl.OC))
    if dtype == FP32:
        x, dy = x.astype(np.float32), dy.astype(np.float32)
        return Inputs(wl, x, dy, np.zeros(wl.OC, np.float32), x, dy, False)
    x, dy = round_to_bf16_bits(x), round_to_bf16_bits(dy)
    return Inputs(wl, bf16_bits_to_f32(x), bf16_bits_to_f32(dy), np.zeros(wl.OC, np.float32),
                  x, dy, True)
