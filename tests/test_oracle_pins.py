"""The oracle against its pins (CPU only).

1. Every pin in pins.py passes on the oracle built from oracle/conv_ref.c.
2. Every plausible mistake planted in a copy of that source (a dropped
   term, a wrong sign or index, a transposed operand, a flipped kernel, a
   precision loss) is caught by at least one pin.  The mistakes are planted
   in the oracle, on the CPU, in a temporary build; the real source is never
   modified.
"""
import os

import numpy as np
import pytest

import oracle
from convolution_implicit_gemm_fwd_amd.workloads import WORKLOADS, make_inputs

from pins import ALL_PINS, brute_conv, assert_close


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_tiny_workload_bruteforce(oracle_lib):
    """All 1,024 outputs of the tiny workload agree with the brute force."""
    wl = WORKLOADS["tiny"]
    for rounded in (True, False):
        inp = make_inputs(wl, seed=0, round_bf16=rounded)
        y, S = oracle_lib.conv2d_fwd(inp.x32, inp.w32, inp.bias, wl.stride, wl.pad, wl.dilation)
        yb, Sb = brute_conv(inp.x32, inp.w32, inp.bias, wl.stride, wl.pad, wl.dilation)
        assert y.shape == (1, 8, 8, 16)
        assert_close(y, yb, 1e-12, 1e-12, "tiny workload")
        assert_close(S, Sb, 1e-12, 1e-12, "tiny workload magnitude")


# (description, text in conv_ref.c, replacement).  Each keeps every memory
# access in bounds so a mutant can run in this process.
MUTANTS = [
    ("padding offset dropped",
     "int ih = oh * s - p + kh * d;", "int ih = oh * s + kh * d;"),
    ("padding sign flipped",
     "int iw = ow * s - p + kw * d;", "int iw = ow * s + p + kw * d;"),
    ("dilation dropped on columns",
     "int iw = ow * s - p + kw * d;", "int iw = ow * s - p + kw;"),
    ("stride applied to the padding",
     "int ih = oh * s - p + kh * d;", "int ih = (oh - p) * s + kh * d;"),
    ("kernel flipped",
     "(((size_t)oc * KH + kh) * KW + kw) * IC",
     "(((size_t)oc * KH + (KH - 1 - kh)) * KW + (KW - 1 - kw)) * IC"),
    ("kh and kw swapped on the input side",
     "int iw = ow * s - p + kw * d;", "int iw = ow * s - p + kh * d;"),
    ("weight channels reversed",
     "double prod = xp[ic] * wp[ic];", "double prod = xp[ic] * wp[IC - 1 - ic];"),
    ("one-based column bound",
     "iw < 0 ||", "iw < 1 ||"),
    ("bias dropped",
     "y_px[oc] = acc + (bias ? bias[oc] : 0.0);", "y_px[oc] = acc;"),
    ("magnitude without abs",
     "mag += fabs(prod);", "mag += prod;"),
    ("single-precision accumulator",
     "double acc = 0.0;", "float acc = 0.0f;"),
    ("output extent rounded up",
     "return (int)((padded - span) / s + 1);", "return (int)((padded - span + s - 1) / s + 1);"),
    ("data backward: padding sign flipped",
     "int th = ih + p - kh * d;", "int th = ih - p - kh * d;"),
    ("data backward: stride remainder ignored",
     "if (th < 0 || th % s != 0 || th / s >= OH)", "if (th < 0 || th / s >= OH)"),
    ("data backward: kernel flipped",
     "((size_t)(oc * KH + kh) * KW + kw) * IC", "((size_t)(oc * KH + (KH - 1 - kh)) * KW + (KW - 1 - kw)) * IC"),
    ("data backward: input channels reversed",
     "double t = gy[oc] * wr[ic];", "double t = gy[oc] * wr[IC - 1 - ic];"),
    ("data backward: column dilation dropped",
     "int tw = iw + p - kw * d;", "int tw = iw + p - kw;"),
    ("data backward: magnitude without abs",
     "a[ic] += fabs(t);", "a[ic] += t;"),
    ("weight backward: padding sign flipped",
     "int jh = oh * s - p + kh * d;", "int jh = oh * s + p + kh * d;"),
    ("weight backward: stride dropped on columns",
     "int jw = ow * s - p + kw * d;", "int jw = ow - p + kw * d;"),
    ("weight backward: row dilation dropped",
     "int jh = oh * s - p + kh * d;", "int jh = oh * s - p + kh;"),
    ("weight backward: kernel flipped",
     "const size_t wrow = (size_t)oc * KH * KW + (size_t)kh * KW + kw;",
     "const size_t wrow = (size_t)oc * KH * KW + (size_t)(KH - 1 - kh) * KW + (KW - 1 - kw);"),
    ("weight backward: input channels reversed",
     "double t = gy * xr[ic];", "double t = gy * xr[IC - 1 - ic];"),
    ("weight backward: magnitude without abs",
     "m[ic] += fabs(t);", "m[ic] += t;"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, desc, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, "mutation %r no longer applies to conv_ref.c" % desc
    mpath = tmp_path / "conv_mut.c"
    mpath.write_text(src.replace(old, new))
    so = str(tmp_path / "libconv_mut.so")
    oracle.compile_source(str(mpath), so)
    mutant = oracle.Oracle(so)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError) as e:
            caught.append((pin.__name__, str(e)[:80]))
            break
    assert caught, "no pin catches the planted mistake: %s" % desc
