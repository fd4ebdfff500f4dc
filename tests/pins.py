"""Pins for the oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with the mathematics.  The same battery runs on the
real oracle (all must pass) and on deliberately broken builds of it (each
must be caught by at least one pin), see test_oracle_pins.py.

Sources of truth used here, none of which calls the oracle's arithmetic:
  * hand-counted fixtures in tests/golden/ (output extents, all-ones values);
  * closed forms (delta kernels reproduce or shift the input, 1x1 conv is a
    matrix product, all-ones counts in-bounds taps);
  * library routines on special cases (numpy matmul, torch conv2d in fp64);
  * an independently written brute-force routine (np.pad + window slicing +
    np.dot) on tiny inputs;
  * linearity in w and x, exact on small-integer data.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- helpers

def brute_conv(x, w, b, s, p, d):
    """Independent brute force: pad, cut each dilated window, dot with w."""
    N, H, W, IC = x.shape
    OC, KH, KW, _ = w.shape
    xp = np.pad(x.astype(np.float64), ((0, 0), (p, p), (p, p), (0, 0)))
    span_h, span_w = d * (KH - 1) + 1, d * (KW - 1) + 1
    OH = len(range(0, xp.shape[1] - span_h + 1, s))
    OW = len(range(0, xp.shape[2] - span_w + 1, s))
    wf = w.astype(np.float64).reshape(OC, -1)
    y = np.zeros((N, OH, OW, OC))
    S = np.zeros((N, OH, OW, OC))
    for n in range(N):
        for i in range(OH):
            for j in range(OW):
                win = xp[n, i * s:i * s + span_h:d, j * s:j * s + span_w:d, :].reshape(-1)
                y[n, i, j] = wf @ win
                S[n, i, j] = np.abs(wf) @ np.abs(win)
    if b is not None:
        y += b.astype(np.float64)
    return y, S


def int_data(rng, shape, lo=-8, hi=8):
    """Small integers: every product and sum below is exact in fp64."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def assert_close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    bad = err > lim
    assert not bad.any(), "%s: %d mismatches, max err %g" % (what, bad.sum(), err.max())


# ---------------------------------------------------------------- pins

def pin_out_dims(o):
    """P1: output extents equal the hand-counted table and a window count."""
    for size, k, s, p, d, want in read_table("out_dims.txt"):
        size, k, s, p, d, want = map(int, (size, k, s, p, d, want))
        got = o.out_dim(size, k, s, p, d)
        assert got == want, "out_dim(%d,%d,%d,%d,%d)=%d, table says %d" % (size, k, s, p, d, got, want)
        span, padded = d * (k - 1) + 1, size + 2 * p
        count = sum(1 for start in range(0, padded, s) if start + span <= padded)
        assert got == (count if count > 0 else -1)
    assert o.out_dim(0, 3, 1, 1, 1) == -1
    assert o.out_dim(5, 3, 0, 1, 1) == -1
    assert o.out_dim(5, 3, 1, -1, 1) == -1
    assert o.out_dim(5, 3, 1, 1, 0) == -1


def pin_matmul_1x1(o):
    """P2: a 1x1 convolution is a matrix product (numpy matmul in fp64),
    with stride picking every s-th pixel."""
    rng = np.random.default_rng(11)
    for (N, H, W, IC, OC, s) in [(2, 5, 7, 9, 6, 1), (1, 9, 6, 4, 3, 2), (3, 4, 4, 16, 16, 3)]:
        x = rng.standard_normal((N, H, W, IC))
        w = rng.standard_normal((OC, 1, 1, IC))
        b = rng.standard_normal(OC)
        y, _ = o.conv2d_fwd(x, w, b, s, 0, 1)
        xs = x[:, ::s, ::s, :]
        want = xs.reshape(-1, IC) @ w.reshape(OC, IC).T + b
        assert_close(y.reshape(-1, OC), want, 1e-12, 1e-12, "1x1 conv vs matmul")


def pin_centered_delta(o):
    """P3: a centred identity kernel with 'same' padding reproduces x + b
    exactly (stride 1, any dilation)."""
    rng = np.random.default_rng(12)
    for (K, d) in [(1, 1), (3, 1), (3, 2), (5, 1), (7, 3)]:
        C = 5
        x = int_data(rng, (2, 9, 8, C))
        b = int_data(rng, (C,))
        w = np.zeros((C, K, K, C))
        c = (K - 1) // 2
        for oc in range(C):
            w[oc, c, c, oc] = 1.0
        y, _ = o.conv2d_fwd(x, w, b, 1, d * c, d)
        assert y.shape == x.shape
        assert np.array_equal(y, x + b), "centred delta K=%d d=%d" % (K, d)


def pin_offcenter_delta(o):
    """P4: an identity kernel at tap (kh0, kw0) gives a pure shift:
    y[n][oh][ow][c] = x[n][oh*s - p + kh0*d][ow*s - p + kw0*d][c] inside the
    image and exactly 0 in the padding.  Non-square kernels and asymmetric
    taps fix the orientation (no flip, no kh/kw swap)."""
    rng = np.random.default_rng(13)
    C = 3
    for (KH, KW, kh0, kw0, s, p, d) in [(3, 3, 0, 0, 1, 1, 1), (3, 5, 0, 4, 1, 2, 1),
                                         (5, 2, 4, 1, 2, 3, 1), (3, 3, 2, 0, 1, 2, 2),
                                         (2, 4, 1, 3, 3, 1, 2)]:
        x = int_data(rng, (2, 7, 9, C), 1, 9)   # nonzero everywhere
        w = np.zeros((C, KH, KW, C))
        for oc in range(C):
            w[oc, kh0, kw0, oc] = 1.0
        y, _ = o.conv2d_fwd(x, w, None, s, p, d)
        N, OH, OW, _ = y.shape
        for oh in range(OH):
            for ow in range(OW):
                ih, iw = oh * s - p + kh0 * d, ow * s - p + kw0 * d
                if 0 <= ih < 7 and 0 <= iw < 9:
                    want = x[:, ih, iw, :]
                else:
                    want = np.zeros((N, C))
                assert np.array_equal(y[:, oh, ow, :], want), \
                    "shift mismatch KH=%d KW=%d tap=(%d,%d) at (%d,%d)" % (KH, KW, kh0, kw0, oh, ow)


def pin_all_ones(o):
    """P5: x = w = 1, b = 0 counts in-bounds taps (hand-counted fixture)."""
    shapes = {}
    for (name, H, W, IC, KH, KW, s, p, d, oh, ow, val) in read_table("all_ones.txt"):
        H, W, IC, KH, KW, s, p, d, oh, ow, val = map(int, (H, W, IC, KH, KW, s, p, d, oh, ow, val))
        key = (H, W, IC, KH, KW, s, p, d)
        if key not in shapes:
            x = np.ones((1, H, W, IC))
            w = np.ones((2, KH, KW, IC))
            shapes[key] = o.conv2d_fwd(x, w, None, s, p, d)[0]
        y = shapes[key]
        assert y[0, oh, ow, 0] == val and y[0, oh, ow, 1] == val, \
            "%s all-ones at (%d,%d): %g, expected %d" % (name, oh, ow, y[0, oh, ow, 0], val)


def pin_bruteforce(o, cases=40, seed=14):
    """P6: agreement with the independent brute force on random tiny shapes
    (every combination of stride, padding, dilation, non-square kernels)."""
    rng = np.random.default_rng(seed)
    done = 0
    while done < cases:
        N = int(rng.integers(1, 3))
        H, W = int(rng.integers(1, 10)), int(rng.integers(1, 10))
        IC, OC = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        KH, KW = int(rng.choice([1, 2, 3, 5])), int(rng.choice([1, 2, 3, 5]))
        s, p, d = int(rng.integers(1, 4)), int(rng.integers(0, 4)), int(rng.integers(1, 3))
        if d * (KH - 1) + 1 > H + 2 * p or d * (KW - 1) + 1 > W + 2 * p:
            continue
        x = rng.standard_normal((N, H, W, IC))
        w = rng.standard_normal((OC, KH, KW, IC))
        b = rng.standard_normal(OC) if rng.integers(0, 2) else None
        y, S = o.conv2d_fwd(x, w, b, s, p, d)
        yb, Sb = brute_conv(x, w, b, s, p, d)
        assert_close(y, yb, 1e-12, 1e-12, "brute force %s" % ((N, H, W, IC, OC, KH, KW, s, p, d),))
        assert_close(S, Sb, 1e-12, 1e-12, "magnitude sum")
        done += 1


def pin_linearity(o):
    """P7: conv is linear in w and in x (exact on small-integer data)."""
    rng = np.random.default_rng(15)
    x = int_data(rng, (2, 6, 7, 4))
    w1, w2 = int_data(rng, (3, 3, 2, 4)), int_data(rng, (3, 3, 2, 4))
    b = int_data(rng, (3,))
    args = (2, 1, 1)
    y1 = o.conv2d_fwd(x, w1, b, *args)[0] - b
    y2 = o.conv2d_fwd(x, w2, b, *args)[0] - b
    y12 = o.conv2d_fwd(x, w1 + w2, b, *args)[0] - b
    assert np.array_equal(y12, y1 + y2), "not additive in w"
    y2x = o.conv2d_fwd(2 * x, w1, b, *args)[0] - b
    assert np.array_equal(y2x, 2 * y1), "not homogeneous in x"


def pin_torch(o):
    """P8: torch.nn.functional.conv2d in fp64 on NCHW views (an independent
    library implementation)."""
    import torch
    rng = np.random.default_rng(16)
    for (N, H, W, IC, OC, KH, KW, s, p, d) in [(2, 11, 9, 6, 5, 3, 3, 1, 1, 1),
                                                (1, 16, 16, 3, 8, 7, 7, 2, 3, 1),
                                                (2, 13, 12, 8, 4, 3, 3, 1, 2, 2),
                                                (1, 10, 7, 5, 6, 2, 4, 3, 2, 2)]:
        x = rng.standard_normal((N, H, W, IC))
        w = rng.standard_normal((OC, KH, KW, IC))
        b = rng.standard_normal(OC)
        y, _ = o.conv2d_fwd(x, w, b, s, p, d)
        t = torch.nn.functional.conv2d(torch.from_numpy(x).permute(0, 3, 1, 2),
                                       torch.from_numpy(w).permute(0, 3, 1, 2),
                                       torch.from_numpy(b), stride=s, padding=p, dilation=d)
        assert_close(y, t.permute(0, 2, 3, 1).numpy(), 1e-12, 1e-12, "torch conv2d")


def pin_magnitude(o):
    """P9: S >= |y - b| everywhere, and S of w = |w|, x = |x| equals y."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((2, 8, 8, 5))
    w = rng.standard_normal((4, 3, 3, 5))
    b = rng.standard_normal(4)
    y, S = o.conv2d_fwd(x, w, b, 1, 1, 1)
    assert (S >= np.abs(y - b) - 1e-12).all(), "triangle inequality"
    ya, _ = o.conv2d_fwd(np.abs(x), np.abs(w), None, 1, 1, 1)
    assert_close(S, ya, 1e-12, 1e-12, "S equals conv of magnitudes")


def pin_pixels(o):
    """The pixel-subset entry agrees with the full output at those pixels."""
    rng = np.random.default_rng(18)
    x = rng.standard_normal((3, 9, 7, 6))
    w = rng.standard_normal((5, 3, 2, 6))
    b = rng.standard_normal(5)
    y, S = o.conv2d_fwd(x, w, b, 2, 1, 2)
    flat_y, flat_S = y.reshape(-1, 5), S.reshape(-1, 5)
    pix = rng.choice(flat_y.shape[0], size=11, replace=False)
    py, pS = o.conv2d_fwd_pixels(x, w, b, 2, 1, 2, pix)
    assert np.array_equal(py, flat_y[pix]) and np.array_equal(pS, flat_S[pix])


# ---- data backward (the gradient with respect to x)

def pin_bwd_adjoint(o, cases=30, seed=19):
    """B1: the data-backward pass is the adjoint of the forward map x -> y - b:
    sum(conv(x, w) * dy) == sum(x * dx(dy, w)) for every dy, x, w.  Small
    integers make both sides exact in fp64, so the check is equality; random
    strides, paddings (also past the window), dilations, non-square kernels."""
    rng = np.random.default_rng(seed)
    done = 0
    while done < cases:
        N, H, W = int(rng.integers(1, 3)), int(rng.integers(1, 10)), int(rng.integers(1, 10))
        IC, OC = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        KH, KW = int(rng.choice([1, 2, 3, 5])), int(rng.choice([1, 2, 3]))
        s, p, d = int(rng.integers(1, 4)), int(rng.integers(0, 4)), int(rng.integers(1, 3))
        OH, OW = o.out_dim(H, KH, s, p, d), o.out_dim(W, KW, s, p, d)
        if OH <= 0 or OW <= 0:
            continue
        x = int_data(rng, (N, H, W, IC))
        w = int_data(rng, (OC, KH, KW, IC))
        dy = int_data(rng, (N, OH, OW, OC))
        y, _ = o.conv2d_fwd(x, w, None, s, p, d)
        dx, S = o.conv2d_bwd_data(dy, w, H, W, s, p, d)
        assert dx.shape == x.shape
        lhs, rhs = float(np.sum(y * dy)), float(np.sum(x * dx))
        assert lhs == rhs, "adjoint identity fails: %r vs %r at %s" % (lhs, rhs, (N, H, W, IC, OC, KH, KW, s, p, d))
        done += 1


def pin_bwd_torch(o):
    """B2: torch.nn.grad.conv2d_input in fp64 on NCHW views (an independent
    library implementation of the same gradient)."""
    import torch
    rng = np.random.default_rng(20)
    for (N, H, W, IC, OC, KH, KW, s, p, d) in [(2, 11, 9, 6, 5, 3, 3, 1, 1, 1),
                                                (1, 16, 16, 3, 8, 7, 7, 2, 3, 1),
                                                (2, 13, 12, 8, 4, 3, 3, 1, 2, 2),
                                                (1, 10, 7, 5, 6, 2, 4, 3, 2, 2)]:
        OH, OW = o.out_dim(H, KH, s, p, d), o.out_dim(W, KW, s, p, d)
        dy = rng.standard_normal((N, OH, OW, OC))
        w = rng.standard_normal((OC, KH, KW, IC))
        dx, _ = o.conv2d_bwd_data(dy, w, H, W, s, p, d)
        t = torch.nn.grad.conv2d_input((N, IC, H, W), torch.from_numpy(w).permute(0, 3, 1, 2),
                                       torch.from_numpy(dy).permute(0, 3, 1, 2),
                                       stride=s, padding=p, dilation=d)
        assert_close(dx, t.permute(0, 2, 3, 1).numpy(), 1e-12, 1e-12, "torch conv2d_input")


def pin_bwd_delta(o):
    """B3: with a centred identity kernel and 'same' padding (stride 1) the
    forward map is the identity, so its gradient is too: dx == dy exactly."""
    rng = np.random.default_rng(21)
    for K, d in ((3, 1), (5, 2), (1, 1)):
        C = 4
        w = np.zeros((C, K, K, C))
        for c in range(C):
            w[c, K // 2, K // 2, c] = 1.0
        dy = rng.standard_normal((2, 7, 6, C))
        dx, _ = o.conv2d_bwd_data(dy, w, 7, 6, 1, d * (K - 1) // 2, d)
        assert np.array_equal(dx, dy), "identity kernel: dx != dy (K=%d, d=%d)" % (K, d)


def pin_bwd_magnitude(o):
    """B4: S >= |dx| everywhere, and S equals the gradient of |dy| through |w|."""
    rng = np.random.default_rng(22)
    dy = rng.standard_normal((2, 8, 8, 5))
    w = rng.standard_normal((5, 3, 3, 4))
    dx, S = o.conv2d_bwd_data(dy, w, 8, 8, 1, 1, 1)
    assert (S >= np.abs(dx) - 1e-12).all(), "triangle inequality"
    da, _ = o.conv2d_bwd_data(np.abs(dy), np.abs(w), 8, 8, 1, 1, 1)
    assert_close(S, da, 1e-12, 1e-12, "S equals the gradient of magnitudes")


def pin_wgt_adjoint(o, cases=30, seed=23):
    """G1: the weight-backward pass is the adjoint of the forward map w -> y - b:
    sum(conv(x, w) * dy) == sum(w * dw(x, dy)) for every x, w, dy.  Small
    integers make both sides exact in fp64; random strides, paddings (also
    past the window), dilations, non-square kernels."""
    rng = np.random.default_rng(seed)
    done = 0
    while done < cases:
        N, H, W = int(rng.integers(1, 3)), int(rng.integers(1, 10)), int(rng.integers(1, 10))
        IC, OC = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        KH, KW = int(rng.choice([1, 2, 3, 5])), int(rng.choice([1, 2, 3]))
        s, p, d = int(rng.integers(1, 4)), int(rng.integers(0, 4)), int(rng.integers(1, 3))
        OH, OW = o.out_dim(H, KH, s, p, d), o.out_dim(W, KW, s, p, d)
        if OH <= 0 or OW <= 0:
            continue
        x = int_data(rng, (N, H, W, IC))
        w = int_data(rng, (OC, KH, KW, IC))
        dy = int_data(rng, (N, OH, OW, OC))
        y, _ = o.conv2d_fwd(x, w, None, s, p, d)
        dw, S = o.conv2d_bwd_weight(x, dy, KH, KW, s, p, d)
        assert dw.shape == w.shape
        lhs, rhs = float(np.sum(y * dy)), float(np.sum(w * dw))
        assert lhs == rhs, "adjoint identity fails: %r vs %r at %s" % (lhs, rhs, (N, H, W, IC, OC, KH, KW, s, p, d))
        done += 1


def pin_wgt_torch(o):
    """G2: torch.nn.grad.conv2d_weight in fp64 on NCHW views (an independent
    library implementation of the same gradient)."""
    import torch
    rng = np.random.default_rng(24)
    for (N, H, W, IC, OC, KH, KW, s, p, d) in [(2, 11, 9, 6, 5, 3, 3, 1, 1, 1),
                                                (1, 16, 16, 3, 8, 7, 7, 2, 3, 1),
                                                (2, 13, 12, 8, 4, 3, 3, 1, 2, 2),
                                                (1, 10, 7, 5, 6, 2, 4, 3, 2, 2)]:
        OH, OW = o.out_dim(H, KH, s, p, d), o.out_dim(W, KW, s, p, d)
        x = rng.standard_normal((N, H, W, IC))
        dy = rng.standard_normal((N, OH, OW, OC))
        dw, _ = o.conv2d_bwd_weight(x, dy, KH, KW, s, p, d)
        t = torch.nn.grad.conv2d_weight(torch.from_numpy(x).permute(0, 3, 1, 2), (OC, IC, KH, KW),
                                        torch.from_numpy(dy).permute(0, 3, 1, 2),
                                        stride=s, padding=p, dilation=d)
        assert_close(dw, t.permute(0, 2, 3, 1).numpy(), 1e-12, 1e-12, "torch conv2d_weight")


def pin_wgt_matmul_1x1(o):
    """G3: a 1x1 window without padding makes the weight gradient a plain
    product over pixels, dw[oc][0][0][:] = dy^T x (x subsampled by the
    stride), checked against numpy's matmul in fp64."""
    rng = np.random.default_rng(25)
    for s in (1, 2, 3):
        x = rng.standard_normal((2, 9, 8, 7))
        OH, OW = o.out_dim(9, 1, s, 0, 1), o.out_dim(8, 1, s, 0, 1)
        dy = rng.standard_normal((2, OH, OW, 5))
        dw, _ = o.conv2d_bwd_weight(x, dy, 1, 1, s, 0, 1)
        xs = x[:, ::s, ::s, :][:, :OH, :OW, :].reshape(-1, 7)
        want = dy.reshape(-1, 5).T @ xs
        assert_close(dw[:, 0, 0, :], want, 1e-12, 1e-12, "1x1 weight gradient, stride %d" % s)


def pin_wgt_magnitude(o):
    """G4: S >= |dw| everywhere, and S equals the weight gradient of |x| and |dy|."""
    rng = np.random.default_rng(26)
    x = rng.standard_normal((2, 8, 8, 4))
    dy = rng.standard_normal((2, 8, 8, 5))
    dw, S = o.conv2d_bwd_weight(x, dy, 3, 3, 1, 1, 1)
    assert (S >= np.abs(dw) - 1e-12).all(), "triangle inequality"
    da, _ = o.conv2d_bwd_weight(np.abs(x), np.abs(dy), 3, 3, 1, 1, 1)
    assert_close(S, da, 1e-12, 1e-12, "S equals the gradient of magnitudes")


ALL_PINS = [pin_out_dims, pin_matmul_1x1, pin_centered_delta, pin_offcenter_delta,
            pin_all_ones, pin_bruteforce, pin_linearity, pin_torch, pin_magnitude, pin_pixels,
            pin_bwd_adjoint, pin_bwd_torch, pin_bwd_delta, pin_bwd_magnitude,
            pin_wgt_adjoint, pin_wgt_torch, pin_wgt_matmul_1x1, pin_wgt_magnitude]
