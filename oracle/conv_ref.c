/*
 * conv_ref.c -- CPU oracle for 2-D convolution forward, NHWC / OHWI / NHWC,
 * and for its data-backward and weight-backward passes.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP library and
 * its Python binding never call it, include it or share any code with it.
 *
 * What it computes
 * ----------------
 * The plain definition of the forward convolution, the single operation that
 * the pages' direct, im2col and implicit-GEMM algorithms all implement
 * interchangeably:
 *   - burn-cubecl "kernel/conv/base.rs" listing, conv_forward_nhwc: the same
 *     call is served by a direct kernel or by an implicit GEMM, with the
 *     input in NHWC and the weight permuted to [OC][KH][KW][IC] (OHWI);
 *     the bias is "added to each channel" and is optional;
 *   - burn PR "Introduce autotuning to conv2d and conv_transpose2d with a new
 *     im2col/GEMM algorithm", Changes: autotune picks among direct, im2col
 *     and implicit GEMM for the same op; the GEMM view has
 *     M = batch*out_h*out_w, N = out_channels, K = in_channels*kernel_h*kernel_w.
 *
 *   y[n][oh][ow][oc] = bias[oc]
 *        + sum_{kh<KH} sum_{kw<KW} sum_{ic<IC}
 *              X(n, oh*s - p + kh*d, ow*s - p + kw*d, ic) * w[oc][kh][kw][ic]
 *   X(n, i, j, c)   = x[n][i][j][c] when 0 <= i < H and 0 <= j < W, else 0
 *   S[n][oh][ow][oc] = sum of |X(...) * w[...]| over the same terms
 *
 * S is the magnitude sum the parity tolerance is scaled by.
 *
 * Readings where the pages are silent (each is pinned by a test):
 *   - no kernel flip (cross-correlation);
 *   - zero padding, symmetric, equal for both spatial axes;
 *   - OH = floor((H + 2p - d(KH-1) - 1)/s) + 1, i.e. the number of window
 *     positions that fit inside the padded input; trailing rows that do not
 *     complete a window are ignored;
 *   - groups = 1 (the listing routes groups != 1 away from the implicit GEMM).
 *
 * Arithmetic: every input arrives as double; products and sums are fp64, in
 * the loop order written below (no blocking, no reordering, no fast-math).
 * The inputs the tests feed it are bf16- or fp32-valued, so each product is
 * exact in fp64 and only the summation rounds.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared conv_ref.c -o libconvref.so
 */
#include <stddef.h>
#include <stdint.h>
#include <math.h>
#include <omp.h>

/* Output extent along one spatial axis; -1 when no window fits or an
 * argument is out of range. */
int oracle_out_dim(int in, int k, int s, int p, int d)
{
    if (in <= 0 || k <= 0 || s <= 0 || p < 0 || d <= 0)
        return -1;
    long long span = (long long)d * (k - 1) + 1;   /* receptive extent */
    long long padded = (long long)in + 2LL * p;
    if (span > padded)
        return -1;
    return (int)((padded - span) / s + 1);
}

/* One output pixel (n, oh, ow): all OC outputs and their magnitude sums.
 * y_px and s_px point at OC doubles; s_px may be NULL. */
static void conv_pixel(const double *x, const double *w, const double *bias,
                       int H, int W, int IC, int OC, int KH, int KW,
                       int s, int p, int d, int n, int oh, int ow,
                       double *y_px, double *s_px)
{
    for (int oc = 0; oc < OC; ++oc) {
        double acc = 0.0;
        double mag = 0.0;
        for (int kh = 0; kh < KH; ++kh) {
            int ih = oh * s - p + kh * d;
            for (int kw = 0; kw < KW; ++kw) {
                int iw = ow * s - p + kw * d;
                if (ih < 0 || ih >= H || iw < 0 || iw >= W)
                    continue;                       /* zero padding */
                const double *xp = x + (((size_t)n * H + ih) * W + iw) * IC;
                const double *wp = w + (((size_t)oc * KH + kh) * KW + kw) * IC;
                for (int ic = 0; ic < IC; ++ic) {
                    double prod = xp[ic] * wp[ic];
                    acc += prod;
                    mag += fabs(prod);
                }
            }
        }
        y_px[oc] = acc + (bias ? bias[oc] : 0.0);
        if (s_px)
            s_px[oc] = mag;
    }
}

static int check_args(int N, int H, int W, int IC, int OC, int KH, int KW,
                      int s, int p, int d, int *OH, int *OW)
{
    if (N <= 0 || H <= 0 || W <= 0 || IC <= 0 || OC <= 0 || KH <= 0 || KW <= 0)
        return -1;
    *OH = oracle_out_dim(H, KH, s, p, d);
    *OW = oracle_out_dim(W, KW, s, p, d);
    if (*OH <= 0 || *OW <= 0)
        return -1;
    return 0;
}

/* Full output: y (and S if non-NULL) hold N*OH*OW*OC doubles, NHWC.
 * bias may be NULL (treated as zeros).  Returns 0, or -1 on bad shapes. */
int oracle_conv2d_fwd(const double *x, const double *w, const double *bias,
                      int N, int H, int W, int IC, int OC, int KH, int KW,
                      int s, int p, int d, double *y, double *S)
{
    int OH, OW;
    if (check_args(N, H, W, IC, OC, KH, KW, s, p, d, &OH, &OW))
        return -1;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n)
        for (int oh = 0; oh < OH; ++oh)
            for (int ow = 0; ow < OW; ++ow) {
                size_t px = ((size_t)n * OH + oh) * OW + ow;
                conv_pixel(x, w, bias, H, W, IC, OC, KH, KW, s, p, d, n, oh, ow,
                           y + px * OC, S ? S + px * OC : NULL);
            }
    return 0;
}

/* Selected output pixels only.  pix[i] is the flat pixel index
 * (n*OH + oh)*OW + ow; y and S (S may be NULL) receive npix*OC doubles in
 * the order of pix.  Returns 0, or -1 on bad shapes or an index out of range. */
int oracle_conv2d_fwd_pixels(const double *x, const double *w, const double *bias,
                             int N, int H, int W, int IC, int OC, int KH, int KW,
                             int s, int p, int d, const int64_t *pix, int64_t npix,
                             double *y, double *S)
{
    int OH, OW;
    if (check_args(N, H, W, IC, OC, KH, KW, s, p, d, &OH, &OW))
        return -1;
    int64_t total = (int64_t)N * OH * OW;
    for (int64_t i = 0; i < npix; ++i)
        if (pix[i] < 0 || pix[i] >= total)
            return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < npix; ++i) {
        int64_t q = pix[i];
        int ow = (int)(q % OW);
        int oh = (int)((q / OW) % OH);
        int n = (int)(q / ((int64_t)OW * OH));
        conv_pixel(x, w, bias, H, W, IC, OC, KH, KW, s, p, d, n, oh, ow,
                   y + i * OC, S ? S + i * OC : NULL);
    }
    return 0;
}

/* Gradient of the forward convolution with respect to its input x (the
 * data-backward pass of the burn-cubecl "kernel/conv/base.rs" listing,
 * conv_data_backward: it takes the output gradient and the weights and
 * returns a tensor of the input's shape).  Since y is linear in x,
 *
 *   dx[n][ih][iw][ic] = sum over (oh, ow, kh, kw, oc) with
 *                         oh*s - p + kh*d == ih and ow*s - p + kw*d == iw
 *                       of dy[n][oh][ow][oc] * w[oc][kh][kw][ic]
 *   S[n][ih][iw][ic]  = the same sum of |dy * w|
 *
 * dy is N x OH x OW x OC with OH, OW the forward output extents of (H, W);
 * dx and S are N x H x W x IC.  For each input pixel the terms are taken in
 * the order kh, kw, oc, with oh = (ih + p - kh*d) / s where that division
 * is exact and 0 <= oh < OH (likewise ow); any stride.  Returns 0, or -1 on
 * bad shapes. */
int oracle_conv2d_bwd_data(const double *dy, const double *w,
                           int N, int H, int W, int IC, int OC, int KH, int KW,
                           int s, int p, int d, double *dx, double *S)
{
    int OH, OW;
    if (check_args(N, H, W, IC, OC, KH, KW, s, p, d, &OH, &OW))
        return -1;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n)
        for (int ih = 0; ih < H; ++ih)
            for (int iw = 0; iw < W; ++iw) {
                size_t px = ((size_t)n * H + ih) * W + iw;
                double *g = dx + px * IC;
                double *a = S ? S + px * IC : NULL;
                for (int ic = 0; ic < IC; ++ic) {
                    g[ic] = 0.0;
                    if (a)
                        a[ic] = 0.0;
                }
                for (int kh = 0; kh < KH; ++kh) {
                    int th = ih + p - kh * d;          /* = oh * s */
                    if (th < 0 || th % s != 0 || th / s >= OH)
                        continue;
                    int oh = th / s;
                    for (int kw = 0; kw < KW; ++kw) {
                        int tw = iw + p - kw * d;      /* = ow * s */
                        if (tw < 0 || tw % s != 0 || tw / s >= OW)
                            continue;
                        int ow = tw / s;
                        const double *gy = dy + (((size_t)n * OH + oh) * OW + ow) * OC;
                        for (int oc = 0; oc < OC; ++oc) {
                            const double *wr = w + ((size_t)(oc * KH + kh) * KW + kw) * IC;
                            for (int ic = 0; ic < IC; ++ic) {
                                double t = gy[oc] * wr[ic];
                                g[ic] += t;
                                if (a)
                                    a[ic] += fabs(t);
                            }
                        }
                    }
                }
            }
    return 0;
}

/* Gradient of the forward convolution with respect to its weights (the
 * weight-backward pass of the burn-cubecl "kernel/conv/base.rs" listing,
 * conv_weight_backward: it takes the input and the output gradient and
 * returns a tensor of the weights' shape).  Since y is linear in w,
 *
 *   dw[oc][kh][kw][ic] = sum_{n<N} sum_{oh<OH} sum_{ow<OW}
 *                          dy[n][oh][ow][oc] * X(n, oh*s - p + kh*d, ow*s - p + kw*d, ic)
 *   S[oc][kh][kw][ic]  = the same sum of |dy * X|
 *
 * with X as for the forward (0 in the padding).  x is N x H x W x IC, dy is
 * N x OH x OW x OC with OH, OW the forward output extents; dw and S are
 * OC x KH x KW x IC.  The terms are taken in the order n, oh, ow; any
 * stride, padding and dilation.  Returns 0, or -1 on bad shapes. */
int oracle_conv2d_bwd_weight(const double *x, const double *dy,
                             int N, int H, int W, int IC, int OC, int KH, int KW,
                             int s, int p, int d, double *dw, double *S)
{
    int OH, OW;
    if (check_args(N, H, W, IC, OC, KH, KW, s, p, d, &OH, &OW))
        return -1;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int oc = 0; oc < OC; ++oc)
        for (int kh = 0; kh < KH; ++kh)
            for (int kw = 0; kw < KW; ++kw) {
                const size_t wrow = (size_t)oc * KH * KW + (size_t)kh * KW + kw;
                double *g = dw + wrow * IC;
                double *m = S ? S + wrow * IC : NULL;
                for (int ic = 0; ic < IC; ++ic) {
                    g[ic] = 0.0;
                    if (m)
                        m[ic] = 0.0;
                }
                for (int n = 0; n < N; ++n)
                    for (int oh = 0; oh < OH; ++oh) {
                        int jh = oh * s - p + kh * d;     /* input row of this tap */
                        if (jh < 0 || jh >= H)
                            continue;
                        for (int ow = 0; ow < OW; ++ow) {
                            int jw = ow * s - p + kw * d; /* input column */
                            if (jw < 0 || jw >= W)
                                continue;
                            double gy = dy[(((size_t)n * OH + oh) * OW + ow) * OC + oc];
                            const double *xr = x + (((size_t)n * H + jh) * W + jw) * IC;
                            for (int ic = 0; ic < IC; ++ic) {
                                double t = gy * xr[ic];
                                g[ic] += t;
                                if (m)
                                    m[ic] += fabs(t);
                            }
                        }
                    }
            }
    return 0;
}

/* Threads the OpenMP loops use; n <= 0 leaves the default.  Returns the
 * count in effect. */
int oracle_set_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
}
