/* Runs the oracle's entry points on small seeded shapes (including
 * paddings wider than the window, strides larger than the window,
 * dilations and non-square windows) so that a sanitizer build catches any
 * out-of-bounds access or undefined behaviour in them.  Exits 0 when every
 * call returned 0; a sanitizer report aborts the run. */
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>

int oracle_out_dim(int in, int k, int s, int p, int d);
int oracle_conv2d_fwd(const double *x, const double *w, const double *b, int N, int H, int W, int IC, int OC,
                      int KH, int KW, int s, int p, int d, double *y, double *S);
int oracle_conv2d_fwd_pixels(const double *x, const double *w, const double *b, int N, int H, int W, int IC,
                             int OC, int KH, int KW, int s, int p, int d, const int64_t *pix, int64_t npix,
                             double *y, double *S);
int oracle_conv2d_bwd_data(const double *dy, const double *w, int N, int H, int W, int IC, int OC, int KH,
                           int KW, int s, int p, int d, double *dx, double *S);
int oracle_conv2d_bwd_weight(const double *x, const double *dy, int N, int H, int W, int IC, int OC, int KH,
                             int KW, int s, int p, int d, double *dw, double *S);

static unsigned long long rng = 88172645463325252ULL;
static int rnd(int lo, int hi) /* in [lo, hi] */
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return lo + (int)(rng % (unsigned long long)(hi - lo + 1));
}

static double *fill(size_t n)
{
    double *a = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i)
        a[i] = rnd(-3, 3);
    return a;
}

int main(void)
{
    int done = 0;
    for (int it = 0; it < 400 && done < 120; ++it) {
        const int N = rnd(1, 2), H = rnd(1, 9), W = rnd(1, 9), IC = rnd(1, 5), OC = rnd(1, 5);
        const int KH = rnd(1, 5), KW = rnd(1, 4), s = rnd(1, 4), p = rnd(0, 5), d = rnd(1, 3);
        const int OH = oracle_out_dim(H, KH, s, p, d), OW = oracle_out_dim(W, KW, s, p, d);
        if (OH <= 0 || OW <= 0)
            continue;
        const size_t nx = (size_t)N * H * W * IC, nw = (size_t)OC * KH * KW * IC, ny = (size_t)N * OH * OW * OC;
        double *x = fill(nx), *w = fill(nw), *b = fill(OC), *dy = fill(ny);
        double *y = malloc(ny * sizeof(double)), *S = malloc(ny * sizeof(double));
        double *dx = malloc(nx * sizeof(double)), *Sx = malloc(nx * sizeof(double));
        double *dw = malloc(nw * sizeof(double)), *Sw = malloc(nw * sizeof(double));
        int64_t pix[3] = {0, (int64_t)(N * OH * OW - 1), (int64_t)(N * OH * OW / 2)};
        double *yp = malloc(3 * OC * sizeof(double)), *Sp = malloc(3 * OC * sizeof(double));
        if (oracle_conv2d_fwd(x, w, (it & 1) ? b : NULL, N, H, W, IC, OC, KH, KW, s, p, d, y, S)
            || oracle_conv2d_fwd_pixels(x, w, b, N, H, W, IC, OC, KH, KW, s, p, d, pix, 3, yp, Sp)
            || oracle_conv2d_bwd_data(dy, w, N, H, W, IC, OC, KH, KW, s, p, d, dx, Sx)
            || oracle_conv2d_bwd_weight(x, dy, N, H, W, IC, OC, KH, KW, s, p, d, dw, Sw)) {
            fprintf(stderr, "an oracle call rejected a valid shape\n");
            return 1;
        }
        free(x), free(w), free(b), free(dy), free(y), free(S), free(dx), free(Sx), free(dw), free(Sw);
        free(yp), free(Sp);
        ++done;
    }
    printf("oracle driver: %d shapes\n", done);
    return done >= 100 ? 0 : 1;
}
