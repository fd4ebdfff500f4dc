// Exercises the host side of libconvimg without a device: the planner on
// seeded shapes for several CU counts (every kernel family's plan
// function), forced plans, and the argument checks of every entry point
// (invalid arguments only, so no call reaches the device).  Built with
// the host pass under AddressSanitizer and UBSan, a report aborts the run;
// exits 0 when every status is one the header allows.
#include "convimg.h"

#include <cstdio>
#include <cstdint>

static unsigned long long rng = 2463534242ULL;
static int rnd(int lo, int hi)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return lo + (int)(rng % (unsigned long long)(hi - lo + 1));
}

static bool allowed(int rc)
{
    return rc == CONVIMG_OK || rc == CONVIMG_ERR_SHAPE || rc == CONVIMG_ERR_RANGE;
}

int main()
{
    const int cus[] = {256, 304, 80, 1};
    int plans = 0;
    for (int it = 0; it < 3000; ++it) {
        const int N = rnd(1, 32), H = rnd(1, 300), W = rnd(1, 300);
        const int IC = rnd(0, 3) == 0 ? rnd(1, 8) : 8 * rnd(1, 80), OC = rnd(1, 600);
        const int K = rnd(1, 7), KW = rnd(0, 3) == 0 ? rnd(1, 7) : K;
        const int s = rnd(1, 4), p = rnd(0, 4), d = rnd(1, 3), dtype = rnd(0, 1);
        convimg_plan pl;
        const int rc = conv2d_fwd_plan(N, H, W, IC, OC, K, KW, s, p, d, dtype, cus[it & 3], &pl);
        if (!allowed(rc)) {
            std::fprintf(stderr, "plan status %d\n", rc);
            return 1;
        }
        if (rc == CONVIMG_OK) {
            ++plans;
            if (pl.grid <= 0 || pl.threads <= 0 || pl.OH <= 0 || pl.OW <= 0) {
                std::fprintf(stderr, "bad plan: grid %d threads %d\n", pl.grid, pl.threads);
                return 1;
            }
        }
        size_t bytes = 0;
        const int rcw = conv2d_fwd_nchw_workspace(N, H, W, IC, OC, K, KW, s, p, d, dtype, &bytes);
        if (!allowed(rcw)) {
            std::fprintf(stderr, "workspace status %d\n", rcw);
            return 1;
        }
    }
    // forced plans: every tile, split-K factor and loader the knob accepts
    for (int t = -1; t < conv2d_fwd_num_tiles(); ++t)
        for (int sp : {-1, 1, 3, 16})
            for (int l = -1; l < 3; ++l) {
                if (conv2d_fwd_force(t, sp, l) != CONVIMG_OK) {
                    std::fprintf(stderr, "force %d %d %d refused\n", t, sp, l);
                    return 1;
                }
                convimg_plan pl;
                const int rc = conv2d_fwd_plan(16, 56, 56, 64, 64, 3, 3, 1, 1, 1, 0, 256, &pl);
                const int rc2 = conv2d_fwd_plan(4, 128, 128, 128, 128, 3, 3, 1, 2, 2, 0, 256, &pl);
                const int rc3 = conv2d_fwd_plan(16, 224, 224, 3, 64, 7, 7, 2, 3, 1, 0, 256, &pl);
                if (rc || rc2 || rc3) {
                    std::fprintf(stderr, "forced plan %d %d %d: %d %d %d\n", t, sp, l, rc, rc2, rc3);
                    return 1;
                }
            }
    conv2d_fwd_force(-1, -1, -1);
    // argument errors: each returns before any device work
    void *const a = (void *)0x1000000, *const b = (void *)0x2000000, *const o = (void *)0x3000000;
    int bad = 0;
    bad += conv2d_fwd(nullptr, b, nullptr, 2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 0, (float *)o, 0) != CONVIMG_ERR_NULL;
    bad += conv2d_fwd(a, b, nullptr, 0, 8, 8, 16, 16, 3, 3, 1, 1, 1, 0, (float *)o, 0) != CONVIMG_ERR_SHAPE;
    bad += conv2d_fwd(a, b, nullptr, 2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 0, (float *)a, 0) != CONVIMG_ERR_ALIAS;
    bad += conv2d_bwd_data(a, b, 2, 8, 8, 16, 16, 3, 3, 2, 1, 1, 0, o, (float *)((char *)a + 64), 0)
           != CONVIMG_ERR_ALIAS;
    bad += conv2d_bwd_data_weights(a, 16, 3, 3, 16, 0, a, 0) != CONVIMG_ERR_ALIAS;
    bad += conv2d_bwd_weight(a, b, 2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 2, (float *)o, nullptr, 0, 0)
           != CONVIMG_ERR_DTYPE;
    bad += conv2d_fwd_nchw(a, b, nullptr, 2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 0, 1, o, (void *)0x6000000, 16, 0)
           != CONVIMG_ERR_WORKSPACE;
    bad += conv2d_fwd_autotune(a, b, nullptr, 2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 7, (float *)o, 0, nullptr, nullptr,
                               nullptr, nullptr) != CONVIMG_ERR_DTYPE;
    conv2d_fwd_autotune_clear();
    for (int code = 0; code < 16; ++code)
        bad += conv2d_strerror(code) == nullptr;
    std::printf("abi driver: %d plans, %d unexpected statuses\n", plans, bad);
    return bad == 0 && plans > 1000 ? 0 : 1;
}
