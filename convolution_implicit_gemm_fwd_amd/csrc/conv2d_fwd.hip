// conv2d_fwd.hip -- the C ABI of libconvimg (declared in include/convimg.h):
// argument checks, output extent, the tile plan, the split-K semaphore pool
// and the kernel launch.  The kernels are in igemm_fwd.hpp.
#include "convimg.h"
#include "igemm_fwd.hpp"

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

using namespace convimg;

namespace {

// ---------------------------------------------------------------------------
// Tile table.  Every entry runs 4 waves; the loader variant is a second,
// independent template argument.
// ---------------------------------------------------------------------------
struct TileCfg {
    int BM, BN, waves_m;
    const char *name;
};

constexpr TileCfg kTiles[] = {
    {128, 64, 2, "128x64"},     // 0: OC <= 64, large M (wave tile 64x32)
    {128, 128, 2, "128x128"},   // 1: OC > 64 (wave tile 64x64)
    {256, 128, 2, "256x128"},   // 2: OC > 64, very large M (wave tile 128x64)
    {64, 64, 2, "64x64"},       // 3: small problems (wave tile 32x32)
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
constexpr int kNumLoaders = 3;

typedef void (*KernelFn)(ConvArgs);

template <int T, int L>
constexpr KernelFn kfn()
{
    return &igemm_fwd_bf16<kTiles[T].BM, kTiles[T].BN, kTiles[T].waves_m, L>;
}

const KernelFn kKernels[kNumTiles][kNumLoaders] = {
    {kfn<0, 0>(), kfn<0, 1>(), kfn<0, 2>()},
    {kfn<1, 0>(), kfn<1, 1>(), kfn<1, 2>()},
    {kfn<2, 0>(), kfn<2, 1>(), kfn<2, 2>()},
    {kfn<3, 0>(), kfn<3, 1>(), kfn<3, 2>()},
};

int lds_bytes_of(int tile)
{
    return 2 * (kTiles[tile].BM + kTiles[tile].BN) * kChunks * 16;
}

// Workgroups of a tile config that can be resident on one CU, from its LDS
// footprint alone (160 KB per CU on gfx950); used by the host-only plan.
int lds_occupancy(int tile)
{
    int n = (160 * 1024) / lds_bytes_of(tile);
    return n < 1 ? 1 : (n > 8 ? 8 : n);
}

std::atomic<int> g_force_tile{-1}, g_force_splits{-1}, g_force_loader{-1};

bool log_enabled()
{
    static const bool on = [] {
        const char *e = std::getenv("CONVIMG_LOG");
        return e && e[0] == '1';
    }();
    return on;
}

// Per-device facts that never change: CU count, occupancy per kernel.
struct DeviceInfo {
    int num_cus = 0;
    int occ[kNumTiles][kNumLoaders] = {};
};
std::mutex g_mu;
std::map<int, DeviceInfo> g_dev;

int device_info(int dev, DeviceInfo **out)
{
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_dev.find(dev);
    if (it == g_dev.end()) {
        DeviceInfo info;
        if (hipDeviceGetAttribute(&info.num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess
            || info.num_cus <= 0)
            return CONVIMG_ERR_DEVICE;
        for (int t = 0; t < kNumTiles; ++t)
            for (int l = 0; l < kNumLoaders; ++l) {
                int nb = 0;
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kKernels[t][l], kThreads, 0) != hipSuccess
                    || nb <= 0)
                    nb = 1;
                info.occ[t][l] = nb;
            }
        it = g_dev.emplace(dev, info).first;
    }
    *out = &it->second;
    return CONVIMG_OK;
}

// Split-K semaphores: one int per output tile plus a status word, per
// (device, stream), kept at zero between calls (the last split of a tile
// resets its own semaphore).
struct SemPool {
    int *ptr = nullptr;
    int n = 0;
};
std::map<std::pair<int, hipStream_t>, SemPool> g_sems;

int get_semaphores(int dev, hipStream_t stream, int need, int **out)
{
    std::lock_guard<std::mutex> lock(g_mu);
    SemPool &p = g_sems[std::make_pair(dev, stream)];
    if (p.n < need) {
        int n = need < 4096 ? 4096 : need;
        if (p.ptr) {
            if (hipStreamSynchronize(stream) != hipSuccess)
                return CONVIMG_ERR_ALLOC;
            (void)hipFree(p.ptr);
            p.ptr = nullptr;
            p.n = 0;
        }
        int *ptr = nullptr;
        if (hipMalloc(&ptr, sizeof(int) * (size_t)n) != hipSuccess)
            return CONVIMG_ERR_ALLOC;
        hipLaunchKernelGGL(fill_zero_i32, dim3((n + 255) / 256), dim3(256), 0, stream, ptr, n);
        if (hipGetLastError() != hipSuccess) {
            (void)hipFree(ptr);
            return CONVIMG_ERR_ALLOC;
        }
        p.ptr = ptr;
        p.n = n;
    }
    *out = p.ptr;
    return CONVIMG_OK;
}

int out_dim(int in, int k, int s, int p, int d)
{
    if (in <= 0 || k <= 0 || s <= 0 || p < 0 || d <= 0)
        return -1;
    const long long span = (long long)d * (k - 1) + 1;
    const long long padded = (long long)in + 2LL * p;
    if (span > padded)
        return -1;
    const long long o = (padded - span) / s + 1;
    return o > 0x7fffffffLL ? -1 : (int)o;
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Problem -> plan.  `occ` (may be NULL) gives resident workgroups per CU for
// each kernel; NULL uses the LDS-only estimate.
int make_plan(int N, int H, int W, int IC, int OC, int KH, int KW, int s, int p, int d,
              int dtype, int num_cus, bool aligned, const int (*occ)[kNumLoaders],
              convimg_plan *pl)
{
    if (N <= 0 || H <= 0 || W <= 0 || IC <= 0 || OC <= 0 || KH <= 0 || KW <= 0
        || s <= 0 || p < 0 || d <= 0)
        return CONVIMG_ERR_SHAPE;
    if (dtype != CONVIMG_BF16 && dtype != CONVIMG_FP32)
        return CONVIMG_ERR_DTYPE;
    const int OH = out_dim(H, KH, s, p, d);
    const int OW = out_dim(W, KW, s, p, d);
    if (OH <= 0 || OW <= 0)
        return CONVIMG_ERR_SHAPE;
    const long long lim = 0x7fffffffLL;
    const long long M = (long long)N * OH * OW;
    const long long K = (long long)IC * KH * KW;
    if ((long long)N * H * W * IC >= lim || K >= lim || (long long)OC * K >= lim || M >= lim
        || M * OC >= lim)
        return CONVIMG_ERR_RANGE;

    std::memset(pl, 0, sizeof(*pl));
    pl->OH = OH;
    pl->OW = OW;
    pl->M = M;
    pl->Ngemm = OC;
    pl->K = (int)K;
    pl->threads = kThreads;

    if (dtype == CONVIMG_FP32) {
        pl->tile_id = -1;
        pl->BM = kF32BM;
        pl->BN = kF32BN;
        pl->BK = kF32BK;
        pl->loader = CONVIMG_LOADER_FP32;
        pl->splits = 1;
        pl->tiles_m = ceil_div(M, kF32BM);
        pl->tiles_n = ceil_div(OC, kF32BN);
        pl->ktiles = ceil_div(K, kF32BK);
        pl->grid = pl->tiles_m * pl->tiles_n;
        pl->lds_bytes = (kF32BM + kF32BN) * (kF32BK + 1) * 4;
        return CONVIMG_OK;
    }

    // loader: widest gather the channel count and alignment allow
    int loader = CONVIMG_LOADER_SCALAR;
    if (aligned && IC % kBK == 0)
        loader = CONVIMG_LOADER_TAP;
    else if (aligned && IC % 8 == 0)
        loader = CONVIMG_LOADER_VEC8;
    const int fl = g_force_loader.load();
    if (fl >= 0) {
        const bool allowed = fl == CONVIMG_LOADER_SCALAR
            || (fl == CONVIMG_LOADER_VEC8 && aligned && IC % 8 == 0)
            || (fl == CONVIMG_LOADER_TAP && aligned && IC % kBK == 0);
        if (allowed)
            loader = fl;
    }

    // tile: cover OC with as few N tiles as possible; shrink for small M
    int tile;
    if (OC <= 64)
        tile = (M <= 64LL * num_cus) ? 3 : 0;
    else
        tile = 1;
    const int ft = g_force_tile.load();
    if (ft >= 0 && ft < kNumTiles)
        tile = ft;

    const int BM = kTiles[tile].BM, BN = kTiles[tile].BN;
    const int tiles_m = ceil_div(M, BM);
    const int tiles_n = ceil_div(OC, BN);
    const int ktiles = ceil_div(K, kBK);
    const long long tiles = (long long)tiles_m * tiles_n;

    // split-K: only when the tiles cannot fill the CUs and K is long.  The
    // grid stays within the resident capacity so every split of every tile
    // is running at once and no wait can depend on an unscheduled block.
    const int resident = (occ ? occ[tile][loader] : lds_occupancy(tile)) * num_cus;
    int splits = 1;
    if (tiles < num_cus && ktiles >= 16) {
        long long sc = resident / tiles;
        long long sk = ktiles / 8;
        splits = (int)(sc < sk ? sc : sk);
        if (splits > 16)
            splits = 16;
        if (splits < 1)
            splits = 1;
    }
    const int fs = g_force_splits.load();
    if (fs >= 1)
        splits = fs;
    if (splits > ktiles)
        splits = ktiles;
    if (splits > 1 && tiles * splits > resident) {
        splits = (int)(resident / tiles);
        if (splits < 1)
            splits = 1;
    }
    const long long tiles_pad = splits > 1 ? (tiles + 7) / 8 * 8 : tiles;
    if (tiles_pad * splits >= lim)
        return CONVIMG_ERR_RANGE;

    pl->tile_id = tile;
    pl->BM = BM;
    pl->BN = BN;
    pl->BK = kBK;
    pl->loader = loader;
    pl->splits = splits;
    pl->tiles_m = tiles_m;
    pl->tiles_n = tiles_n;
    pl->ktiles = ktiles;
    pl->grid = (int)(tiles_pad * splits);
    pl->lds_bytes = lds_bytes_of(tile);
    return CONVIMG_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace

extern "C" {

int conv2d_fwd_out_dim(int in, int k, int stride, int pad, int dilation)
{
    return out_dim(in, k, stride, pad, dilation);
}

int conv2d_fwd_num_tiles(void) { return kNumTiles; }

int conv2d_fwd_force(int tile_id, int splits, int loader)
{
    if (tile_id >= kNumTiles || loader >= kNumLoaders)
        return CONVIMG_ERR_SHAPE;
    g_force_tile.store(tile_id < 0 ? -1 : tile_id);
    g_force_splits.store(splits < 1 ? -1 : splits);
    g_force_loader.store(loader < 0 ? -1 : loader);
    return CONVIMG_OK;
}

int conv2d_fwd_plan(int N, int H, int W, int IC, int OC, int KH, int KW,
                    int stride, int pad, int dilation, int dtype, int num_cus,
                    convimg_plan *plan)
{
    if (!plan)
        return CONVIMG_ERR_NULL;
    const int(*occ)[kNumLoaders] = nullptr;
    if (num_cus <= 0) {
        int dev = 0;
        DeviceInfo *info = nullptr;
        if (hipGetDevice(&dev) != hipSuccess)
            return CONVIMG_ERR_DEVICE;
        int rc = device_info(dev, &info);
        if (rc != CONVIMG_OK)
            return rc;
        num_cus = info->num_cus;
        occ = info->occ;
    }
    return make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, num_cus, true,
                     occ, plan);
}

int conv2d_fwd(const void *x, const void *w, const float *bias,
               int N, int H, int W, int IC, int OC, int KH, int KW,
               int stride, int pad, int dilation, int dtype,
               float *out, hipStream_t stream)
{
    if (!x || !w || !out)
        return CONVIMG_ERR_NULL;
    // shape checks first: they need no device
    convimg_plan pl;
    int rc = make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, 1, true, nullptr, &pl);
    if (rc != CONVIMG_OK)
        return rc;
    const size_t esz = dtype == CONVIMG_BF16 ? 2 : 4;
    const size_t nx = (size_t)N * H * W * IC * esz;
    const size_t nw = (size_t)OC * pl.K * esz;
    const size_t no = (size_t)pl.M * OC * 4;
    if (overlaps(out, no, x, nx) || overlaps(out, no, w, nw)
        || (bias && overlaps(out, no, bias, (size_t)OC * 4)))
        return CONVIMG_ERR_ALIAS;

    int dev = 0;
    DeviceInfo *info = nullptr;
    if (hipGetDevice(&dev) != hipSuccess)
        return CONVIMG_ERR_DEVICE;
    rc = device_info(dev, &info);
    if (rc != CONVIMG_OK)
        return rc;
    const bool aligned = (((uintptr_t)x | (uintptr_t)w) & 15) == 0;
    rc = make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, info->num_cus, aligned,
                   info->occ, &pl);
    if (rc != CONVIMG_OK)
        return rc;

    ConvArgs a;
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.out = out;
    a.sem = nullptr;
    a.N = N;
    a.H = H;
    a.W = W;
    a.IC = IC;
    a.OC = OC;
    a.KH = KH;
    a.KW = KW;
    a.stride = stride;
    a.pad = pad;
    a.dil = dilation;
    a.OH = pl.OH;
    a.OW = pl.OW;
    a.M = (int)pl.M;
    a.K = pl.K;
    a.tiles_m = pl.tiles_m;
    a.tiles_n = pl.tiles_n;
    a.ktiles = pl.ktiles;
    a.splits = pl.splits;
    a.tiles_pad = pl.grid / pl.splits;
    a.remap = pl.splits == 1 ? 1 : 0;

    if (pl.splits > 1) {
        rc = get_semaphores(dev, stream, pl.tiles_m * pl.tiles_n + 1, &a.sem);
        if (rc != CONVIMG_OK)
            return rc;
    }
    if (log_enabled())
        std::fprintf(stderr,
                     "convimg: N=%d H=%d W=%d IC=%d OC=%d K=%dx%d s=%d p=%d d=%d -> "
                     "tile=%d(%dx%dx%d) loader=%d splits=%d grid=%d lds=%d\n",
                     N, H, W, IC, OC, KH, KW, stride, pad, dilation, pl.tile_id, pl.BM, pl.BN,
                     pl.BK, pl.loader, pl.splits, pl.grid, pl.lds_bytes);

    if (dtype == CONVIMG_FP32)
        hipLaunchKernelGGL(igemm_fwd_f32, dim3(pl.grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(kKernels[pl.tile_id][pl.loader], dim3(pl.grid), dim3(kThreads), 0,
                           stream, a);
    if (hipGetLastError() != hipSuccess)
        return CONVIMG_ERR_LAUNCH;
    return CONVIMG_OK;
}

int conv2d_fwd_status(hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return CONVIMG_ERR_DEVICE;
    int *ptr = nullptr;
    int n = 0;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_sems.find(std::make_pair(dev, stream));
        if (it == g_sems.end())
            return CONVIMG_OK;
        ptr = it->second.ptr;
        n = it->second.n;
    }
    if (hipStreamSynchronize(stream) != hipSuccess)
        return CONVIMG_ERR_DEVICE;
    // the status word follows the semaphores of the largest grid seen; a
    // timeout leaves semaphores out of step, so any nonzero word anywhere
    // means: report it and reset the whole array
    int *host = (int *)std::malloc(sizeof(int) * (size_t)n);
    if (!host)
        return CONVIMG_ERR_ALLOC;
    int status = CONVIMG_OK;
    if (hipMemcpy(host, ptr, sizeof(int) * (size_t)n, hipMemcpyDeviceToHost) != hipSuccess)
        status = CONVIMG_ERR_DEVICE;
    else {
        for (int i = 0; i < n; ++i)
            if (host[i] != 0) {
                status = CONVIMG_ERR_TIMEOUT;
                break;
            }
        if (status != CONVIMG_OK) {
            hipLaunchKernelGGL(fill_zero_i32, dim3((n + 255) / 256), dim3(256), 0, stream, ptr, n);
            (void)hipStreamSynchronize(stream);
        }
    }
    std::free(host);
    return status;
}

void conv2d_release(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    for (auto &kv : g_sems) {
        if (kv.second.ptr) {
            int cur = 0;
            (void)hipGetDevice(&cur);
            (void)hipSetDevice(kv.first.first);
            (void)hipDeviceSynchronize();
            (void)hipFree(kv.second.ptr);
            (void)hipSetDevice(cur);
        }
    }
    g_sems.clear();
}

const char *conv2d_strerror(int status)
{
    switch (status) {
    case CONVIMG_OK: return "ok";
    case CONVIMG_ERR_NULL: return "null pointer argument";
    case CONVIMG_ERR_SHAPE: return "invalid shape, stride, padding or dilation (or no output pixel)";
    case CONVIMG_ERR_DTYPE: return "unsupported dtype";
    case CONVIMG_ERR_RANGE: return "an element count reaches 2^31";
    case CONVIMG_ERR_ALIAS: return "out overlaps an input";
    case CONVIMG_ERR_ALLOC: return "could not allocate split-K semaphores";
    case CONVIMG_ERR_LAUNCH: return "kernel launch failed";
    case CONVIMG_ERR_DEVICE: return "no usable HIP device";
    case CONVIMG_ERR_TIMEOUT: return "a split-K workgroup timed out waiting for its turn";
    default: return "unknown status";
    }
}

}  // extern "C"
