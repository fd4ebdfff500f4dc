// conv2d_fwd.hip -- the C ABI of libconvimg (declared in include/convimg.h):
// argument checks, output extent, the tile plan, the split-K semaphore pool
// and the kernel launches.  The kernels are in the igemm_*.hpp headers.
#include "convimg.h"
#include "igemm_image.hpp"
#include "igemm_patch.hpp"
#include "igemm_pipe.hpp"
#include "igemm_regs.hpp"
#include "igemm_resident.hpp"
#include "igemm_dgrad.hpp"
#include "igemm_layout.hpp"
#include "igemm_strip.hpp"
#include "igemm_window.hpp"
#include "igemm_wgrad.hpp"

#include <algorithm>
#include <vector>
#include <array>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <type_traits>

using namespace convimg;

namespace {

// ---------------------------------------------------------------------------
// Tile table.  kRegs entries use the register-staged kernel (every loader,
// including the element-wise edge path); kPipe entries use the direct-to-LDS
// pipelined kernel (vector loaders only); kPatch entries the pipelined kernel
// with an LDS patch of input rows; kStrip entries the strip kernel (BM is the
// largest chunk of pixels: 4 waves x BM / 128 blocks of 32 rows); the
// kWindow entry the few-channel kernel (every loader slot); the kResident
// entry the kernel with weights and input rows resident in LDS; the kImage
// entry the kernel for deep layers on small images (one workgroup per image
// and 32 output channels, K in chunks of 64 channels).
// ---------------------------------------------------------------------------
enum Kind { kRegs = 0, kPipe = 1, kPatch = 2, kStrip = 3, kWindow = 4, kResident = 5, kImage = 6 };

struct TileCfg {
    int kind, BM, BN, WM, WN, stages, ms;
    const char *name;
    int patch_px;   // kPatch: input pixels the LDS patch holds
};

constexpr TileCfg kTiles[] = {
    {kRegs, 128, 64, 2, 2, 2, 16, "regs 128x64"},           // 0
    {kRegs, 128, 128, 2, 2, 2, 16, "regs 128x128"},         // 1
    {kRegs, 256, 128, 2, 2, 2, 16, "regs 256x128"},         // 2
    {kRegs, 64, 64, 2, 2, 2, 16, "regs 64x64"},             // 3
    {kPipe, 128, 64, 2, 2, 3, 16, "pipe16 128x64 s3"},      // 4
    {kPipe, 128, 64, 2, 2, 4, 16, "pipe16 128x64 s4"},      // 5
    {kPipe, 128, 128, 2, 2, 3, 16, "pipe16 128x128 s3"},    // 6
    {kPipe, 256, 128, 4, 2, 3, 16, "pipe16 256x128 w8"},    // 7
    {kPipe, 64, 64, 2, 2, 4, 16, "pipe16 64x64 s4"},        // 8
    {kPipe, 256, 64, 4, 2, 3, 16, "pipe16 256x64 w8"},      // 9
    {kPipe, 128, 128, 2, 4, 3, 16, "pipe16 128x128 w8"},    // 10
    {kPipe, 128, 64, 4, 2, 3, 16, "pipe16 128x64 w8"},      // 11
    {kPipe, 256, 128, 2, 2, 3, 32, "pipe32 256x128 w4"},    // 12: wave 128x64
    {kPipe, 256, 128, 4, 2, 3, 32, "pipe32 256x128 w8"},    // 13: wave 64x64
    {kPipe, 128, 128, 2, 2, 3, 32, "pipe32 128x128 s3"},    // 14: wave 64x64
    {kPipe, 128, 128, 2, 2, 2, 32, "pipe32 128x128 s2"},    // 15: wave 64x64, 2 WG/CU
    {kPipe, 128, 64, 2, 2, 3, 32, "pipe32 128x64 s3"},      // 16: wave 64x32
    {kPipe, 256, 64, 4, 1, 3, 32, "pipe32 256x64 w4"},      // 17: wave 64x64
    {kPipe, 128, 64, 4, 1, 3, 32, "pipe32 128x64 w4x1"},    // 18: wave 32x64
    {kPipe, 128, 128, 2, 4, 3, 32, "pipe32 128x128 w8"},    // 19: wave 64x32
    {kPipe, 64, 64, 2, 2, 4, 32, "pipe32 64x64 s4"},        // 20: wave 32x32
    {kPipe, 128, 128, 2, 2, 4, 32, "pipe32 128x128 s4"},    // 21
    {kPatch, 128, 64, 2, 2, 3, 32, "patch 128x64", 384},    // 22: wave 64x32
    {kPatch, 256, 64, 4, 1, 3, 32, "patch 256x64", 512},    // 23: wave 64x64
    {kPatch, 256, 128, 2, 2, 3, 32, "patch 256x128 w4", 768}, // 24: wave 128x64
    {kPatch, 256, 128, 4, 2, 3, 32, "patch 256x128 w8", 768}, // 25: wave 64x64
    {kPatch, 128, 128, 2, 2, 3, 32, "patch 128x128", 640},  // 26: wave 64x64
    {kPatch, 128, 64, 4, 1, 3, 32, "patch 128x64 w4x1", 384}, // 27: wave 32x64
    {kPatch, 256, 64, 4, 1, 9, 32, "patch 256x64 s9", 512},  // 28: all 3x3 weight taps in flight
    {kPatch, 128, 64, 2, 2, 9, 32, "patch 128x64 s9", 384},  // 29
    {kStrip, 256, 64, 4, 1, 1, 32, "strip 256"},            // 30: chunks of up to 256 pixels
    {kStrip, 128, 64, 4, 1, 1, 32, "strip 128"},            // 31
    {kWindow, 128, 64, 4, 1, 1, 32, "window"},              // 32: few input channels
    {kResident, 32, 64, 8, 1, 1, 32, "resident"},           // 33: weights + input rows in LDS
    {kImage, 32, 32, 8, 1, 2, 32, "image"},                 // 34: one image x 32 channels per workgroup
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
constexpr int kLdsBytes = 160 * 1024;     // LDS per CU (and per workgroup) on gfx950
constexpr int kWindowTile = 32;           // the kWindow entry
constexpr int kResidentTile = 33;         // the kResident entry
constexpr int kImageTile = 34;            // the kImage entry
constexpr int kTwoPerCuTile = 15;         // pipe32 128x128, 2 stages: two workgroups per CU
constexpr int kSmallPipeTile = 20;        // pipe32 64x64, 4 stages: problems with few 128x128 tiles
constexpr int kTallPipeTile = 4;          // pipe16 128x64, 3 stages: few 128x128 tiles but enough 128x64
constexpr int kImgMaxMB = 8;              // image kernel: at most 8 blocks of 32 output pixels
constexpr int kNumLoaders = 3;

typedef void (*KernelFn)(ConvArgs);

template <int T, int L>
constexpr KernelFn kfn()
{
    constexpr TileCfg c = kTiles[T];
    if constexpr (c.kind == kRegs)
        return &igemm_regs_bf16<c.BM, c.BN, c.WM, L>;
    else if constexpr (c.kind == kWindow)
        return &igemm_window_bf16<kWinMaxKH>;      // stands for the family; launches pick by KH
    else if constexpr (c.kind == kResident)
        return &igemm_resident_bf16<9, 4>;         // stands for the family; launches pick by IC
    else if constexpr (c.kind == kImage)
        return &igemm_image_bf16<kImgMaxMB>;       // stands for the family; launches pick by MB
    else if constexpr (c.kind == kStrip)
        return L == kLoaderTap ? &igemm_strip_bf16<c.BM / 128> : nullptr;   // FM
    else if constexpr (c.kind == kPatch)
        return L == kLoaderTap ? &igemm_patch_bf16<c.BM, c.BN, c.WM, c.WN, c.stages, c.patch_px>
                               : nullptr;
    else if constexpr (L == kLoaderScalar)
        return nullptr;
    else
        return &igemm_pipe_bf16<c.BM, c.BN, c.WM, c.WN, c.stages, c.ms, L>;
}

template <int T>
constexpr std::array<KernelFn, kNumLoaders> krow()
{
    return {kfn<T, 0>(), kfn<T, 1>(), kfn<T, 2>()};
}

template <int... T>
constexpr std::array<std::array<KernelFn, kNumLoaders>, sizeof...(T)> ktable(std::integer_sequence<int, T...>)
{
    return {krow<T>()...};
}

const std::array<std::array<KernelFn, kNumLoaders>, kNumTiles> kKernels =
    ktable(std::make_integer_sequence<int, kNumTiles>{});

// Window kernels by kernel height (1 .. kWinMaxKH).
const KernelFn kWinKernels[kWinMaxKH + 1] = {
    nullptr, &igemm_window_bf16<1>, &igemm_window_bf16<2>, &igemm_window_bf16<3>,
    &igemm_window_bf16<4>, &igemm_window_bf16<5>, &igemm_window_bf16<6>, &igemm_window_bf16<7>,
};
static_assert(kWinMaxKH == 7, "window kernel table");

// Resident kernels (3x3) by IC / 16 = 1, 2, 4, 8.
const KernelFn kResKernels[4] = {
    &igemm_resident_bf16<9, 1>, &igemm_resident_bf16<9, 2>, &igemm_resident_bf16<9, 4>,
    &igemm_resident_bf16<9, 8>,
};
// The same with x and out in NCHW order: [fp32 out, bf16 out][IC / 16 = 1, 2, 4, 8].
const KernelFn kResNchwKernels[2][4] = {
    {&igemm_resident_bf16<9, 1, kResNchwF32>, &igemm_resident_bf16<9, 2, kResNchwF32>,
     &igemm_resident_bf16<9, 4, kResNchwF32>, &igemm_resident_bf16<9, 8, kResNchwF32>},
    {&igemm_resident_bf16<9, 1, kResNchwBf16>, &igemm_resident_bf16<9, 2, kResNchwBf16>,
     &igemm_resident_bf16<9, 4, kResNchwBf16>, &igemm_resident_bf16<9, 8, kResNchwBf16>},
};
// Image kernels by blocks of 32 output pixels per image (1 .. kImgMaxMB).
const KernelFn kImgKernels[kImgMaxMB + 1] = {
    nullptr, &igemm_image_bf16<1>, &igemm_image_bf16<2>, &igemm_image_bf16<3>, &igemm_image_bf16<4>,
    &igemm_image_bf16<5>, &igemm_image_bf16<6>, &igemm_image_bf16<7>, &igemm_image_bf16<8>,
};
static_assert(kImgMaxMB == 8, "image kernel table");

int res_index(int IC)
{
    return IC == 16 ? 0 : IC == 32 ? 1 : IC == 64 ? 2 : IC == 128 ? 3 : -1;
}

int threads_of(int tile)
{
    return kTiles[tile].kind == kStrip ? kStripThreads
         : kTiles[tile].kind == kWindow ? kWinThreads
         : kTiles[tile].kind == kResident ? kResThreads
         : kTiles[tile].kind == kImage ? kImgThreads
         : kTiles[tile].WM * kTiles[tile].WN * 64;
}

int lds_bytes_of(int tile)
{
    const TileCfg &c = kTiles[tile];
    if (c.kind == kPatch)
        return (c.patch_px + 1) * kChunks * 16 + c.stages * c.BN * kChunks * 16;
    if (c.kind == kStrip || c.kind == kWindow || c.kind == kResident || c.kind == kImage)
        return kLdsBytes;       // sized per problem; one workgroup per CU
    return c.stages * (c.BM + c.BN) * kChunks * 16;
}

// Largest patch (input rows x W pixels) any BM-pixel tile of this problem
// reads; -1 when there are too many tiles to check.
long long max_patch_px(long long M, int BM, int H, int W, int OH, int OW, int KH, int s, int p,
                       int d)
{
    const long long tiles = (M + BM - 1) / BM;
    if (tiles > (1 << 20))
        return -1;
    long long best = 0;
    for (long long t = 0; t < tiles; ++t) {
        const int m0 = (int)(t * BM);
        const int m1 = (int)(m0 + BM < M ? m0 + BM : M);
        const PatchRows r = patch_rows(m0, m1, H, OH, OW, KH, s, p, d);
        const long long px = (long long)(r.hi - r.lo + 1) * W;
        if (px > best)
            best = px;
    }
    return best;
}

// Workgroups of a tile config that can be resident on one CU, from its LDS
// footprint alone (160 KB per CU on gfx950); used by the host-only plan.
int lds_occupancy(int tile)
{
    int n = kLdsBytes / lds_bytes_of(tile);
    return n < 1 ? 1 : (n > 8 ? 8 : n);
}

std::atomic<int> g_force_tile{-1}, g_force_splits{-1}, g_force_loader{-1};
std::atomic<int> g_spin_limit{kSpinLimit};     // split-K wait bound (tests shorten it)

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
    std::array<int, kNumLoaders> occ[kNumTiles] = {};
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
            for (int l = 0; l < kNumLoaders; ++l)
                if ((kTiles[t].kind == kStrip || kTiles[t].kind == kWindow) && kKernels[t][l] != nullptr)
                    (void)hipFuncSetAttribute((const void *)kKernels[t][l],
                                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        for (int kh = 1; kh <= kWinMaxKH; ++kh)
            (void)hipFuncSetAttribute((const void *)kWinKernels[kh],
                                      hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        for (KernelFn f : kResKernels)
            (void)hipFuncSetAttribute((const void *)f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        for (const auto &row : kResNchwKernels)
            for (KernelFn f : row)
                (void)hipFuncSetAttribute((const void *)f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        for (int mb = 1; mb <= kImgMaxMB; ++mb)
            (void)hipFuncSetAttribute((const void *)kImgKernels[mb],
                                      hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        wgrad_set_attributes();
        for (int t = 0; t < kNumTiles; ++t)
            for (int l = 0; l < kNumLoaders; ++l) {
                int nb = 1;
                if (kKernels[t][l] != nullptr
                    && (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kKernels[t][l], threads_of(t), 0)
                            != hipSuccess
                        || nb <= 0))
                    nb = 1;
                info.occ[t][l] = nb;
            }
        it = g_dev.emplace(dev, info).first;
    }
    *out = &it->second;
    return CONVIMG_OK;
}

// The current device and its facts.  The last device a host thread used is
// remembered per thread, so the hot path takes no lock (entries of g_dev are
// never removed, so the pointer stays valid).
int current_device(int *dev, DeviceInfo **info)
{
    thread_local int t_dev = -1;
    thread_local DeviceInfo *t_info = nullptr;
    if (hipGetDevice(dev) != hipSuccess)
        return CONVIMG_ERR_DEVICE;
    if (*dev == t_dev && t_info != nullptr) {
        *info = t_info;
        return CONVIMG_OK;
    }
    const int rc = device_info(*dev, info);
    if (rc == CONVIMG_OK) {
        t_dev = *dev;
        t_info = *info;
    }
    return rc;
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

// Strip kernel plan: one workgroup per CU for each 64-channel slice, strips
// of equal length, chunks of at most 256 pixels; LDS holds a zero block, the
// slice's weights for the whole K, the largest patch any chunk needs and the
// epilogue scratch.
struct StripPlan {
    int tile = -1;
    int strip_px = 0, chunk_px = 0, tiles_m = 0, tiles_n = 0;
    int lds_zero = 0, lds_patch = 0, lds_scratch = 0, lds_flags = 0, lds_bytes = 0;
};

bool fill_strip(StripPlan *sp, long long strip, long long chunk, int tiles_m, int tiles_n,
                long long zero, long long wbytes, long long patch);

// Window kernel plan (few input channels): one kernel row of the receptive
// field fits in 32 k values, windows start at even elements for every pixel
// and row (s*IC and W*IC even), x reached with 32-bit offsets in 16-byte
// chunks, out with 32-bit store offsets.  (Odd s*IC or W*IC would need two
// weight layouts; those shapes keep the element-wise gather.)  One workgroup per CU per 64
// channels; units (up to 128 pixels of one output row) split evenly.
struct WinPlan {
    int seg = 0, segs = 0, sh = 0, wp = 0, rb = 0, sets = 0;
    int tiles_m = 0, tiles_n = 0, lds_rows = 0, lds_bytes = 0;
};

bool plan_window(int N, int H, int W, int IC, int OC, int KH, int KW, int s, int p, int d,
                 int OH, int OW, long long M, int num_cus, WinPlan *wp)
{
    const long long lim = 0x7fffffffLL;
    const int sh = (p * IC) & 1;
    const long long span = ((long long)(KW - 1) * d + 1) * IC;
    if (KH > kWinMaxKH || span + sh > 32 || (s * IC) % 2 != 0 || (W * IC) % 2 != 0)
        return false;
    // (a 16-byte copy may run past the end of x: buffer loads check the
    // range per dword, so the dwords inside x still arrive)
    const long long xbytes = (long long)N * H * W * IC * 2;
    const long long wbytes = (long long)OC * KH * KW * IC * 2;
    if (xbytes % 4 != 0 || xbytes >= lim || wbytes >= lim || M * OC * 4 >= lim)
        return false;
    const int segs = ceil_div(OW, kWinSeg);
    const int seg = ceil_div(OW, segs);
    // every wave reads its 32 pixels' windows, also past the unit's last
    // pixel (those results are not stored): size the row buffers for 128.
    // The run starts up to 14 bytes into its buffer (the copy starts at the
    // 16-byte boundary below it) and ends 2 * jall bytes later.
    const long long jall = (long long)(kWinSeg - 1) * s * IC + 32;
    const long long rb = (16 + 2 * jall + 1023) / 1024 * 1024;
    // LDS: the weight staging rows (later the epilogue scratch), then the
    // row-buffer sets.  Prefer kWinOcc workgroups per CU, then 3 sets (rows
    // of two units in flight) over 2.
    const int wrow = ((KH * 32 + 8) * 2 + 15) / 16 * 16;
    const int rows_at = 64 * wrow > kWinScrBytes ? 64 * wrow : kWinScrBytes;
    int occ = 0, sets = 0;
    for (int o = kWinOcc; o >= 1 && sets == 0; --o)
        for (int st = 3; st >= 2 && sets == 0; --st)
            if ((rows_at + (long long)st * KH * rb) * o <= kLdsBytes) {
                occ = o;
                sets = st;
            }
    if (sets == 0)
        return false;
    const int tiles_n = ceil_div(OC, 64);
    long long gm = (long long)occ * num_cus / tiles_n;
    if (gm < 1)
        gm = 1;
    const long long units = (long long)N * OH * segs;
    // the kernel's 32-bit row offsets, float-reciprocal unit divisions and
    // 32-bit unit-range products (units times the group count)
    if (xbytes >= (1LL << 30) || units >= (1LL << 21) || units * (units < gm ? units : gm) >= (1LL << 31))
        return false;
    wp->seg = seg;
    wp->segs = segs;
    wp->sh = sh;
    wp->wp = wrow;
    wp->rb = (int)rb;
    wp->sets = sets;
    wp->tiles_m = (int)(units < gm ? units : gm);      // groups of units (an even split)
    wp->tiles_n = tiles_n;
    wp->lds_rows = rows_at;
    wp->lds_bytes = (int)(rows_at + (long long)sets * KH * rb);
    return true;
}

struct ResPlan {
    int tiles_m = 0, tiles_n = 0, lds_rows = 0, zero = 0, lds_bytes = 0, rows = 0, scr = -1;
};

// Resident kernel plan (3x3, IC = 16, 32, 64 or 128, x and w 16-byte
// aligned): the 64-channel weight slice (K bf16 + one spare chunk per
// record) and the input rows of the largest of the tiles_m pixel ranges
// (IC bf16 + one spare chunk per pixel) must fit in LDS with one zero
// record.  The ranges split M evenly, larger shares first, as the kernel
// does.
bool plan_resident(int N, int H, int W, int IC, int OC, int KH, int KW, int s, int p, int d,
                   int OH, int OW, long long M, int num_cus, ResPlan *rp)
{
    const long long lim = 0x7fffffffLL;
    if (KH * KW != 9 || res_index(IC) < 0)
        return false;
    if ((long long)N * H * W * IC * 2 >= lim || (long long)OC * KH * KW * IC * 2 >= lim || M * OC * 4 >= lim)
        return false;
    if (M >= (1LL << 21))           // the kernel's float-reciprocal divisions of pixel indices
        return false;
    const long long prec = IC * 2 + 16;
    const long long wbytes = 64 * ((long long)KH * KW * IC * 2 + 16);
    if (wbytes + 1024 + prec > kLdsBytes)
        return false;
    const int tiles_n = ceil_div(OC, 64);
    long long tm = num_cus / tiles_n;
    if (tm < 1)
        tm = 1;
    if (tm > M)
        tm = M;
    const long long per = M / tm, extra = M - per * tm;
    const long long ohw = (long long)OH * OW;
    long long max_rows = 0;
    for (long long g = 0; g < tm; ++g) {
        const long long m_a = g * per + (g < extra ? g : extra);
        const long long m_b = m_a + per + (g < extra ? 1 : 0);
        const long long n_a = m_a / ohw, oh_a = (m_a - n_a * ohw) / OW;
        const long long n_b = (m_b - 1) / ohw, oh_b = (m_b - 1 - n_b * ohw) / OW;
        const long long lo = n_a * H + std::max<long long>(oh_a * s - p, 0);
        const long long hi = n_b * H + std::min<long long>(oh_b * s - p + (long long)(KH - 1) * d, H - 1);
        max_rows = std::max(max_rows, hi - lo + 1);
    }
    const long long rows_bytes = (max_rows * W * prec + 1023) / 1024 * 1024;
    const long long lds = wbytes + rows_bytes + prec;
    if (lds > kLdsBytes)
        return false;
    rp->tiles_m = (int)tm;
    rp->tiles_n = tiles_n;
    rp->lds_rows = (int)wbytes;
    rp->zero = (int)(wbytes + rows_bytes);
    rp->lds_bytes = (int)lds;
    // the store scratch (results leave as 16-byte stores) where it fits
    if (lds + kResScrBytes <= kLdsBytes) {
        rp->scr = (int)lds;
        rp->lds_bytes = (int)(lds + kResScrBytes);
    }
    rp->rows = (int)max_rows;
    return true;
}

struct ImgPlan {
    int mb = 0, set = 0, wofs = 0, lds_bytes = 0, tiles_n = 0, ti = 1, ts = 1;
};

// Image kernel plan (3x3, IC % 64 == 0, x and w 16-byte aligned): one
// image's output (at most kImgMaxMB blocks of 32 pixels) per workgroup;
// two buffer sets of (zero-padded image, 64 records of 144 bytes per pixel;
// 9 x 32 weight records) must fit in LDS, as must the 4 partial tiles of
// the final reduction.
bool plan_image(int N, int H, int W, int IC, int OC, int KH, int KW, int p, int OH, int OW,
                ImgPlan *ip)
{
    const long long lim = 0x7fffffffLL;
    if (KH != 3 || KW != 3 || IC % 64 != 0)
        return false;
    if ((long long)N * H * W * IC * 2 >= lim || (long long)OC * 9 * IC * 2 >= lim
        || (long long)N * OH * OW * OC * 4 >= lim)
        return false;
    const int mb = ceil_div(OH * OW, 32);
    if (mb > kImgMaxMB)
        return false;
    // the kernel's 24-bit products and float-reciprocal divisions
    if (IC > 65536 || (long long)N * ceil_div(OC, kImgBN) >= (1LL << 21))
        return false;
    // padded rows of img_row_units chunks (at least one copy instruction's
    // 64 chunks), then the weight chunks; no copy writes past its region
    if (W + 2LL * p > 4096 || H + 2LL * p > 4096)
        return false;
    long long pchunks = (long long)(H + 2 * p) * img_row_units(W + 2 * p, OW);
    if (pchunks < 64)
        pchunks = 64;
    const long long patch = pchunks * 16;
    const long long wts = (long long)kImgWChunks * 16;
    const long long set = patch + wts;
    long long lds = 2 * set;
    const long long red = 4LL * 32 * mb * kImgRedRow * 4;
    if (red > lds)
        lds = red;
    if (lds > kLdsBytes)
        return false;
    const long long copies = (pchunks + 63) / 64 + (kImgWChunks + 63) / 64;
    if ((copies + kImgWaves - 1) / kImgWaves > kImgMaxCopies)
        return false;
    ip->mb = mb;
    ip->set = (int)set;
    ip->wofs = (int)patch;
    ip->lds_bytes = (int)lds;
    ip->tiles_n = ceil_div(OC, kImgBN);
    // workgroup blocks of ti images x ts slices (about one XCD's 32 workgroups)
    for (int g : {4, 2, 1})
        if (N % g == 0) {
            ip->ti = g;
            break;
        }
    for (int g : {8, 4, 2, 1})
        if (ip->tiles_n % g == 0) {
            ip->ts = g;
            break;
        }
    return true;
}

bool plan_strip(long long M, int H, int W, int OH, int OW, int IC, int OC, int KH, int KW,
                int s, int p, int d, long long K, int num_cus, StripPlan *sp)
{
    const int cpp = IC / 8;
    if (IC % kBK != 0)
        return false;
    const long long zero = ((IC * 2 > 1024 ? IC * 2 : 1024) + 1023) / 1024 * 1024;
    const int rec = cpp + 1;                    // LDS record: cpp chunks and a spare
    const long long wbytes = (long long)kStripBN * KH * KW * rec * 16;
    if (zero + wbytes + kStripScratchBytes >= kLdsBytes)
        return false;
    const int tiles_n = ceil_div(OC, kStripBN);
    int gm = num_cus / tiles_n;
    if (gm < 1)
        gm = 1;
    long long strip = (M + gm - 1) / gm;
    if (strip < 32)
        strip = 32;
    const int tiles_m = ceil_div(M, strip);
    // the largest chunk whose patch fits next to the weights (at most 256
    // pixels: 2 blocks of 32 rows per M-group keep a compute wave within the
    // registers of 3 waves per SIMD)
    for (int cap = 256; cap >= 128; cap /= 2) {
        const long long nc = (strip + cap - 1) / cap;
        if ((long long)tiles_m * nc > (1 << 22))
            return false;
        const long long chunk = (strip + nc - 1) / nc;
        long long patch = 0;
        for (long long g = 0; g < tiles_m; ++g) {
            const long long e = (g + 1) * strip < M ? (g + 1) * strip : M;
            for (long long c0 = g * strip; c0 < e; c0 += chunk) {
                const long long c1 = c0 + chunk < e ? c0 + chunk : e;
                const StripSeg sg = strip_seg((int)c0, (int)c1, H, W, OH, OW, KH, s, p, d, rec);
                if (sg.total_chunks * 16 > patch)
                    patch = sg.total_chunks * 16;
            }
        }
        const long long total = zero + wbytes + patch + kStripScratchBytes + kStripTailBytes;
        if (total <= kLdsBytes)
            return fill_strip(sp, strip, chunk, tiles_m, tiles_n, zero, wbytes, patch);
    }
    return false;
}

bool fill_strip(StripPlan *sp, long long strip, long long chunk, int tiles_m, int tiles_n,
                long long zero, long long wbytes, long long patch)
{
    const long long blocks = (chunk + 31) / 32;     // 32-row blocks over 4 M-groups
    sp->tile = blocks > 4 ? 30 : 31;
    sp->strip_px = (int)strip;
    sp->chunk_px = (int)chunk;
    sp->tiles_m = tiles_m;
    sp->tiles_n = tiles_n;
    sp->lds_zero = (int)zero;
    sp->lds_patch = (int)(zero + wbytes);
    sp->lds_scratch = (int)(zero + wbytes + patch);
    sp->lds_flags = (int)(zero + wbytes + patch + kStripScratchBytes);
    sp->lds_bytes = (int)(zero + wbytes + patch + kStripScratchBytes + kStripTailBytes);
    return true;
}

// Problem -> plan.  `aligned`: x and w start on 16-byte boundaries (the
// vector loaders need it).  `occ` (may be NULL) gives resident workgroups per
// CU for each kernel; NULL uses the LDS-only estimate.
int make_plan_uncached(int N, int H, int W, int IC, int OC, int KH, int KW, int s, int p, int d,
                       int dtype, int num_cus, bool aligned,
                       const std::array<int, kNumLoaders> *occ, convimg_plan *pl, StripPlan *spo,
                       WinPlan *wpo, ResPlan *rpo, ImgPlan *ipo, int ft, int fs, int fl)
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
    pl->threads = kRegsThreads;

    if (dtype == CONVIMG_FP32) {
        pl->tile_id = -1;
        pl->BM = kF32BM;
        pl->BN = OC <= kF32BNSmall ? kF32BNSmall : kF32BN;
        pl->BK = kF32BK;
        pl->loader = CONVIMG_LOADER_FP32;
        pl->splits = 1;
        pl->tiles_m = ceil_div(M, kF32BM);
        pl->tiles_n = ceil_div(OC, pl->BN);
        pl->ktiles = ceil_div(K, kF32BK);
        pl->grid = pl->tiles_m * pl->tiles_n;
        pl->lds_bytes = (kF32BM + pl->BN) * kF32Row * 4;
        return CONVIMG_OK;
    }

    // loader: widest gather the channel count and alignment allow
    int loader = CONVIMG_LOADER_SCALAR;
    if (aligned && IC % kBK == 0)
        loader = CONVIMG_LOADER_TAP;
    else if (aligned && IC % 8 == 0)
        loader = CONVIMG_LOADER_VEC8;
    if (fl >= 0) {
        const bool allowed = fl == CONVIMG_LOADER_SCALAR
            || (fl == CONVIMG_LOADER_VEC8 && aligned && IC % 8 == 0)
            || (fl == CONVIMG_LOADER_TAP && aligned && IC % kBK == 0);
        if (allowed)
            loader = fl;
    }

    // The pipelined kernel addresses x and w through 32-bit buffer offsets
    // with an out-of-range sentinel at 2^31 bytes.
    const long long esz = 2;
    const bool pipe_ok = loader != CONVIMG_LOADER_SCALAR
        && (long long)N * H * W * IC * esz < lim && (long long)OC * K * esz < lim;

    // Tile choice, from measured sweeps on MI355X (every table entry timed on
    // each shape class): the resident kernel wherever its weights and input
    // rows fit in LDS (3x3, IC 16 .. 128); else the image kernel for 3x3
    // layers on images of at most 256 output pixels (IC % 64 == 0, the
    // padded image fits twice in LDS); else 128x64 with 8 waves wherever
    // OC <= 64 or the M x N tiles cannot fill the CUs (then split-K fills
    // them); 256x128 with 8 waves when there are enough large tiles for
    // every CU; the window kernel for few input channels.
    StripPlan sp;
    const bool strip_ok = pipe_ok && loader == CONVIMG_LOADER_TAP
        && plan_strip(M, H, W, OH, OW, IC, OC, KH, KW, s, p, d, K, num_cus, &sp);
    WinPlan wnp;
    const bool window_ok = aligned
        && plan_window(N, H, W, IC, OC, KH, KW, s, p, d, OH, OW, M, num_cus, &wnp);
    ResPlan rsp;
    const bool resident_ok = pipe_ok && aligned
        && plan_resident(N, H, W, IC, OC, KH, KW, s, p, d, OH, OW, M, num_cus, &rsp);
    ImgPlan imp;
    const bool image_ok = pipe_ok && aligned && plan_image(N, H, W, IC, OC, KH, KW, p, OH, OW, &imp);
    int tile;
    if (pipe_ok) {
        // 128x128 tiles, two workgroups per CU, wherever they give every CU
        // at least one (one workgroup's copies overlap the other's MFMAs:
        // measured 7 % faster than 256x128 on the dilated layer, and on a
        // 1x1 stride-2 layer with 1.5 a CU 9.4 us against 14.9 for
        // 128x64); fewer than that with OC > 64: 128x64 tiles (3 stages)
        // where those fill the CUs (1x1 256 -> 1024 on 14x14: 7.1 us
        // against 9.2 for 64x64), else 64x64 tiles, split over K up to the
        // CU count (3x3 stride-2 layers with 16 images, 56x56x128, 28x28x256
        // and 14x14x512: 11.0 / 15.4 / 20.9 us against 16.9 / 28.2 / 57.6
        // for 128x64 with every resident slot split); OC <= 64: 128x64
        // (with split-K where K is large)
        const long long mid = ((M + 127) / 128) * ((OC + 127) / 128);
        const long long tall = ((M + 127) / 128) * ((OC + 63) / 64);
        tile = (OC > 64 && mid >= num_cus) ? kTwoPerCuTile
             : OC > 64 ? (tall >= num_cus ? kTallPipeTile : kSmallPipeTile) : 11;
    } else if (OC <= 64) {
        tile = (M <= 64LL * num_cus) ? 3 : 0;
    } else {
        tile = 1;
    }
    if (image_ok)
        tile = kImageTile;      // deep layer on small images: measured faster on every such shape
    if (resident_ok)
        tile = kResidentTile;   // weights and input rows fit in LDS: measured faster on every such shape
    if (window_ok && loader == CONVIMG_LOADER_SCALAR)
        tile = kWindowTile;     // few channels: the window kernel instead of the element-wise gather
    if (ft >= 0 && ft < kNumTiles)
        tile = ft;
    if (kTiles[tile].kind == kWindow) {
        if (window_ok) {
            pl->tile_id = tile;
            pl->BM = wnp.seg;
            pl->BN = 64;
            pl->BK = 32;
            pl->loader = loader;
            pl->splits = 1;
            pl->tiles_m = wnp.tiles_m;
            pl->tiles_n = wnp.tiles_n;
            pl->ktiles = KH;            // K laid out as KH steps of 32
            pl->grid = wnp.tiles_m * wnp.tiles_n;
            pl->threads = kWinThreads;
            pl->lds_bytes = wnp.lds_bytes;
            if (wpo)
                *wpo = wnp;
            return CONVIMG_OK;
        }
        tile = pipe_ok ? 11 : 0;    // a forced window the problem cannot use
    }
    if (kTiles[tile].kind == kImage) {
        if (image_ok) {
            pl->tile_id = tile;
            pl->BM = 32 * imp.mb;           // one image's output pixels
            pl->BN = kImgBN;
            pl->BK = 64;
            pl->loader = loader;
            pl->splits = 1;
            pl->tiles_m = N;
            pl->tiles_n = imp.tiles_n;
            pl->ktiles = IC / 64;
            pl->grid = N * imp.tiles_n;
            pl->threads = kImgThreads;
            pl->lds_bytes = imp.lds_bytes;
            if (ipo)
                *ipo = imp;
            return CONVIMG_OK;
        }
        tile = pipe_ok ? 11 : 0;    // a forced image tile the problem cannot use
    }
    if (kTiles[tile].kind == kResident) {
        if (resident_ok) {
            pl->tile_id = tile;
            pl->BM = 32;                // pixels per wave unit
            pl->BN = 64;
            pl->BK = 16;
            pl->loader = loader;
            pl->splits = 1;
            pl->tiles_m = rsp.tiles_m;
            pl->tiles_n = rsp.tiles_n;
            pl->ktiles = (int)(K / 16);
            pl->grid = rsp.tiles_m * rsp.tiles_n;
            pl->threads = kResThreads;
            pl->lds_bytes = rsp.lds_bytes;
            if (rpo)
                *rpo = rsp;
            return CONVIMG_OK;
        }
        tile = pipe_ok ? 11 : 0;    // a forced resident tile the problem cannot use
    }
    if (kTiles[tile].kind == kStrip) {
        if (strip_ok) {
            pl->tile_id = sp.tile;
            pl->BM = kTiles[sp.tile].BM;
            pl->BN = kStripBN;
            pl->BK = kBK;
            pl->loader = loader;
            pl->splits = 1;
            pl->tiles_m = sp.tiles_m;
            pl->tiles_n = sp.tiles_n;
            pl->ktiles = ceil_div(K, kBK);
            pl->grid = sp.tiles_m * sp.tiles_n;
            pl->threads = kStripThreads;
            pl->lds_bytes = sp.lds_bytes;
            if (spo)
                *spo = sp;
            return CONVIMG_OK;
        }
        tile = pipe_ok ? 11 : 0;    // a forced strip the problem cannot use
    }
    if (kTiles[tile].kind == kPipe && !pipe_ok)
        tile = 0;       // a forced pipelined tile the problem cannot use
    if (kTiles[tile].kind == kPatch) {
        const long long px = max_patch_px(M, kTiles[tile].BM, H, W, OH, OW, KH, s, p, d);
        if (!pipe_ok || loader != CONVIMG_LOADER_TAP || px < 0 || px > kTiles[tile].patch_px)
            tile = pipe_ok ? 4 : 0;   // the patch would not fit: the pipelined gather instead
    }
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
        // the 64x64 tile splits only until the CU count is reached and
        // while each split keeps 16 K tiles (its serial turns cost more than
        // the slots left idle: 14x14x512 stride-2 layer 20.9 us with 2
        // splits, 24.2 us with 9; 1x1 1024 -> 256 on 14x14, 16 K tiles, 9.3
        // us whole, 11.8 us in 2); the others fill every resident slot
        const bool small = tile == kSmallPipeTile;
        long long sc = small ? (num_cus + tiles - 1) / tiles : resident / tiles;
        long long sk = ktiles / (small ? 16 : 8);
        splits = (int)(sc < sk ? sc : sk);
        if (splits > 16)
            splits = 16;
        if (splits < 1)
            splits = 1;
    }
    if (fs >= 1)
        splits = fs;
    if (splits > ktiles)
        splits = ktiles;
    if (M * OC * 4 >= lim || kTiles[tile].kind == kPatch)
        splits = 1;     // the in-place reduction addresses out with 32-bit offsets
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
    pl->threads = threads_of(tile);
    pl->lds_bytes = lds_bytes_of(tile);
    return CONVIMG_OK;
}

// Choices made by conv2d_fwd_autotune, per problem (shape, dtype, CU count,
// alignment): the tile and split-K factor that timed fastest.  Consulted by
// the planner only while the table is not empty.
typedef std::array<int, 13> TuneKey;
std::mutex g_tune_mu;
std::map<TuneKey, std::pair<int, int>> g_tuned;
std::atomic<int> g_tuned_count{0};
thread_local int t_try_tile = -1, t_try_splits = -1;   // set while a candidate is timed

TuneKey tune_key(int N, int H, int W, int IC, int OC, int KH, int KW, int s, int p, int d, int dtype,
                 int num_cus, bool aligned)
{
    return TuneKey{N, H, W, IC, OC, KH, KW, s, p, d, dtype, num_cus, aligned ? 1 : 0};
}

void tuned_choice(int N, int H, int W, int IC, int OC, int KH, int KW, int s, int p, int d, int dtype,
                  int num_cus, bool aligned, int *ft, int *fs)
{
    std::lock_guard<std::mutex> lock(g_tune_mu);
    auto it = g_tuned.find(tune_key(N, H, W, IC, OC, KH, KW, s, p, d, dtype, num_cus, aligned));
    if (it != g_tuned.end()) {
        *ft = it->second.first;
        *fs = it->second.second;
    }
}

// Plans of recent problems, per host thread (no lock): planning evaluates
// every kernel family (several microseconds for some shapes), which would
// otherwise be paid on each call of a layer that is run over and over.  The
// key holds every input of the planner, the forced settings included.
constexpr int kPlanCacheWays = 8;
struct PlanCacheEntry {
    int key[16] = {};
    const void *occ = nullptr;
    bool valid = false;
    int rc = 0;
    convimg_plan pl = {};
    StripPlan sp;
    WinPlan wp;
    ResPlan rp;
    ImgPlan ip;
};
thread_local PlanCacheEntry t_plans[kPlanCacheWays];
thread_local unsigned t_plan_next = 0;

int make_plan(int N, int H, int W, int IC, int OC, int KH, int KW, int s, int p, int d,
              int dtype, int num_cus, bool aligned,
              const std::array<int, kNumLoaders> *occ, convimg_plan *pl, StripPlan *spo = nullptr,
              WinPlan *wpo = nullptr, ResPlan *rpo = nullptr, ImgPlan *ipo = nullptr)
{
    // the tile / split-K / loader to force: the test knob, else a plan the
    // autotuner is timing (this thread), else a tuned choice for the problem
    int ft = g_force_tile.load(), fs = g_force_splits.load(), fl = g_force_loader.load();
    if (ft < 0 && fs < 0 && fl < 0) {
        if (t_try_tile >= 0) {
            ft = t_try_tile;
            fs = t_try_splits;
        } else if (g_tuned_count.load() > 0) {
            tuned_choice(N, H, W, IC, OC, KH, KW, s, p, d, dtype, num_cus, aligned, &ft, &fs);
        }
    }
    const int key[16] = {N, H, W, IC, OC, KH, KW, s, p, d, dtype, num_cus, aligned ? 1 : 0, ft, fs, fl};
    PlanCacheEntry *e = nullptr;
    for (PlanCacheEntry &c : t_plans)
        if (c.valid && c.occ == (const void *)occ && std::memcmp(c.key, key, sizeof(key)) == 0) {
            e = &c;
            break;
        }
    if (!e) {
        e = &t_plans[t_plan_next++ % kPlanCacheWays];
        e->valid = false;
        e->sp = StripPlan();
        e->wp = WinPlan();
        e->rp = ResPlan();
        e->ip = ImgPlan();
        e->rc = make_plan_uncached(N, H, W, IC, OC, KH, KW, s, p, d, dtype, num_cus, aligned, occ,
                                   &e->pl, &e->sp, &e->wp, &e->rp, &e->ip, ft, fs, fl);
        std::memcpy(e->key, key, sizeof(key));
        e->occ = occ;
        e->valid = true;
    }
    if (e->rc == CONVIMG_OK) {
        *pl = e->pl;
        if (spo)
            *spo = e->sp;
        if (wpo)
            *wpo = e->wp;
        if (rpo)
            *rpo = e->rp;
        if (ipo)
            *ipo = e->ip;
    }
    return e->rc;
}

FastDiv make_fast_div(int v)
{
    if (v < 1)
        v = 1;   // (callers pass divisors >= 1; a 0 from an unused plan field stays harmless)
    int l = 0;
    while ((1LL << l) < v)
        ++l;
    const unsigned long long num = 1ULL << (31 + l);
    FastDiv f;
    f.mul = (unsigned)((num + (unsigned long long)v - 1) / (unsigned long long)v);
    f.shift = 31 + l;
    return f;
}

// Weight-backward plan: 64 x 192 output tiles; the pixels split into
// contiguous ranges so that tiles x ranges fills the CUs evenly, at least
// four steps of 8 pixel groups per range, partial sums (ranges x OC x
// KH*KW*IC fp32) kept under 1 GiB.
struct WgPlan {
    int OH = 0, OW = 0, M = 0, KKIC = 0, bpr = 0, groups = 0, tiles_m = 0, tiles_n = 0, splits = 1, chunk = 0;
    int tr_stages = 4;            // LDS stages of the transpose-read kernel
    int inplace = 0;              // 1: the ranges add into dw in turn (no workspace)
    // the row-window kernel's own tiles and ranges (row = 1 where the shape
    // allows it; it runs where x and dy are also 16-byte aligned)
    int row = 0, row_xi = 16, row_stages = 3, row_rl = 0, row_rsp = 0, row_rr = 0, row_nseg = 1, row_steps = 0;
    int row_tiles_n = 0, row_splits = 1, row_chunk = 0, row_inplace = 0;
    size_t ws_bytes = 0;          // enough for whichever kernel the call's alignment selects
};

int plan_wgrad(int N, int H, int W, int IC, int OC, int KH, int KW, int s, int p, int d, int dtype,
               int num_cus, WgPlan *wp)
{
    convimg_plan fwd;
    int rc = make_plan(N, H, W, IC, OC, KH, KW, s, p, d, dtype, 1, true, nullptr, &fwd);
    if (rc != CONVIMG_OK)
        return rc;
    const long long lim = 0x7fffffffLL;
    const int esz = dtype == CONVIMG_FP32 ? 4 : 2;
    // x and dy are read through buffer resources with 32-bit byte offsets
    if ((long long)N * H * W * IC * esz >= lim || fwd.M * OC * esz >= lim)
        return CONVIMG_ERR_RANGE;
    wp->OH = fwd.OH;
    wp->OW = fwd.OW;
    wp->M = (int)fwd.M;
    wp->KKIC = fwd.K;
    wp->bpr = ceil_div(fwd.OW, 8);
    const long long groups = (long long)N * fwd.OH * wp->bpr;
    if (groups * 8 >= lim)
        return CONVIMG_ERR_RANGE;
    wp->groups = (int)groups;
    wp->tiles_m = ceil_div(OC, kWgBM);
    if (dtype == CONVIMG_FP32) {
        // fp32 storage: the fp32 kernel's 64 x 64 tiles; ranges for two
        // workgroups per CU, and at most kWgF32MaxSteps steps (8192 pixel
        // slots) each, so that a range's fp32 sum adds at most 8192
        // products per output before the ranges are added in order
        wp->tiles_n = ceil_div(fwd.K, kWgF32BN);
        const long long tiles = (long long)wp->tiles_m * wp->tiles_n;
        const long long steps = (groups + 7) / 8;
        const long long per = (long long)OC * fwd.K * 4;
        long long S = tiles < 2LL * num_cus ? 2LL * num_cus / tiles : 1;
        if (S > steps)
            S = steps;
        if (S < (steps + kWgF32MaxSteps - 1) / kWgF32MaxSteps)
            S = (steps + kWgF32MaxSteps - 1) / kWgF32MaxSteps;
        if (S < 1)
            S = 1;
        const long long chunk = (steps + S - 1) / S * 8;
        S = (groups + chunk - 1) / chunk;
        if (tiles * S >= lim || S * per > (1LL << 30))      // (the workspace stays within 1 GiB)
            return CONVIMG_ERR_RANGE;
        wp->splits = (int)S;
        wp->chunk = (int)chunk;
        wp->inplace = 0;
        wp->row = 0;
        wp->ws_bytes = S > 1 ? (size_t)(S * per) : 0;
        return CONVIMG_OK;
    }
    wp->tiles_n = ceil_div(fwd.K, kWgBN);
    const long long tiles = (long long)wp->tiles_m * wp->tiles_n;
    const long long steps = (groups + 7) / 8;
    // ranges per tile: as many as fit one workgroup per CU (rounded down, so
    // no CU gets a second workgroup while others idle); where the tiles
    // alone fill half the CUs, as many as fit two per CU (the LDS allows
    // two).  Measured: a 12-tile layer ran 90 us with 22 ranges (264
    // workgroups on 256 CUs), 66 us with 32 and 62 us with 21; a 192-tile
    // layer 62 us with one range and 57 us with two.
    // The transpose-read kernel (IC % 64 == 0, OC % 8 == 0) runs with four
    // LDS stages (one workgroup per CU) where the ranges are short, and with
    // two stages (two workgroups per CU, each hiding the other's waits)
    // where a range at one workgroup per CU would still be 16 steps or
    // more.  Measured: the 512-channel 14x14 layer (56 steps a range) 45.5
    // -> 43.0 us, a dilated 128-channel layer (49 steps) 45.0 -> 37.5 us,
    // a 64-channel 56x56 layer (10 steps) 21.0 -> 22.0 us (kept at four).
    const bool tr = wgrad_tr_shape(IC, OC);
    const long long per = (long long)OC * fwd.K * 4;
    auto ranges = [&](long long per_cu) {
        long long S = tiles < per_cu * num_cus ? per_cu * num_cus / tiles : 1;
        if (S > steps / 4)
            S = steps / 4;
        if (S * per > (1LL << 30))
            S = (1LL << 30) / per;
        return S < 1 ? 1LL : S;
    };
    long long S = ranges(tr ? 1 : (2 * tiles >= num_cus ? 2 : 1));
    wp->tr_stages = kWtStagesDeep;
    if (tr && steps / S >= 16) {
        wp->tr_stages = kWtStagesPair;
        S = ranges(2);
    }
    const long long chunk = (steps + S - 1) / S * 8;     // groups per range
    S = (groups + chunk - 1) / chunk;
    if (tiles * S >= lim)
        return CONVIMG_ERR_RANGE;
    wp->splits = (int)S;
    wp->chunk = (int)chunk;
    // a few ranges add into dw in turn; the plan keeps every workgroup
    // resident at once (tiles x ranges within the occupancy used above), so
    // a range's predecessor is always running
    wp->inplace = (S > 1 && S <= kWgInplaceMax && per < (long long)kOutOfRange) ? 1 : 0;
    wp->ws_bytes = (S > 1 && !wp->inplace) ? (size_t)(S * per) : 0;

    // Row-window kernel: units of rl output pixels (a whole row where OW <=
    // 64, else rnseg equal segments; unequal ones are left to the kernels
    // above), rr units in a step's 128 slots; 128 x rows a stage where that
    // holds as many units as 192 rows would (three or four stages, whichever
    // gives the shorter longest range), else 192 (three stages).  Ranges:
    // one workgroup per CU (8 waves, 96-128 KB of LDS), in whole rounds of
    // the stages.
    if (wgrad_row_shape(IC, OC, KW, s)) {
        const int OW = fwd.OW;
        const int nseg = ceil_div(OW, 64);
        const int rl = OW / nseg, rsp = rl + 2 * d;
        // (rows - 1: the last x row stays zero; empty slots read it)
        auto fit = [&](int rows) { return std::min(kWrSlots / rl, (rows - 1) / rsp); };
        const int r16 = fit(128), r24 = fit(192);
        const int xi = (r16 >= 1 && r16 == r24) ? 16 : (r24 >= 1 ? 24 : 0);
        const long long units = (long long)N * fwd.OH * nseg;
        // (units below 2^21: the kernel divides with float reciprocals)
        if (OW % nseg == 0 && xi && units < (1LL << 21)) {
            const int rr = xi == 16 ? r16 : r24;
            const long long rsteps = (units + rr - 1) / rr;
            const long long rtiles = (long long)wp->tiles_m * KH * (IC / 64);
            auto ranges_for = [&](int stages, long long *chunk) {
                long long R = rtiles < num_cus ? num_cus / rtiles : 1;
                if (R > rsteps / stages)
                    R = rsteps / stages;
                if (R * per > (1LL << 30))
                    R = (1LL << 30) / per;
                if (R < 1)
                    R = 1;
                *chunk = ((rsteps + R - 1) / R + stages - 1) / stages * stages;
                return (rsteps + *chunk - 1) / *chunk;
            };
            long long c3 = 0, c4 = 0;
            const long long R3 = ranges_for(3, &c3), R4 = xi == 16 ? ranges_for(4, &c4) : 0;
            const int stages = (xi == 16 && c4 <= c3) ? 4 : 3;
            const long long R = stages == 4 ? R4 : R3, rchunk = stages == 4 ? c4 : c3;
            if (rtiles * R < lim) {
                wp->row = 1;
                wp->row_xi = xi;
                wp->row_stages = stages;
                wp->row_rl = rl;
                wp->row_rsp = rsp;
                wp->row_rr = rr;
                wp->row_nseg = nseg;
                wp->row_steps = (int)rsteps;
                wp->row_tiles_n = KH * (IC / 64);
                wp->row_splits = (int)R;
                wp->row_chunk = (int)rchunk;
                wp->row_inplace = (R > 1 && R <= kWgInplaceMax && per < (long long)kOutOfRange) ? 1 : 0;
                const size_t ws_row = (R > 1 && !wp->row_inplace) ? (size_t)(R * per) : 0;
                if (ws_row > wp->ws_bytes)
                    wp->ws_bytes = ws_row;
            }
        }
    }
    return CONVIMG_OK;
}

// Workspace of the NCHW entry point: NHWC copy of x, OHWI copy of w, fp32
// NHWC result, each starting on a 256-byte boundary.
struct NchwLayout {
    size_t w_off = 0, y_off = 0, bytes = 0;
};

NchwLayout nchw_layout(const convimg_plan &pl, int N, int H, int W, int IC, int OC, int dtype)
{
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t esz = dtype == CONVIMG_BF16 ? 2 : 4;
    NchwLayout l;
    l.w_off = up((size_t)N * H * W * IC * esz);
    l.y_off = up(l.w_off + (size_t)OC * pl.K * esz);
    l.bytes = up(l.y_off + (size_t)pl.M * OC * 4);
    return l;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// The argument errors of the weight transform (returned before any work is
// queued); *grid: its launch grid.
int flip_args(const void *w, int OC, int KH, int KW, int IC, int dtype, const void *wt, dim3 *grid)
{
    if (!w || !wt)
        return CONVIMG_ERR_NULL;
    if (OC <= 0 || KH <= 0 || KW <= 0 || IC <= 0)
        return CONVIMG_ERR_SHAPE;
    if (dtype != CONVIMG_BF16 && dtype != CONVIMG_FP32)
        return CONVIMG_ERR_DTYPE;
    if ((long long)OC * KH * KW * IC >= 0x7fffffffLL)
        return CONVIMG_ERR_RANGE;
    const size_t esz = dtype == CONVIMG_BF16 ? 2 : 4;
    const size_t nw = (size_t)OC * KH * KW * IC * esz;
    if (overlaps(wt, nw, w, nw))
        return CONVIMG_ERR_ALIAS;
    *grid = dim3((IC + kFlipTile - 1) / kFlipTile, (OC + kFlipTile - 1) / kFlipTile, KH * KW);
    if (grid->y > 65535u || grid->z > 65535u)
        return CONVIMG_ERR_RANGE;
    return CONVIMG_OK;
}

// Where the split-K semaphores of a call come from.
enum SemSource { kSemPool, kSemScratch };

int fwd_call(const void *x, const void *w, const float *bias,
             int N, int H, int W, int IC, int OC, int KH, int KW,
             int stride, int pad, int dilation, int dtype,
             float *out, hipStream_t stream, SemSource sems, int flipw = 0, int nchw = 0);

}  // namespace

// Scratch of conv2d_fwd_noalloc: its split-K semaphores (one int per output
// tile and a status word), a fixed array in each device's memory, so the
// entry point never allocates.  The plan keeps tiles x splits within what is
// resident at once (a few thousand workgroups on this chip), far below this.
constexpr int kScratchInts = 4096;
static __device__ __align__(256) int scratch[kScratchInts];

namespace {

// Device address of `scratch` on device `dev` (the current device), looked
// up once per device with that device current and kept: in host code the
// array's name is only a stand-in for the symbol, never a device address.
std::mutex g_scratch_mu;
std::map<int, int *> g_scratch;

int scratch_of(int dev, int **out)
{
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch.find(dev);
    if (it == g_scratch.end()) {
        int *ptr = nullptr;
        if (hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return CONVIMG_ERR_DEVICE;
        it = g_scratch.emplace(dev, ptr).first;
    }
    *out = it->second;
    return CONVIMG_OK;
}

}  // namespace

extern "C" {

int conv2d_fwd_out_dim(int in, int k, int stride, int pad, int dilation)
{
    return out_dim(in, k, stride, pad, dilation);
}

int conv2d_fwd_num_tiles(void) { return kNumTiles; }

int conv2d_fwd_tile_kind(int tile_id)
{
    if (tile_id < 0 || tile_id >= kNumTiles)
        return -1;
    static_assert(kRegs == CONVIMG_KIND_REGS && kPipe == CONVIMG_KIND_PIPE
                      && kPatch == CONVIMG_KIND_PATCH && kStrip == CONVIMG_KIND_STRIP
                      && kWindow == CONVIMG_KIND_WINDOW && kResident == CONVIMG_KIND_RESIDENT
                      && kImage == CONVIMG_KIND_IMAGE,
                  "kind codes");
    static_assert(kTiles[kWindowTile].kind == kWindow, "window tile index");
    static_assert(kTiles[kResidentTile].kind == kResident, "resident tile index");
    static_assert(kTiles[kImageTile].kind == kImage, "image tile index");
    return kTiles[tile_id].kind;
}

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
    const std::array<int, kNumLoaders> *occ = nullptr;
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
    return fwd_call(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out, stream,
                    kSemPool);
}

int conv2d_fwd_noalloc(const void *x, const void *w, const float *bias,
                       int N, int H, int W, int IC, int OC, int KH, int KW,
                       int stride, int pad, int dilation, int dtype,
                       float *out, hipStream_t stream)
{
    return fwd_call(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out, stream,
                    kSemScratch);
}

int conv2d_fwd_test_spin_limit(int iterations)
{
    const int prev = g_spin_limit.load();
    g_spin_limit.store(iterations < 1 ? kSpinLimit : iterations);
    return prev;
}

}  // extern "C"

namespace {

// conv2d_fwd and conv2d_fwd_noalloc: checks, plan, launch.  `sems` says
// where split-K semaphores come from: the library's per-stream pool (may
// allocate on first use) or the device's static scratch array (never
// allocates).  flipw: the data backward's in-LDS weight flip (see below).
// nchw (1: fp32 out, 2: bf16 out): x, w and out in NCHW, OIHW and NCHW
// order, computed by the resident kernel's NCHW variant;
// CONVIMG_ERR_UNSUPPORTED before any launch where that kernel does not
// serve the problem.
int fwd_call(const void *x, const void *w, const float *bias,
             int N, int H, int W, int IC, int OC, int KH, int KW,
             int stride, int pad, int dilation, int dtype,
             float *out, hipStream_t stream, SemSource sems, int flipw, int nchw)
{
    if (!x || !w || !out)
        return CONVIMG_ERR_NULL;
    int dev = 0;
    DeviceInfo *info = nullptr;
    const int rc_dev = current_device(&dev, &info);
    convimg_plan pl;
    StripPlan sp;
    WinPlan wnp;
    ResPlan rsp;
    ImgPlan imp;
    // one plan per call: with the device's facts when there is a device,
    // else host-only, so that argument errors still come before the device
    // error
    const bool aligned = (((uintptr_t)x | (uintptr_t)w) & 15) == 0;
    int rc = rc_dev == CONVIMG_OK
        ? make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, info->num_cus, aligned,
                    info->occ, &pl, &sp, &wnp, &rsp, &imp)
        : make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, 1, true, nullptr, &pl);
    if (rc != CONVIMG_OK)
        return rc;
    const size_t esz = dtype == CONVIMG_BF16 ? 2 : 4;
    const size_t nx = (size_t)N * H * W * IC * esz;
    const size_t nw = (size_t)OC * pl.K * esz;
    const size_t no = (size_t)pl.M * OC * (nchw == 2 ? 2 : 4);
    if (overlaps(out, no, x, nx) || overlaps(out, no, w, nw)
        || (bias && overlaps(out, no, bias, (size_t)OC * 4)))
        return CONVIMG_ERR_ALIAS;
    if (rc_dev != CONVIMG_OK)
        return rc_dev;
    if (nchw) {
        // the NCHW variant: resident plans, 8-pixel runs of whole rows, out
        // 16-byte aligned, the range's 8 x 8 blocks within its loader's rounds
        const int kind = pl.tile_id >= 0 ? kTiles[pl.tile_id].kind : -1;
        if (kind != kResident || dtype != CONVIMG_BF16 || W % 8 != 0 || (((uintptr_t)x | (uintptr_t)out) & 15) != 0
            || (long long)rsp.rows * (W / 8) * (IC / 8) > (long long)kResThreads * kResNchwRounds)
            return CONVIMG_ERR_UNSUPPORTED;
    }

    ConvArgs a;
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.out = out;
    a.sem = nullptr;
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    a.x_bytes = (unsigned)(nx < 0xffffffffu ? nx : 0xffffffffu);
    a.w_bytes = (unsigned)(nw < 0xffffffffu ? nw : 0xffffffffu);
    // masked output lanes store to offset kOutOfRange: it must lie past the
    // extent the buffer resource allows (larger outputs use 64-bit stores)
    a.out_bytes = (unsigned)(no < (size_t)kOutOfRange ? no : (size_t)kOutOfRange);
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
    a.vec_out = (((uintptr_t)out & 15) == 0 && OC % 4 == 0) ? 1 : 0;
    a.div_ohw = make_fast_div(pl.OH * pl.OW);
    a.div_ow = make_fast_div(pl.OW);
    a.remap = pl.splits == 1 ? 1 : 0;
    a.nfast = (pl.splits > 1 && nw > nx) ? 1 : 0;
    a.strip_px = sp.strip_px;
    a.chunk_px = sp.chunk_px;
    a.lds_zero = sp.lds_zero;
    a.lds_patch = sp.lds_patch;
    a.lds_scratch = sp.lds_scratch;
    a.lds_flags = sp.lds_flags;
    a.win_seg = wnp.seg;
    a.win_segs = wnp.segs;
    a.win_sets = wnp.sets;
    a.win_div_g = make_fast_div(std::max(wnp.tiles_m, 1));      // (0 when the plan is not a window one)
    a.win_div_q = make_fast_div(std::max(wnp.tiles_m >> 3, 1));
    a.win_div_q1 = make_fast_div((wnp.tiles_m >> 3) + 1);
    a.win_sh = wnp.sh;
    a.win_wp = wnp.wp;
    a.win_rb = wnp.rb;
    a.res_zero = rsp.zero;
    a.res_scr = (a.vec_out || nchw) ? rsp.scr : -1;   // (the NCHW variant needs only out 16-byte aligned, checked above)
    a.res_flipw = 0;
    a.img_flipw = 0;
    if (flipw) {
        // the resident kernel (the 64 x 64 slice) and the image kernel flip
        // the weights of a square kernel in LDS themselves; elsewhere the
        // caller runs the separate transform instead
        const int kind = pl.tile_id >= 0 ? kTiles[pl.tile_id].kind : -1;
        if (KH != KW || dtype != CONVIMG_BF16)
            return CONVIMG_ERR_UNSUPPORTED;
        if (kind == kResident && IC == 64 && OC == 64)
            a.res_flipw = 1;
        else if (kind == kImage)
            a.img_flipw = 1;
        else
            return CONVIMG_ERR_UNSUPPORTED;
    }
    a.img_set = imp.set;
    a.img_wofs = imp.wofs;
    a.img_ti = imp.ti;
    a.img_ts = imp.ts;
    a.lds_rows = pl.tile_id >= 0 && kTiles[pl.tile_id].kind == kResident ? rsp.lds_rows : wnp.lds_rows;

    if (pl.splits > 1) {
        const int need = pl.tiles_m * pl.tiles_n + 1;
        if (sems == kSemScratch) {
            // the device's static array: cleared here, since every call on
            // this device shares it and a call that timed out leaves it dirty
            if (need > kScratchInts)
                return CONVIMG_ERR_SCRATCH;
            rc = scratch_of(dev, &a.sem);
            if (rc != CONVIMG_OK)
                return rc;
            hipLaunchKernelGGL(fill_zero_i32, dim3((need + 255) / 256), dim3(256), 0, stream, a.sem, need);
            if (hipGetLastError() != hipSuccess)
                return CONVIMG_ERR_LAUNCH;
        } else {
            rc = get_semaphores(dev, stream, need, &a.sem);
            if (rc != CONVIMG_OK)
                return rc;
        }
    }
    if (log_enabled())
        std::fprintf(stderr,
                     "convimg: N=%d H=%d W=%d IC=%d OC=%d K=%dx%d s=%d p=%d d=%d -> "
                     "tile=%d(%dx%dx%d) loader=%d splits=%d grid=%d lds=%d\n",
                     N, H, W, IC, OC, KH, KW, stride, pad, dilation, pl.tile_id, pl.BM, pl.BN,
                     pl.BK, pl.loader, pl.splits, pl.grid, pl.lds_bytes);

    if (dtype == CONVIMG_FP32)
        hipLaunchKernelGGL(pl.BN == kF32BNSmall ? igemm_fwd_f32<kF32BNSmall> : igemm_fwd_f32<kF32BN>,
                           dim3(pl.grid), dim3(kRegsThreads), 0, stream, a);
    else if (kTiles[pl.tile_id].kind == kWindow)
        hipLaunchKernelGGL(kWinKernels[KH], dim3(pl.grid), dim3(pl.threads), (unsigned)pl.lds_bytes,
                           stream, a);
    else if (kTiles[pl.tile_id].kind == kResident && nchw)
        hipLaunchKernelGGL(kResNchwKernels[nchw - 1][res_index(IC)], dim3(pl.grid), dim3(pl.threads),
                           (unsigned)pl.lds_bytes, stream, a);
    else if (kTiles[pl.tile_id].kind == kResident)
        hipLaunchKernelGGL(kResKernels[res_index(IC)], dim3(pl.grid), dim3(pl.threads),
                           (unsigned)pl.lds_bytes, stream, a);
    else if (kTiles[pl.tile_id].kind == kImage)
        hipLaunchKernelGGL(kImgKernels[imp.mb], dim3(pl.grid), dim3(pl.threads), (unsigned)pl.lds_bytes,
                           stream, a);
    else if (kTiles[pl.tile_id].kind == kStrip)
        hipLaunchKernelGGL(kKernels[pl.tile_id][pl.loader], dim3(pl.grid), dim3(pl.threads),
                           (unsigned)pl.lds_bytes, stream, a);
    else
        hipLaunchKernelGGL(kKernels[pl.tile_id][pl.loader], dim3(pl.grid), dim3(pl.threads), 0,
                           stream, a);
    if (hipGetLastError() != hipSuccess)
        return CONVIMG_ERR_LAUNCH;
    return CONVIMG_OK;
}

}  // namespace

extern "C" {

int conv2d_fwd_nchw_workspace(int N, int H, int W, int IC, int OC, int KH, int KW, int stride, int pad,
                              int dilation, int dtype, size_t *bytes)
{
    if (!bytes)
        return CONVIMG_ERR_NULL;
    convimg_plan pl;
    const int rc = make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, 1, true, nullptr, &pl);
    if (rc != CONVIMG_OK)
        return rc;
    *bytes = nchw_layout(pl, N, H, W, IC, OC, dtype).bytes;
    return CONVIMG_OK;
}

int conv2d_fwd_nchw(const void *x, const void *w, const float *bias, int N, int H, int W, int IC, int OC,
                    int KH, int KW, int stride, int pad, int dilation, int dtype, int out_dtype, void *out,
                    void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!x || !w || !out || !ws)
        return CONVIMG_ERR_NULL;
    convimg_plan pl;
    int rc = make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, 1, true, nullptr, &pl);
    if (rc != CONVIMG_OK)
        return rc;
    if (out_dtype != CONVIMG_BF16 && out_dtype != CONVIMG_FP32)
        return CONVIMG_ERR_DTYPE;
    const NchwLayout l = nchw_layout(pl, N, H, W, IC, OC, dtype);
    if (ws_bytes < l.bytes)
        return CONVIMG_ERR_WORKSPACE;
    const size_t esz = dtype == CONVIMG_BF16 ? 2 : 4;
    const size_t nx = (size_t)N * H * W * IC * esz, nw = (size_t)OC * pl.K * esz;
    const size_t no = (size_t)pl.M * OC * (out_dtype == CONVIMG_BF16 ? 2 : 4), nb = bias ? (size_t)OC * 4 : 0;
    if (overlaps(out, no, x, nx) || overlaps(out, no, w, nw) || (bias && overlaps(out, no, bias, nb))
        || overlaps(out, no, ws, l.bytes) || overlaps(ws, l.bytes, x, nx) || overlaps(ws, l.bytes, w, nw)
        || (bias && overlaps(ws, l.bytes, bias, nb)))
        return CONVIMG_ERR_ALIAS;
    const int HW = H * W, OHW = pl.OH * pl.OW, KK = KH * KW;
    auto tiles = [](int v) { return (unsigned)((v + kPermTile - 1) / kPermTile); };
    if (N > 65535 || OC > 65535 || tiles(IC) > 65535u || tiles(OHW) > 65535u)
        return CONVIMG_ERR_RANGE;
    char *wsb = (char *)ws;
    // the resident kernel's NCHW variant where it serves the problem: one
    // launch, no permute (the workspace is not used)
    rc = fwd_call(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, (float *)out, stream,
                  kSemPool, 0, out_dtype == CONVIMG_BF16 ? 2 : 1);
    if (rc != CONVIMG_ERR_UNSUPPORTED)
        return rc;
    const dim3 blk(kPermThreads);
    // x [N][IC][H*W] -> [N][H*W][IC] and w [OC][IC][KH*KW] -> [OC][KH*KW][IC],
    // one launch
    const TransposeJob jx{IC, HW, (int)tiles(HW), (int)tiles(IC)}, jw{IC, KK, (int)tiles(KK), (int)tiles(IC)};
    const long long t1 = (long long)jx.cx * jx.ry * N, t2 = (long long)jw.cx * jw.ry * OC;
    if (t1 + t2 >= 0x7fffffffLL)
        return CONVIMG_ERR_RANGE;
    if (dtype == CONVIMG_BF16)
        hipLaunchKernelGGL(transpose_batched2<unsigned short>, dim3((unsigned)(t1 + t2)), blk, 0, stream,
                           (const unsigned short *)x, (unsigned short *)wsb, jx, (int)t1, (const unsigned short *)w,
                           (unsigned short *)(wsb + l.w_off), jw);
    else
        hipLaunchKernelGGL(transpose_batched2<float>, dim3((unsigned)(t1 + t2)), blk, 0, stream, (const float *)x,
                           (float *)wsb, jx, (int)t1, (const float *)w, (float *)(wsb + l.w_off), jw);
    if (hipGetLastError() != hipSuccess)
        return CONVIMG_ERR_LAUNCH;
    rc = conv2d_fwd(wsb, wsb + l.w_off, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype,
                    (float *)(wsb + l.y_off), stream);
    if (rc != CONVIMG_OK)
        return rc;
    // y [N][OH*OW][OC] -> out [N][OC][OH*OW], in out_dtype
    if (out_dtype == CONVIMG_BF16)
        hipLaunchKernelGGL((transpose_batched<float, unsigned short>), dim3(tiles(OC), tiles(OHW), N), blk, 0,
                           stream, (const float *)(wsb + l.y_off), (unsigned short *)out, OHW, OC);
    else
        hipLaunchKernelGGL((transpose_batched<float, float>), dim3(tiles(OC), tiles(OHW), N), blk, 0, stream,
                           (const float *)(wsb + l.y_off), (float *)out, OHW, OC);
    if (hipGetLastError() != hipSuccess)
        return CONVIMG_ERR_LAUNCH;
    return CONVIMG_OK;
}

int conv2d_fwd_autotune(const void *x, const void *w, const float *bias, int N, int H, int W, int IC, int OC,
                        int KH, int KW, int stride, int pad, int dilation, int dtype, float *out,
                        hipStream_t stream, int *tile_out, int *splits_out, float *us_best, float *us_default)
{
    if (!x || !w || !out)
        return CONVIMG_ERR_NULL;
    convimg_plan pl;
    int rc = make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, 1, true, nullptr, &pl);
    if (rc != CONVIMG_OK)
        return rc;
    int dev = 0;
    DeviceInfo *info = nullptr;
    if (hipGetDevice(&dev) != hipSuccess)
        return CONVIMG_ERR_DEVICE;
    rc = device_info(dev, &info);
    if (rc != CONVIMG_OK)
        return rc;
    const bool aligned = (((uintptr_t)x | (uintptr_t)w) & 15) == 0;
    const TuneKey key = tune_key(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, info->num_cus, aligned);
    {
        // time the static choice, not an earlier tuned one
        std::lock_guard<std::mutex> lock(g_tune_mu);
        if (g_tuned.erase(key))
            g_tuned_count.fetch_sub(1);
    }
    // candidates: what the planner makes of each forced tile (it falls back
    // where a tile cannot serve the problem), with its split-K factor, half
    // of it and none; the static choice first
    std::vector<std::pair<int, int>> cand;
    auto add = [&](int t, int sp) {
        for (auto &c : cand)
            if (c.first == t && c.second == sp)
                return;
        cand.emplace_back(t, sp);
    };
    rc = make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, info->num_cus, aligned, info->occ, &pl);
    if (rc != CONVIMG_OK)
        return rc;
    add(pl.tile_id, pl.splits);
    if (dtype == CONVIMG_BF16) {
        for (int t = 0; t < kNumTiles; ++t) {
            convimg_plan c;
            t_try_tile = t;
            t_try_splits = -1;
            rc = make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, info->num_cus, aligned,
                           info->occ, &c);
            t_try_tile = -1;
            if (rc != CONVIMG_OK)
                continue;
            add(c.tile_id, c.splits);
            if (c.splits > 1) {
                add(c.tile_id, c.splits / 2);
                add(c.tile_id, 1);
            }
        }
    }
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess)
        return CONVIMG_ERR_DEVICE;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return CONVIMG_ERR_DEVICE;
    }
    constexpr int kWarm = 2, kReps = 5;
    float best = 0.f, first = 0.f;
    int best_i = -1;
    rc = CONVIMG_OK;
    for (size_t i = 0; i < cand.size() && rc == CONVIMG_OK; ++i) {
        t_try_tile = cand[i].first;
        t_try_splits = cand[i].second;
        for (int r = 0; r < kWarm && rc == CONVIMG_OK; ++r)
            rc = conv2d_fwd(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out, stream);
        if (rc == CONVIMG_OK && hipEventRecord(e0, stream) != hipSuccess)
            rc = CONVIMG_ERR_DEVICE;
        for (int r = 0; r < kReps && rc == CONVIMG_OK; ++r)
            rc = conv2d_fwd(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out, stream);
        float ms = 0.f;
        if (rc == CONVIMG_OK && (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess
                                 || hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
            rc = CONVIMG_ERR_DEVICE;
        t_try_tile = t_try_splits = -1;
        if (rc != CONVIMG_OK)
            break;
        const float us = ms * 1000.f / kReps;
        if (i == 0)
            first = us;
        if (best_i < 0 || us < best) {
            best = us;
            best_i = (int)i;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (rc != CONVIMG_OK)
        return rc;
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        if (g_tuned.emplace(key, cand[best_i]).second)
            g_tuned_count.fetch_add(1);
    }
    // leave the tuned plan's result in out
    rc = conv2d_fwd(x, w, bias, N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, out, stream);
    if (rc != CONVIMG_OK)
        return rc;
    if (tile_out)
        *tile_out = cand[best_i].first;
    if (splits_out)
        *splits_out = cand[best_i].second;
    if (us_best)
        *us_best = best;
    if (us_default)
        *us_default = first;
    return CONVIMG_OK;
}

void conv2d_fwd_autotune_clear(void)
{
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tuned.clear();
    g_tuned_count.store(0);
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

int conv2d_bwd_data_weights(const void *w, int OC, int KH, int KW, int IC, int dtype, void *wt,
                            hipStream_t stream)
{
    dim3 grid;
    const int rc = flip_args(w, OC, KH, KW, IC, dtype, wt, &grid);
    if (rc != CONVIMG_OK)
        return rc;
    const size_t esz = dtype == CONVIMG_BF16 ? 2 : 4;
    const int vlen = (int)(16 / esz);
    const int vec_in = (IC % vlen == 0 && ((uintptr_t)w & 15) == 0) ? 1 : 0;
    const int vec_out = (OC % vlen == 0 && ((uintptr_t)wt & 15) == 0) ? 1 : 0;
    if (dtype == CONVIMG_BF16)
        hipLaunchKernelGGL(flip_transpose<unsigned short>, grid, dim3(kFlipThreads), 0, stream,
                           (const unsigned short *)w, (unsigned short *)wt, OC, KH * KW, IC,
                           vec_in, vec_out);
    else
        hipLaunchKernelGGL(flip_transpose<unsigned>, grid, dim3(kFlipThreads), 0, stream,
                           (const unsigned *)w, (unsigned *)wt, OC, KH * KW, IC, vec_in, vec_out);
    if (hipGetLastError() != hipSuccess)
        return CONVIMG_ERR_LAUNCH;
    return CONVIMG_OK;
}

int conv2d_bwd_data(const void *dy, const void *w, int N, int H, int W, int IC, int OC, int KH, int KW,
                    int stride, int pad, int dilation, int dtype, void *wt, float *dx, hipStream_t stream)
{
    if (!dy || !w || !wt || !dx)
        return CONVIMG_ERR_NULL;
    // the forward problem this maps to: first every check conv2d_fwd makes
    // on the shapes (the output extent OH x OW of dy included)
    convimg_plan fwd;
    int rc = make_plan(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, 1, true, nullptr, &fwd);
    if (rc != CONVIMG_OK)
        return rc;
    if (stride != 1 || KH != KW || pad > dilation * (KH - 1)) {
        // the fallback route: the gradient from its definition, any stride,
        // kernel shape and padding (wt unused), by phases of the stride or
        // element by element
        const size_t esz = dtype == CONVIMG_BF16 ? 2 : 4;
        const size_t nw = (size_t)OC * KH * KW * IC * esz;
        const size_t ny = (size_t)fwd.M * OC * esz;
        const size_t nx = (size_t)N * H * W * IC * 4;
        if (overlaps(dx, nx, w, nw) || overlaps(dx, nx, dy, ny))
            return CONVIMG_ERR_ALIAS;
        const size_t lim = 0x7fffffff;
        const long long M = (long long)N * H * W;
        const long long tiles = (long long)ceil_div(M, 64) * ceil_div(IC, 64);
        if (nw >= lim || ny >= lim || nx >= lim || tiles >= (long long)lim)
            return CONVIMG_ERR_RANGE;
        int dev = 0;
        DeviceInfo *info = nullptr;
        rc = current_device(&dev, &info);
        if (rc != CONVIMG_OK)
            return rc;
        if (dtype == CONVIMG_BF16 && OC % 8 == 0 && ((uintptr_t)dy & 15) == 0) {
            // bf16 with 16-byte runs of dy: the kernel by phases (only the
            // taps that reach each phase of the stride)
            int gsd = stride, r = dilation;
            while (r != 0) {
                const int t = gsd % r;
                gsd = r;
                r = t;
            }
            DgPhArgs q;
            q.dy = dy;
            q.w = w;
            q.dx = dx;
            q.N = N;
            q.H = H;
            q.W = W;
            q.IC = IC;
            q.OC = OC;
            q.KH = KH;
            q.KW = KW;
            q.s = stride;
            q.p = pad;
            q.d = dilation;
            q.OH = fwd.OH;
            q.OW = fwd.OW;
            q.dk = stride / gsd;
            q.dq = dilation / gsd;
            q.Hp = ceil_div(H, stride);
            q.Wp = ceil_div(W, stride);
            const long long Mp = (long long)N * q.Hp * q.Wp;
            const long long tiles_p = ceil_div(Mp, 64);
            const long long tiles_m = (long long)stride * stride * tiles_p;
            const long long grid = tiles_m * ceil_div(IC, 64);
            if (grid >= (long long)lim || tiles_p * 64 >= (long long)lim)   // (pixel indices of a phase fit an int)
                return CONVIMG_ERR_RANGE;
            q.Mp = (int)Mp;
            q.tiles_p = (int)tiles_p;
            q.tiles_m = (int)tiles_m;
            q.ob = ceil_div(OC, 64);
            q.dy_bytes = (unsigned)ny;
            q.w_bytes = (unsigned)nw;
            q.dx_bytes = (unsigned)nx;
            q.div_tp = make_fast_div(q.tiles_p);
            q.div_hwp = make_fast_div(q.Hp * q.Wp);
            q.div_wp = make_fast_div(q.Wp);
            q.div_s = make_fast_div(stride);
            if (IC % 8 == 0 && ((uintptr_t)w & 15) == 0)
                hipLaunchKernelGGL(igemm_dgrad_phase_bf16<true>, dim3((unsigned)grid), dim3(256), 0, stream, q);
            else
                hipLaunchKernelGGL(igemm_dgrad_phase_bf16<false>, dim3((unsigned)grid), dim3(256), 0, stream, q);
            return hipGetLastError() == hipSuccess ? CONVIMG_OK : CONVIMG_ERR_LAUNCH;
        }
        DgArgs g;
        g.dy = dy;
        g.w = w;
        g.dx = dx;
        g.N = N;
        g.H = H;
        g.W = W;
        g.IC = IC;
        g.OC = OC;
        g.KH = KH;
        g.KW = KW;
        g.s = stride;
        g.p = pad;
        g.d = dilation;
        g.OH = fwd.OH;
        g.OW = fwd.OW;
        g.M = (int)M;
        g.K = KH * KW * OC;
        g.tiles_m = ceil_div(M, 64);
        g.dy_bytes = (unsigned)ny;
        g.w_bytes = (unsigned)nw;
        g.dx_bytes = (unsigned)nx;
        g.div_oc = make_fast_div(OC);
        g.div_kw = make_fast_div(KW);
        g.div_hw = make_fast_div(H * W);
        g.div_w = make_fast_div(W);
        if (dtype == CONVIMG_BF16)
            hipLaunchKernelGGL(igemm_dgrad_any<true>, dim3((unsigned)tiles), dim3(256), 0, stream, g);
        else
            hipLaunchKernelGGL(igemm_dgrad_any<false>, dim3((unsigned)tiles), dim3(256), 0, stream, g);
        return hipGetLastError() == hipSuccess ? CONVIMG_OK : CONVIMG_ERR_LAUNCH;
    }
    const int pt = dilation * (KH - 1) - pad;
    convimg_plan pl;
    rc = make_plan(N, fwd.OH, fwd.OW, OC, IC, KH, KW, 1, pt, dilation, dtype, 1, true, nullptr, &pl);
    if (rc != CONVIMG_OK)
        return rc;
    if (pl.OH != H || pl.OW != W)      // (cannot happen for stride 1)
        return CONVIMG_ERR_SHAPE;
    const size_t esz = dtype == CONVIMG_BF16 ? 2 : 4;
    const size_t nw = (size_t)OC * KH * KW * IC * esz;
    const size_t ny = (size_t)N * fwd.OH * fwd.OW * OC * esz;
    const size_t nx = (size_t)N * H * W * IC * 4;
    if (overlaps(wt, nw, dy, ny) || overlaps(dx, nx, w, nw) || overlaps(dx, nx, dy, ny)
        || overlaps(dx, nx, wt, nw))
        return CONVIMG_ERR_ALIAS;
    // the transform's own argument errors first (before any device work,
    // whichever path runs)
    {
        dim3 grid;
        rc = flip_args(w, OC, KH, KW, IC, dtype, wt, &grid);
        if (rc != CONVIMG_OK)
            return rc;
    }
    // where the mapped problem runs on the resident kernel (64 -> 64
    // channels) or the image kernel, the kernel flips and transposes the
    // forward weights in LDS (one launch, wt untouched); else the transform
    // into wt, then the forward on the mapped problem
    if (dtype == CONVIMG_BF16) {
        rc = fwd_call(dy, w, nullptr, N, fwd.OH, fwd.OW, OC, IC, KH, KW, 1, pt, dilation, dtype, dx, stream,
                      kSemPool, 1);
        if (rc != CONVIMG_ERR_UNSUPPORTED)
            return rc;
    }
    rc = conv2d_bwd_data_weights(w, OC, KH, KW, IC, dtype, wt, stream);
    if (rc != CONVIMG_OK)
        return rc;
    return conv2d_fwd(dy, wt, nullptr, N, fwd.OH, fwd.OW, OC, IC, KH, KW, 1, pt, dilation, dtype, dx, stream);
}

int conv2d_bwd_weight_workspace(int N, int H, int W, int IC, int OC, int KH, int KW, int stride, int pad,
                                int dilation, int dtype, size_t *bytes)
{
    if (!bytes)
        return CONVIMG_ERR_NULL;
    WgPlan wp;
    int rc = plan_wgrad(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, 1, &wp);
    if (rc != CONVIMG_OK)
        return rc;
    int dev = 0;
    DeviceInfo *info = nullptr;
    if (hipGetDevice(&dev) != hipSuccess)
        return CONVIMG_ERR_DEVICE;
    rc = device_info(dev, &info);
    if (rc != CONVIMG_OK)
        return rc;
    rc = plan_wgrad(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, info->num_cus, &wp);
    if (rc != CONVIMG_OK)
        return rc;
    *bytes = wp.ws_bytes;
    return CONVIMG_OK;
}

int conv2d_bwd_weight(const void *x, const void *dy, int N, int H, int W, int IC, int OC, int KH, int KW,
                      int stride, int pad, int dilation, int dtype, float *dw, void *ws, size_t ws_bytes,
                      hipStream_t stream)
{
    if (!x || !dy || !dw)
        return CONVIMG_ERR_NULL;
    // argument errors first: they need no device
    WgPlan wp;
    int rc = plan_wgrad(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, 1, &wp);
    if (rc != CONVIMG_OK)
        return rc;
    const size_t esz = dtype == CONVIMG_FP32 ? 4 : 2;
    const size_t nx = (size_t)N * H * W * IC * esz;
    const size_t ny = (size_t)wp.M * OC * esz;
    const size_t nw = (size_t)OC * wp.KKIC * 4;
    if (overlaps(dw, nw, x, nx) || overlaps(dw, nw, dy, ny))
        return CONVIMG_ERR_ALIAS;
    int dev = 0;
    DeviceInfo *info = nullptr;
    if (hipGetDevice(&dev) != hipSuccess)
        return CONVIMG_ERR_DEVICE;
    rc = device_info(dev, &info);
    if (rc != CONVIMG_OK)
        return rc;
    rc = plan_wgrad(N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype, info->num_cus, &wp);
    if (rc != CONVIMG_OK)
        return rc;
    if (wp.ws_bytes > 0) {
        if (!ws)
            return CONVIMG_ERR_NULL;
        if (ws_bytes < wp.ws_bytes)
            return CONVIMG_ERR_WORKSPACE;
        if (overlaps(ws, wp.ws_bytes, x, nx) || overlaps(ws, wp.ws_bytes, dy, ny)
            || overlaps(ws, wp.ws_bytes, dw, nw))
            return CONVIMG_ERR_ALIAS;
    }
    const bool vx = IC % 8 == 0 && ((uintptr_t)x & 15) == 0;
    const bool vdy = OC % 8 == 0 && ((uintptr_t)dy & 15) == 0;
    // the row-window kernel, else the transpose-read kernel, where the shape
    // and the alignment allow (the workspace fits either plan)
    const bool row = wp.row && vx && vdy;
    const int tiles_n = row ? wp.row_tiles_n : wp.tiles_n;
    const int splits = row ? wp.row_splits : wp.splits;
    const int inplace = row ? wp.row_inplace : wp.inplace;
    WgArgs a;
    a.x = (const unsigned short *)x;
    a.dy = (const unsigned short *)dy;
    a.dst = (splits > 1 && !inplace) ? (float *)ws : dw;
    a.inplace = inplace;
    a.sem = nullptr;
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    if (inplace) {
        rc = get_semaphores(dev, stream, wp.tiles_m * tiles_n + 1, &a.sem);
        if (rc != CONVIMG_OK)
            return rc;
    }
    a.N = N;
    a.H = H;
    a.W = W;
    a.IC = IC;
    a.OC = OC;
    a.KH = KH;
    a.KW = KW;
    a.s = stride;
    a.p = pad;
    a.d = dilation;
    a.OH = wp.OH;
    a.OW = wp.OW;
    a.M = wp.M;
    a.KKIC = wp.KKIC;
    a.tiles_m = wp.tiles_m;
    a.tiles_n = tiles_n;
    a.splits = splits;
    a.chunk = row ? wp.row_chunk : wp.chunk;
    a.bpr = wp.bpr;
    a.groups = wp.groups;
    a.div_bpr = make_fast_div(wp.bpr);
    a.div_oh = make_fast_div(wp.OH);
    a.div_s = make_fast_div(stride);
    a.div_ic = make_fast_div(IC);
    a.div_kw = make_fast_div(KW);
    a.x_bytes = (unsigned)nx;
    a.dy_bytes = (unsigned)ny;
    a.rl = wp.row_rl;
    a.rsp = wp.row_rsp;
    a.rr = wp.row_rr;
    a.rnseg = wp.row_nseg;
    a.rsteps = wp.row_steps;
    a.nicb = IC / 64;
    a.NR = N * wp.OH;
    a.div_rnseg = make_fast_div(wp.row_nseg);
    const int grid = wp.tiles_m * tiles_n * splits;
    const hipError_t le = dtype == CONVIMG_FP32 ? wgrad_f32_launch(a, grid, stream)
                        : row ? wgrad_row_launch(a, grid, wp.row_xi, wp.row_stages, stream)
                        : (wgrad_tr_shape(IC, OC) && vx && vdy) ? wgrad_tr_launch(a, grid, wp.tr_stages, stream)
                                                                : wgrad_launch(a, vx, vdy, grid, stream);
    if (le != hipSuccess)
        return CONVIMG_ERR_LAUNCH;
    if (splits > 1 && !inplace) {
        const int n = OC * wp.KKIC;
        const int vec = (n % 4 == 0 && ((uintptr_t)ws & 15) == 0 && ((uintptr_t)dw & 15) == 0) ? 1 : 0;
        if (wgrad_reduce_launch((const float *)ws, dw, n, splits, vec, wgrad_reduce_log2_groups(splits), stream)
            != hipSuccess)
            return CONVIMG_ERR_LAUNCH;
    }
    return CONVIMG_OK;
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
    case CONVIMG_ERR_UNSUPPORTED:
        return "unsupported by the backward passes (data: stride 1, KH == KW, pad <= dilation*(KH-1); "
               "weights: bf16 storage)";
    case CONVIMG_ERR_WORKSPACE: return "workspace smaller than conv2d_bwd_weight_workspace reports";
    case CONVIMG_ERR_SCRATCH:
        return "conv2d_fwd_noalloc: the plan needs more split-K semaphores than its fixed scratch holds";
    default: return "unknown status";
    }
}

}  // extern "C"
