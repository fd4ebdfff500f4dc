// igemm_wgrad.hpp -- weight backward (gradient with respect to w) as an
// implicit GEMM.
//
// burn-cubecl "kernel/conv/base.rs" listing, conv_weight_backward: the
// implicit-GEMM route serves every groups = 1 problem.  The gradient is
//
//   dw[oc][kh][kw][ic] = sum_{n,oh,ow} dy[n][oh][ow][oc] * X(n, oh*s-p+kh*d, ow*s-p+kw*d, ic)
//
// a GEMM with M = OC (rows, from dy), N = KH*KW*IC (columns j = t*IC + ic
// with tap t = kh*KW + kw, from the im2col gather of x) and the reduction
// over the N*OH*OW output pixels.  Both operands lie pixel-major in memory
// (channels contiguous), while the MFMA wants 8 consecutive reduction
// values per lane: each loader thread reads an 8-pixel x 8-channel block
// with 16-byte loads, transposes it in registers and writes one 16-byte
// LDS record per channel, so the LDS holds channel rows of 64 pixels.
//
// The pixels are walked in groups of 8 consecutive pixels of one output
// row (a row of OW pixels is ceil(OW/8) groups, the last one masked), so a
// group needs one row decode and its 8 gathers are one base offset plus a
// constant stride.
//
// Workgroup: 256 threads, a 64 (oc) x 192 (j) tile, 8 groups (64 pixel
// slots) per step, two LDS stages (the next step's loads are in flight
// while the current one runs on the MFMAs), one barrier per step.  Wave w
// computes all 64 rows x columns [48w, 48w+48) with 16x16x32 bf16 MFMAs.
// The groups are split into `splits` contiguous ranges.  With one range
// the tile goes straight to dw; with at most kWgInplaceMax ranges they take
// turns on a per-tile semaphore and add into dw in range order (the
// forward's serial split-K, so the sum has a fixed order); with more, each
// range's partial tile goes to a workspace and a second kernel sums the
// ranges in order.  Either way every call gives the same bits.
#pragma once

#include <type_traits>

namespace convimg {

constexpr int kWgBM = 64;           // output channels per tile
constexpr int kWgBN = 192;          // (tap, input channel) columns per tile
constexpr int kWgBK = 64;           // pixels per step
constexpr int kWgThreads = 256;
constexpr int kWgRows = kWgBM + kWgBN;           // LDS rows per stage (A rows, then B rows)
// one row: 64 pixels of one channel, padded by one 16-byte record (measured)
constexpr int kWgRowBytes = kWgBK * 2 + 16;
constexpr int kWgStageBytes = kWgRows * kWgRowBytes;
constexpr int kWgLdsBytes = 2 * kWgStageBytes;
constexpr int kWgReduceThreads = 256;
constexpr int kWgRedMaxGroups = 32;                     // range groups per column, at most
constexpr int kWgRedBatch = 8;                          // loads a thread issues before adding
#ifndef CONVIMG_WG_RED_LOADS
#define CONVIMG_WG_RED_LOADS 5
#endif
constexpr int kWgRedLoads = CONVIMG_WG_RED_LOADS;       // ranges a reduce thread loads, at most

// Range groups for the reduce over `splits` ranges, as log2: the fewest (a
// power of two, at most kWgRedMaxGroups) that leave each thread at most
// kWgRedLoads ranges to load.  Measured: groups of about five ranges beat
// both longer groups (fewer workgroups, each thread's loads in more
// rounds) and shorter ones (more workgroups than are resident at once).
inline int wgrad_reduce_log2_groups(int splits)
{
    int lg = 0;
    while ((1 << lg) < kWgRedMaxGroups && (splits + (1 << lg) - 1) >> lg > kWgRedLoads)
        ++lg;
    return lg;
}
#ifndef CONVIMG_WG_PF
#define CONVIMG_WG_PF 1
#endif
constexpr int kWgPF = CONVIMG_WG_PF;    // steps of loads in flight (measured)

struct WgArgs {
    const unsigned short *x;     // [N][H][W][IC] bf16 (fp32 for the fp32-storage kernel)
    const unsigned short *dy;    // [N][OH][OW][OC] bf16 (likewise)
    float *dst;                  // dw [OC][KKIC], or partial sums [splits][OC][KKIC]
    int *sem;                    // in place: one int per tile, then a status word
    int spin_limit;              // in place: polls before a range gives up its turn
    int inplace;                 // 1: the ranges add into dw in turn (dst = dw)
    int N, H, W, IC, OC, KH, KW, s, p, d, OH, OW;
    int M, KKIC;                 // pixels N*OH*OW; columns KH*KW*IC
    int bpr, groups;             // 8-pixel groups per output row; N*OH*bpr
    int tiles_m, tiles_n, splits, chunk;   // chunk: groups per split, a multiple of 8
    unsigned x_bytes, dy_bytes;            // both below 2^31
    FastDiv div_bpr, div_oh, div_s, div_ic, div_kw;
    // row-window kernel only: a step is rr units of rl output pixels (whole
    // rows when rnseg == 1, else one of a row's rnseg equal segments), a
    // unit's x span rsp = rl + 2d input pixels; rsteps steps in all (chunk
    // is then steps per range); nicb = IC / 64; NR = N * OH output rows
    int rl, rsp, rr, rnseg, rsteps, nicb, NR;
    FastDiv div_rnseg;
};

// The transpose-read kernel (below) serves IC % 64 == 0 and OC % 8 == 0
// with 16-byte aligned x and dy.  Its LDS ring holds kWtStagesDeep stages
// of 32 KB (one workgroup per CU) or kWtStagesPair (two per CU).
constexpr int kWtStagesDeep = 4;
constexpr int kWtStagesPair = 2;

inline bool wgrad_tr_shape(int IC, int OC)
{
    return IC % 64 == 0 && OC % 8 == 0;
}

// The row-window kernel (below): stride 1, KW == 3, IC % 64 == 0,
// OC % 8 == 0, 16-byte aligned x and dy.  Eight waves; a stage holds 128 dy
// slots and 8 XI x rows (XI = 16 or 24), in three or four stages.
constexpr int kWrThreads = 512;
constexpr int kWrSlots = 128;

inline bool wgrad_row_shape(int IC, int OC, int KW, int s)
{
    return IC % 64 == 0 && OC % 8 == 0 && KW == 3 && s == 1;
}

// Most pixel ranges that add into dw in turn (more go through a workspace:
// each turn waits for the previous range's stores).
constexpr int kWgInplaceMax = 4;

// The fp32-storage kernel (below): 64 x 64 tiles, LDS rows of 80 floats
// (a pixel slot's 64 values and 16 floats of padding: the four slots an
// MFMA operand read spans fall on four disjoint bank quarters), at most
// kWgF32MaxSteps steps (64 pixel slots each) a range.
constexpr int kWgF32BN = 64;
constexpr int kWgF32Row = 80;
constexpr int kWgF32MaxSteps = 128;

// The kernels are compiled in conv2d_wgrad.hip only; other units see the
// argument block and the launchers.
#ifdef CONVIMG_WGRAD_KERNELS

// LDS byte offset of 16-byte record `chunk` (8 pixels) of row `row`: rows
// of 9 records (one of padding) and the chunk XORed with bits 3..5 of the
// row.  One pass of the transposed writes (16 lanes: 8 chunks x 2 rows 8
// apart) then falls on 16 distinct bank groups; the 16 consecutive rows of
// an MFMA operand read on 9 (one 2-way conflict).
__device__ __forceinline__ int wg_rec(int row, int chunk)
{
    return row * kWgRowBytes + ((chunk ^ ((row >> 3) & 7)) << 4);
}

// A wave's results: acc[i][j] (i < NI, j < NJ) is the 16x16 block at rows
// oc0 + 16 i, columns jc[j] .. jc[j] + 15 of dw; lane l holds rows 4 (l >> 4) .. +3 of
// column jc[j] + (l & 15).  Without `inplace`, range `split` writes its
// partial tile (dst + split * OC * KKIC).  In place, the range waits until
// the tile's semaphore equals `split` (every wave's first lane polls, with a
// bound: a wave that gives up sets the status word after the semaphores and
// writes NaN over its part), then range 0 stores and later ranges add to
// what is there, with agent-coherent (sc1) loads and stores, which reach the
// other XCDs' workgroups; after its stores are acknowledged and the
// workgroup has met, thread 0 passes the turn on (the last range resets it
// to 0).  Every thread of the workgroup calls this (it holds barriers).
template <int NI, int NJ>
__device__ __forceinline__ void wg_store(const WgArgs &a, const floatx4_t (&acc)[NI][NJ], int oc0,
                                         const int (&jc)[NJ], int split, int tile)
{
    const int lane = threadIdx.x & 63;
    if (!a.inplace) {
        // One range: dw itself, with streaming stores (the forward's output
        // policy; with the default one the tile stays dirty in the XCD's L2
        // until the kernel ends and is written back then: 512-channel layer
        // -2 %).  Partial tiles keep the default policy, which the reduce
        // that reads them measured slightly faster with.  dw is below 2 GiB
        // (the plan checks).
        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
            a.dst + (size_t)split * a.OC * a.KKIC, 0, (unsigned)((size_t)a.OC * a.KKIC * 4), kRsrcWord3);
        auto store = [&](auto aux) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int jj = jc[j] + (lane & 15);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int oc = oc0 + 16 * i + 4 * (lane >> 4) + v;
                        const unsigned off = (oc < a.OC && jj < a.KKIC) ? 4u * (unsigned)(oc * a.KKIC + jj)
                                                                        : kOutOfRange;
                        __builtin_amdgcn_raw_buffer_store_b32(f32_bits(acc[i][j][v]), rd, off, 0,
                                                              decltype(aux)::value);
                    }
                }
            }
        };
        if (a.splits == 1)
            store(std::integral_constant<int, kOutAux>{});
        else
            store(std::integral_constant<int, 0>{});
        return;
    }
    int *sem = a.sem + tile;
    int late = 0;
    if (lane == 0) {
        int spins = 0;
        while (__hip_atomic_load(sem, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != split) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins >= a.spin_limit) {
                __hip_atomic_store(a.sem + a.tiles_m * a.tiles_n, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                late = 1;
                break;
            }
        }
    }
    late = __builtin_amdgcn_readfirstlane(late);
    // dw is below 2 GiB (the plan checks), so every offset and the
    // out-of-range offset of masked lanes fit the buffer resource
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        a.dst, 0, (unsigned)((size_t)a.OC * a.KKIC * 4), kRsrcWord3);
    auto offset = [&](int i, int j, int v) {
        const int jj = jc[j] + (lane & 15), oc = oc0 + 16 * i + 4 * (lane >> 4) + v;
        return (oc < a.OC && jj < a.KKIC) ? 4u * (unsigned)(oc * a.KKIC + jj) : kOutOfRange;
    };
    if (late) {
#pragma unroll 1
        for (int q = 0; q < NI * NJ * 4; ++q)
            __builtin_amdgcn_raw_buffer_store_b32(0x7fc00000u, rd, offset(q / (4 * NJ), (q / 4) % NJ, q % 4), 0,
                                                  kCoherent);
        __syncthreads();
        return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        // one block row at a time: its loads go out as one batch
        float prev[NJ][4];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                prev[j][v] = split == 0 ? 0.f
                    : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, offset(i, j, v), 0, kCoherent));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                __builtin_amdgcn_raw_buffer_store_b32(f32_bits(prev[j][v] + acc[i][j][v]), rd, offset(i, j, v), 0,
                                                      kCoherent);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this thread's stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(sem, (split + 1 == a.splits) ? 0 : split + 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// VX: IC % 8 == 0 and x 16-byte aligned (16-byte gathers of x), else
// element-wise.  VDY: OC % 8 == 0 and dy 16-byte aligned, likewise.  PF:
// steps whose loads are in flight while a step runs on the MFMAs (1 or 2).
// Every load is a buffer load whose masked lanes take an offset past the
// buffer's end and read zeros, so the loads issue back to back, unbranched.
template <bool VX, bool VDY, int PF>
__global__ __launch_bounds__(kWgThreads) void igemm_wgrad_bf16(WgArgs a)
{
    extern __shared__ __align__(16) unsigned char wg_lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // uniform: the roles below are per wave
    const int tiles = a.tiles_m * a.tiles_n;
    // ranges of one tile column share their dy rows and x windows: keep the
    // workgroups of one range together on one XCD
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int split = bid / tiles, tile = bid - split * tiles;
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int oc0 = tm * kWgBM, j0 = tn * kWgBN;
    const int g_begin = split * a.chunk;
    const int g_end = min(a.groups, g_begin + a.chunk);
    const int steps = (g_end - g_begin + 7) / 8;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc((void *)a.dy, 0, a.dy_bytes, kRsrcWord3);

    // loader role: waves 0..2 gather 8 columns of x per thread, wave 3 8 rows of dy
    const bool is_b = wave < 3;
    const int li = is_b ? tid : tid - 192;
    // neighbouring lanes take neighbouring 8-channel groups of one pixel
    // group, so each gather instruction reads whole cache lines with 8
    // consecutive lanes each (measured 6-16 % faster than neighbouring
    // lanes taking neighbouring pixel groups)
    const int grp = (li & ~63) / 8 + (li & 7);              // 8-channel group of the tile
    const int pg = (li & 63) >> 3;                          // pixel group of the step
    const int row0 = is_b ? kWgBM + grp * 8 : grp * 8;    // first LDS row written

    // fixed per thread: the columns (tap, channel) or rows (oc) it loads
    const int col = j0 + grp * 8;                 // first column (B) of the group
    const int orow = oc0 + grp * 8;               // first output channel (A) of the group
    int dh[VX ? 1 : 8], dwc[VX ? 1 : 8], icc[VX ? 1 : 8];
    bool colok[VX ? 1 : 8];
    if (is_b) {
#pragma unroll
        for (int c = 0; c < (VX ? 1 : 8); ++c) {
            const int j = col + c;
            colok[c] = j < a.KKIC;
            const int jj = colok[c] ? j : 0;
            const int t = fast_div(jj, a.div_ic);
            const int kh = fast_div(t, a.div_kw);
            icc[c] = jj - t * a.IC;
            dh[c] = kh * a.d - a.p;
            dwc[c] = (t - kh * a.KW) * a.d - a.p;
        }
    }
    const unsigned sic = (unsigned)(a.s * a.IC);  // x elements between consecutive pixels of a row

    // bit e set: pixel e of the group reads input column iw0 + e*s inside
    // [0, W) and is an output pixel (ow0 + e < OW)
    auto col_mask = [&](int iw0, int valid_px) {
        int lo = 0;
        if (iw0 < 0)
            lo = fast_div(-iw0 + a.s - 1, a.div_s);
        int hi = a.W - iw0 > 0 ? fast_div(a.W - iw0 + a.s - 1, a.div_s) : 0;
        hi = min(hi, valid_px);
        return hi > lo ? (int)((0xffu >> (8 - hi)) & (0xffu << lo)) : 0;
    };

    auto load = [&](int st, u32x4_t (&v)[8]) {
        const int g = g_begin + st * 8 + pg;
        const bool gok = g < g_end;
        const int gg = gok ? g : g_begin;
        const int r = fast_div(gg, a.div_bpr);            // output row n*OH + oh
        const int ow0 = (gg - r * a.bpr) * 8;
        const int valid_px = gok ? min(8, a.OW - ow0) : 0;
        if (VX && VDY) {
            // both roles: 8 16-byte loads at base + e*stride; the role only
            // picks base, stride, mask and buffer (all wave-uniform choices
            // but the values), so the loads sit in one straight line
            unsigned base, stride;
            int mask;
            if (is_b) {
                const int n = fast_div(r, a.div_oh);
                const int oh = r - n * a.OH;
                const int ih = oh * a.s + dh[0], iw0 = ow0 * a.s + dwc[0];
                const bool rowok = colok[0] && ih >= 0 && ih < a.H;
                mask = rowok ? col_mask(iw0, valid_px) : 0;
                base = 2u * ((unsigned)((n * a.H + ih) * a.W + iw0) * a.IC + icc[0]);
                stride = 2u * sic;
            } else {
                mask = orow < a.OC ? (int)(0xffu >> (8 - valid_px)) : 0;
                base = 2u * ((unsigned)(r * a.OW + ow0) * a.OC + orow);
                stride = 2u * (unsigned)a.OC;
            }
            const __amdgpu_buffer_rsrc_t rs = is_b ? rx : rdy;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((mask >> e) & 1) ? base + stride * e : kOutOfRange,
                                                             0, 0);
        } else if (is_b) {
            const int n = fast_div(r, a.div_oh);
            const int oh = r - n * a.OH;
            if (VX) {
                const int ih = oh * a.s + dh[0], iw0 = ow0 * a.s + dwc[0];
                const bool rowok = colok[0] && ih >= 0 && ih < a.H;
                const int mask = rowok ? col_mask(iw0, valid_px) : 0;
                const unsigned base = 2u * ((unsigned)((n * a.H + ih) * a.W + iw0) * a.IC + icc[0]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned off = ((mask >> e) & 1) ? base + 2u * sic * e : kOutOfRange;
                    v[e] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int ih = oh * a.s + dh[c], iw0 = ow0 * a.s + dwc[c];
                    const bool rowok = colok[c] && ih >= 0 && ih < a.H;
                    const int mask = rowok ? col_mask(iw0, valid_px) : 0;
                    const unsigned base = 2u * ((unsigned)((n * a.H + ih) * a.W + iw0) * a.IC + icc[c]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const unsigned off = ((mask >> e) & 1) ? base + 2u * sic * e : kOutOfRange;
                        const unsigned h = __builtin_amdgcn_raw_buffer_load_b16(rx, off, 0, 0);
                        v[e][c >> 1] |= h << ((c & 1) * 16);
                    }
                }
            }
        } else {
            const unsigned base = (unsigned)(r * a.OW + ow0) * a.OC + orow;
            const int mask = orow < a.OC ? (int)(0xffu >> (8 - valid_px)) : 0;
            if (VDY) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned off = ((mask >> e) & 1) ? 2u * (base + (unsigned)a.OC * e) : kOutOfRange;
                    v[e] = __builtin_amdgcn_raw_buffer_load_b128(rdy, off, 0, 0);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    u32x4_t val = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const bool ok = ((mask >> e) & 1) && orow + c < a.OC;
                        const unsigned off = ok ? 2u * (base + (unsigned)a.OC * e + c) : kOutOfRange;
                        const unsigned h = __builtin_amdgcn_raw_buffer_load_b16(rdy, off, 0, 0);
                        val[c >> 1] |= h << ((c & 1) * 16);
                    }
                    v[e] = val;
                }
            }
        }
    };
    auto store = [&](int stage, const u32x4_t (&v)[8]) {
        u32x4_t t[8];
        transpose8x8(v, t);
        unsigned char *base = wg_lds + stage * kWgStageBytes;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            *(u32x4_t *)(base + wg_rec(row0 + c, pg)) = t[c];
    };

    floatx4_t acc[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const int lrow = lane & 15, lchk = lane >> 4;
    auto compute = [&](int stage) {
        const unsigned char *base = wg_lds + stage * kWgStageBytes;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int ch = kb * 4 + lchk;
            bf16x8_t fa[4], fb[3];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = *(const bf16x8_t *)(base + wg_rec(i * 16 + lrow, ch));
#pragma unroll
            for (int j = 0; j < 3; ++j)
                fb[j] = *(const bf16x8_t *)(base + wg_rec(kWgBM + wave * 48 + j * 16 + lrow, ch));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };

    // Register slot q holds the loads of the steps congruent to q mod PF:
    // steps st+1 .. st+PF are in flight while step st runs on the MFMAs.
    // The barriers wait for the LDS writes only (a workgroup fence would
    // also wait for those loads).
    u32x4_t v[PF][8];
    load(0, v[0]);
    store(0, v[0]);
#pragma unroll
    for (int q = 1; q <= PF; ++q)
        load(q, v[q % PF]);
    wait_lgkmcnt0();
    lds_barrier();
    for (int st0 = 0; st0 < steps; st0 += PF) {
#pragma unroll
        for (int q = 0; q < PF; ++q) {
            const int st = st0 + q;
            if (st >= steps)
                break;
            compute(st & 1);
            // unconditional: past the last step the groups are out of range,
            // every lane reads zeros and the stage written is not read again;
            // straight-line code lets the compiler wait for the oldest loads
            // only (vmcnt counts), not for all of them
            store((st + 1) & 1, v[(q + 1) % PF]);
            load(st + 1 + PF, v[(q + 1) % PF]);
            wait_lgkmcnt0();
            lds_barrier();
        }
    }

    const int jc[3] = {j0 + 48 * wave, j0 + 48 * wave + 16, j0 + 48 * wave + 32};
    wg_store<4, 3>(a, acc, oc0, jc, split, tile);
}

// ---------------------------------------------------------------------------
// Transpose-read weight backward (IC % 64 == 0, OC % 8 == 0, x and dy 16-byte
// aligned).  Same GEMM, tile (64 oc x 192 columns) and pixel walk (row-aligned
// groups of 8 output pixels, 64 pixels a step) as the kernel above, but no
// register transposes: the loaders copy raw pixel rows straight into LDS
// (16 bytes a lane, buffer loads to LDS), and the MFMA fragments are read
// with the gfx950 LDS transpose read ds_read_b64_tr_b16.
//
// That read (measured with an in-bounds probe): within each group of 16
// lanes, lane r fetches 4 consecutive 16-bit values at its own address; if
// those are viewed as a 16 x 4 matrix F (rows = lanes), lane l receives
// F[4e + (l >> 2)][l & 3] for e = 0..3.  So when lane r points at pixel row
// kb + (r >> 2), column m0 + 4 (r & 3) of a pixel-major tile, lane l gets the
// values of column m0 + l at pixels kb .. kb + 3: two such reads give the 8
// consecutive reduction values a lane feeds to v_mfma_f32_16x16x32_bf16.
//
// LDS stage: four regions of 64 pixel rows x 64 bf16 (128 bytes a row): dy's
// 64 output channels, then x's 192 columns as three regions of 64 (one tap's
// 64-channel slice each, since IC % 64 == 0).  The 16-byte chunk c of row r
// is stored at position c ^ s(r), s(r) = 2 (bit 1 of r) + 4 (bit 3 of r): the
// 4 rows x 32 bytes a 16-lane transpose read touches, and those of the next
// group 8 rows on, fall on distinct banks.  A copy instruction fills one
// region's 8 rows of one pixel group (1 KB): lane l takes pixel l >> 3 and
// physical chunk l & 7.
//
// STAGES stages in a ring: the copies of step st + STAGES - 1 are issued
// after the barrier of step st, which certifies that every wave is done
// with step st - 1's stage.  The step loop is unrolled by STAGES, so every
// stage offset is a constant: the compiler can then tell the stage a copy
// writes from the one the MFMA fragments are read from, and does not wait
// for the copies in flight before those reads.
constexpr int kWtRegion = kWgBK * 128;           // bytes: 64 pixel rows x 64 bf16
constexpr int kWtStage = 4 * kWtRegion;          // dy, then three 64-column regions of x
constexpr int kWtCopies = 8;                     // copy instructions per wave per step

__device__ __forceinline__ int wt_swz(int row)
{
    return (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
}

template <int STAGES>
__global__ __launch_bounds__(kWgThreads) void igemm_wgrad_tr_bf16(WgArgs a)
{
    static_assert(STAGES >= 2 && STAGES <= 5 && (STAGES - 1) * kWtCopies < 64, "vmcnt range");
    // one LDS variable per stage: the compiler then knows that a copy into
    // one stage and the fragment reads of another do not overlap (with one
    // array it waited for every copy in flight before each step's reads)
    __shared__ __align__(16) unsigned char lds0[kWtStage];
    __shared__ __align__(16) unsigned char lds1[kWtStage];
    __shared__ __align__(16) unsigned char lds2[STAGES > 2 ? kWtStage : 16];
    __shared__ __align__(16) unsigned char lds3[STAGES > 3 ? kWtStage : 16];
    __shared__ __align__(16) unsigned char lds4[STAGES > 4 ? kWtStage : 16];
    auto stage_base = [&](int stage) -> unsigned char * {
        return stage == 0 ? lds0 : stage == 1 ? lds1 : stage == 2 ? lds2 : stage == 3 ? lds3 : lds4;
    };
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tiles = a.tiles_m * a.tiles_n;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int split = bid / tiles, tile = bid - split * tiles;
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int oc0 = tm * kWgBM, j0 = tn * kWgBN;
    const int g_begin = split * a.chunk;
    const int g_end = min(a.groups, g_begin + a.chunk);
    const int steps = (g_end - g_begin + 7) / 8;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc((void *)a.dy, 0, a.dy_bytes, kRsrcWord3);

    // ---- copy roles.  Wave w copies pixel groups 2w and 2w + 1 of every
    // step: per group one dy instruction and three x instructions.  Lane:
    // pixel e = lane >> 3 of the group, physical chunk lane & 7, so logical
    // chunk cq[q] = (lane & 7) ^ s(8 (2w + q) + e).
    const int e = lane >> 3;
    int cq[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
        cq[q] = (lane & 7) ^ ((((e >> 1) & 1) << 1) | (q << 2));
    // x regions: the columns j0 + 64 ci .. + 63 are input channels
    // icb .. icb + 63 of one tap (kh, kw) (uniform values)
    int rdh[3], rdw[3], ricb[3];
    bool rok[3];
#pragma unroll
    for (int ci = 0; ci < 3; ++ci) {
        const int j = j0 + 64 * ci;
        rok[ci] = j < a.KKIC;
        const int jj = rok[ci] ? j : 0;
        const int t = fast_div(jj, a.div_ic);
        const int kh = fast_div(t, a.div_kw);
        ricb[ci] = jj - t * a.IC;
        rdh[ci] = kh * a.d - a.p;
        rdw[ci] = (t - kh * a.KW) * a.d - a.p;
    }
    const unsigned xpix = 2u * (unsigned)a.IC;          // bytes between neighbouring pixels of x
    auto issue = [&](int st, int stage) {
        unsigned char *const sbase = stage_base(stage);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int gi = 2 * wave + q;
            const int g = g_begin + st * 8 + gi;
            const bool gok = g < g_end;
            const int gg = gok ? g : g_begin;
            const int r = fast_div(gg, a.div_bpr);          // output row n*OH + oh
            const int ow0 = (gg - r * a.bpr) * 8;
            const int n = fast_div(r, a.div_oh);
            const int oh = r - n * a.OH;
            const bool pok = gok && ow0 + e < a.OW;
            const int oc = oc0 + 8 * cq[q];
            const unsigned aoff = (pok && oc < a.OC)
                ? 2u * ((unsigned)(r * a.OW + ow0 + e) * (unsigned)a.OC + (unsigned)oc) : kOutOfRange;
            dma16(rdy, (u32x4_t *)(sbase + gi * 1024), aoff);
#pragma unroll
            for (int ci = 0; ci < 3; ++ci) {
                const int ih = oh * a.s + rdh[ci];
                const int iw = (ow0 + e) * a.s + rdw[ci];
                const bool ok = pok && rok[ci] && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
                const unsigned xoff = ok
                    ? (unsigned)((n * a.H + ih) * a.W + iw) * xpix + 2u * (unsigned)(ricb[ci] + 8 * cq[q]) : kOutOfRange;
                dma16(rx, (u32x4_t *)(sbase + (1 + ci) * kWtRegion + gi * 1024), xoff);
            }
        }
    };

    // ---- fragment addresses (bytes within a stage, before the k-step and
    // half offsets).  Lane: group g16 = lane >> 4, r16 = lane & 15; it points
    // at row 8 g16 + (r16 >> 2) (+ 32 ks + 4 h), column m0 + 4 (r16 & 3).
    const int g16 = lane >> 4, r16 = lane & 15;
    const int sl = (((r16 >> 3) & 1) << 1) | ((g16 & 1) << 2);     // s(row), the same for every ks and h
    const int rowb = (8 * g16 + (r16 >> 2)) * 128 + 8 * (r16 & 1);
    const int b1 = (r16 & 3) >> 1;
    int abase[4], bbase[3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        abase[i] = rowb + 16 * ((2 * i + b1) ^ sl);
#pragma unroll
    for (int jb = 0; jb < 3; ++jb) {
        const int col = 48 * wave + 16 * jb;           // this wave's columns, within the tile
        bbase[jb] = (1 + (col >> 6)) * kWtRegion + rowb + 16 * ((((col & 63) >> 3) + b1) ^ sl);
    }

    floatx4_t acc[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    auto tr = [&](const unsigned char *p) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
    };
    auto frag = [&](const unsigned char *p) {
        const v4i16 lo = tr(p), hi = tr(p + 4 * 128);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto compute = [&](int stage) {
        const unsigned char *const sbase = stage_base(stage);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8_t fa[4], fb[3];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = frag(sbase + abase[i] + ks * 32 * 128);
#pragma unroll
            for (int j = 0; j < 3; ++j)
                fb[j] = frag(sbase + bbase[j] + ks * 32 * 128);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };

    // ---- pipeline: steps past the last one are issued too (every lane of
    // them is out of range: they write zeros into stages that are not read
    // again), so every wave always has STAGES - 1 steps of copies in flight
    // and the counted wait is a constant
#pragma unroll
    for (int q = 0; q < STAGES - 1; ++q)
        issue(q, q);
    // Whole rounds of STAGES steps with no branch inside (with a branch
    // around each step the compiler waited for the copies of the steps
    // ahead before the fragment reads of most steps), then the last partial
    // round step by step.
    auto step = [&](int st, auto q) __attribute__((always_inline)) {
        wait_vmcnt<(STAGES - 2) * kWtCopies>();    // step st has landed (this wave's part)
        lds_barrier();
        issue(st + STAGES - 1, (decltype(q)::value + STAGES - 1) % STAGES);
        compute(decltype(q)::value);
    };
    const int full = steps - steps % STAGES;
    for (int st0 = 0; st0 < full; st0 += STAGES) {
        step(st0, std::integral_constant<int, 0>{});
        step(st0 + 1, std::integral_constant<int, 1>{});
        if constexpr (STAGES > 2)
            step(st0 + 2, std::integral_constant<int, 2>{});
        if constexpr (STAGES > 3)
            step(st0 + 3, std::integral_constant<int, 3>{});
        if constexpr (STAGES > 4)
            step(st0 + 4, std::integral_constant<int, 4>{});
    }
    if (full < steps)
        step(full, std::integral_constant<int, 0>{});
    if constexpr (STAGES > 2)
        if (full + 1 < steps)
            step(full + 1, std::integral_constant<int, 1>{});
    if constexpr (STAGES > 3)
        if (full + 2 < steps)
            step(full + 2, std::integral_constant<int, 2>{});
    if constexpr (STAGES > 4)
        if (full + 3 < steps)
            step(full + 3, std::integral_constant<int, 3>{});
    wait_vmcnt<0>();       // (the copies past the last step: done before the workgroup ends)

    const int jc[3] = {j0 + 48 * wave, j0 + 48 * wave + 16, j0 + 48 * wave + 32};
    wg_store<4, 3>(a, acc, oc0, jc, split, tile);
}

// Row-window kernel.  A tile is 64 output channels x the three taps of one
// kernel row kh at one block of 64 input channels: columns (kh, kw, 64 icb
// + c) for kw = 0..2, c < 64.  At stride 1 those three taps read one input
// row, shifted by d pixels from tap to tap, so a step copies, beside dy,
// each unit's input row segment once (rsp = rl + 2d pixels for rl output
// pixels) instead of three gathered slices (half the bytes of the
// transpose-read kernel above).  The MFMA fragments are read with
// ds_read_b64_tr_b16 as there; a lane's x row is its pixel slot's, shifted
// by kw d.
//
// A step is 128 pixel slots holding rr units; a unit is rl consecutive
// output pixels of one output row (the whole row where OW <= 64, else one of
// rnseg equal segments), units numbered row by row.  Slot p = i rl + c (unit
// i, column c); slots from rr rl on are empty (dy zero, x read from a zero
// row, so a non-finite x value never meets them).
//
// LDS stage: 128 dy rows (slot p: 64 output channels, 128 bytes), then 8 XI
// x rows (unit i's span at rows i rsp .. i rsp + rsp - 1: 64 input
// channels), the 16-byte chunks of every row swizzled by wt_swz.  A copy
// instruction fills 8 rows (1 KB): wave w issues dy copies w, w + 8 and x
// copies w, w + 8, ...; rows past the step's data are copied as zeros, so
// every wave issues the same number each step and the counted wait is a
// constant.
//
// Waves: 8, two a SIMD.  Wave w computes the 64 x 96 block of columns
// 96 (w & 1) .. + 95 over slots 32 (w >> 1) .. + 31 of every step (one k
// step of v_mfma_f32_16x16x32_bf16: 4 A and 6 B fragments for 24 MFMAs,
// against 7 for 12 with 64 x 48 blocks).  After the last step the four
// waves of a column half add their blocks through LDS in wave order, each
// keeping 16 rows, and store them.
template <int XI, int STAGES, bool SEG>
__global__ __launch_bounds__(kWrThreads) void igemm_wgrad_row_bf16(WgArgs a)
{
    constexpr int kXRows = 8 * XI;
    constexpr int kXBase = kWrSlots * 128;           // x rows follow the dy slots
    constexpr int kStage = kXBase + kXRows * 128;
    constexpr int kDyCopies = kWrSlots / 64;         // dy copy instructions a wave issues per step
    constexpr int kCpw = kDyCopies + XI / 8;         // copy instructions a wave issues per step
    constexpr int kSlot = 9 * 64 * 16;               // exchange bytes a wave writes per column triple
    static_assert((XI == 16 || XI == 24) && STAGES >= 3 && STAGES <= 4 && (STAGES - 1) * kCpw < 64, "shape");
    static_assert(((8 + STAGES - 1) / STAGES) * kSlot <= kStage, "exchange slots fit the stages");
    __shared__ __align__(16) unsigned char lds0[kStage];
    __shared__ __align__(16) unsigned char lds1[kStage];
    __shared__ __align__(16) unsigned char lds2[kStage];
    __shared__ __align__(16) unsigned char lds3[STAGES > 3 ? kStage : 16];
    auto stage_base = [&](int stage) -> unsigned char * {
        return stage == 0 ? lds0 : stage == 1 ? lds1 : stage == 2 ? lds2 : lds3;
    };
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cw = wave & 1, ksw = wave >> 1;
    const int tiles = a.tiles_m * a.tiles_n;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int split = bid / tiles, tile = bid - split * tiles;
    // (run-time divisions as float-reciprocal ones: every quotient in this
    // kernel is below 2^21, and an integer division costs dozens of VALU
    // instructions a lane)
    const float inv_rl = __builtin_amdgcn_rcpf((float)a.rl), inv_rsp = __builtin_amdgcn_rcpf((float)a.rsp);
    const int tn = tile / a.tiles_m, tm = tile - tn * a.tiles_m;
    const int kh = tn / a.nicb, icb = tn - kh * a.nicb;
    const int oc0 = tm * kWgBM;
    const int s_begin = split * a.chunk;
    const int s_end = min(a.rsteps, s_begin + a.chunk);
    const int steps = s_end - s_begin;
    const int ih_off = kh * a.d - a.p;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc((void *)a.dy, 0, a.dy_bytes, kRsrcWord3);

    // ---- copy roles.  Lane: row e8 = lane >> 3 of the instruction's 8,
    // physical chunk lane & 7.  Units are rl pixels wide and numbered row by
    // row, so slot p of the step whose first unit is u0 holds output pixel
    // u0 rl + p: a dy offset is a per-step scalar plus a per-lane constant.
    // Divisions by run-time values use float reciprocals (small_div: every
    // quotient here is below 2^21) and the products 24-bit multiplies (x
    // holds fewer than 2^24 pixels since IC >= 64 and it is below 2 GiB),
    // both full-rate, where 64-bit and 32-bit integer multiplies are not.
    const int e8 = lane >> 3;
    const int units = a.NR * a.rnseg;
    unsigned doff[kDyCopies];
    int dlim[kDyCopies];
#pragma unroll
    for (int k = 0; k < kDyCopies; ++k) {
        const int pd = 8 * (wave + 8 * k) + e8;      // dy slot
        const int du = small_div(pd, inv_rl);
        const int doc = oc0 + 8 * ((lane & 7) ^ wt_swz(pd));
        doff[k] = 2u * ((unsigned)pd * (unsigned)a.OC + (unsigned)doc);
        dlim[k] = (du < a.rr && doc < a.OC) ? du : units;   // valid while u0 + dlim < units
    }
    int xu[XI / 8], xpos[XI / 8];
    unsigned xch[XI / 8];
#pragma unroll
    for (int k = 0; k < XI / 8; ++k) {
        const int q = 8 * (wave + 8 * k) + e8;       // x row
        const int u = small_div(q, inv_rsp);
        xpos[k] = q - u * a.rsp - a.p;
        // rows past the units never valid; whole-row units: the column is
        // the same every step, so its bounds test is made here
        xu[k] = (u < a.rr && (SEG || (unsigned)xpos[k] < (unsigned)a.W)) ? u : units;
        xch[k] = 2u * (unsigned)(icb * 64 + 8 * ((lane & 7) ^ wt_swz(q)));
    }
    const float inv_nseg = __builtin_amdgcn_rcpf((float)a.rnseg), inv_oh = __builtin_amdgcn_rcpf((float)a.OH);
    const unsigned xpix = 2u * (unsigned)a.IC;
    const unsigned dy_unit = 2u * (unsigned)a.rl * (unsigned)a.OC;  // dy bytes a unit
    auto issue = [&](int st, int stage) {
        unsigned char *const sb = stage_base(stage);
        const int gs = s_begin + st;
        const int u0 = gs < s_end ? gs * a.rr : units;           // past the range: nothing valid
#pragma unroll
        for (int k = 0; k < kDyCopies; ++k) {
            const unsigned off = u0 + dlim[k] < units ? (unsigned)u0 * dy_unit + doff[k] : kOutOfRange;
            dma16(rdy, (u32x4_t *)(sb + (wave + 8 * k) * 1024), off);
        }
#pragma unroll
        for (int k = 0; k < XI / 8; ++k) {
            const int u = u0 + xu[k];
            const int r = SEG ? small_div(u, inv_nseg) : u;        // output row n OH + oh
            const int n = small_div(r, inv_oh);
            const int ih = r - (int)__umul24(n, a.OH) + ih_off;
            const int iw = SEG ? (int)__umul24(u - (int)__umul24(r, a.rnseg), a.rl) + xpos[k] : xpos[k];
            const bool ok = u < units && (unsigned)ih < (unsigned)a.H && (!SEG || (unsigned)iw < (unsigned)a.W);
            const unsigned pix = __umul24(__umul24(n, a.H) + ih, a.W) + iw;
            const unsigned off = ok ? __umul24(pix, xpix) + xch[k] : kOutOfRange;
            dma16(rx, (u32x4_t *)(sb + kXBase + (wave + 8 * k) * 1024), off);
        }
    };

    // ---- fragment addresses.  Lane: group g16 = lane >> 4, r16 = lane & 15
    // fetches slot prow (+ 4 for the second half), columns 4 (r16 & 3) ..
    // of its 16-column block; it receives slots kb .. kb + 3 of column l.
    // A slot past the step's pixels fetches x from the last x row, which no
    // unit reaches (the plan leaves it), so it holds zeros: dy is zero there
    // too, and a non-finite x value never meets an empty slot.
    const int g16 = lane >> 4, r16 = lane & 15;
    const int b1 = (r16 & 3) >> 1;
    const int prow = 32 * ksw + 8 * g16 + (r16 >> 2);
    int abase[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        abase[i] = prow * 128 + 16 * ((2 * i + b1) ^ wt_swz(prow)) + 8 * (r16 & 1);
    int xb[2][6];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int p = prow + 4 * h;
        const int i = small_div(p, inv_rl), c = p - i * a.rl;
#pragma unroll
        for (int jb = 0; jb < 6; ++jb) {
            const int col = 96 * cw + 16 * jb;
            const int xr = i < a.rr ? i * a.rsp + c + (col >> 6) * a.d : kXRows - 1;
            xb[h][jb] = kXBase + xr * 128 + 16 * ((((col & 63) >> 3) + b1) ^ wt_swz(xr)) + 8 * (r16 & 1);
        }
    }

    floatx4_t acc[4][6];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 6; ++j)
            acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    auto tr = [&](const unsigned char *p) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
    };
    auto compute = [&](int stage) {
        const unsigned char *const sb = stage_base(stage);
        bf16x8_t fa[4], fb[6];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v4i16 lo = tr(sb + abase[i]), hi = tr(sb + abase[i] + 4 * 128);
            fa[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            const v4i16 lo = tr(sb + xb[0][j]), hi = tr(sb + xb[1][j]);
            fb[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 6; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };

    // ---- pipeline in whole rounds of STAGES steps: steps past the range's
    // last copy zeros and add nothing (the plan sizes the ranges in whole
    // rounds where it can).  A branch around a step made the compiler wait
    // for nearly every copy in flight before the next step's fragment reads.
#pragma unroll
    for (int q = 0; q < STAGES - 1; ++q)
        issue(q, q);
    for (int st0 = 0; st0 < steps; st0 += STAGES) {
#pragma unroll
        for (int q = 0; q < STAGES; ++q) {
            wait_vmcnt<(STAGES - 2) * kCpw>();        // step st0 + q has landed (this wave's part)
            lds_barrier();
            issue(st0 + q + STAGES - 1, (q + STAGES - 1) % STAGES);
            compute(q);
        }
    }
    wait_vmcnt<0>();
    lds_barrier();          // every copy has landed and every fragment read is done

    // ---- the four waves of a column half: in two passes of three column
    // blocks, every wave writes the three row blocks the others keep to its
    // own slot, then wave w adds row block w >> 1 of the four waves in wave
    // order (its own from registers).  One copy of this code per row block
    // kept (ksw is the same for the whole wave): with ksw a run-time index
    // into the accumulators the compiler branched around every access.
    floatx4_t keep[1][6];
    auto exchange = [&](auto kept) {
        constexpr int KS = decltype(kept)::value;
        unsigned char *const mine = stage_base(wave % STAGES) + (wave / STAGES) * kSlot;
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i == KS)
                    continue;
                const int idx = i - (i > KS ? 1 : 0);
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    ((floatx4_t *)mine)[(3 * idx + j) * 64 + lane] = acc[i][3 * jp + j];
            }
            lds_barrier();
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int jj = 3 * jp + j;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int src = 2 * k + cw;
                    const floatx4_t *const theirs =
                        (const floatx4_t *)(stage_base(src % STAGES) + (src / STAGES) * kSlot);
                    const floatx4_t v = k == KS ? acc[KS][jj] : theirs[(3 * (KS - (KS > k ? 1 : 0)) + j) * 64 + lane];
                    keep[0][jj] = k == 0 ? v : keep[0][jj] + v;
                }
            }
            lds_barrier();
        }
    };
    switch (ksw) {
    case 0: exchange(std::integral_constant<int, 0>{}); break;
    case 1: exchange(std::integral_constant<int, 1>{}); break;
    case 2: exchange(std::integral_constant<int, 2>{}); break;
    default: exchange(std::integral_constant<int, 3>{}); break;
    }
    int jc[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
        const int col = 96 * cw + 16 * j;
        jc[j] = (kh * 3 + (col >> 6)) * a.IC + 64 * icb + (col & 63);
    }
    wg_store<1, 6>(a, keep, oc0 + 16 * ksw, jc, split, tile);
}

// dw = the sum of the pixel ranges' partial tiles, part[s][i] for s < splits.
// A workgroup covers 256 >> LG consecutive 4-element columns; thread t takes
// column t % cols and range group t / cols (ranges split evenly and in
// order over 2^LG groups), loads all of its group's ranges before adding
// them in order, and the groups' sums are then added in group order through
// LDS: a fixed order for a given LG, so every call of a problem gives the
// same bits.  LG is a compile-time constant so that every index here is a
// shift and the groups' sums are read at once (a 64-bit division by a
// run-time group count before the first load, and the sums read one after
// another, measured 0.4 us slower on the ResNet-style layer).  vec: n % 4
// == 0 and both buffers 16-byte aligned (16-byte accesses), else element by
// element.
template <int LG>
__global__ __launch_bounds__(kWgReduceThreads) void wgrad_reduce(const float *__restrict__ part,
                                                                 float *__restrict__ dw, int n, int splits,
                                                                 int vec)
{
    constexpr int LC = 8 - LG;                   // log2 of the columns a workgroup covers
    __shared__ floatx4_t red[kWgReduceThreads];
    const int t = threadIdx.x;
    const int col = t & ((1 << LC) - 1), g = t >> LC;
    const int i = (int)(((unsigned)blockIdx.x << LC) + (unsigned)col) * 4;
    const int s0 = (int)(((long long)splits * g) >> LG), s1 = (int)(((long long)splits * (g + 1)) >> LG);
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (i < n) {
        if (vec) {
            // buffer loads, ranges past the group's reading zeros through an
            // offset past the workspace (below 1 GiB, so every offset fits):
            // no branch around a load, which made the compiler wait for each
            const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
                (void *)part, 0, (unsigned)((size_t)splits * n * 4), kRsrcWord3);
            floatx4_t v[kWgRedBatch];
            for (int sb = s0; sb < s1; sb += kWgRedBatch) {
#pragma unroll
                for (int q = 0; q < kWgRedBatch; ++q) {
                    const unsigned off = sb + q < s1 ? 4u * ((unsigned)(sb + q) * (unsigned)n + (unsigned)i) : kOutOfRange;
                    v[q] = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, 0));
                }
#pragma unroll
                for (int q = 0; q < kWgRedBatch; ++q)
                    acc += v[q];
            }
        } else {
            const int cnt = min(4, n - i);
            for (int s = s0; s < s1; ++s)
                for (int e = 0; e < cnt; ++e)
                    acc[e] += part[(size_t)s * n + i + e];
        }
    }
    red[t] = acc;
    __syncthreads();
    if (g == 0 && i < n) {
        floatx4_t sum = red[col];
#pragma unroll
        for (int q = 1; q < (1 << LG); ++q)
            sum += red[(q << LC) + col];
        if (vec) {
            *(floatx4_t *)(dw + i) = sum;
        } else {
            const int cnt = min(4, n - i);
            for (int e = 0; e < cnt; ++e)
                dw[i + e] = sum[e];
        }
    }
}

// fp32 storage (CONVIMG_FP32): 64 (oc) x 64 (j) tiles of dw over the same
// pixel ranges as the general kernel (groups of 8 pixels of one output row,
// 64 pixel slots a step), the products and sums in fp32 with
// v_mfma_f32_16x16x4_f32, four waves of 32 x 32.  A step stages dy and the
// im2col gather of x in LDS, pixel-major (slot rows of 64 values), one
// element a lane: a thread keeps one column (tap, channel) and one output
// channel for the whole range and takes 16 slots a step, whose pixel
// decodes the step's first 64 threads write to LDS beforehand.  Buffer loads
// whose masked lanes read zero past the end of the buffer; the loads of
// step st + 1 are in flight during step st's MFMAs.
__global__ __launch_bounds__(kWgThreads) void igemm_wgrad_f32(WgArgs a)
{
    __shared__ float sA[64 * kWgF32Row];      // [slot][oc - oc0]
    __shared__ float sB[64 * kWgF32Row];      // [slot][j - j0]
    __shared__ int4 pinf[2][64];              // per slot: pixel m (-1: none), n H, oh s, ow s

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tiles = a.tiles_m * a.tiles_n;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int split = bid / tiles, tile = bid - split * tiles;
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int oc0 = tm * kWgBM, j0 = tn * kWgF32BN;
    const int g_begin = split * a.chunk;
    const int g_end = min(a.groups, g_begin + a.chunk);
    const int steps = (g_end - g_begin + 7) / 8;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc((void *)a.dy, 0, a.dy_bytes, kRsrcWord3);

    // this thread's column c (j = j0 + c) and output channel oc0 + c; its
    // slots (tid >> 6) + 4 k
    const int c = tid & 63;
    const int j = j0 + c;
    const bool cok = j < a.KKIC, ook = oc0 + c < a.OC;
    int dh = 0, dwc = 0, ic = 0;
    if (cok) {
        const int t = fast_div(j, a.div_ic);
        const int kh = fast_div(t, a.div_kw);
        ic = j - t * a.IC;
        dh = kh * a.d - a.p;
        dwc = (t - kh * a.KW) * a.d - a.p;
    }
    // threads 0..63: slot `tid` of step st
    auto decode = [&](int st, int buf) {
        const int g = g_begin + st * 8 + (tid >> 3);
        int4 pi = make_int4(-1, 0, 0, 0);
        if (g < g_end) {
            const int r = fast_div(g, a.div_bpr);            // output row n OH + oh
            const int ow = (g - r * a.bpr) * 8 + (tid & 7);
            if (ow < a.OW) {
                const int n = fast_div(r, a.div_oh), oh = r - n * a.OH;
                pi = make_int4(r * a.OW + ow, n * a.H, oh * a.s, ow * a.s);
            }
        }
        pinf[buf][tid] = pi;
    };
    float va[16], vb[16];
    auto load = [&](int buf) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int4 pi = pinf[buf][(tid >> 6) + 4 * k];
            const bool mok = pi.x >= 0;
            const int ih = pi.z + dh, iw = pi.w + dwc;
            const bool xok = mok && cok && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
            const unsigned oa = (mok && ook) ? 4u * (unsigned)(pi.x * a.OC + oc0 + c) : kOutOfRange;
            const unsigned ob = xok ? 4u * (unsigned)(((pi.y + ih) * a.W + iw) * a.IC + ic) : kOutOfRange;
            va[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdy, oa, 0, 0));
            vb[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, ob, 0, 0));
        }
    };

    const int wm = wave & 1, wn = wave >> 1;
    const int lrow = lane & 15, lk = lane >> 4;
    floatx4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
            acc[i][jb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    if (steps > 0) {
        if (tid < 64)
            decode(0, 0);
        __syncthreads();
        load(0);
    }
    for (int st = 0; st < steps; ++st) {
        const int buf = st & 1;
        __syncthreads();            // the previous step's operand reads are done
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int ps = (tid >> 6) + 4 * k;
            sA[ps * kWgF32Row + c] = va[k];
            sB[ps * kWgF32Row + c] = vb[k];
        }
        if (tid < 64 && st + 1 < steps)
            decode(st + 1, buf ^ 1);
        __syncthreads();
        if (st + 1 < steps)
            load(buf ^ 1);
#pragma unroll 4
        for (int kk = 0; kk < 16; ++kk) {
            const int row = (4 * kk + lk) * kWgF32Row;
            float af[2], bfv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = sA[row + 32 * wm + 16 * i + lrow];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
                bfv[jb] = sB[row + 32 * wn + 16 * jb + lrow];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfv[jb], acc[i][jb], 0, 0, 0);
        }
    }
    const int jc[2] = {j0 + 32 * wn, j0 + 32 * wn + 16};
    wg_store<2, 2>(a, acc, oc0 + 32 * wm, jc, split, tile);
}

#endif  // CONVIMG_WGRAD_KERNELS

// Launchers, defined in conv2d_wgrad.hip (its own translation unit: it is
// compiled with the MFMA accumulators in VGPRs, which measured fewer
// register copies for this kernel than the default AGPR form).
void wgrad_set_attributes();
hipError_t wgrad_launch(const WgArgs &a, bool vx, bool vdy, int grid, hipStream_t stream);
hipError_t wgrad_tr_launch(const WgArgs &a, int grid, int stages, hipStream_t stream);
hipError_t wgrad_row_launch(const WgArgs &a, int grid, int xi, int stages, hipStream_t stream);
hipError_t wgrad_f32_launch(const WgArgs &a, int grid, hipStream_t stream);
hipError_t wgrad_reduce_launch(const float *part, float *dw, int n, int splits, int vec, int lg,
                               hipStream_t stream);

}  // namespace convimg
