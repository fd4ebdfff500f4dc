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
// The groups are split into `splits` contiguous ranges; each range's
// partial tile goes to a workspace and a second kernel sums the ranges in
// order (deterministic), or straight to dw when there is one range.
#pragma once

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
constexpr int kWgReduceThreads = 512;
#ifndef CONVIMG_WG_PF
#define CONVIMG_WG_PF 1
#endif
constexpr int kWgPF = CONVIMG_WG_PF;    // steps of loads in flight (measured)

// Division by a run-time constant with one 64-bit multiply (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// for 0 <= n < 2^31 and divisor v >= 1, with l = ceil(log2 v),
// mul = ceil(2^(31+l) / v) < 2^32 gives n / v = (n * mul) >> (31 + l).
struct FastDiv {
    unsigned mul;
    int shift;
};

__device__ __forceinline__ int fast_div(int n, FastDiv f)
{
    return (int)(((unsigned long long)(unsigned)n * f.mul) >> f.shift);
}

struct WgArgs {
    const unsigned short *x;     // [N][H][W][IC] bf16
    const unsigned short *dy;    // [N][OH][OW][OC] bf16
    float *dst;                  // dw [OC][KKIC], or partial sums [splits][OC][KKIC]
    int N, H, W, IC, OC, KH, KW, s, p, d, OH, OW;
    int M, KKIC;                 // pixels N*OH*OW; columns KH*KW*IC
    int bpr, groups;             // 8-pixel groups per output row; N*OH*bpr
    int tiles_m, tiles_n, splits, chunk;   // chunk: groups per split, a multiple of 8
    unsigned x_bytes, dy_bytes;            // both below 2^31
    FastDiv div_bpr, div_oh, div_s, div_ic, div_kw;
};

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

// v[e] holds 8 channels of pixel e (channel 2h in the low half of dword h);
// out[c] receives 8 pixels of channel c (pixel 2q in the low half of dword q).
__device__ __forceinline__ void transpose8x8(const u32x4_t (&v)[8], u32x4_t (&out)[8])
{
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // byte selects over {hi, lo}: lo bytes are 0-3, hi bytes 4-7
            const unsigned lo = v[2 * q][h], hi = v[2 * q + 1][h];
            out[2 * h][q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);       // low halves
            out[2 * h + 1][q] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);   // high halves
        }
    }
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

    // D[row = 4*(lane/16) + v][col = lane % 16] of each 16x16 block
    float *dst = a.dst + (size_t)split * a.OC * a.KKIC;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int jj = j0 + wave * 48 + j * 16 + lrow;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int oc = oc0 + i * 16 + 4 * lchk + e;
                if (oc < a.OC && jj < a.KKIC)
                    dst[(size_t)oc * a.KKIC + jj] = acc[i][j][e];
            }
        }
    }
}

// dw = the sum of the pixel ranges' partial tiles, part[s][i] for s < splits.
// One workgroup covers 256 consecutive elements (4 per lane); its 8 waves
// each add an eighth of the ranges in order, then wave 0 adds the eight
// partial sums in wave order: a fixed order, so every call gives the same
// bits.  vec: n % 4 == 0 and both buffers 16-byte aligned (16-byte
// accesses), else element by element.
__global__ __launch_bounds__(kWgReduceThreads) void wgrad_reduce(const float *__restrict__ part,
                                                                 float *__restrict__ dw, int n, int splits,
                                                                 int vec)
{
    constexpr int kWaves = kWgReduceThreads / 64;
    __shared__ floatx4_t red[kWaves][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i = (blockIdx.x * 64 + lane) * 4;
    const int s0 = (int)((long long)splits * w / kWaves), s1 = (int)((long long)splits * (w + 1) / kWaves);
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (i < n) {
        if (vec) {
#pragma unroll 4
            for (int s = s0; s < s1; ++s)
                acc += *(const floatx4_t *)(part + (size_t)s * n + i);
        } else {
            const int cnt = min(4, n - i);
            for (int s = s0; s < s1; ++s)
                for (int e = 0; e < cnt; ++e)
                    acc[e] += part[(size_t)s * n + i + e];
        }
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w == 0 && i < n) {
        floatx4_t t = red[0][lane];
#pragma unroll
        for (int q = 1; q < kWaves; ++q)
            t += red[q][lane];
        if (vec) {
            *(floatx4_t *)(dw + i) = t;
        } else {
            const int cnt = min(4, n - i);
            for (int e = 0; e < cnt; ++e)
                dw[i + e] = t[e];
        }
    }
}

#endif  // CONVIMG_WGRAD_KERNELS

// Launchers, defined in conv2d_wgrad.hip (its own translation unit: it is
// compiled with the MFMA accumulators in VGPRs, which measured fewer
// register copies for this kernel than the default AGPR form).
void wgrad_set_attributes();
hipError_t wgrad_launch(const WgArgs &a, bool vx, bool vdy, int grid, hipStream_t stream);
hipError_t wgrad_reduce_launch(const float *part, float *dw, int n, int splits, int vec, int blocks,
                               hipStream_t stream);

}  // namespace convimg
