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
// Workgroup: 256 threads, a 64 (oc) x 192 (j) tile, 64 pixels per step,
// two LDS stages of 32 KB (the next step's loads are in flight while the
// current one runs on the MFMAs), one barrier per step.  Wave w computes
// all 64 rows x columns [48w, 48w+48) with 16x16x32 bf16 MFMAs.  The
// pixels are split into `splits` contiguous ranges; each range's partial
// tile goes to a workspace and a second kernel sums the ranges in order
// (deterministic), or straight to dw when there is one range.
#pragma once

namespace convimg {

constexpr int kWgBM = 64;           // output channels per tile
constexpr int kWgBN = 192;          // (tap, input channel) columns per tile
constexpr int kWgBK = 64;           // pixels per step
constexpr int kWgThreads = 256;
constexpr int kWgRows = kWgBM + kWgBN;           // LDS rows per stage (A rows, then B rows)
constexpr int kWgRowBytes = kWgBK * 2;           // one row: 64 pixels of one channel
constexpr int kWgStageBytes = kWgRows * kWgRowBytes;
constexpr int kWgLdsBytes = 2 * kWgStageBytes;
constexpr int kWgReduceThreads = 256;

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
    int tiles_m, tiles_n, splits, chunk;   // chunk: pixels per split, a multiple of kWgBK
    FastDiv div_ohw, div_ow, div_ic, div_kw;
};

// LDS byte offset of 16-byte record `chunk` (8 pixels) of row `row`; the
// XOR keeps the 16 rows one MFMA operand read touches on distinct banks.
__device__ __forceinline__ int wg_rec(int row, int chunk)
{
    return row * kWgRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// v[e] holds 8 channels of pixel e (channel 2h in the low half of dword h);
// out[c] receives 8 pixels of channel c (pixel 2q in the low half of dword q).
__device__ __forceinline__ void transpose8x8(const u32x4_t (&v)[8], u32x4_t (&out)[8])
{
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned lo = v[2 * q][h], hi = v[2 * q + 1][h];
            out[2 * h][q] = (lo & 0xffffu) | (hi << 16);
            out[2 * h + 1][q] = (lo >> 16) | (hi & 0xffff0000u);
        }
    }
}

// VX: IC % 8 == 0 and x 16-byte aligned (16-byte gathers of x), else
// element-wise.  VDY: OC % 8 == 0 and dy 16-byte aligned, likewise.
template <bool VX, bool VDY>
__global__ __launch_bounds__(kWgThreads) void igemm_wgrad_bf16(WgArgs a)
{
    extern __shared__ __align__(16) unsigned char wg_lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tiles = a.tiles_m * a.tiles_n;
    // ranges of one tile column share their dy rows and x windows: keep the
    // workgroups of one range together on one XCD
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int split = bid / tiles, tile = bid - split * tiles;
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int oc0 = tm * kWgBM, j0 = tn * kWgBN;
    const int m_begin = split * a.chunk;
    const int m_end = min(a.M, m_begin + a.chunk);
    const int steps = (m_end - m_begin + kWgBK - 1) / kWgBK;

    // loader role: threads 0..191 gather 8 columns of x, 192..255 8 rows of dy
    const bool is_b = tid < 3 * 64;
    const int grp = is_b ? tid % 24 : (tid - 192) % 8;
    const int pg = is_b ? tid / 24 : (tid - 192) / 8;      // 8-pixel group of the step
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

    u32x4_t v[8];
    auto load = [&](int st) {
        const int mb = m_begin + st * kWgBK + pg * 8;
        int n = 0, oh = 0, ow = 0;
        if (mb < m_end) {
            n = fast_div(mb, a.div_ohw);
            const int r = mb - n * a.OH * a.OW;
            oh = fast_div(r, a.div_ow);
            ow = r - oh * a.OW;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool pix = mb + e < m_end;
            u32x4_t val = {0u, 0u, 0u, 0u};
            if (is_b) {
                if (VX) {
                    const int ih = oh * a.s + dh[0], iw = ow * a.s + dwc[0];
                    if (pix && colok[0] && ih >= 0 && ih < a.H && iw >= 0 && iw < a.W)
                        val = *(const u32x4_t *)(a.x + (size_t)((n * a.H + ih) * a.W + iw) * a.IC + icc[0]);
                } else {
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const int ih = oh * a.s + dh[c], iw = ow * a.s + dwc[c];
                        unsigned h = 0;
                        if (pix && colok[c] && ih >= 0 && ih < a.H && iw >= 0 && iw < a.W)
                            h = a.x[(size_t)((n * a.H + ih) * a.W + iw) * a.IC + icc[c]];
                        val[c >> 1] |= h << ((c & 1) * 16);
                    }
                }
            } else {
                const unsigned short *src = a.dy + (size_t)(mb + e) * a.OC + orow;
                if (VDY) {
                    if (pix && orow < a.OC)
                        val = *(const u32x4_t *)src;
                } else {
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        unsigned h = 0;
                        if (pix && orow + c < a.OC)
                            h = src[c];
                        val[c >> 1] |= h << ((c & 1) * 16);
                    }
                }
            }
            v[e] = val;
            // next pixel
            if (++ow == a.OW) {
                ow = 0;
                if (++oh == a.OH) {
                    oh = 0;
                    ++n;
                }
            }
        }
    };
    auto store = [&](int stage) {
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

    load(0);
    store(0);
    __syncthreads();
    const int lrow = lane & 15, lchk = lane >> 4;
    for (int st = 0; st < steps; ++st) {
        const bool more = st + 1 < steps;
        if (more)
            load(st + 1);
        const unsigned char *base = wg_lds + (st & 1) * kWgStageBytes;
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
        if (more)
            store((st + 1) & 1);
        __syncthreads();
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

// dw[i] = sum over s = 0..splits-1, in that order, of part[s][i]; four
// consecutive elements per thread.  vec: n % 4 == 0 and both buffers
// 16-byte aligned (16-byte accesses), else element by element.
__global__ __launch_bounds__(kWgReduceThreads) void wgrad_reduce(const float *__restrict__ part,
                                                                 float *__restrict__ dw, int n, int splits,
                                                                 int vec)
{
    const int i = (blockIdx.x * kWgReduceThreads + threadIdx.x) * 4;
    if (i >= n)
        return;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    if (vec) {
        for (int s = 0; s < splits; ++s) {
            const floatx4_t v = *(const floatx4_t *)(part + (size_t)s * n + i);
            s0 += v[0];
            s1 += v[1];
            s2 += v[2];
            s3 += v[3];
        }
        *(floatx4_t *)(dw + i) = floatx4_t{s0, s1, s2, s3};
    } else {
        const int cnt = min(4, n - i);
        for (int e = 0; e < cnt; ++e) {
            float acc = 0.f;
            for (int s = 0; s < splits; ++s)
                acc += part[(size_t)s * n + i + e];
            dw[i + e] = acc;
        }
    }
}

}  // namespace convimg
