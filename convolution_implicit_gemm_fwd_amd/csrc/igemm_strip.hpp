// igemm_strip.hpp -- implicit-GEMM kernel for layers whose weight slice fits
// in LDS next to the input rows of a strip of output pixels.
//
// One workgroup (4 waves, one per SIMD) owns a contiguous strip of output
// pixels (GEMM rows) and a 64-wide slice of the output channels.  It copies
// the slice's weights for the whole K into LDS once, and for each chunk of
// the strip every input row the chunk reads; the im2col gather then happens
// in the LDS addresses the MFMA operands are read from.  Each input pixel
// crosses the CU's memory path once per chunk instead of once per tap (the
// pipelined kernel's im2col tile re-reads it for each of the KH*KW taps), and
// the weights once per workgroup instead of once per tile.  The launch has
// one workgroup per CU and strips of equal length, so every CU does the same
// work.
//
// The copies are direct-to-LDS (buffer_load ... lds, 1 KB per wave
// instruction), so LDS areas are copied as contiguous runs of 16-byte
// chunks:
//   * weights: tap-major, [KH*KW][64 channel rows][IC]; chunk c of row r of
//     a tap is stored at position c ^ (r & 7) within its group of 8;
//   * patch: the input rows of each image the chunk touches, one contiguous
//     run per image ("segment", rounded up to whole 1 KB blocks); chunk c of
//     pixel p of a segment is stored at position c ^ (p & 7);
// so the 8 lanes that read one chunk column of 8 consecutive pixels (or
// channels) hit 8 distinct 4-bank groups.  Padding taps read a zero block at
// LDS offset 0.
#pragma once

#include "igemm_common.hpp"
#include "igemm_pipe.hpp"

namespace convimg {

constexpr int kStripBN = 64;      // output channels per workgroup
constexpr int kStripWaves = 4;
constexpr int kStripScratchStride = 68;   // floats per epilogue scratch row (64 + pad)
constexpr int kStripScratchBytes = kStripWaves * 16 * kStripScratchStride * 4;

// Input rows [lo, hi] that output rows oh_lo..oh_hi of one image read,
// clipped to the image; returns the row count (0 if all of it is padding).
__host__ __device__ inline int strip_rows(int oh_lo, int oh_hi, int H, int KH, int s, int p,
                                          int d, int *ih_lo)
{
    int lo = oh_lo * s - p;
    int hi = oh_hi * s - p + (KH - 1) * d;
    if (lo < 0)
        lo = 0;
    if (hi > H - 1)
        hi = H - 1;
    *ih_lo = lo;
    return hi >= lo ? hi - lo + 1 : 0;
}

__host__ __device__ inline long long strip_round(long long chunks)
{
    return (chunks + 63) / 64 * 64;
}

// LDS layout of the patch of output pixels [c0, c1): segments for images
// n_a..n_b.  The first starts at input row ih_a of image n_a; the others at
// row 0.  Segment offsets (in 16-byte chunks): 0 for n_a, then first_chunks
// + (n - n_a - 1) * full_chunks.
struct StripSeg {
    int n_a, n_b;
    int oh_a, oh_b;          // first output row in image n_a, last in image n_b
    int ih_a, rows_a;        // first segment: first input row, row count
    long long first_chunks;  // first segment, rounded up to whole 1 KB blocks
    long long full_chunks;   // a segment of a whole image, rounded
    long long total_chunks;
};

__host__ __device__ inline StripSeg strip_seg(int c0, int c1, int H, int W, int OH, int OW,
                                              int KH, int s, int p, int d, int cpp)
{
    StripSeg g;
    const int q_a = c0 / OW, q_b = (c1 - 1) / OW;   // flattened output rows n*OH + oh
    g.n_a = q_a / OH;
    g.n_b = q_b / OH;
    g.oh_a = q_a - g.n_a * OH;
    g.oh_b = q_b - g.n_b * OH;
    const long long rowc = (long long)W * cpp;       // chunks per input row
    int lo;
    if (g.n_a == g.n_b) {
        g.rows_a = strip_rows(g.oh_a, g.oh_b, H, KH, s, p, d, &lo);
        g.ih_a = lo;
        g.first_chunks = strip_round(g.rows_a * rowc);
        g.full_chunks = 0;
        g.total_chunks = g.first_chunks;
        return g;
    }
    g.rows_a = strip_rows(g.oh_a, OH - 1, H, KH, s, p, d, &lo);
    g.ih_a = lo;
    g.first_chunks = strip_round(g.rows_a * rowc);
    g.full_chunks = strip_round(strip_rows(0, OH - 1, H, KH, s, p, d, &lo) * rowc);
    const long long last = strip_round(strip_rows(0, g.oh_b, H, KH, s, p, d, &lo) * rowc);
    g.total_chunks = g.first_chunks + (long long)(g.n_b - g.n_a - 1) * g.full_chunks + last;
    return g;
}

// s_waitcnt vmcnt(n) for a count known only at run time (the instruction
// takes an immediate); n >= 63 needs no wait, since at most 63 vector memory
// instructions of a wave are ever outstanding.
__device__ __forceinline__ void wait_vmcnt_rt(int n)
{
    switch (n) {
#define CONVIMG_W(k) case k: wait_vmcnt<k>(); break;
#define CONVIMG_W8(k) CONVIMG_W(k) CONVIMG_W(k + 1) CONVIMG_W(k + 2) CONVIMG_W(k + 3) \
                      CONVIMG_W(k + 4) CONVIMG_W(k + 5) CONVIMG_W(k + 6) CONVIMG_W(k + 7)
        CONVIMG_W8(0) CONVIMG_W8(8) CONVIMG_W8(16) CONVIMG_W8(24)
        CONVIMG_W8(32) CONVIMG_W8(40) CONVIMG_W8(48)
        CONVIMG_W(56) CONVIMG_W(57) CONVIMG_W(58) CONVIMG_W(59) CONVIMG_W(60) CONVIMG_W(61)
        CONVIMG_W(62)
#undef CONVIMG_W8
#undef CONVIMG_W
    default:
        break;
    }
}

// FM: 32-row MFMA blocks per wave (a chunk is at most 128 * FM pixels).
// v_mfma_f32_32x32x16_bf16 throughout: with one wave per SIMD it keeps the
// matrix core busier than the 16x16x32 shape.
template <int FM>
__global__ __launch_bounds__(256) void igemm_strip_bf16(ConvArgs a)
{
    constexpr int FN = kStripBN / 32;
    extern __shared__ u32x4_t dsm[];
    char *const lds = (char *)dsm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lk = lane >> 5;      // k chunk this lane feeds
    const int lr = lane & 31;      // row / column this lane feeds

    int bid = blockIdx.x;
    if (a.remap)
        bid = xcd_remap(bid, gridDim.x);
    const int gn = bid / a.tiles_m;
    const int gm = bid - gn * a.tiles_m;
    const int n0 = gn * kStripBN;
    const int p_begin = gm * a.strip_px;
    if (p_begin >= a.M)
        return;
    const int p_end = min(p_begin + a.strip_px, a.M);

    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)a.w, 0, a.w_bytes, kRsrcWord3);

    const int cpp = a.IC >> 3;              // 16-byte chunks per input pixel
    const int cs = a.cpp_shift;             // log2(cpp)
    const int KCH = a.K >> 3;               // 16-byte chunks per weight row
    const int zb = a.lds_zero;              // zero block bytes (at LDS offset 0)
    const int pb = a.lds_patch;             // patch offset (bytes)
    const int OHW = a.OH * a.OW;

    // ---- zero block
    for (int i = tid; i < (zb >> 4); i += 256)
        dsm[i] = u32x4_t{0u, 0u, 0u, 0u};

    // bias of the columns this lane writes
    float bv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int oc = n0 + j * 32 + lr;
        bv[j] = (a.bias != nullptr && oc < a.OC) ? a.bias[oc] : 0.f;
    }

    // B fragment of channel row j*32 + lr, step t of tap tap (chunks 2t + lk):
    // wrow[j] + tap * tapb + ((t << 5) ^ v16)
    const int tapb = kStripBN * cpp * 16;       // bytes per tap of the weight slice
    int wrow[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
        wrow[j] = zb + (j * 32 + lr) * cpp * 16;
    const int v16 = (lk ^ (lr & 7)) << 4;
    const int ntaps = a.KH * a.KW;
    const int wpt = cpp >> 2;                   // weight copies per wave per tap

    float *const scratch = (float *)(lds + a.lds_scratch) + wave * 16 * kStripScratchStride;

    for (int c0 = p_begin; c0 < p_end; c0 += a.chunk_px) {
        const int c1 = min(c0 + a.chunk_px, p_end);
        if (c0 != p_begin)
            __syncthreads();    // every wave is done with the previous patch

        // ---- patch: one contiguous run of input rows per image
        const StripSeg g = strip_seg(c0, c1, a.H, a.W, a.OH, a.OW, a.KH, a.stride, a.pad, a.dil, cpp);
        {
            long long off_n = 0;
            for (int n = g.n_a; n <= g.n_b; ++n) {
                int ih_lo, rows;
                if (n == g.n_a) {
                    ih_lo = g.ih_a;
                    rows = g.rows_a;
                } else {
                    rows = strip_rows(0, n == g.n_b ? g.oh_b : a.OH - 1, a.H, a.KH, a.stride,
                                      a.pad, a.dil, &ih_lo);
                }
                const int seg_chunks = rows * a.W * cpp;
                const int gbase = ((n * a.H + ih_lo) * a.W) * cpp;
                u32x4_t *dst = (u32x4_t *)(lds + pb) + off_n;
                const int nblk = (seg_chunks + 63) >> 6;
                for (int blk = wave; blk < nblk; blk += kStripWaves) {
                    const int P = blk * 64 + lane;
                    const unsigned off = P < seg_chunks
                        ? 16u * (unsigned)(gbase + (P ^ ((P >> cs) & 7))) : kOutOfRange;
                    dma16(rx, dst + blk * 64, off);
                }
                off_n += (n == g.n_a) ? g.first_chunks : g.full_chunks;
            }
        }

        // ---- weights (first chunk only), after the patch, tap by tap: tap
        // tau is cpp blocks of 1 KB; block b, lane l holds row (64b + l) >> cs,
        // position (64b + l) & (cpp - 1).  Each wave issues wpt copies per tap,
        // so before tap tau a wave waits until at most
        // (ntaps - 1 - tau) * wpt of its copies are outstanding.
        if (c0 == p_begin) {
            for (int tap = 0; tap < ntaps; ++tap) {
                for (int blk = wave; blk < cpp; blk += kStripWaves) {
                    const int P = blk * 64 + lane;
                    const int row = P >> cs, c = P & (cpp - 1);
                    const int oc = n0 + row;
                    const unsigned off = oc < a.OC
                        ? 16u * (unsigned)(oc * KCH + tap * cpp + (c ^ (row & 7))) : kOutOfRange;
                    dma16(rw, (u32x4_t *)(lds + zb + tap * tapb) + blk * 64, off);
                }
            }
        }

        // ---- per-block pixel geometry (block i of this wave: rows
        // c0 + (wave * FM + i) * 32 + lr)
        int pix0[FM], ih0[FM], iw0[FM], segb[FM];
        bool vm[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = c0 + (wave * FM + i) * 32 + lr;
            vm[i] = m < c1;
            const int mm = vm[i] ? m : c0;
            const int n = mm / OHW;
            const int r = mm - n * OHW;
            const int oh = r / a.OW;
            const int ow = r - oh * a.OW;
            ih0[i] = oh * a.stride - a.pad;
            iw0[i] = ow * a.stride - a.pad;
            int ihl;
            long long so;
            if (n == g.n_a) {
                ihl = g.ih_a;
                so = 0;
            } else {
                ihl = 0;
                so = g.first_chunks + (long long)(n - g.n_a - 1) * g.full_chunks;
            }
            pix0[i] = (ih0[i] - ihl) * a.W + iw0[i];
            segb[i] = pb + (int)so * 16;
        }

        floatx16_t acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = floatx16_t{};

        // patch and the first tap's weights; on later chunks every weight
        // copy is long complete and nothing newer than the patch is in flight
        wait_vmcnt_rt(c0 == p_begin ? (ntaps - 1) * wpt : 0);
        __syncthreads();

        // ---- K loop: taps in (kh, kw) order, T = IC / 16 MFMA k steps per
        // tap (a multiple of 4).  The fragments of step k + 1 are read from
        // LDS while the MFMAs of step k run (two register sets, and a
        // scheduling barrier that keeps the reads ahead of the MFMAs), so
        // LDS latency hides behind matrix work with one wave per SIMD.
        // A fragment of pixel pix, chunk 2t + lk of the tap: the tap's
        // address (t = 0) ^ (t << 5), since the chunk's low 3 bits are XORed
        // with pix & 7 and the pixel record is cpp * 16 bytes aligned.
        const int T = a.IC >> 4;
        int akh = 0, akw = 0;       // tap whose A addresses are computed next
        auto tap_addr = [&](int (&aa)[FM]) {
            const int dh = akh * a.dil, dw = akw * a.dil;
            const int dpix = dh * a.W + dw;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int pix = pix0[i] + dpix;
                const bool ok = vm[i] && (unsigned)(ih0[i] + dh) < (unsigned)a.H
                    && (unsigned)(iw0[i] + dw) < (unsigned)a.W;
                aa[i] = ok ? segb[i] + (pix << (cs + 4)) + (((pix & 7) ^ lk) << 4) : 0;
            }
            if (++akw == a.KW) {
                akw = 0;
                ++akh;
            }
        };
        // wofs: tap * tapb + ((t << 5) ^ v16) of the step to read
        auto load = [&](const int (&aa)[FM], int wofs, bf16x8_t (&fa)[FM], bf16x8_t (&fb)[FN]) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(lds + aa[i]));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(lds + wrow[j] + wofs));
        };
        auto mma = [&](const bf16x8_t (&fa)[FM], const bf16x8_t (&fb)[FN]) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        };

        int a_cur[FM], a_nxt[FM], a_ld[FM];
        tap_addr(a_cur);
        bf16x8_t fa0[FM], fb0[FN], fa1[FM], fb1[FN];
        load(a_cur, v16, fa0, fb0);
        for (int tap = 0; tap < ntaps; ++tap) {
            const int tofs = tap * tapb;
            if (tap + 1 < ntaps)
                tap_addr(a_nxt);
            else
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    a_nxt[i] = a_cur[i];    // harmless reads past the last step
            for (int t = 0; t < T; t += 2) {
                // fa0/fb0 hold step t of this tap
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    a_ld[i] = a_cur[i] ^ ((t + 1) << 5);
                load(a_ld, tofs + (((t + 1) << 5) ^ v16), fa1, fb1);
                __builtin_amdgcn_sched_barrier(0);  // the reads go out before the MFMAs
                mma(fa0, fb0);
                const bool last = t + 2 == T;
                if (last && c0 == p_begin && tap + 1 < ntaps) {
                    wait_vmcnt_rt((ntaps - 2 - tap) * wpt);   // next tap's weights
                    __syncthreads();
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    a_ld[i] = last ? a_nxt[i] : (a_cur[i] ^ ((t + 2) << 5));
                load(a_ld, last ? tofs + tapb + v16 : tofs + (((t + 2) << 5) ^ v16), fa0, fb0);
                __builtin_amdgcn_sched_barrier(0);
                mma(fa1, fb1);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a_cur[i] = a_nxt[i];
        }

        // ---- epilogue: + bias, through the wave's scratch (16 rows at a
        // time) into 16-byte stores of whole 64-channel row segments.  Value
        // v of block (i, j) is row 8*(v >> 2) + 4*lk + (v & 3), column
        // j*32 + lr; half h holds v = 8h .. 8h + 7, rows 16h .. 16h + 15.
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int v = 8 * h; v < 8 * h + 8; ++v)
                        scratch[(8 * ((v >> 2) - 2 * h) + 4 * lk + (v & 3)) * kStripScratchStride
                                + j * 32 + lr] = acc[i][j][v] + bv[j];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int f = t * 64 + lane;
                    const int row = f >> 4, c4 = (f & 15) * 4;
                    const floatx4_t val = *(const floatx4_t *)(scratch + row * kStripScratchStride + c4);
                    const int m = c0 + (wave * FM + i) * 32 + 16 * h + row;
                    const int oc = n0 + c4;
                    if (m < c1) {
                        float *o = a.out + (long long)m * a.OC + oc;
                        if (a.vec_out && oc + 3 < a.OC) {
                            *(floatx4_t *)o = val;
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (oc + e < a.OC)
                                    o[e] = val[e];
                        }
                    }
                }
            }
        }
    }
}

}  // namespace convimg
