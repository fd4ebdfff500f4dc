// igemm_resident.hpp -- implicit-GEMM kernel for layers whose 64-channel
// weight slice and whose input rows for one CU's share of the output pixels
// fit in LDS together (a ResNet 3x3 layer: 64 -> 64 channels on 56x56 maps
// needs 73 KB of weights and at most 6 input rows, 47 KB).
//
// One workgroup (8 waves) per CU takes a contiguous range of output pixels
// m (an even split of M).  Its prologue copies, direct to LDS:
//   * the weight slice, channel rows n0 .. n0+63, each a record of K bf16
//     plus a spare 16-byte chunk, so lanes reading the same k of 32
//     consecutive rows fall on distinct banks;
//   * every input row g = n*H + ih the range reads (one contiguous run of
//     x in NHWC order), each pixel a record of IC bf16 plus a spare chunk;
// and zeroes one pixel record that stands for every padding pixel.  After
// one barrier the waves work independently: wave w takes 32-pixel units
// w, w+8, ...; lane (lk, lr) finds, for each tap (kh, kw), the record of the
// input pixel of output pixel lr of the unit (or the zero record), and the
// K loop runs over all taps, IC/16 MFMA steps per tap, with
// v_mfma_f32_32x32x16_bf16 against both 32-channel halves of the slice
// (A and B from LDS, next step's fragments loaded during this step's
// MFMAs; even and odd steps into separate accumulators).  Results (+ bias)
// leave through a per-wave LDS scratch as 16-byte stores (or one dword a
// lane where the output does not allow them); no copy or barrier follows
// the prologue, so one wave's stores overlap the other waves' MFMAs.
//
// With LAYOUT kResNchwF32 or kResNchwBf16 the same kernel reads x in NCHW
// order and writes out in NCHW order (fp32, or bf16 rounded to nearest
// even): the input rows arrive as 16-byte runs of 8 pixels of one channel,
// eight channels a lane, which the lane transposes in registers into the
// 16-byte chunks of 8 pixel records; and each lane's accumulators already
// hold, for one output channel, four runs of 4 consecutive pixels, stored
// as they are.  The NCHW entry point then needs no input or output permute
// around the GEMM; the weights then come in OIHW order too, and each
// weight record is reordered in LDS after the copies.
//
// Measured on MI355X (ResNet 3x3 layer above), this order beat the
// alternatives tried: copying the rows before the weights, tap-major weight
// records with a barrier per tap or per kernel row (MFMAs starting before
// the later taps have landed), 16 waves, and 64-pixel units (one wave per
// SIMD cannot hide the LDS and MFMA latencies that two waves per SIMD do).
#pragma once

#include "igemm_common.hpp"
#include "igemm_pipe.hpp"

namespace convimg {

constexpr int kResThreads = 512;
constexpr int kResWaves = kResThreads / 64;
constexpr int kResScrRow = 36;                                 // floats per pixel row of the store scratch
constexpr int kResScrBytes = kResWaves * 32 * kResScrRow * 4;  // one 32-pixel x 32-channel block per wave
#ifndef CONVIMG_RES_PF
#define CONVIMG_RES_PF 1
#endif
constexpr int kResPF = CONVIMG_RES_PF;     // k steps whose fragments are in flight ahead of the MFMAs
constexpr int kResNchwRounds = 2;          // NCHW x: 8 x 8 blocks a thread (the plan checks the rows fit)

// Layouts of x and out: NHWC with fp32 out (the forward's), or NCHW with
// fp32 or bf16 out.
constexpr int kResNhwc = 0, kResNchwF32 = 1, kResNchwBf16 = 2;

// NT: taps (KH * KW); CPS: 16-wide k steps per tap (IC / 16).
template <int NT, int CPS, int LAYOUT = kResNhwc>
__global__ __launch_bounds__(kResThreads, 1) void igemm_resident_bf16(ConvArgs a)
{
    extern __shared__ u32x4_t dsm[];
    char *const lds = (char *)dsm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lk = lane >> 5;
    const int lr = lane & 31;
    // the arguments the set-up reads, loaded in one batch: the compiler
    // otherwise loads them as they are needed, one dependent round trip
    // after another
    asm volatile("" ::"s"(a.tiles_m), "s"(a.tiles_n), "s"(a.M), "s"(a.IC), "s"(a.H), "s"(a.W), "s"(a.K),
                 "s"(a.stride), "s"(a.pad), "s"(a.dil), "s"(a.OH), "s"(a.OW), "s"(a.KH), "s"(a.x), "s"(a.w),
                 "s"(a.x_bytes), "s"(a.w_bytes), "s"(a.lds_rows), "s"(a.res_zero), "s"(a.OC), "s"(a.bias));
    // ranges in XCD order: neighbouring ranges share input rows, which then
    // meet in one L2 (the grid: tiles_m ranges per 64-channel slice)
    const int bid = xcd_remap(blockIdx.x, a.tiles_m * a.tiles_n);
    const int gn = bid / a.tiles_m;
    const int gm = bid - gn * a.tiles_m;
    const int n0 = gn * 64;
    const int per = a.M / a.tiles_m, extra = a.M - per * a.tiles_m;
    const int m_a = gm * per + min(gm, extra);
    const int m_b = m_a + per + (gm < extra ? 1 : 0);
    if (m_a >= m_b)
        return;
    const int IC = a.IC, H = a.H, W = a.W, K = a.K;
    const int s = a.stride, p = a.pad, d = a.dil;
    const int ohw = a.OH * a.OW;
    // input rows of the range: first tap row of its first output row to the
    // last tap row of its last output row (rows between, of any image, too)
    int g_lo, g_hi;
    {
        const int n_a = m_a / ohw, oh_a = (m_a - n_a * ohw) / a.OW;
        const int n_b = (m_b - 1) / ohw, oh_b = (m_b - 1 - n_b * ohw) / a.OW;
        g_lo = n_a * H + max(oh_a * s - p, 0);
        g_hi = n_b * H + min(oh_b * s - p + (a.KH - 1) * d, H - 1);
    }
    const int nrows = max(g_hi - g_lo + 1, 0);      // the plan sized LDS for the largest range
    const int wchunks = K / 8 + 1;
    const int wrec = 16 * wchunks;
    const int pchunks = IC / 8 + 1;
    const int prec = 16 * pchunks;
    char *const rows = lds + a.lds_rows;
    char *const zero = lds + a.res_zero;
    // ---- prologue: weight records, then pixel records; slot q of a region
    // is its q-th 16-byte chunk (copy instruction q / 64, lane q % 64).  The
    // address arithmetic uses float-reciprocal divisions and 24-bit products
    // (the plan keeps x and w under 2 GB): the copies wait on it.  A weight
    // row at or past OC lies past the end of w and reads zeros.
    {
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)a.w, 0, a.w_bytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
        const int wins = wchunks;
        const int rins = (nrows * W * pchunks + 63) / 64;
        const float inv_wch = __builtin_amdgcn_rcpf((float)wchunks);
        const float inv_pch = __builtin_amdgcn_rcpf((float)pchunks);
        const unsigned wbase = (unsigned)n0 * (unsigned)K * 2u;
        const unsigned xbase = (unsigned)g_lo * (unsigned)W * (unsigned)IC * 2u;
        const int npx = nrows * W;
        // NCHW x: a lane takes 8 channels (block cb) of 8 pixels (group pg,
        // within one row: W % 8 == 0) of the range's rows, eight 16-byte
        // loads from the channel planes; blocks numbered cb fastest, so 16
        // consecutive lanes write 16 distinct bank groups.  All loads are
        // issued before the weight copies; the transposed writes follow
        // them (the plan's LDS rows hold at most kResThreads * kResNchwRounds
        // blocks).
        constexpr int CB = 2 * CPS;
        u32x4_t xv[LAYOUT != kResNhwc ? kResNchwRounds : 1][8];
        int xrec[LAYOUT != kResNhwc ? kResNchwRounds : 1];
        if constexpr (LAYOUT != kResNhwc) {
            const int nblk = (npx >> 3) * CB;
            const unsigned plane = (unsigned)(H * W) * 2u;
            const float inv_w = __builtin_amdgcn_rcpf((float)W), inv_h = __builtin_amdgcn_rcpf((float)H);
            const int n_lo = g_lo / H, ih_lo = g_lo - n_lo * H;
#pragma unroll
            for (int r = 0; r < kResNchwRounds; ++r) {
                const int q = r * kResThreads + tid;
                const int cb = q & (CB - 1), px0 = 8 * (q / CB);
                const int gr = small_div(px0, inv_w), iw0 = px0 - gr * W;
                const int t = small_div(ih_lo + gr, inv_h);
                const int n = n_lo + t, ih = ih_lo + gr - t * H;
                const bool ok = q < nblk;
                xrec[r] = ok ? a.lds_rows + px0 * prec + 16 * cb : -1;
                const unsigned off = 2u * ((unsigned)((n * IC + 8 * cb) * H + ih) * (unsigned)W + (unsigned)iw0);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    xv[r][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? off + (unsigned)j * plane : kOutOfRange,
                                                                     0, 0);
            }
        }
        for (int i = wave; i < (LAYOUT == kResNhwc ? wins + rins : wins); i += kResWaves) {
            if (i < wins) {
                const int q = i * 64 + lane;
                const int r = small_div(q, inv_wch), c = q - (int)__umul24(r, wchunks);
                dma16(rw, dsm + i * 64, c < K / 8 ? wbase + __umul24(r, 2u * K) + 16u * c : kOutOfRange);
            } else {
                const int j = i - wins;
                const int q = j * 64 + lane;
                const int px = small_div(q, inv_pch), c = q - (int)__umul24(px, pchunks);
                const bool ok = c < IC / 8 && px < npx;
                dma16(rx, (u32x4_t *)rows + j * 64, ok ? xbase + __umul24(px, 2u * IC) + 16u * c : kOutOfRange);
            }
        }
        if (tid < pchunks)
            ((u32x4_t *)zero)[tid] = u32x4_t{0u, 0u, 0u, 0u};
        if constexpr (LAYOUT != kResNhwc) {
            wait_vmcnt<0>();
#pragma unroll
            for (int r = 0; r < kResNchwRounds; ++r) {
                if (xrec[r] < 0)
                    continue;
                u32x4_t t[8];
                transpose8x8(xv[r], t);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *(u32x4_t *)(lds + xrec[r] + e * prec) = t[e];
            }
        }
    }
    float bv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int oc = n0 + j * 32 + lr;
        bv[j] = (a.bias != nullptr && oc < a.OC) ? a.bias[oc] : 0.f;
    }
    wait_vmcnt<0>();
    __syncthreads();
    if constexpr (LAYOUT != kResNhwc) {
        // The weights came in OIHW order: record oc holds w[oc][ic][t] at
        // element 9 ic + t.  Reorder each record in place to element
        // t IC + ic (the OHWI record the k steps read).  A task is the
        // channel pair 2p, 2p + 1 of one record: its 18 elements are the 9
        // dwords at byte 36 p, and output dword t pairs (2p, t) with
        // (2p + 1, t), at byte 2 (t IC + 2p).  Every read completes before
        // any write.
        static_assert(NT == 9, "the NCHW variant serves 3x3 kernels");
        constexpr int ICN = 16 * CPS, PAIRS = ICN / 2, NTASK = 64 * PAIRS / kResThreads;
        unsigned d[NTASK][NT];
#pragma unroll
        for (int k = 0; k < NTASK; ++k) {
            const int T = k * kResThreads + tid;
            const char *const src = lds + (T / PAIRS) * wrec + 36 * (T % PAIRS);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                d[k][j] = *(const unsigned *)(src + 4 * j);
        }
        wait_lgkmcnt0();
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NTASK; ++k) {
            const int T = k * kResThreads + tid;
            char *const dst = lds + (T / PAIRS) * wrec + 4 * (T % PAIRS);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *(unsigned *)(dst + 2 * ICN * t) =
                    __builtin_amdgcn_perm(d[k][(NT + t) >> 1], d[k][t >> 1], (t & 1) ? 0x05040302u : 0x07060100u);
        }
        wait_lgkmcnt0();
        __syncthreads();
    }
    if (a.res_flipw) {
        // The data backward's mapped problem, its weights copied as the
        // forward's are (64 x 64 channels): record oc holds w[oc][t][ic].
        // Flip and transpose them in place, so that record ic holds, at tap
        // NT - 1 - t, w[oc][t][ic] for oc = 0 .. 63: the mapped problem's
        // weights (the transform a separate launch would otherwise write).
        // The 64 x 64 x NT elements are 64 NT tiles of 4 (oc) x 16 (ic),
        // one per 16-lane group and read: ds_read_b64_tr_b16 gives lane l
        // the 4 rows oc .. oc + 3 of column ic0 + l, which are 8 contiguous
        // bytes of record ic0 + l.  Every read completes before any write.
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        constexpr int NQ = 2 * NT;                  // reads a wave (64 NT tiles over 8 waves x 4 groups)
        const int G = lane >> 4, r = lane & 15;
        v4i16 v[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int T = (wave * NQ + q) * 4 + G;
            const int t = T >> 6, ocq = (T >> 2) & 15, icb = T & 3;
            v[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(
                lds + (4 * ocq + (r >> 2)) * wrec + 2 * (64 * t + 16 * icb + 4 * (r & 3))));
        }
        wait_lgkmcnt0();
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int T = (wave * NQ + q) * 4 + G;
            const int t = T >> 6, ocq = (T >> 2) & 15, icb = T & 3;
            *(v4i16 *)(lds + (16 * icb + r) * wrec + 2 * (64 * (NT - 1 - t) + 4 * ocq)) = v[q];
        }
        wait_lgkmcnt0();
        __syncthreads();
    }
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.out_bytes, kRsrcWord3);
    // units of 32 pixels from the range's start; in NCHW order from the
    // 32-pixel boundary at or before it, so that where OH * OW % 32 == 0 a
    // whole unit's run of each channel is one aligned 128-byte line (fp32)
    // or half of one (bf16).  Pixels of a unit outside the range are
    // computed from an in-range pixel and never stored.
    const int ubase = LAYOUT == kResNhwc ? m_a : (m_a & ~31);
    const int nunits = (m_b - ubase + 31) / 32;
    const float inv_ohw = __builtin_amdgcn_rcpf((float)ohw), inv_ow = __builtin_amdgcn_rcpf((float)a.OW);
    // this lane's part of each output offset: row 4 lk of a unit, channel lr
    const unsigned lane_out = 4u * (__umul24(4 * lk, a.OC) + (unsigned)lr);
    // B fragment of step st = tap * CPS + c: weight record j*32 + lr, bytes 32 st + 16 lk
    const char *const b0 = lds + lr * wrec + 16 * lk;
    const char *const b1 = b0 + 32 * wrec;
    for (int u = wave; u < nunits; u += kResWaves) {
        const int m0 = ubase + 32 * u;
        // this lane's output pixel (past the range: any pixel, never stored)
        const int m = min(max(m0 + lr, m_a), m_b - 1);
        const int n = small_div(m, inv_ohw);
        const int rem = m - (int)__umul24(n, ohw);
        const int oh = small_div(rem, inv_ow);
        const int ow = rem - (int)__umul24(oh, a.OW);
        int tap[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int kh = t / a.KW, kw = t - kh * a.KW;
            const int ih = oh * s - p + kh * d, iw = ow * s - p + kw * d;
            const bool ok = (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W;
            tap[t] = (ok ? a.lds_rows + (int)__umul24(__umul24(n * H + ih - g_lo, W) + iw, prec) : a.res_zero) + 16 * lk;
        }
        // even and odd k steps go to separate accumulators: four independent
        // MFMA chains per wave, so a wave that runs alone on its SIMD (the
        // other has no unit left) still issues back to back
        floatx16_t acc0 = floatx16_t{}, acc1 = floatx16_t{}, acc2 = floatx16_t{}, acc3 = floatx16_t{};
        // step st = t * CPS + c: A at tap record t + 32 c, B at 32 st; the
        // next step's fragments load during this step's MFMAs
        auto afrag = [&](int st) {
            return __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(lds + tap[st / CPS] + 32 * (st % CPS)));
        };
        auto bfrag = [&](const char *b, int st) {
            return __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(b + 32 * st));
        };
        // fragments of step st live in slot st % (PF + 1): steps st+1 ..
        // st+PF are in flight while step st multiplies
        constexpr int NS = NT * CPS;
        bf16x8_t fa[kResPF + 1], fb0[kResPF + 1], fb1[kResPF + 1];
#pragma unroll
        for (int st = 0; st < kResPF && st < NS; ++st) {
            fa[st] = afrag(st);
            fb0[st] = bfrag(b0, st);
            fb1[st] = bfrag(b1, st);
        }
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            constexpr int R = kResPF + 1;
            if (st + kResPF < NS) {
                fa[(st + kResPF) % R] = afrag(st + kResPF);
                fb0[(st + kResPF) % R] = bfrag(b0, st + kResPF);
                fb1[(st + kResPF) % R] = bfrag(b1, st + kResPF);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (st % 2 == 0) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st % R], fb0[st % R], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st % R], fb1[st % R], acc1, 0, 0, 0);
            } else {
                acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st % R], fb0[st % R], acc2, 0, 0, 0);
                acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st % R], fb1[st % R], acc3, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        acc0 += acc2;
        acc1 += acc3;
        if constexpr (LAYOUT != kResNhwc) {
            // NCHW: value v of block j is channel oc = n0 + 32 j + lr at pixel
            // m0 + 8 (v >> 2) + 4 lk + (v & 3).
            constexpr int ES = LAYOUT == kResNchwBf16 ? 2 : 4;
            if (a.res_scr >= 0) {
                // Through this wave's scratch, channel-major (36 floats a
                // channel: the 16 lanes of a 128-bit write pass fall on 16
                // distinct bank groups), read back as 16 bytes a lane: 4
                // (fp32) or 8 (bf16) consecutive pixels of one channel.  A
                // unit wholly inside the range, in one image, on a 32-pixel
                // boundary of it (OH * OW % 32 == 0) stores 16 bytes a lane:
                // whole lines (fp32, streaming stores) or half lines (bf16,
                // the default policy: streaming stores of partial lines cost
                // more than the kernel's MFMAs here); other units store
                // element by element, their lines shared with the
                // neighbouring range's first or last unit.
                float *const scr = (float *)(lds + a.res_scr) + wave * (32 * kResScrRow);
                const bool full = m0 >= m_a && m0 + 32 <= m_b && ohw % 32 == 0;
                const int nu = small_div(max(m0, m_a), inv_ohw);
                const int p0 = m0 - (int)__umul24(nu, ohw);
                constexpr int LPC = ES == 4 ? 8 : 4;          // lanes a channel run
                constexpr int PPL = 32 / LPC;                 // pixels a lane
                const int cl = lane / LPC, q = lane % LPC;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const floatx16_t &acc = j == 0 ? acc0 : acc1;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *(floatx4_t *)(scr + lr * kResScrRow + 8 * i + 4 * lk) =
                            floatx4_t{acc[4 * i] + bv[j], acc[4 * i + 1] + bv[j], acc[4 * i + 2] + bv[j],
                                      acc[4 * i + 3] + bv[j]};
#pragma unroll
                    for (int i = 0; i < 32 / (64 / LPC); ++i) {
                        const int c = i * (64 / LPC) + cl;
                        const int oc = n0 + 32 * j + c;
                        float v[PPL];
#pragma unroll
                        for (int h4 = 0; h4 < PPL / 4; ++h4) {
                            const floatx4_t t = *(const floatx4_t *)(scr + c * kResScrRow + PPL * q + 4 * h4);
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                v[4 * h4 + b] = t[b];
                        }
                        if (full) {
                            const unsigned off = oc < a.OC
                                ? ES * ((unsigned)(nu * a.OC + oc) * (unsigned)ohw + (unsigned)(p0 + PPL * q))
                                : kOutOfRange;
                            u32x4_t val;
                            if constexpr (ES == 2) {
#pragma unroll
                                for (int b = 0; b < 4; ++b)
                                    val[b] = (unsigned)bf16_rne(v[2 * b]) | ((unsigned)bf16_rne(v[2 * b + 1]) << 16);
                            } else {
#pragma unroll
                                for (int b = 0; b < 4; ++b)
                                    val[b] = __float_as_uint(v[b]);
                            }
                            // streaming where the unit's run is a whole line
                            if constexpr (ES == 4)
                                __builtin_amdgcn_raw_buffer_store_b128(val, ro, off, 0, kOutAux);
                            else
                                __builtin_amdgcn_raw_buffer_store_b128(val, ro, off, 0, 0);
                        } else {
#pragma unroll
                            for (int b = 0; b < PPL; ++b) {
                                const int mm = m0 + PPL * q + b;
                                const int nb = small_div(min(max(mm, m_a), m_b - 1), inv_ohw);
                                const int pb = mm - (int)__umul24(nb, ohw);
                                const unsigned off = (mm >= m_a && mm < m_b && oc < a.OC)
                                    ? ES * ((unsigned)(nb * a.OC + oc) * (unsigned)ohw + (unsigned)pb) : kOutOfRange;
                                if constexpr (ES == 2)
                                    __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(v[b]), ro, off, 0, 0);
                                else
                                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[b]), ro, off, 0, 0);
                            }
                        }
                    }
                }
                continue;
            }
            // else from the accumulators: values 4 i .. 4 i + 3 are 4
            // consecutive pixels; one 16-byte (fp32) or 8-byte (bf16) store
            // where they lie inside the range, in one image, on a 4-pixel
            // boundary of it (out is 16-byte aligned), else one element at
            // a time; default policy (the pieces of a line meet in L2).
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mq = m0 + 8 * i + 4 * lk;
                const int nq = small_div(min(max(mq, m_a), m_b - 1), inv_ohw);
                const int pq = mq - (int)__umul24(nq, ohw);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int oc = n0 + 32 * j + lr;
                    const floatx16_t &acc = j == 0 ? acc0 : acc1;
                    float v[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        v[b] = acc[4 * i + b] + bv[j];
                    if (mq >= m_a && mq + 3 < m_b && oc < a.OC && (pq & 3) == 0 && pq + 3 < ohw) {
                        const unsigned off = ES * ((unsigned)(nq * a.OC + oc) * (unsigned)ohw + (unsigned)pq);
                        if constexpr (ES == 2) {
                            const unsigned lo = (unsigned)bf16_rne(v[0]) | ((unsigned)bf16_rne(v[1]) << 16);
                            const unsigned hi = (unsigned)bf16_rne(v[2]) | ((unsigned)bf16_rne(v[3]) << 16);
                            typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
                            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, ro, off, 0, 0);
                        } else {
                            __builtin_amdgcn_raw_buffer_store_b128(
                                u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                        __float_as_uint(v[3])},
                                ro, off, 0, 0);
                        }
                    } else {
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const int mm = mq + b;
                            const int nb = small_div(min(max(mm, m_a), m_b - 1), inv_ohw);
                            const int pb = mm - (int)__umul24(nb, ohw);
                            const unsigned off = (mm >= m_a && mm < m_b && oc < a.OC)
                                ? ES * ((unsigned)(nb * a.OC + oc) * (unsigned)ohw + (unsigned)pb) : kOutOfRange;
                            if constexpr (ES == 2)
                                __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(v[b]), ro, off, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[b]), ro, off, 0, 0);
                        }
                    }
                }
            }
            continue;
        }
        // value v of block j: pixel m0 + 8*(v >> 2) + 4*lk + (v & 3), channel
        // n0 + j*32 + lr
        if (a.res_scr >= 0) {
            // through this wave's scratch: block j written pixel-major (36
            // floats a pixel: the lane halves, 4 pixels apart, share 16 of
            // 64 banks, the two pixels a 16-lane read serves share 4), then
            // read back as 16 bytes a lane: lane group g = lane / 8 takes
            // pixel 8 i + g, channels 4 (lane & 7) .. +4.  One wave's LDS
            // operations complete in order, so block 1's writes follow
            // block 0's reads.
            float *const scr = (float *)(lds + a.res_scr) + wave * (32 * kResScrRow);
            const int q4 = 4 * (lane & 7);
            const int px0 = lane >> 3;
            const unsigned vbase = 4u * ((unsigned)(m0 + px0) * (unsigned)a.OC + (unsigned)(n0 + q4));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    scr[(8 * (v >> 2) + 4 * lk + (v & 3)) * kResScrRow + lr] = (j == 0 ? acc0[v] : acc1[v]) + bv[j];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int px = 8 * i + px0;
                    const u32x4_t val = *(const u32x4_t *)(scr + px * kResScrRow + q4);
                    const unsigned off = (m0 + px < m_b && n0 + 32 * j + q4 < a.OC)
                        ? vbase + 4u * (unsigned)(8 * i * a.OC + 32 * j) : kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b128(val, ro, off, 0, kOutAux);
                }
            }
            continue;
        }
        // else one dword a lane per value, at ubase + lane_out + 4 ((8 (v >> 2) + (v & 3)) OC + 32 j)
        const unsigned ubase = 4u * ((unsigned)m0 * (unsigned)a.OC + (unsigned)n0) + lane_out;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int mv = m0 + 8 * (v >> 2) + 4 * lk + (v & 3);
            const unsigned vofs = 4u * (unsigned)((8 * (v >> 2) + (v & 3)) * a.OC);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int oc = n0 + j * 32 + lr;
                const unsigned off = (mv < m_b && oc < a.OC) ? ubase + vofs + 128u * j : kOutOfRange;
                const float val = (j == 0 ? acc0[v] : acc1[v]) + bv[j];
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, val), ro, off, 0, kOutAux);
            }
        }
    }
}

}  // namespace convimg
