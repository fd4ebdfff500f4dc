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

// NT: taps (KH * KW); CPS: 16-wide k steps per tap (IC / 16).
template <int NT, int CPS>
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
        for (int i = wave; i < wins + rins; i += kResWaves) {
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
    }
    float bv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int oc = n0 + j * 32 + lr;
        bv[j] = (a.bias != nullptr && oc < a.OC) ? a.bias[oc] : 0.f;
    }
    wait_vmcnt<0>();
    __syncthreads();
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
    const int nunits = (m_b - m_a + 31) / 32;
    const float inv_ohw = __builtin_amdgcn_rcpf((float)ohw), inv_ow = __builtin_amdgcn_rcpf((float)a.OW);
    // this lane's part of each output offset: row 4 lk of a unit, channel lr
    const unsigned lane_out = 4u * (__umul24(4 * lk, a.OC) + (unsigned)lr);
    // B fragment of step st = tap * CPS + c: weight record j*32 + lr, bytes 32 st + 16 lk
    const char *const b0 = lds + lr * wrec + 16 * lk;
    const char *const b1 = b0 + 32 * wrec;
    for (int u = wave; u < nunits; u += kResWaves) {
        const int m0 = m_a + 32 * u;
        // this lane's output pixel (past the range: any pixel, never stored)
        const int m = min(m0 + lr, m_b - 1);
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
