// igemm_regs.hpp -- register-staged implicit-GEMM kernels.
//
// The general kernel of the family: any channel count (including the
// element-wise gather of the masked edge path, e.g. IC = 3 with K = 147),
// any alignment, any buffer size.  Global loads of K tile t+1 go to
// registers while the waves run MFMA on K tile t from LDS, then are written
// to the other of two LDS buffers; one barrier per K tile (LDS reads and
// matrix operations as overlapping stages, the structure of the rocMLIR PR
// "Double buffering improvements").  Also the fp32-storage kernel.
#pragma once

#include "igemm_common.hpp"

namespace convimg {

constexpr int kRegsThreads = 256;   // 4 waves of 64

// ---------------------------------------------------------------------------
// bf16 implicit GEMM.  BM x BN tile, WAVES_M x (4 / WAVES_M) waves.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WAVES_M, int LOADER>
__global__ __launch_bounds__(kRegsThreads) void igemm_regs_bf16(ConvArgs a)
{
    constexpr int WAVES_N = 4 / WAVES_M;
    constexpr int WTM = BM / WAVES_M;
    constexpr int WTN = BN / WAVES_N;
    constexpr int FM = WTM / 16;
    constexpr int FN = WTN / 16;
    constexpr int AR = BM / 32;     // A rows loaded per thread
    constexpr int BR = BN / 32;     // B rows loaded per thread
    static_assert(WAVES_M * WAVES_N == 4, "four waves");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must hold 16x16 blocks");
    static_assert(BM % 32 == 0 && BN % 32 == 0, "loader covers 32 rows per pass");

    __shared__ u32x4_t sA[2][BM * kChunks];
    __shared__ u32x4_t sB[2][BN * kChunks];

    const unsigned short *__restrict__ x = (const unsigned short *)a.x;
    const unsigned short *__restrict__ w = (const unsigned short *)a.w;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WAVES_M;
    const int wn = wave / WAVES_M;

    // ---- which tile and which K range
    const TileCoord tc = tile_coord<BM, BN>(a);
    if (!tc.valid)
        return;             // padding slot: the whole workgroup leaves together
    const int split = tc.split, tile = tc.tile, m0 = tc.m0, n0 = tc.n0;
    const int kt_begin = tc.kt_begin, kt_end = tc.kt_end;

    // ---- per-thread gather rows: decode m -> (n, oh, ow) once
    const int cA = tid & 7;         // 16-byte chunk of the row this thread loads
    const int rA = tid >> 3;        // first row (0..31), then +32 per pass
    const int OHW = a.OH * a.OW;
    int xoff[AR], ih0[AR], iw0[AR];
    bool mok[AR];                   // row is a real output pixel (m < M)
#pragma unroll
    for (int j = 0; j < AR; ++j) {
        const int m = m0 + rA + 32 * j;
        mok[j] = m < a.M;
        const int mm = mok[j] ? m : 0;
        const int n = mm / OHW;
        const int r = mm - n * OHW;
        const int oh = r / a.OW;
        const int ow = r - oh * a.OW;
        xoff[j] = n * a.H * a.W * a.IC;
        ih0[j] = oh * a.stride - a.pad;
        iw0[j] = ow * a.stride - a.pad;
    }
    int woff[BR];
    bool wok[BR];
#pragma unroll
    for (int j = 0; j < BR; ++j) {
        const int oc = n0 + rA + 32 * j;
        wok[j] = oc < a.OC;
        woff[j] = wok[j] ? oc * a.K : 0;
    }

    // ---- tap-aligned loader state (IC % 64 == 0): tap (kh, kw), channel c0
    int t_kh = 0, t_kw = 0, t_c0 = 0;
    if (LOADER == kLoaderTap) {
        const int kflat = kt_begin * kBK;
        const int tap = kflat / a.IC;
        t_c0 = kflat - tap * a.IC;
        t_kh = tap / a.KW;
        t_kw = tap - t_kh * a.KW;
    }

    u32x4_t ra[AR], rb[BR];
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};

    auto load_tile = [&](int kt) {
        if (LOADER == kLoaderTap) {
            const int dh = t_kh * a.dil, dw = t_kw * a.dil;
            const int cofs = t_c0 + cA * 8;
#pragma unroll
            for (int j = 0; j < AR; ++j) {
                const int ih = ih0[j] + dh, iw = iw0[j] + dw;
                const bool ok = mok[j] && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
                ra[j] = zero4;
                if (ok)
                    ra[j] = *(const u32x4_t *)(x + xoff[j] + (ih * a.W + iw) * a.IC + cofs);
            }
            const int k = kt * kBK + cA * 8;
#pragma unroll
            for (int j = 0; j < BR; ++j) {
                rb[j] = zero4;
                if (wok[j])
                    rb[j] = *(const u32x4_t *)(w + woff[j] + k);
            }
            // advance to the next 64-channel slice / tap
            t_c0 += kBK;
            if (t_c0 == a.IC) {
                t_c0 = 0;
                if (++t_kw == a.KW) {
                    t_kw = 0;
                    ++t_kh;
                }
            }
        } else if (LOADER == kLoaderVec8) {
            const int k = kt * kBK + cA * 8;
            const bool okk = k < a.K;
            const int tap = k / a.IC;
            const int ic = k - tap * a.IC;
            const int kh = tap / a.KW;
            const int kw = tap - kh * a.KW;
            const int dh = kh * a.dil, dw = kw * a.dil;
#pragma unroll
            for (int j = 0; j < AR; ++j) {
                const int ih = ih0[j] + dh, iw = iw0[j] + dw;
                const bool ok = okk && mok[j] && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
                ra[j] = zero4;
                if (ok)
                    ra[j] = *(const u32x4_t *)(x + xoff[j] + (ih * a.W + iw) * a.IC + ic);
            }
#pragma unroll
            for (int j = 0; j < BR; ++j) {
                rb[j] = zero4;
                if (okk && wok[j])
                    rb[j] = *(const u32x4_t *)(w + woff[j] + k);
            }
        } else {
            // element-wise gather: the 8 k values of this thread's chunk are
            // decoded once and shared by all rows it loads
            const int k0 = kt * kBK + cA * 8;
            int tap = k0 / a.IC;
            int ic = k0 - tap * a.IC;
            int kh = tap / a.KW;
            int kw = tap - kh * a.KW;
            int koff[8], dh[8], dw[8];
            bool okk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                okk[e] = (k0 + e) < a.K;
                dh[e] = kh * a.dil;
                dw[e] = kw * a.dil;
                koff[e] = (dh[e] * a.W + dw[e]) * a.IC + ic;
                if (++ic == a.IC) {
                    ic = 0;
                    if (++kw == a.KW) {
                        kw = 0;
                        ++kh;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < AR; ++j) {
                const int base = xoff[j] + (ih0[j] * a.W + iw0[j]) * a.IC;
                unsigned int v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ih = ih0[j] + dh[e], iw = iw0[j] + dw[e];
                    const bool ok = okk[e] && mok[j] && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
                    const unsigned int h = ok ? (unsigned int)x[base + koff[e]] : 0u;
                    v[e >> 1] |= h << (16 * (e & 1));
                }
                ra[j] = u32x4_t{v[0], v[1], v[2], v[3]};
            }
#pragma unroll
            for (int j = 0; j < BR; ++j) {
                unsigned int v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool ok = okk[e] && wok[j];
                    const unsigned int h = ok ? (unsigned int)w[woff[j] + k0 + e] : 0u;
                    v[e >> 1] |= h << (16 * (e & 1));
                }
                rb[j] = u32x4_t{v[0], v[1], v[2], v[3]};
            }
        }
    };

    auto stage_tile = [&](int buf) {
#pragma unroll
        for (int j = 0; j < AR; ++j)
            sA[buf][swz(rA + 32 * j, cA)] = ra[j];
#pragma unroll
        for (int j = 0; j < BR; ++j)
            sB[buf][swz(rA + 32 * j, cA)] = rb[j];
    };

    floatx4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // Lane l feeds row (l & 15) of a 16x16 block with the 8 consecutive k of
    // chunk (l >> 4) of each 32-wide k step; A and B use the same k chunks,
    // so every product pairs x and w at the same k.
    const int lrow = lane & 15;
    const int lchk = lane >> 4;

    auto compute_tile = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int ck = ks * 4 + lchk;
            bf16x8_t af[FM], bfg[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = __builtin_bit_cast(bf16x8_t, sA[buf][swz(wm * WTM + i * 16 + lrow, ck)]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfg[j] = __builtin_bit_cast(bf16x8_t, sB[buf][swz(wn * WTN + j * 16 + lrow, ck)]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfg[j], acc[i][j], 0, 0, 0);
        }
    };

    // ---- main loop: prefetch K tile t+1 into registers while tile t is
    // consumed from LDS; one barrier per K tile
    if (kt_begin < kt_end) {
        load_tile(kt_begin);
        stage_tile(0);
    }
    __syncthreads();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
        const int buf = (kt - kt_begin) & 1;
        const bool more = kt + 1 < kt_end;
        if (more)
            load_tile(kt + 1);
        compute_tile(buf);
        if (more)
            stage_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue
    float bv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int oc = n0 + wn * WTN + j * 16 + lrow;
        bv[j] = (a.bias != nullptr && oc < a.OC) ? a.bias[oc] : 0.f;
    }
    if (a.splits == 1 && a.vec_out) {
        // the loop's last barrier passed: every wave is done with sA / sB
        static_assert(4 * EpiScratch<16, WTN>::floats * 4 <= (int)sizeof(sA), "epilogue scratch");
        store_tile_vec<16, FM, FN, WTN>(a, acc, bv, m0 + wm * WTM, n0 + wn * WTN,
                                        (float *)&sA[0][0] + wave * EpiScratch<16, WTN>::floats);
        return;
    }
    store_tile<16, FM, FN>(a, acc, bv, m0 + wm * WTM + acc_row0<16>(lane),
                           n0 + wn * WTN + acc_col0<16>(lane), split, tile);
}

// ---------------------------------------------------------------------------
// fp32 storage: the same implicit GEMM with fp32 tiles and
// v_mfma_f32_16x16x4_f32 (products and sums in fp32).  64 x BN tiles (BN =
// 64, or 16 where OC <= 16: four waves of 16 rows then do no dead work on
// channels past OC), no split.
// K goes through LDS in chunks of kF32BK = 144 (a whole 3x3 x 16-channel K
// in one): each chunk's element-wise gathers are all in flight together
// before one barrier, so a small problem pays about one memory round trip
// per chunk instead of one per 16-wide K step.
// ---------------------------------------------------------------------------
constexpr int kF32BM = 64, kF32BN = 64, kF32BNSmall = 16, kF32BK = 144;
constexpr int kF32Row = kF32BK + 1;             // LDS row stride (floats)
constexpr int kF32Cols = kF32BK / 4;            // chunk columns per thread

template <int BN>
__global__ __launch_bounds__(kRegsThreads) void igemm_fwd_f32(ConvArgs a)
{
    // waves WMW x WNW, each FM x FN blocks of 16 x 16
    constexpr int WNW = BN == 64 ? 2 : 1, WMW = 4 / WNW;
    constexpr int FM = kF32BM / (16 * WMW), FN = BN / (16 * WNW);
    __shared__ float sA[kF32BM][kF32Row];
    __shared__ float sB[BN][kF32Row];
    const float *__restrict__ x = (const float *)a.x;
    const float *__restrict__ w = (const float *)a.w;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WMW, wn = wave / WMW;
    const int tm = blockIdx.x % a.tiles_m;
    const int tn = blockIdx.x / a.tiles_m;
    const int m0 = tm * kF32BM, n0 = tn * BN;
    const int OHW = a.OH * a.OW;

    // each thread loads row tid / 4 of the A and B tiles, chunk columns
    // (tid & 3) + 4 j
    const int row = tid >> 2, c0 = tid & 3;
    const int m = m0 + row;
    const bool mok = m < a.M;
    int xoff, ih0, iw0;
    {
        const int mm = mok ? m : 0;
        const int n = mm / OHW;
        const int r = mm - n * OHW;
        const int oh = r / a.OW;
        const int ow = r - oh * a.OW;
        xoff = n * a.H * a.W * a.IC;
        ih0 = oh * a.stride - a.pad;
        iw0 = ow * a.stride - a.pad;
    }
    const int oc_row = n0 + row;
    const bool wok = row < BN && oc_row < a.OC;
    const int woff = wok ? oc_row * a.K : 0;

    floatx4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const int lrow = lane & 15, lchk = lane >> 4;
    // x and w below 2 GiB: buffer loads (masked lanes read zero from past
    // the end); else plain loads guarded per element
    const bool small = a.x_bytes < kOutOfRange && a.w_bytes < kOutOfRange;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)a.w, 0, a.w_bytes, kRsrcWord3);
    for (int k0 = 0; k0 < a.K; k0 += kF32BK) {
        // the whole chunk's loads first (k past K reads as zero).  This
        // thread's k values step by 4: (kh, kw, ic) is decoded once per
        // chunk and then advanced (integer division by a run-time value
        // costs tens of instructions, and there are 36 columns)
        float va[kF32Cols], vb[kF32Cols];
        int ic, kh, kw;
        {
            const int kk = k0 + c0;
            const int tap = kk / a.IC;
            ic = kk - tap * a.IC;
            kh = tap / a.KW;
            kw = tap - kh * a.KW;
        }
        if (small) {
            // buffer loads: a masked lane's offset lies past the buffer and
            // reads zero, so no branch surrounds a load and all 72 go out
            // back to back
#pragma unroll
            for (int j = 0; j < kF32Cols; ++j) {
                const int k = k0 + c0 + 4 * j;
                const bool okk = k < a.K;
                const int ih = ih0 + kh * a.dil, iw = iw0 + kw * a.dil;
                const bool ok = okk && mok && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
                va[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    rx, ok ? 4u * (unsigned)(xoff + (ih * a.W + iw) * a.IC + ic) : kOutOfRange, 0, 0));
                vb[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    rw, (okk && wok) ? 4u * (unsigned)(woff + k) : kOutOfRange, 0, 0));
                ic += 4;
                while (ic >= a.IC) {
                    ic -= a.IC;
                    if (++kw == a.KW) {
                        kw = 0;
                        ++kh;
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kF32Cols; ++j) {
                const int k = k0 + c0 + 4 * j;
                const bool okk = k < a.K;
                const int ih = ih0 + kh * a.dil, iw = iw0 + kw * a.dil;
                const bool ok = okk && mok && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
                va[j] = ok ? x[xoff + (ih * a.W + iw) * a.IC + ic] : 0.f;
                vb[j] = (okk && wok) ? w[woff + k] : 0.f;
                ic += 4;
                while (ic >= a.IC) {
                    ic -= a.IC;
                    if (++kw == a.KW) {
                        kw = 0;
                        ++kh;
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kF32Cols; ++j) {
            sA[row][c0 + 4 * j] = va[j];
            if (row < BN)
                sB[row][c0 + 4 * j] = vb[j];
        }
        __syncthreads();
#pragma unroll 4
        for (int ks = 0; ks < kF32BK / 4; ++ks) {
            float af[FM], bfg[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = sA[wm * 16 * FM + i * 16 + lrow][ks * 4 + lchk];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfg[j] = sB[wn * 16 * FN + j * 16 + lrow][ks * 4 + lchk];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfg[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int oc = n0 + wn * 16 * FN + j * 16 + lrow;
        const float bv = (a.bias != nullptr && oc < a.OC) ? a.bias[oc] : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int mo = m0 + wm * 16 * FM + i * 16 + lchk * 4 + v;
                if (mo < a.M && oc < a.OC)
                    a.out[mo * a.OC + oc] = acc[i][j][v] + bv;
            }
    }
}

}  // namespace convimg
