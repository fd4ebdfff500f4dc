// igemm_pipe.hpp -- implicit-GEMM kernel with a multi-stage direct-to-LDS
// pipeline (vector loaders: IC a multiple of 64 or of 8, 16-byte aligned
// buffers smaller than 2 GB).
//
// gfx950 can load 16 bytes per lane from a buffer straight into LDS
// (buffer_load_dwordx4 ... lds): lane l of a wave writes bytes
// [16*l, 16*l + 16) after the wave's LDS base, and an offset past the
// buffer's extent writes zeros.  So the im2col gather costs no registers,
// and the padding / tail masking is an out-of-range offset:
//   * one wave instruction fills a contiguous 1 KB block = 8 LDS rows of 8
//     chunks; lane l fills row 8 b + (l >> 3) (b: the block's index), physical
//     chunk (l & 7), so it loads logical chunk (l & 7) ^ ((row >> 1) & 7) of
//     that row (the XOR swizzle is applied on the global side);
//   * STAGES LDS buffers: K tiles t+1 .. t+STAGES-1 are in flight while the
//     waves read K tile t from LDS and run MFMA on it (the rocMLIR PR "Double
//     buffering improvements" splits LDS reads and matrix ops into
//     overlapping stages; here the global->LDS copies are a third stage, and
//     deeper);
//   * one barrier per K tile: each wave waits (vmcnt) for its own copies of
//     tile t, the barrier then publishes every wave's copies and certifies
//     that every wave has finished reading tile t-1, whose buffer the next
//     copies overwrite.  The barrier is the bare s_barrier, so the compiler
//     adds no wait for the copies still in flight.
#pragma once

#include "igemm_common.hpp"

namespace convimg {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt 7 and lgkmcnt 15
// mean "do not wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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

// s_waitcnt lgkmcnt(0): this wave's LDS reads and writes have completed.
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

__device__ __forceinline__ void lds_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // no compiler motion of LDS accesses across
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}


// floor(x / d) for 0 <= x < 2^21, inv = v_rcp_f32(d): the quotient of
// x + 0.5 is at least 0.5 / d from an integer, and its float error is below
// that for such x.
__device__ __forceinline__ int small_div(int x, float inv)
{
    return (int)(((float)x + 0.5f) * inv);
}

// floor(x / 9) for 0 <= x < 16384 (7282 / 65536 exceeds 1/9 by under
// 1/16384 per unit of x).
__device__ __forceinline__ int div9(int x)
{
    return (int)(__umul24(x, 7282u) >> 16);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, u32x4_t *lds, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds,
                                             16, off, 0, 0, 0);
}

// MS: MFMA block size, 16 (v_mfma_f32_16x16x32_bf16) or 32
// (v_mfma_f32_32x32x16_bf16).
template <int MS>
struct Mfma;

template <>
struct Mfma<16> {
    typedef floatx4_t acc_t;
    static constexpr int kstep = 32;
    __device__ static __forceinline__ acc_t run(bf16x8_t a, bf16x8_t b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mfma<32> {
    typedef floatx16_t acc_t;
    static constexpr int kstep = 16;
    __device__ static __forceinline__ acc_t run(bf16x8_t a, bf16x8_t b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <int BM, int BN, int WM, int WN, int STAGES, int MS, int LOADER>
__global__ __launch_bounds__(WM * WN * 64) void igemm_pipe_bf16(ConvArgs a)
{
    typedef Mfma<MS> MF;
    typedef typename MF::acc_t acc_t;
    constexpr int NW = WM * WN;
    constexpr int NT = NW * 64;
    constexpr int WTM = BM / WM;
    constexpr int WTN = BN / WN;
    constexpr int FM = WTM / MS;
    constexpr int FN = WTN / MS;
    constexpr int KSTEPS = kBK / MF::kstep;     // MFMA k steps per K tile
    constexpr int LGRP = MS;                    // lanes per k chunk group
    constexpr int RPP = NT / 8;                 // LDS rows one pass of all lanes fills
    constexpr int AP = BM / RPP;                // copies per lane per stage, A
    constexpr int BP = BN / RPP;                // copies per lane per stage, B
    constexpr int A_CH = BM * kChunks;
    constexpr int STAGE_CH = (BM + BN) * kChunks;
    constexpr int PER_STAGE = AP + BP;
    static_assert(LOADER == kLoaderTap || LOADER == kLoaderVec8, "vector loaders only");
    static_assert(WTM % MS == 0 && WTN % MS == 0, "wave tile must hold whole MFMA blocks");
    static_assert(BM % RPP == 0 && BN % RPP == 0, "a pass fills whole rows");
    static_assert(STAGES >= 2 && (STAGES - 2) * PER_STAGE < 64, "vmcnt range");

    __shared__ u32x4_t smem[STAGES * STAGE_CH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // (uniform: the copies' LDS addresses are then scalar, with no
    // readfirstlane per copy instruction)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;
    const int wn = wave / WM;

    const TileCoord tc = tile_coord<BM, BN>(a);
    if (!tc.valid)
        return;
    const int m0 = tc.m0, n0 = tc.n0;
    const int kt_begin = tc.kt_begin;
    const int nk = tc.kt_end - tc.kt_begin;

    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)a.w, 0, a.w_bytes, kRsrcWord3);

    const int lrow = lane % LGRP;               // row / column of an MFMA block this lane feeds
    const int lchk = lane / LGRP;               // k chunk within an MFMA k step

    // ---- the rows this lane copies: row (pass * RPP + wave * 8 + lane / 8).
    // RPP is a multiple of 16, so bits 1..3 of the row are those of
    // wave * 8 + lane / 8: the logical chunk is the same for every pass.
    const int lr = lane >> 3;
    const int cl = (lane & 7) ^ ((4 * (wave & 1)) | (lr >> 1));   // logical chunk this lane loads
    static_assert(RPP % 16 == 0, "rows of one pass keep bits 1..3 of the row");
    const int OHW = a.OH * a.OW;
    // xbase[j]: byte offset of this lane's chunk of row j at tap (0, 0),
    // channel 0 (negative where the tap falls in the top or left padding);
    // the tap-aligned loader adds one per-tile scalar to it, with no
    // multiply per copy
    // (the row decode divides by the host's multiply-shift constants: an
    // integer division by a run-time value is a chain of quarter-rate
    // multiplies, and all of it comes before the first copy)
    int xoff[AP], ih0[AP], iw0[AP], xbase[AP];
    bool mok[AP];
#pragma unroll
    for (int j = 0; j < AP; ++j) {
        const int m = m0 + j * RPP + wave * 8 + lr;
        mok[j] = m < a.M;
        const int mm = mok[j] ? m : 0;
        const int n = fast_div(mm, a.div_ohw);
        const int r = mm - n * OHW;
        const int oh = fast_div(r, a.div_ow);
        const int ow = r - oh * a.OW;
        xoff[j] = n * a.H * a.W * a.IC;
        ih0[j] = oh * a.stride - a.pad;
        iw0[j] = ow * a.stride - a.pad;
        xbase[j] = 2 * (xoff[j] + (ih0[j] * a.W + iw0[j]) * a.IC + cl * 8);
    }
    int woff[BP];
    bool wok[BP];
#pragma unroll
    for (int j = 0; j < BP; ++j) {
        const int oc = n0 + j * RPP + wave * 8 + lr;
        wok[j] = oc < a.OC;
        woff[j] = wok[j] ? oc * a.K : 0;
    }

    // tap-aligned loader state (IC % 64 == 0): tap (kh, kw), channel c0
    int t_kh = 0, t_kw = 0, t_c0 = 0;
    if (LOADER == kLoaderTap) {
        const int kflat = kt_begin * kBK;
        const int tap = kflat / a.IC;
        t_c0 = kflat - tap * a.IC;
        t_kh = tap / a.KW;
        t_kw = tap - t_kh * a.KW;
    }

    // Issue the copies of K tile kt into LDS stage `st`.  Tiles are issued in
    // increasing kt, which the tap-aligned state relies on.
    auto issue = [&](int kt, int st) {
        u32x4_t *sa = smem + st * STAGE_CH + wave * 64;
        u32x4_t *sb = smem + st * STAGE_CH + A_CH + wave * 64;
        int dh, dw, cofs;
        bool okk;
        const int k = kt * kBK + cl * 8;
        if (LOADER == kLoaderTap) {
            dh = t_kh * a.dil;
            dw = t_kw * a.dil;
            cofs = t_c0 + cl * 8;
            okk = true;
            t_c0 += kBK;
            if (t_c0 == a.IC) {
                t_c0 = 0;
                if (++t_kw == a.KW) {
                    t_kw = 0;
                    ++t_kh;
                }
            }
        } else {
            okk = k < a.K;
            const int tap = k / a.IC;
            cofs = k - tap * a.IC;
            const int kh = tap / a.KW;
            dh = kh * a.dil;
            dw = (tap - kh * a.KW) * a.dil;
        }
        // tap-aligned: the tap's row and column shift and the channel block
        // are the same for every lane (one scalar); else per lane
        const int sdelta = LOADER == kLoaderTap ? 2 * ((dh * a.W + dw) * a.IC + cofs - cl * 8) : 0;
#pragma unroll
        for (int j = 0; j < AP; ++j) {
            const int ih = ih0[j] + dh, iw = iw0[j] + dw;
            const bool ok = okk && mok[j] && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
            const unsigned off = !ok ? kOutOfRange
                : LOADER == kLoaderTap ? (unsigned)(xbase[j] + sdelta)
                                       : 2u * (unsigned)(xoff[j] + (ih * a.W + iw) * a.IC + cofs);
            dma16(rx, sa + j * RPP * kChunks, off);
        }
#pragma unroll
        for (int j = 0; j < BP; ++j) {
            const unsigned off = (okk && wok[j]) ? 2u * (unsigned)(woff[j] + k) : kOutOfRange;
            dma16(rw, sb + j * RPP * kChunks, off);
        }
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = acc_t{};

    // Fragments of k step ks+1 are read from LDS before the MFMAs of k step
    // ks are issued, so LDS latency overlaps matrix work within the wave.
    auto load_frags = [&](const u32x4_t *sa, const u32x4_t *sb, int ks, bf16x8_t (&af)[FM],
                          bf16x8_t (&bfg)[FN]) {
        const int ck = ks * (64 / LGRP) + lchk;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = __builtin_bit_cast(bf16x8_t, sa[swz(wm * WTM + i * MS + lrow, ck)]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bfg[j] = __builtin_bit_cast(bf16x8_t, sb[swz(wn * WTN + j * MS + lrow, ck)]);
    };
    auto compute = [&](int st) {
        const u32x4_t *sa = smem + st * STAGE_CH;
        const u32x4_t *sb = sa + A_CH;
        bf16x8_t af[2][FM], bfg[2][FN];
        load_frags(sa, sb, 0, af[0], bfg[0]);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if (ks + 1 < KSTEPS)
                load_frags(sa, sb, ks + 1, af[(ks + 1) & 1], bfg[(ks + 1) & 1]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = MF::run(af[ks & 1][i], bfg[ks & 1][j], acc[i][j]);
        }
    };

    // ---- pipeline
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk)
            issue(kt_begin + s, s);

    // Bias through a bounds-checked buffer load (no branch; a missing bias is
    // a buffer of extent 0, which reads as zeros), issued after the prologue
    // copies so that its latency hides under theirs.
    const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.bias, 0, (a.bias != nullptr && tc.split == 0) ? a.OC * 4 : 0, kRsrcWord3);
    float bv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int oc = n0 + wn * WTN + j * MS + lrow;
        bv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              rbias, oc < a.OC ? 4u * oc : kOutOfRange, 0, 0));
    }

    for (int i = 0; i < nk; ++i) {
        if (i + STAGES - 2 < nk)
            wait_vmcnt<(STAGES - 2) * PER_STAGE>();   // tile i landed; later tiles may not have
        else
            wait_vmcnt<0>();
        lds_barrier();
        if (i + STAGES - 1 < nk)
            issue(kt_begin + i + STAGES - 1, (i + STAGES - 1) % STAGES);
        compute(i % STAGES);
    }

    if (a.splits == 1 && a.vec_out) {
        static_assert(NW * EpiScratch<MS, WTN>::floats * 4 <= (int)sizeof(smem), "epilogue scratch");
        __syncthreads();    // every wave is done reading the last stage
        store_tile_vec<MS, FM, FN, WTN>(a, acc, bv, m0 + wm * WTM, n0 + wn * WTN,
                                        (float *)smem + wave * EpiScratch<MS, WTN>::floats);
        return;
    }
    store_tile<MS, FM, FN>(a, acc, bv, m0 + wm * WTM + acc_row0<MS>(lane),
                           n0 + wn * WTN + acc_col0<MS>(lane), tc.split, tc.tile);
}

}  // namespace convimg
