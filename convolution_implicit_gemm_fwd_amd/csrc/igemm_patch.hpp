// igemm_patch.hpp -- implicit GEMM with the im2col gather done inside LDS.
//
// The A operand of a workgroup's BM output pixels (consecutive m) draws, for
// every tap, on the same few input rows: the tile's output rows times the
// stride plus the kernel's dilated extent.  Gathering A from global memory
// tap by tap (the other kernels) re-reads each input pixel once per tap;
// here each 64-channel slice of those input rows -- the "patch", whole rows,
// all columns -- is copied into LDS once, and the MFMA A fragments are read
// from it with im2col addressing:
//     pixel (n, oh, ow), tap (kh, kw)  ->  patch row n*H + oh*s - p + kh*d - row0,
//                                          patch column ow*s - p + kw*d
// (a tap that falls into the zero padding reads a zeroed LDS chunk).  So no
// im2col matrix exists anywhere, not even in LDS: the conversion is address
// arithmetic on the read side.
//
// Weights stream through a ring of STAGES LDS buffers, one 64-channel slice
// of one tap per K tile, copied straight from global memory into LDS as in
// igemm_pipe.hpp.  K is ordered (channel slice, tap) here, the same order for
// A and B, so the sum covers every (tap, channel) pair once.
//
// Patch layout: pixel p of the patch (p = patch_row * W + column) occupies 8
// chunks of 16 bytes; logical chunk c sits at position c ^ (p & 7), so eight
// lanes reading one chunk of eight consecutive pixels hit distinct banks.
#pragma once

#include "igemm_pipe.hpp"

namespace convimg {

// First and last input row (flattened n*H + ih) the pixels [m0, m1) read.
struct PatchRows {
    int lo, hi;
};

__host__ __device__ inline int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

__host__ __device__ inline PatchRows patch_rows(int m0, int m1, int H, int OH, int OW, int KH,
                                                int s, int p, int d)
{
    const int fo_f = m0 / OW, fo_l = (m1 - 1) / OW;     // flattened output rows n*OH + oh
    const int n_f = fo_f / OH, oh_f = fo_f - n_f * OH;
    const int n_l = fo_l / OH, oh_l = fo_l - n_l * OH;
    PatchRows r;
    r.lo = n_f * H + clampi(oh_f * s - p, 0, H - 1);
    r.hi = n_l * H + clampi(oh_l * s - p + (KH - 1) * d, 0, H - 1);
    return r;
}

template <int BM, int BN, int WM, int WN, int STAGES, int PATCH_PX>
__global__ __launch_bounds__(WM * WN * 64) void igemm_patch_bf16(ConvArgs a)
{
    constexpr int MS = 32;
    typedef Mfma<MS> MF;
    typedef typename MF::acc_t acc_t;
    constexpr int NW = WM * WN;
    constexpr int NT = NW * 64;
    constexpr int WTM = BM / WM;
    constexpr int WTN = BN / WN;
    constexpr int FM = WTM / MS;
    constexpr int FN = WTN / MS;
    constexpr int KSTEPS = kBK / MF::kstep;
    constexpr int RPP = NT / 8;                       // weight rows one pass fills
    constexpr int BP = BN / RPP;                      // weight copies per lane per stage
    constexpr int PATCH_CH = PATCH_PX * kChunks;
    constexpr int PP = PATCH_CH / NT;                 // patch copies per lane per slice
    constexpr int ZERO_CH = 8;                        // one zeroed pixel (8 chunks)
    constexpr int B_CH = BN * kChunks;
    static_assert(WTM % MS == 0 && WTN % MS == 0, "wave tile must hold whole MFMA blocks");
    static_assert(BN % RPP == 0, "a pass fills whole weight rows");
    static_assert(PATCH_CH % NT == 0, "patch copies are whole passes");
    static_assert(STAGES >= 2 && (STAGES - 2) * BP < 64 && PP + STAGES * BP < 64, "vmcnt range");

    __shared__ u32x4_t patch[PATCH_CH + ZERO_CH];
    __shared__ u32x4_t wring[STAGES * B_CH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;

    const TileCoord tc = tile_coord<BM, BN>(a);
    if (!tc.valid)
        return;
    const int m0 = tc.m0, n0 = tc.n0;
    const int m1 = m0 + BM < a.M ? m0 + BM : a.M;
    const PatchRows pr = patch_rows(m0, m1, a.H, a.OH, a.OW, a.KH, a.stride, a.pad, a.dil);
    const int patch_px = (pr.hi - pr.lo + 1) * a.W;   // the host guarantees <= PATCH_PX
    const int taps = a.KH * a.KW;
    const int nk = a.ktiles;                           // (IC / 64) slices x taps

    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)a.w, 0, a.w_bytes, kRsrcWord3);

    if (tid < ZERO_CH)
        patch[PATCH_CH + tid] = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();            // the zero chunk is visible before any copy is in flight

    const int lrow = lane & 31;
    const int lchk = lane >> 5;

    // ---- copies.  Lane l of a wave instruction fills slot (base + l): row
    // (slot >> 3), physical chunk (l & 7), i.e. logical chunk (l & 7) ^ f(row):
    // f(row) = (row >> 1) & 7 for the weight rows (the swizzle of swz()),
    // row & 7 for the patch pixels (their reads follow the im2col pattern).
    const int lr = lane >> 3;
    // weight rows j * RPP + wave * 8 + lr (RPP a multiple of 16): bits 1..3 of
    // the row are those of wave * 8 + lr, so the logical chunk is (lane & 7)
    // ^ ((row >> 1) & 7) for every pass
    const int cl_w = (lane & 7) ^ ((4 * (wave & 1)) | (lr >> 1));
    static_assert(RPP % 16 == 0, "weight rows of one pass keep bits 1..3 of the row");
    int woff[BP];
    bool wok[BP];
#pragma unroll
    for (int j = 0; j < BP; ++j) {
        const int oc = n0 + j * RPP + wave * 8 + lr;
        wok[j] = oc < a.OC;
        woff[j] = wok[j] ? oc * a.K : 0;
    }
    // weight K tile kt = slice * taps + tap holds w[oc][tap][slice*64 .. +64)
    auto issue_w = [&](int kt, int st) {
        const int slice = kt / taps;
        const int tap = kt - slice * taps;
        const int k = tap * a.IC + slice * kBK + cl_w * 8;
        u32x4_t *sb = wring + st * B_CH + wave * 64;
#pragma unroll
        for (int j = 0; j < BP; ++j)
            dma16(rw, sb + j * RPP * kChunks, wok[j] ? 2u * (unsigned)(woff[j] + k) : kOutOfRange);
    };
    const int x_rows = a.N * a.H;
    auto issue_patch = [&](int slice) {
#pragma unroll
        for (int j = 0; j < PP; ++j) {
            const int slot = j * NT + wave * 64 + lane;
            const int px = slot >> 3;
            const int c = (slot & 7) ^ (px & 7);
            const int frow = pr.lo + px / a.W;
            const bool ok = px < patch_px && frow < x_rows;
            const unsigned off = ok ? 2u * (unsigned)((pr.lo * a.W + px) * a.IC + slice * kBK + c * 8)
                                    : kOutOfRange;
            dma16(rx, patch + j * NT + wave * 64, off);
        }
    };

    // ---- this lane's pixels: block i covers rows wm*WTM + i*32 + (lane & 31)
    const int OHW = a.OH * a.OW;
    int ih0[FM], iw0[FM], pbase[FM];
    bool mok[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WTM + i * MS + lrow;
        mok[i] = m < a.M;
        const int mm = mok[i] ? m : m0;
        const int n = mm / OHW;
        const int r = mm - n * OHW;
        const int oh = r / a.OW;
        const int ow = r - oh * a.OW;
        ih0[i] = oh * a.stride - a.pad;
        iw0[i] = ow * a.stride - a.pad;
        pbase[i] = (n * a.H + ih0[i] - pr.lo) * a.W + iw0[i];   // patch pixel of tap (0, 0)
    }

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = acc_t{};

    // A fragments of tap (kh, kw): per block, the LDS chunk index of chunk 0
    // of the pixel (or of the zero pixel) and its swizzle key.
    auto a_index = [&](int kh, int kw, int (&pix)[FM]) {
        const int dh = kh * a.dil, dw = kw * a.dil;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int ih = ih0[i] + dh, iw = iw0[i] + dw;
            const bool ok = mok[i] && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
            const int px = pbase[i] + dh * a.W + dw;
            pix[i] = (ok && px < PATCH_PX) ? px : -1;   // the bound holds by plan; never read past it
        }
    };
    auto load_frags = [&](const u32x4_t *sb, const int (&pix)[FM], int ks, bf16x8_t (&af)[FM],
                          bf16x8_t (&bfg)[FN]) {
        const int ck = ks * 2 + lchk;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int idx = pix[i] >= 0 ? pix[i] * kChunks + (ck ^ (pix[i] & 7)) : PATCH_CH + ck;
            af[i] = __builtin_bit_cast(bf16x8_t, patch[idx]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bfg[j] = __builtin_bit_cast(bf16x8_t, sb[swz(wn * WTN + j * MS + lrow, ck)]);
    };
    auto compute = [&](int st, int kh, int kw) {
        const u32x4_t *sb = wring + st * B_CH;
        int pix[FM];
        a_index(kh, kw, pix);
        bf16x8_t af[2][FM], bfg[2][FN];
        load_frags(sb, pix, 0, af[0], bfg[0]);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if (ks + 1 < KSTEPS)
                load_frags(sb, pix, ks + 1, af[(ks + 1) & 1], bfg[(ks + 1) & 1]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = MF::run(af[ks & 1][i], bfg[ks & 1][j], acc[i][j]);
        }
    };

    // ---- pipeline over K tiles kt = slice * taps + tap.  The patch of a slice
    // is copied when the slice starts; weights run STAGES-1 tiles ahead.
    issue_patch(0);
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk)
            issue_w(s, s);

    const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.bias, 0, a.bias != nullptr ? a.OC * 4 : 0, kRsrcWord3);
    float bv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int oc = n0 + wn * WTN + j * MS + lrow;
        bv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              rbias, oc < a.OC ? 4u * oc : kOutOfRange, 0, 0));
    }

    int tap = 0, kh = 0, kw = 0, slice = 0;
    for (int kt = 0; kt < nk; ++kt) {
        if (tap == 0 && slice > 0) {
            // new channel slice: every wave is done with the old patch
            lds_barrier();
            issue_patch(slice);
        }
        if (tap == 0 || kt + STAGES - 2 >= nk)
            wait_vmcnt<0>();                      // the patch (and everything before it)
        else
            wait_vmcnt<(STAGES - 2) * BP>();      // weight tile kt landed
        lds_barrier();
        if (kt + STAGES - 1 < nk)
            issue_w(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
        compute(kt % STAGES, kh, kw);
        if (++kw == a.KW) {
            kw = 0;
            if (++kh == a.KH) {
                kh = 0;
            }
        }
        if (++tap == taps) {
            tap = 0;
            ++slice;
        }
    }

    if (a.vec_out) {
        static_assert(NW * EpiScratch<MS, WTN>::floats * 4 <= (int)sizeof(patch), "epilogue scratch");
        __syncthreads();    // every wave is done reading the patch
        store_tile_vec<MS, FM, FN, WTN>(a, acc, bv, m0 + wm * WTM, n0 + wn * WTN,
                                        (float *)patch + wave * EpiScratch<MS, WTN>::floats);
        return;
    }
    store_tile<MS, FM, FN>(a, acc, bv, m0 + wm * WTM + acc_row0<MS>(lane),
                           n0 + wn * WTN + acc_col0<MS>(lane), 0, tc.tile);
}

}  // namespace convimg
