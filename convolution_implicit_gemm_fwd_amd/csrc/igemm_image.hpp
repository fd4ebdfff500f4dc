// igemm_image.hpp -- implicit-GEMM kernel for deep layers on small images
// (the large-K case: 512 -> 512 channels on 14x14 maps, K = 4608), where the
// output tile of one image is small and K is long.
//
// One workgroup (8 waves) computes one image's output pixels (MB blocks of
// 32) against 32 output channels, over all of K, with no split-K.  K is
// walked in chunks of 64 input channels.  Per chunk, direct-to-LDS copies
// bring in
//   * the image zero-padded by p on every side, each pixel a record of the
//     chunk's 64 channels plus a spare 16-byte chunk (copy lanes that fall
//     on the frame or the spare chunk read zeros), so every tap of every
//     output pixel addresses a record with no bounds test.  Each padded row
//     ends in a gap that makes the row stride, in 16-byte units, congruent
//     to 9 OW mod 16: the 16 lanes an LDS 128-bit read serves together then
//     cover all 64 banks even where their output pixels wrap to the next
//     row (without the gap, pixel (oh+1, 0) shares banks with (oh, 0));
//   * the chunk's weights: per tap, 32 records of 64 channels plus a spare
//     chunk;
// into one of two buffer sets: chunk c+1's copies are issued between chunk
// c's MFMAs, after the one barrier per chunk that tells every wave chunk c
// has landed and the other set is free.  Waves 0-3 take the first ceil(MB/2) pixel blocks and waves
// 4-7 the rest (each SIMD holds one wave of each group, so every SIMD does
// the same MFMA work); within a group, wave w takes channels 16 (w & 3) ..
// +16 of every chunk, for all taps, with v_mfma_f32_32x32x16_bf16 (A and B
// from LDS; each B fragment serves the group's blocks).  Each wave's code is
// straight-line over the taps (no branch around an MFMA: the compiler
// duplicates the accumulators across such branches).  After the last chunk
// the 4 partial sums of each output are added through LDS by all threads,
// bias added, and stored 16 bytes a thread where the output allows.
#pragma once

#include <type_traits>

#include "igemm_common.hpp"
#include "igemm_pipe.hpp"

namespace convimg {

constexpr int kImgThreads = 512;
constexpr int kImgWaves = 8;
constexpr int kImgNT = 9;                      // taps (3x3)
constexpr int kImgRec = 144;                   // LDS record: 64 bf16 + a spare 16-byte chunk
constexpr int kImgBN = 32;                     // output channels per workgroup
constexpr int kImgMaxCopies = 11;              // copies per wave per chunk at most (the plan checks)
constexpr int kImgWChunks = kImgNT * kImgBN * 9;  // 16-byte chunks of a chunk's weights
constexpr int kImgFlipChunks = kImgNT * 64 * 4;   // the same, copied as forward-weight rows (flipw)
constexpr int kImgFlipReads = kImgNT * 16 * 2 / (kImgWaves * 4);   // transposed reads a wave per chunk (flipw)
static_assert(kImgFlipChunks * 16 <= kImgWChunks * 16, "the rows fit the records' area");
constexpr int kImgRedRow = 40;                     // floats per pixel of the partial sums in LDS
#ifndef CONVIMG_IMG_SPREAD
#define CONVIMG_IMG_SPREAD 22
#endif
constexpr int kImgCopySpread = CONVIMG_IMG_SPREAD;  // MFMA slots a chunk's copies are spread over

// Padded-image row stride in 16-byte units: PW records of 9 units, then a
// gap of 0..15 units so that the stride is congruent to 9 * OW modulo 16.
__host__ __device__ constexpr int img_row_units(int PW, int OW)
{
    return 9 * PW + ((9 * OW - 9 * PW) & 15);
}

// MB: 32-pixel blocks per image (OH * OW <= 32 MB).
template <int MB>
__global__ __launch_bounds__(kImgThreads, 1) void igemm_image_bf16(ConvArgs a)
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
    asm volatile("" ::"s"(a.img_ti), "s"(a.img_ts), "s"(a.tiles_n), "s"(a.N), "s"(a.H), "s"(a.W), "s"(a.IC), "s"(a.pad),
                 "s"(a.OW), "s"(a.OH), "s"(a.img_set), "s"(a.img_wofs), "s"(a.x), "s"(a.w), "s"(a.x_bytes),
                 "s"(a.w_bytes), "s"(a.dil), "s"(a.stride));

    // workgroups in XCD order (each XCD runs a contiguous range), tiled in
    // blocks of img_ti images x img_ts channel slices (about one XCD's
    // share), so the images and the weight slices a block reads are shared
    // within one L2
    // (ti and ts are powers of two; the few divisions left go through
    // small_div: the prologue runs before any copy is in flight, so every
    // instruction in it is on the critical path)
    const int bid = xcd_remap(blockIdx.x, a.N * a.tiles_n);   // (the grid: one workgroup per image and slice)
    const int lti = __builtin_ctz(a.img_ti), lts = __builtin_ctz(a.img_ts);
    const int blk = bid >> (lti + lts), inb = bid & ((1 << (lti + lts)) - 1);
    const int nbs = a.tiles_n >> lts;               // blocks along the slices
    const int bi = small_div(blk, __builtin_amdgcn_rcpf((float)nbs)), bs = blk - bi * nbs;
    const int n = (bi << lti) + (inb & ((1 << lti) - 1));
    const int ot = (bs << lts) + (inb >> lti);
    const int n0 = ot * kImgBN;

    const int H = a.H, W = a.W, IC = a.IC, p = a.pad;
    const int PW = W + 2 * p;                       // padded row width
    const int RU = img_row_units(PW, a.OW);         // padded row stride, 16-byte units
    const int PC = (H + 2 * p) * RU;                // patch chunks
    const int ohw = a.OH * a.OW;
    const int nchunks = IC / 64;
    // LDS: buffer set b at b * a.img_set: patch (PC chunks), then weights
    const int set_bytes = a.img_set;
    const int wofs = a.img_wofs;                    // weights' offset within a set

    // ---- copies of chunk c into set b: instruction j of the chunk's
    // patch instructions then weight instructions; wave w issues j = w, w+8, ...
    // Instruction j of a region copies its chunks 64 j .. 64 j + 63, the last
    // one moved back to end on the region's last chunk (its first lanes copy
    // again what the one before copied: the same bytes), so no copy writes
    // past its region.  Each lane's source offsets are worked out once:
    // chunk c only adds c * 128 bytes (64 channels) to every one, and an
    // out-of-range offset stays out of range.
    // flipw: w holds the forward weights of a data backward's mapped problem
    // (rows = the mapped input channels); a chunk's weights are then copied
    // as they are, 64-byte pieces w[oc][t][n0 .. n0 + 31], into rows (t, oc)
    // of the set's weight area, and flipped and transposed into the records
    // after the chunk's barrier (flip_weights below)
    const bool flipw = a.img_flipw != 0;
    const int wch = flipw ? kImgFlipChunks : kImgWChunks;     // 16-byte chunks of a chunk's weights
    const unsigned cstride = flipw ? 64u * (unsigned)kImgNT * 2u * (unsigned)a.OC : 128u;  // bytes a chunk moves them
    const int pins = (PC + 63) / 64;
    const int wins = (wch + 63) / 64;
    const int cins = pins + wins;
    auto first = [&](int j, int n) { return min(64 * j, max(n - 64, 0)); };
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)a.w, 0, a.w_bytes, kRsrcWord3);
    // Byte offsets: pixel (ih, iw) of image n at xbase + (ih W + iw) IC2,
    // weight row oc, tap t at oc K2 + t IC2.  All 24-bit products (the plan
    // keeps x and w under 2 GB and the image under 2^24 pixels).  A weight
    // row at or past OC lies past the end of w and reads zeros.  Chunk 0 is
    // copied as soon as each offset is known.
    const unsigned IC2 = 2u * (unsigned)IC, K2 = (unsigned)kImgNT * IC2;
    const unsigned xbase = (unsigned)n * (unsigned)(H * W) * IC2, wbase = (unsigned)n0 * K2;
    const float inv_ru = __builtin_amdgcn_rcpf((float)RU);
    unsigned soff[kImgMaxCopies];
#pragma unroll
    for (int k = 0; k < kImgMaxCopies; ++k) {
        const int j = wave + kImgWaves * k;
        unsigned off = kOutOfRange;
        if (j < pins) {
            // chunk q: padded row q / RU, record (q mod RU) / 9 of it (past
            // the row's PW records: the gap), 16-byte part (q mod RU) mod 9
            const int q = first(j, PC) + lane;
            const int pr = small_div(q, inv_ru), within = q - (int)__umul24(pr, RU);
            const int pc = div9(within), sub = within - 9 * pc;
            const int ih = pr - p, iw = pc - p;
            if (sub < 8 && (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W)
                off = xbase + __umul24(__umul24(ih, W) + iw, IC2) + 16u * sub;
        } else if (j < cins && !flipw) {
            const int q = first(j - pins, kImgWChunks) + lane;
            const int rec = div9(q), sub = q - 9 * rec;             // rec = tap * 32 + r
            const int t = rec >> 5, r = rec & 31;
            if (sub < 8)
                off = wbase + __umul24(r, K2) + __umul24(t, IC2) + 16u * sub;
        } else if (j < cins) {
            // row (t, oc) of 64 bytes: w[oc][t][n0 .. n0 + 31] (past the end
            // of w: zeros; past OC in a row: channels never stored)
            const int q = first(j - pins, kImgFlipChunks) + lane;
            const int row = q >> 2, t = row >> 6, oc = row & 63;
            off = __umul24(oc * kImgNT + t, 2u * (unsigned)a.OC) + 2u * (unsigned)n0 + 16u * (q & 3);
        }
        soff[k] = off;
        if (j < pins)
            dma16(rx, dsm + first(j, PC), off);
        else if (j < cins)
            dma16(rw, (u32x4_t *)(lds + wofs) + first(j - pins, wch), off);
    }
    // copy k of chunk c into set b.  lp, lc, lpc: pins, cins and PC as the
    // chunk's own copies (see run), so that the few scalar operations that
    // place each copy are redone per chunk instead of being kept, for all
    // eleven copies and both sets, in registers the loop then spilled
    auto issue_one = [&](int k, int c, int b, int lp, int lc, int lpc, int lwch) {
        const int j = wave + kImgWaves * k;
        char *const base = lds + b * set_bytes;
        if (j < lp)
            dma16(rx, (u32x4_t *)base + first(j, lpc), soff[k] + 128u * c);
        else if (j < lc)
            dma16(rw, (u32x4_t *)(base + wofs) + first(j - lp, lwch), soff[k] + cstride * c);
    };
    // flipw: rows (t, oc) of set b's weight area -> records (NT - 1 - t) * 32
    // + ic, bytes 2 oc.  288 tiles of 4 (oc) x 16 (ic), one per 16-lane group
    // and read (9 reads a wave): ds_read_b64_tr_b16 gives lane l the 4 rows
    // oc .. oc + 3 of column ic0 + l, 8 contiguous bytes of record ic0 + l.
    // Every read completes before any write (the two layouts overlap).
    auto flip_weights = [&](int b) {
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        char *const wb = lds + b * set_bytes + wofs;
        const int G = lane >> 4, r = lane & 15;
        v4i16 v[kImgFlipReads];
#pragma unroll
        for (int q = 0; q < kImgFlipReads; ++q) {
            const int T = (wave * kImgFlipReads + q) * 4 + G;
            const int t = T >> 5, ocq = (T >> 1) & 15, icb = T & 1;
            v[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(
                wb + (t * 64 + 4 * ocq + (r >> 2)) * 64 + 2 * (16 * icb + 4 * (r & 3))));
        }
        wait_lgkmcnt0();
        lds_barrier();
#pragma unroll
        for (int q = 0; q < kImgFlipReads; ++q) {
            const int T = (wave * kImgFlipReads + q) * 4 + G;
            const int t = T >> 5, ocq = (T >> 1) & 15, icb = T & 1;
            *(v4i16 *)(wb + ((kImgNT - 1 - t) * 32 + 16 * icb + r) * kImgRec + 8 * ocq) = v[q];
        }
        wait_lgkmcnt0();
        lds_barrier();
    };

    auto tap_off = [&](int t) { return ((t / 3) * a.dil * RU + (t % 3) * a.dil * 9) * 16; };
    // this wave's 16-channel slice (w & 3) and k half lk
    const int sub16 = 32 * (wave & 3) + 16 * lk;
    // B fragment of tap t: weight record t*32 + lr of the set, same slice
    const int brec = wofs + lr * kImgRec + sub16;
    float *const red = (float *)lds;
    const float inv_ow = __builtin_amdgcn_rcpf((float)a.OW);

    // Blocks [I0, I1) (compile time) for the whole K loop, then the partial
    // sums to LDS: wave slice s, pixel m, channel c at float index
    // (s * 32 MB + m) * kImgRedRow + c (40 floats a pixel: the two lane
    // halves of a write, 4 pixels apart, fall on disjoint banks).
    auto body = [&](auto i0_tag, auto i1_tag) {
        constexpr int I0 = decltype(i0_tag)::value, I1 = decltype(i1_tag)::value, NB = I1 - I0;
        constexpr int NA = NB > 0 ? NB : 1;         // (a group with no block still copies and meets)
        // per lane: padded-patch record of each block's output pixel at tap
        // (0, 0); tap (kh, kw) adds the same kh*d rows and kw*d records for
        // every lane
        int abase[NA];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int m = min(32 * (I0 + i) + lr, ohw - 1);   // past the image: any pixel, never stored
            const int oh = small_div(m, inv_ow), ow = m - oh * a.OW;
            abase[i] = (int)(__umul24(__umul24(oh, a.stride), RU) + __umul24(ow, 9 * a.stride)) * 16 + sub16;
        }
        floatx16_t acc[NA];
#pragma unroll
        for (int i = 0; i < NB; ++i)
            acc[i] = floatx16_t{};
        // all taps of the chunk in buffer set B, while chunk cn's copies go
        // into the other set (when cn < nchunks), spread over the first
        // MFMAs so that the copy unit works beside the matrix cores instead
        // of holding the waves at a burst of copies.  Each block's A
        // fragment for the next tap loads right after its MFMA has read the
        // current one; the next B fragment loads at the start of the tap.
        auto run = [&](auto b_tag, int cn) {
            constexpr int B = decltype(b_tag)::value;
            constexpr int M = kImgNT * NB;                              // MFMAs of the chunk
            constexpr int S = M < kImgCopySpread ? M : kImgCopySpread;  // MFMA slots the copies use
            const bool more = cn < nchunks;
            // (opaque copies: the compiler cannot hoist what depends on them
            // out of the chunk loop)
            int lp = pins, lc = cins, lpc = PC, lwch = wch;
            asm volatile("" : "+s"(lp), "+s"(lc), "+s"(lpc), "+s"(lwch));
            // copies k with slot(k) == m follow MFMA m (slot(k) = k S / K)
            auto copies_after = [&](int m) {
                if (!more)
                    return;
#pragma unroll
                for (int k = 0; k < kImgMaxCopies; ++k)
                    if ((k * S) / kImgMaxCopies == m)
                        issue_one(k, cn, B ^ 1, lp, lc, lpc, lwch);
            };
            const char *const sb = lds + B * set_bytes;
            auto af = [&](int i, int t) {
                return __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(sb + abase[i] + tap_off(t)));
            };
            auto bf = [&](int t) {
                return __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(sb + brec + t * 32 * kImgRec));
            };
            if constexpr (NB == 0) {
                if (more) {
#pragma unroll
                    for (int k = 0; k < kImgMaxCopies; ++k)
                        issue_one(k, cn, B ^ 1, lp, lc, lpc, lwch);
                }
                return;
            }
            bf16x8_t fb = bf(0), fa[NA];
#pragma unroll
            for (int i = 0; i < NB; ++i)
                fa[i] = af(i, 0);
#pragma unroll
            for (int t = 0; t < kImgNT; ++t) {
                bf16x8_t nb;
                if (t + 1 < kImgNT)
                    nb = bf(t + 1);
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    __builtin_amdgcn_sched_barrier(0);
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb, acc[i], 0, 0, 0);
                    if (t + 1 < kImgNT)
                        fa[i] = af(i, t + 1);
                    copies_after(t * NB + i);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (t + 1 < kImgNT)
                    fb = nb;
            }
        };
        auto chunk = [&](int c, auto b_tag) {
            // this wave's copies of chunk c (the only ones in flight) have
            // landed; after the barrier all of chunk c has, and every wave
            // is done with the other set (chunk c - 1), which chunk c + 1
            // then refills
            wait_vmcnt<0>();
            lds_barrier();
            if (flipw)
                flip_weights(decltype(b_tag)::value);
            run(b_tag, c + 1);
        };
        for (int c = 0; c < nchunks; c += 2) {
            chunk(c, std::integral_constant<int, 0>{});
            if (c + 1 < nchunks)
                chunk(c + 1, std::integral_constant<int, 1>{});
        }
        // the partial sums overwrite both sets: every wave's reads first
        wait_lgkmcnt0();
        lds_barrier();
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                red[((wave & 3) * 32 * MB + 32 * (I0 + i) + 8 * (v >> 2) + 4 * lk + (v & 3)) * kImgRedRow + lr] = acc[i][v];
        (void)abase;
    };
    constexpr int MB0 = (MB + 1) / 2;
    if (wave < 4)
        body(std::integral_constant<int, 0>{}, std::integral_constant<int, MB0>{});
    else
        body(std::integral_constant<int, MB0>{}, std::integral_constant<int, MB>{});
    wait_lgkmcnt0();
    lds_barrier();

    // every output pixel m of the image: the 4 partials + bias, stored by
    // all 512 threads; four channels (16 bytes) a thread where the output
    // allows 16-byte stores, else one
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.out_bytes, kRsrcWord3);
    const unsigned obase = 4u * ((unsigned)n * (unsigned)ohw * (unsigned)a.OC + (unsigned)n0);
    if (a.vec_out) {
        const int q4 = 4 * (tid & 7);
        floatx4_t b4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            b4[e] = (a.bias != nullptr && n0 + q4 + e < a.OC) ? a.bias[n0 + q4 + e] : 0.f;
        for (int m = tid >> 3; m < ohw; m += kImgThreads / 8) {
            floatx4_t sum = b4;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                sum += *(const floatx4_t *)(red + (w * 32 * MB + m) * kImgRedRow + q4);
            const unsigned off = n0 + q4 < a.OC ? obase + 4u * (unsigned)(m * a.OC + q4) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, sum), ro, off, 0, kOutAux);
        }
    } else {
        const int c = tid & 31;
        const float bv = (a.bias != nullptr && n0 + c < a.OC) ? a.bias[n0 + c] : 0.f;
        for (int m = tid >> 5; m < ohw; m += kImgThreads / 32) {
            float sum = bv;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                sum += red[(w * 32 * MB + m) * kImgRedRow + c];
            const unsigned off = n0 + c < a.OC ? obase + 4u * (unsigned)(m * a.OC + c) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, sum), ro, off, 0, kOutAux);
        }
    }
}

}  // namespace convimg
