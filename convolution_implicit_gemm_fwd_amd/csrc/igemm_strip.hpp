// igemm_strip.hpp -- implicit-GEMM kernel for layers whose weight slice fits
// in LDS next to the input rows of a strip of output pixels.
//
// One workgroup (8 compute waves, 4 copy waves) owns a contiguous strip of output
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
// instruction), so LDS areas are filled as contiguous runs of 16-byte chunks.
// Both operands use records of cpp + 1 chunks (cpp = IC / 8): cpp chunks of
// data and one spare, so that consecutive pixels (or channel rows) start 4
// banks apart and the 8 lanes that read one chunk of 8 consecutive records hit
// 8 distinct 4-bank groups, while the chunk a k step reads is a fixed byte
// offset from the record start (an immediate of the LDS read, no per-step
// address arithmetic):
//   * weights: tap-major, [KH*KW][64 channel rows][cpp + 1 chunks];
//   * patch: the input rows of each image the chunk touches, one contiguous
//     run of pixel records per image ("segment", rounded up to whole 1 KB
//     blocks);
// a copy lane that lands on a spare chunk loads nothing (an out-of-range
// offset, which writes zeros).  Padding taps read a zero block at LDS
// offset 0.
#pragma once

#include "igemm_common.hpp"
#include "igemm_pipe.hpp"

namespace convimg {

constexpr int kStripBN = 64;      // output channels per workgroup
constexpr int kStripWaves = 8;    // compute waves: 4 M-groups x 2 tap halves
constexpr int kStripCopyWaves = 4;  // copy waves, one per SIMD
constexpr int kStripThreads = (kStripWaves + kStripCopyWaves) * 64;
constexpr int kStripScratchStride = 68;   // floats per epilogue scratch row (64 + pad)
constexpr int kStripScratchBytes = 4 * 16 * kStripScratchStride * 4;   // one 16-row tile per M-group
constexpr int kStripTailBytes = 16 + kStripBN * 4;   // progress counters, then the slice's bias

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

// FM: 32-row MFMA blocks per M-group (a chunk is at most 128 * FM pixels).
//
// Waves: 4 copy waves (0-3) and 8 compute waves (4-11), two per SIMD.
// Compute wave w computes M-group w & 3 (rows [(w & 3) * FM * 32, ...) of
// the chunk, all 64 channels) over half of the taps: waves 4-7 the first
// ceil(KH*KW / 2), waves 8-11 the rest; the two waves of a SIMD share one output block, so the SIMD
// interleaves two instruction streams while LDS reads stay those of one wave
// per block, and the two partial sums meet in LDS in the epilogue.
// v_mfma_f32_32x32x16_bf16.
//
// The copy waves issue every global->LDS copy (1 KB blocks dealt
// round-robin), in the order the compute waves need the data: the chunk's
// patch, then the weights tap by tap (tap i of the first half, then tap
// nt0 + i of the second), a few taps ahead.  A wave keeps only a few copies
// in flight, so four of them share the work.  Each waits for its own copies
// (vmcnt) and then adds 1 to an LDS progress counter; the compute waves poll
// the counters instead of meeting at a barrier, so they never stall on a
// copy instruction and only wait for data that has not landed yet.  A copy
// completes before its wave's vmcnt wait returns and the counter is bumped
// after that wait, so a compute wave that sees the count also sees the data.
template <int FM>
__global__ __launch_bounds__(kStripThreads) void igemm_strip_bf16(ConvArgs a)
{
    constexpr int FN = kStripBN / 32;
    extern __shared__ u32x4_t dsm[];
    char *const lds = (char *)dsm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // waves 0-3 copy (the oldest waves of a SIMD win its issue arbitration),
    // waves 4-11 compute
    const bool copier = wave < kStripCopyWaves;
    const int cw = wave;                    // copy wave index
    const int grp = wave & 3;               // M-group (and SIMD) of a compute wave
    const int half = ((wave - kStripCopyWaves) >> 2) & 1;  // tap half of a compute wave
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

    const int cpp = a.IC >> 3;              // 16-byte data chunks per input pixel
    const int rec = cpp + 1;                // chunks per LDS record (one spare)
    const int recb = rec * 16;              // bytes per LDS record
    const unsigned rmagic = 0xffffffffu / (unsigned)rec + 1u;   // P / rec == umulhi(P, rmagic) for P < 2^16
    const int KCH = a.K >> 3;               // 16-byte chunks per weight row
    const int zb = a.lds_zero;              // zero block bytes (at LDS offset 0)
    const int pb = a.lds_patch;             // patch offset (bytes)
    const int OHW = a.OH * a.OW;
    const int ntaps = a.KH * a.KW;
    const int nt0 = (ntaps + 1) >> 1;       // tap iterations (taps of the first half)
    const int tapb = kStripBN * recb;       // bytes per tap of the weight slice
    // Tap order, rotated per CU: every CU of an XCD copies the same weights,
    // and if all started with the same tap they would all wait on the same
    // few L2 channels.  Iteration i of the first half computes tap
    // (i + rot0) % nt0, of the second half tap nt0 + (i + rot1) % n1.
    const int n1 = ntaps - nt0;
    const int cu_rank = (int)(blockIdx.x >> 3);
    const int rot0 = cu_rank % nt0, rot1 = n1 > 0 ? cu_rank % n1 : 0;
    auto tap_of = [&](int h, int i) {        // -1: no such tap
        if (h == 0)
            return i < nt0 ? (i + rot0 >= nt0 ? i + rot0 - nt0 : i + rot0) : -1;
        return i < n1 ? nt0 + (i + rot1 >= n1 ? i + rot1 - n1 : i + rot1) : -1;
    };
    // progress counters, each bumped once per copy wave per step: [0] by
    // chunks whose patch has landed, [1] by weight taps (order positions).
    // Typed as LDS so that polls and bumps are LDS instructions (a generic
    // pointer would make them flat accesses through the vector memory path
    // the copies use).
    typedef __attribute__((address_space(3))) int lds_int;
    lds_int *const prog = (lds_int *)(lds + a.lds_flags);

    // ---- zero block, progress words
    for (int i = tid; i < (zb >> 4); i += kStripThreads)
        dsm[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (tid == 0) {
        __hip_atomic_store(prog, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_store(prog + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();

    // The slice's 64 bias values go to LDS (after the progress counters)
    // with the first patch: a global load here would make every wave wait
    // for it at the chunk loop's entry.  A missing bias is a buffer of
    // extent 0, which reads as zeros.
    float *const bias_lds = (float *)(lds + a.lds_flags + 16);

    // Copy waves: the weights of order position pos (2i: the first half's
    // tap of iteration i, 2i + 1: the second half's), rec blocks of 1 KB;
    // chunk P of the tap's area is chunk P % rec of channel row P / rec.
    // Copy wave cw takes blocks cw, cw + 4, ...
    const int wpc = (rec - cw + kStripCopyWaves - 1) / kStripCopyWaves;  // its blocks per tap
    auto issue_w = [&](int pos) {
        if (pos >= ntaps)
            return;
        const int tap = tap_of(pos & 1, pos >> 1);
        for (int blk = cw; blk < rec; blk += kStripCopyWaves) {
            const int P = blk * 64 + lane;
            const int row = (int)__umulhi((unsigned)P, rmagic), c = P - row * rec;
            const int oc = n0 + row;
            const unsigned off = (oc < a.OC && c < cpp)
                ? 16u * (unsigned)(oc * KCH + tap * cpp + c) : kOutOfRange;
            dma16(rw, (u32x4_t *)(lds + zb + tap * tapb) + blk * 64, off);
        }
    };
    auto publish = [&](int idx) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0)
            __hip_atomic_fetch_add(prog + idx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    // Compute waves: wait until progress counter idx reaches need (bounded:
    // a wave gives up after kSpinLimit sleeps rather than hang).
    auto await = [&](int idx, int need) {
        for (int spins = 0;
             __hip_atomic_load(prog + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < need
             && spins < kSpinLimit;
             ++spins)
            __builtin_amdgcn_s_sleep(1);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // B fragment of channel row j*32 + lr, step t of tap tap (chunks 2t + lk):
    // wrow[j] + tap * tapb + 32 t
    int wrow[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
        wrow[j] = zb + (j * 32 + lr) * recb + lk * 16;

    float *const scratch = (float *)(lds + a.lds_scratch) + grp * 16 * kStripScratchStride;

    int chunk = 0;
    for (int c0 = p_begin; c0 < p_end; c0 += a.chunk_px, ++chunk) {
        const int c1 = min(c0 + a.chunk_px, p_end);
        const bool first = c0 == p_begin;
        if (!first)
            __syncthreads();    // every wave is done with the previous patch

        const StripSeg g = strip_seg(c0, c1, a.H, a.W, a.OH, a.OW, a.KH, a.stride, a.pad, a.dil, rec);
        floatx16_t acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = floatx16_t{};

        if (copier) {
            if (first && cw == 0) {
                const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)a.bias, 0, a.bias != nullptr ? a.OC * 4 : 0, kRsrcWord3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (__attribute__((address_space(3))) void *)bias_lds, 4,
                    n0 + lane < a.OC ? 4u * (unsigned)(n0 + lane) : kOutOfRange, 0, 0, 0);
            }
            // ---- patch: one contiguous run of input rows per image
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
                const int seg_chunks = rows * a.W * rec;
                const int gbase = ((n * a.H + ih_lo) * a.W) * cpp;
                u32x4_t *dst = (u32x4_t *)(lds + pb) + off_n;
                const int nblk = (seg_chunks + 63) >> 6;
                for (int blk = cw; blk < nblk; blk += kStripCopyWaves) {
                    const int P = blk * 64 + lane;
                    const int px = (int)__umulhi((unsigned)P, rmagic), c = P - px * rec;
                    const unsigned off = (P < seg_chunks && c < cpp)
                        ? 16u * (unsigned)(gbase + px * cpp + c) : kOutOfRange;
                    dma16(rx, dst + blk * 64, off);
                }
                off_n += (n == g.n_a) ? g.first_chunks : g.full_chunks;
            }
            if (first) {
                // weights, 3 taps ahead of the one being waited for; the
                // patch is older than every weight copy
                for (int pos = 0; pos < 3; ++pos)
                    issue_w(pos);
                for (int k = 0; k < ntaps; ++k) {
                    wait_vmcnt_rt((min(k + 2, ntaps - 1) - k) * wpc);
                    if (k == 0)
                        publish(0);
                    publish(1);
                    issue_w(k + 3);
                }
            } else {
                wait_vmcnt<0>();
                publish(0);
            }
        } else {
            // ---- per-block pixel geometry (block i: rows c0 + (grp*FM + i)*32 + lr)
            int pix0[FM], ih0[FM], iw0[FM], segb[FM];
            bool vm[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = c0 + (grp * FM + i) * 32 + lr;
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
                segb[i] = pb + (int)so * 16 + lk * 16;
            }

            // ---- K loop: tap iterations x 64-channel slices x 4 MFMA k
            // steps.  The fragments of step k + 1 are read from LDS while the
            // MFMAs of step k run (two register sets, and a scheduling barrier
            // that keeps the reads ahead of the MFMAs).  Step t of a slice
            // reads chunk 2t + lk of the slice: the slice's address + 32 t, an
            // immediate offset.
            const int nsl = a.IC >> 6;
            int abase[FM];          // record of the block's pixel at tap (0, 0), + lk chunk
#pragma unroll
            for (int i = 0; i < FM; ++i)
                abase[i] = segb[i] + pix0[i] * recb;
            // A addresses of tap tp (tp < 0: the zero block)
            auto tap_addr = [&](int tp, int (&aa)[FM]) {
                const int kh = tp >= 0 ? tp / a.KW : 0, kw = tp >= 0 ? tp - kh * a.KW : 0;
                const int dh = kh * a.dil, dw = kw * a.dil;
                const int dofs = (dh * a.W + dw) * recb;
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const bool ok = tp >= 0 && vm[i] && (unsigned)(ih0[i] + dh) < (unsigned)a.H
                        && (unsigned)(iw0[i] + dw) < (unsigned)a.W;
                    aa[i] = ok ? abase[i] + dofs : 0;
                }
            };
            auto load = [&](const int (&aa)[FM], int wofs, int imm, bf16x8_t (&fa)[FM], bf16x8_t (&fb)[FN]) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(lds + aa[i] + imm));
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(lds + wrow[j] + wofs + imm));
            };
            auto mma = [&](const bf16x8_t (&fa)[FM], const bf16x8_t (&fb)[FN]) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            };

            await(0, kStripCopyWaves * (chunk + 1));            // the patch
            if (first)
                await(1, kStripCopyWaves * min(2, ntaps));      // the first iteration's taps
            int a_sl[FM], a_nxt[FM], a_nsl[FM];
            int tap = tap_of(half, 0);              // tap of this wave's current iteration
            tap_addr(tap, a_sl);
            bf16x8_t fa0[FM], fb0[FN], fa1[FM], fb1[FN];
            int w_sl = max(tap, 0) * tapb;          // B offset of the current slice
            load(a_sl, w_sl, 0, fa0, fb0);
            for (int it = 0; it < nt0; ++it) {
                const bool act = tap >= 0;          // the second half may have one tap fewer
                const int tap_n = tap_of(half, it + 1);
                const int nofs = max(tap_n, 0) * tapb;  // next tap (a valid area if none)
                tap_addr(tap_n, a_nxt);
                for (int sl = 0; sl < nsl; ++sl) {
                    const bool last_sl = sl + 1 == nsl;
                    // fa0/fb0 hold step 0 of this slice
                    load(a_sl, w_sl, 32, fa1, fb1);
                    __builtin_amdgcn_sched_barrier(0);  // the reads go out before the MFMAs
                    if (act)
                        mma(fa0, fb0);
                    load(a_sl, w_sl, 64, fa0, fb0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (act)
                        mma(fa1, fb1);
                    load(a_sl, w_sl, 96, fa1, fb1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (act)
                        mma(fa0, fb0);
                    if (last_sl && first && it + 1 < nt0)
                        await(1, kStripCopyWaves * min(2 * it + 4, ntaps));  // the next iteration's taps
#pragma unroll
                    for (int i = 0; i < FM; ++i)
                        a_nsl[i] = last_sl ? a_nxt[i] : a_sl[i] + 128;
                    const int w_nsl = last_sl ? nofs : w_sl + 128;
                    load(a_nsl, w_nsl, 0, fa0, fb0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (act)
                        mma(fa1, fb1);
#pragma unroll
                    for (int i = 0; i < FM; ++i)
                        a_sl[i] = a_nsl[i];
                    w_sl = w_nsl;
                }
                tap = tap_n;
            }
        }

        // ---- epilogue: the two partial sums of each block meet in the
        // group's scratch (16 rows at a time); the owner of a round adds its
        // own part and the bias and stores whole 64-channel row segments with
        // 16-byte stores.  Value v of block (i, j) is row 8*(v >> 2) + 4*lk +
        // (v & 3), column j*32 + lr; half h of a block holds v = 8h .. 8h + 7,
        // rows 16h .. 16h + 15.  Rounds alternate the owner between the waves;
        // the copy wave only keeps the barrier count.
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool owner = !copier && half == h;
                if (!copier && !owner) {
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int v = 8 * h; v < 8 * h + 8; ++v)
                            scratch[(8 * ((v >> 2) - 2 * h) + 4 * lk + (v & 3)) * kStripScratchStride
                                    + j * 32 + lr] = acc[i][j][v];
                }
                __syncthreads();
                if (owner) {
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int v = 8 * h; v < 8 * h + 8; ++v) {
                            float *e = scratch + (8 * ((v >> 2) - 2 * h) + 4 * lk + (v & 3)) * kStripScratchStride
                                + j * 32 + lr;
                            *e = *e + acc[i][j][v] + bias_lds[j * 32 + lr];
                        }
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int f = t * 64 + lane;
                        const int row = f >> 4, c4 = (f & 15) * 4;
                        const floatx4_t val = *(const floatx4_t *)(scratch + row * kStripScratchStride + c4);
                        const int m = c0 + (grp * FM + i) * 32 + 16 * h + row;
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
                __syncthreads();
            }
        }
    }
}

}  // namespace convimg
