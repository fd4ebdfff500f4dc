// igemm_window.hpp -- implicit-GEMM kernel for layers with few input
// channels (the fast case of the masked edge path: an RGB stem with IC = 3,
// 7x7, stride 2 has K = 147, which breaks every 8- or 16-channel grouping).
//
// When one kernel row of the receptive field, span = ((KW - 1) * d + 1) * IC
// input elements, fits in 32 k values, the KW * IC products of kernel row kh
// for output pixel (oh, ow) read one contiguous run ("window") of input row
// ih = oh*s - p + kh*d, starting at element (ow*s - p) * IC of that row.
// K is laid out as KH steps of 32: position jj of step kh multiplies window
// element jj - sh, where sh (0 or 1) makes every window start at an even
// element, so a lane's 8 consecutive k values are a 4-byte aligned 16-byte
// run of the LDS copy of the input row.  Weight positions that are not on
// the (kw, c) grid of the window are zero.
//
// A workgroup (4 waves) keeps the 64-channel weight slice in registers (each
// lane holds the B fragments of every k step) and walks a contiguous range
// of "units": up to 128 pixels of one output row.  Per unit the KH input rows
// it reads are copied into LDS (direct-to-LDS, 16-byte chunks) into one of
// `win_sets` buffer sets, so the rows of the next win_sets - 1 units are in
// flight while this unit computes; elements outside the image row are then
// zeroed in LDS.  Wave w computes pixels [32w, 32w + 32) of the unit against
// all 64 channels with v_mfma_f32_32x32x16_bf16 (A from LDS, B from
// registers).  The results go out as 16-byte stores after a transpose
// through a per-wave LDS scratch (over the weight staging area, free once
// the weights are in registers), or as 4-byte stores straight from the
// accumulators when out is not 16-byte aligned or OC % 4 != 0.  Every store
// is issued unconditionally: a masked element's offset is out of range, so
// the store is dropped and each wave's count of memory instructions per unit
// is fixed.  Two workgroups share a CU, so one's per-unit bookkeeping
// overlaps the other's MFMAs and stores; KH is a template argument so the
// MFMA loop has no branches.
#pragma once

#include "igemm_common.hpp"
#include "igemm_pipe.hpp"

namespace convimg {

constexpr int kWinThreads = 256;
constexpr int kWinMaxKH = 7;                   // B fragments of up to 14 k steps in registers
constexpr int kWinOcc = 2;                     // workgroups per CU the plan aims for
constexpr int kWinSeg = 128;                   // pixels per unit at most (4 waves x 32)
constexpr int kWinStores = 2 * 16;             // 4-byte stores per wave per unit
constexpr int kWinVecStores = 8;               // 16-byte stores per wave per unit
constexpr int kWinScrRow = 72;                 // floats per pixel row of the epilogue scratch
constexpr int kWinScrBytes = 4 * 32 * kWinScrRow * 4;   // epilogue scratch of the 4 waves

template <int KH>
__global__ __launch_bounds__(kWinThreads, kWinOcc) void igemm_window_bf16(ConvArgs a)
{
    extern __shared__ u32x4_t dsm[];
    char *const lds = (char *)dsm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lk = lane >> 5;      // k chunk this lane feeds
    const int lr = lane & 31;      // pixel row / channel column this lane feeds

    // Unit ranges.  With one 64-channel slice, XCD x (workgroups b with
    // b % 8 == x, the order the dispatcher deals them in) takes a contiguous
    // block of units, so input rows that neighbouring units share meet in
    // its L2; within the XCD the first half of its workgroups (the first
    // slot of each of its CUs: every CU is filled once before any takes a
    // second workgroup) take the larger shares of an even split, so the two
    // workgroups of a CU sum to about the same count on every CU.  With
    // several slices: an even split in launch order, larger shares first.
    // the arguments the set-up reads, loaded in one batch: the compiler
    // otherwise loads them as they are needed, one dependent round trip
    // after another
    asm volatile("" ::"s"(a.N), "s"(a.OH), "s"(a.OW), "s"(a.win_segs), "s"(a.win_seg), "s"(a.tiles_n),
                 "s"(a.tiles_m), "s"(a.IC), "s"(a.KW), "s"(a.stride), "s"(a.pad), "s"(a.dil), "s"(a.H), "s"(a.W),
                 "s"(a.win_sh), "s"(a.win_wp), "s"(a.win_rb), "s"(a.win_sets), "s"(a.x), "s"(a.x_bytes),
                 "s"(a.lds_rows), "s"(a.K));
    const int units = a.N * a.OH * a.win_segs;
    int gn, u_begin, u_end;
    // (divisions by the host's multiply-shift constants: the plan keeps
    // units * tiles_m below 2^31; an integer division by a run-time value
    // is a long chain of quarter-rate VALU multiplies, all of it before the
    // first row copy goes out)
    if (a.tiles_n == 1) {
        const int G = a.tiles_m, q = G >> 3, r = G & 7;      // (the grid: tiles_m groups of units)
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
        const int cnt = q + (x < r ? 1 : 0);                      // workgroups of XCD x
        const int base = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
        const int ux0 = fast_div(units * base, a.win_div_g);
        const int ux1 = fast_div(units * (base + cnt), a.win_div_g);
        const int per = fast_div(ux1 - ux0, x < r ? a.win_div_q1 : a.win_div_q);
        const int extra = (ux1 - ux0) - per * cnt;
        gn = 0;
        u_begin = ux0 + j * per + min(j, extra);
        u_end = u_begin + per + (j < extra ? 1 : 0);
    } else {
        gn = fast_div(blockIdx.x, a.win_div_g);
        const int gm = blockIdx.x - gn * a.tiles_m;
        const int per = fast_div(units, a.win_div_g), extra = units - per * a.tiles_m;
        u_begin = gm * per + min(gm, extra);
        u_end = u_begin + per + (gm < extra ? 1 : 0);
    }
    const int n0 = gn * 64;
    if (u_begin >= u_end)
        return;

    const int IC = a.IC, KW = a.KW;
    const int sic = a.stride * IC;          // elements between neighbouring pixels' windows
    const int WIC = a.W * IC;               // elements per input row
    const int sh = a.win_sh;
    const int wp = a.win_wp;                // LDS bytes per weight row
    const int rb = a.win_rb;                // LDS bytes per input-row buffer
    const int nsets = a.win_sets;
    constexpr int nsteps = 2 * KH;          // 16-wide MFMA k steps
    const int jcap = (a.win_seg - 1) * sic + 32;    // row elements a unit reads

    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.out_bytes, kRsrcWord3);
    char *const rows = lds + a.lds_rows;

    // Geometry of unit u: output row q = n*OH + oh, first pixel ow0, the
    // first element e_lo of the run of each input row it reads, and gb0, the
    // byte offset in x of element e_lo of input row oh*s - p of image n
    // (negative at the top-left corner); kernel row kh adds kh * rowstep.
    // Divisions go through float reciprocals (the plan keeps the unit count
    // under 2^21): this bookkeeping runs once per unit on every wave.
    struct Unit {
        int n, oh, ow0, q, e_lo, gb0;
    };
    const float inv_segs = __builtin_amdgcn_rcpf((float)a.win_segs);
    const float inv_oh = __builtin_amdgcn_rcpf((float)a.OH);
    const int rowstep = 2 * a.dil * WIC;
    auto unit_of = [&](int u) {
        Unit g;
        g.q = small_div(u, inv_segs);
        const int seg = u - g.q * a.win_segs;
        g.n = small_div(g.q, inv_oh);
        g.oh = g.q - g.n * a.OH;
        g.ow0 = seg * a.win_seg;
        g.e_lo = (g.ow0 * a.stride - a.pad) * IC - sh;      // even
        g.gb0 = 2 * ((g.n * a.H + g.oh * a.stride - a.pad) * WIC + g.e_lo);
        return g;
    };
    // Byte offset within the row buffer of the run's first element of row
    // kh: the copy starts at the 16-byte boundary below it.
    auto row_delta = [&](const Unit &g, int kh) { return (g.gb0 + kh * rowstep) & 15; };
    // Copy the KH input rows of unit u into buffer set `set`: per row
    // rb / 1024 instructions of 64 16-byte chunks, dealt round-robin over
    // the waves; rows outside the image and chunks outside x read zeros.
    // Lanes past the run the unit reads get an out-of-range offset (no
    // memory request); the instruction count per wave stays fixed.
    const int bpr = rb >> 10;               // 1 KB copies per row
    const float inv_bpr = __builtin_amdgcn_rcpf((float)bpr);
    auto issue_rows = [&](int u, int set) {
        const Unit g = unit_of(u);
        for (int idx = wave; idx < KH * bpr; idx += 4) {
            const int kh = small_div(idx, inv_bpr), b = idx - kh * bpr;
            const int ih = g.oh * a.stride - a.pad + kh * a.dil;
            const int gb = g.gb0 + kh * rowstep;
            const int chunk = b * 64 + lane;
            const int src = (gb & ~15) + 16 * chunk;
            // a chunk that runs past the end of x still brings its dwords
            // inside x (the buffer range check is per dword)
            const bool ok = (unsigned)ih < (unsigned)a.H && src >= 0 && (unsigned)src < a.x_bytes
                && 16 * chunk < (gb & 15) + 2 * jcap;
            dma16(rx, (u32x4_t *)(rows + (set * KH + kh) * rb) + b * 64, ok ? (unsigned)src : kOutOfRange);
        }
    };
    // vector memory instructions of this wave per unit: row copies, stores
    const int ndma = wave < KH * bpr ? (KH * bpr - 1 - wave) / 4 + 1 : 0;
    const int nst = a.vec_out ? kWinVecStores : kWinStores;
    const int ahead = nsets - 1;            // units whose rows are in flight

    // the rows of the first units are in flight while the weights load
    for (int i = 0; i < ahead && u_begin + i < u_end; ++i)
        issue_rows(u_begin + i, i);

    // ---- weight slice -> LDS (zeros off the window grid), then registers.
    // Thread k (K <= KH * 32 <= 256) reads column k of the 64 channel rows
    // (one wave's 64 loads of a row are one contiguous run of w), every
    // load issued before the first is waited for; rows past OC read zeros.
    // Column-per-thread keeps the LDS writes below on neighbouring banks.
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)a.w, 0, a.w_bytes, kRsrcWord3);
    unsigned short wcol[64];
    if (tid < a.K) {
#pragma unroll
        for (int r = 0; r < 64; ++r) {
            const int oc = n0 + r;
            const unsigned off = oc < a.OC ? 2u * (unsigned)(oc * a.K + tid) : kOutOfRange;
            wcol[r] = __builtin_amdgcn_raw_buffer_load_b16(rw, off, 0, 0);
        }
    }
    for (int i = tid; i < 64 * wp / 16; i += kWinThreads)
        dsm[i] = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();
    if (tid < a.K) {
        const int kwic = KW * IC;
        const int kh = small_div(tid, __builtin_amdgcn_rcpf((float)kwic));
        const int rem = tid - kh * kwic;
        const int kw = small_div(rem, __builtin_amdgcn_rcpf((float)IC));
        const int c = rem - kw * IC;
        char *const col = lds + 2 * (kh * 32 + sh + kw * a.dil * IC + c);
#pragma unroll
        for (int r = 0; r < 64; ++r)
            *(unsigned short *)(col + r * wp) = wcol[r];
    }
    float bv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int oc = n0 + j * 32 + lr;
        bv[j] = (a.bias != nullptr && oc < a.OC) ? a.bias[oc] : 0.f;
    }
    __syncthreads();
    // B fragment of step t, block j: channel row j*32 + lr, positions 16t + 8lk .. + 8
    bf16x8_t breg[2 * KH][2];
#pragma unroll
    for (int t = 0; t < 2 * KH; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            breg[t][j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(lds + (j * 32 + lr) * wp + 2 * (16 * t + 8 * lk)));

    floatx16_t acc[2];
    int set = 0;
    for (int u = u_begin; u < u_end; ++u) {
        const Unit g = unit_of(u);
        // Unit u's rows have landed once at most this many of this wave's
        // later instructions are outstanding: the copies of units u+1 ..
        // u+ahead-1 and the stores of the last `ahead` units (vector memory
        // instructions complete in order; a smaller count only waits longer).
        // The barriers here carry no memory fence: a fence would also wait
        // for the rows still in flight for later units.  Each wave's waits
        // give the order instead.
        {
            const int later = min(u + ahead - 1, u_end - 1) - u;
            const int done = u - max(u - ahead, u_begin);
            wait_vmcnt_rt(min(later * ndma + done * nst, 63));
        }
        lds_barrier();
        // zero the elements of each row run that lie outside the image row
        // (left: j < -e_lo, right: j >= WIC - e_lo), all rows in one pass
        {
            const int left = min(max(-g.e_lo, 0), jcap);
            const int right0 = max(min(WIC - g.e_lo, jcap), 0);
            const int nfix = left + (jcap - right0);
            if (nfix > 0) {
#pragma unroll
                for (int kh = 0; kh < KH; ++kh) {
                    char *const rowp = rows + (set * KH + kh) * rb + row_delta(g, kh);
                    for (int e = tid; e < nfix; e += kWinThreads) {
                        const int j = e < left ? e : right0 + (e - left);
                        *(unsigned short *)(rowp + 2 * j) = 0;
                    }
                }
            }
        }
        wait_lgkmcnt0();
        lds_barrier();
        if (u + ahead < u_end)
            issue_rows(u + ahead, set == 0 ? ahead : set - 1);

        // A fragment of step t: row buffer t >> 1, bytes
        // delta + 2 * (pixel * sic + 16 (t & 1) + 8 lk), 4-byte aligned
        int abase[KH];
#pragma unroll
        for (int kh = 0; kh < KH; ++kh)
            abase[kh] = (set * KH + kh) * rb + row_delta(g, kh) + 2 * ((32 * wave + lr) * sic + 8 * lk);
        auto aload = [&](int t) {
            const unsigned *p = (const unsigned *)(rows + abase[t >> 1] + 32 * (t & 1));
            return __builtin_bit_cast(bf16x8_t, u32x4_t{p[0], p[1], p[2], p[3]});
        };
        acc[0] = floatx16_t{};
        acc[1] = floatx16_t{};
        bf16x8_t fa0 = aload(0), fa1;
#pragma unroll
        for (int t = 0; t < nsteps; t += 2) {
            fa1 = aload(t + 1);
            __builtin_amdgcn_sched_barrier(0);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, breg[t][0], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, breg[t][1], acc[1], 0, 0, 0);
            if (t + 2 < nsteps)
                fa0 = aload(t + 2);
            __builtin_amdgcn_sched_barrier(0);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, breg[t + 1][0], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, breg[t + 1][1], acc[1], 0, 0, 0);
        }

        // ---- stores: value v of block j is pixel 32*wave + 8*(v >> 2) +
        // 4*lk + (v & 3), channel n0 + j*32 + lr
        const int ow_end = min(g.ow0 + a.win_seg, a.OW);
        if (a.vec_out) {
            // transpose through this wave's scratch rows (pixel-major, 72
            // floats apart so the two lane halves hit different banks), then
            // lane l stores channels 4(l & 15) .. +4 of pixel 4i + (l >> 4)
            float *const scr = (float *)lds + wave * (32 * kWinScrRow);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    scr[(8 * (v >> 2) + 4 * lk + (v & 3)) * kWinScrRow + j * 32 + lr] = acc[j][v] + bv[j];
            // (the LDS operations of one wave complete in order)
            const int c4 = 4 * (lane & 15);
            const int oc = n0 + c4;
#pragma unroll
            for (int i = 0; i < kWinVecStores; ++i) {
                const int px = 4 * i + (lane >> 4);
                const u32x4_t val = *(const u32x4_t *)(scr + px * kWinScrRow + c4);
                const int ow = g.ow0 + 32 * wave + px;
                const unsigned off = (ow < ow_end && oc < a.OC)
                    ? 4u * (unsigned)((g.q * a.OW + ow) * a.OC + oc) : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b128(val, ro, off, 0, kOutAux);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int oc = n0 + j * 32 + lr;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int ow = g.ow0 + 32 * wave + 8 * (v >> 2) + 4 * lk + (v & 3);
                    const int m = g.q * a.OW + ow;
                    const unsigned off = (ow < ow_end && oc < a.OC) ? 4u * (unsigned)(m * a.OC + oc) : kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, acc[j][v] + bv[j]), ro,
                                                          off, 0, kOutAux);
                }
            }
        }
        set = set == ahead ? 0 : set + 1;
    }
}

}  // namespace convimg
