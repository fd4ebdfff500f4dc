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
// it reads are copied into LDS (direct-to-LDS, 16-byte chunks, double
// buffered: the next unit's rows are in flight while this unit computes);
// elements outside the image row are then zeroed in LDS.  Wave w computes
// pixels [32w, 32w + 32) of the unit against all 64 channels with
// v_mfma_f32_32x32x16_bf16 (A from LDS, B from registers) and stores the
// results straight from the accumulators (fixed count of buffer stores; a
// masked element's offset is out of range, so the store is dropped).
#pragma once

#include "igemm_common.hpp"
#include "igemm_pipe.hpp"

namespace convimg {

constexpr int kWinThreads = 256;
constexpr int kWinMaxKH = 7;                   // B fragments of up to 14 k steps in registers
constexpr int kWinSeg = 128;                   // pixels per unit at most (4 waves x 32)
constexpr int kWinStores = 2 * 16;             // buffer stores per wave per unit

__global__ __launch_bounds__(kWinThreads) void igemm_window_bf16(ConvArgs a)
{
    extern __shared__ u32x4_t dsm[];
    char *const lds = (char *)dsm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lk = lane >> 5;      // k chunk this lane feeds
    const int lr = lane & 31;      // pixel row / channel column this lane feeds

    int bid = blockIdx.x;
    if (a.remap)
        bid = xcd_remap(bid, gridDim.x);
    const int gn = bid / a.tiles_m;
    const int gm = bid - gn * a.tiles_m;
    const int n0 = gn * 64;
    const int nunits = a.N * a.OH * a.win_segs;
    const int u_begin = gm * a.win_per;
    if (u_begin >= nunits)
        return;
    const int u_end = min(u_begin + a.win_per, nunits);

    const int IC = a.IC, KH = a.KH, KW = a.KW;
    const int sic = a.stride * IC;          // elements between neighbouring pixels' windows
    const int WIC = a.W * IC;               // elements per input row
    const int sh = a.win_sh;
    const int wp = a.win_wp;                // LDS bytes per weight row
    const int rb = a.win_rb;                // LDS bytes per input-row buffer
    const int nsteps = 2 * KH;              // 16-wide MFMA k steps
    const int jcap = (a.win_seg - 1) * sic + 32;    // row elements a unit reads

    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, a.x_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.out_bytes, kRsrcWord3);
    char *const rows = lds + a.lds_rows;

    // ---- weight slice -> LDS (zeros off the window grid), then registers
    for (int i = tid; i < 64 * wp / 16; i += kWinThreads)
        dsm[i] = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();
    {
        // thread tid handles k = tid, tid + 256, ... of every channel row
        const unsigned short *w = (const unsigned short *)a.w;
        const int kwic = KW * IC;
        for (int k = tid; k < a.K; k += kWinThreads) {
            const int kh = k / kwic;
            const int rem = k - kh * kwic;
            const int kw = rem / IC;
            const int c = rem - kw * IC;
            const int pos = 2 * (kh * 32 + sh + kw * a.dil * IC + c);
#pragma unroll 8
            for (int r = 0; r < 64; ++r) {
                const int oc = n0 + r;
                const unsigned short v = oc < a.OC ? w[(long long)oc * a.K + k] : (unsigned short)0;
                *(unsigned short *)(lds + r * wp + pos) = v;
            }
        }
    }
    float bv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int oc = n0 + j * 32 + lr;
        bv[j] = (a.bias != nullptr && oc < a.OC) ? a.bias[oc] : 0.f;
    }
    __syncthreads();
    // B fragment of step t, block j: channel row j*32 + lr, positions 16t + 8lk .. + 8
    bf16x8_t breg[2 * kWinMaxKH][2];
#pragma unroll
    for (int t = 0; t < 2 * kWinMaxKH; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            breg[t][j] = t < nsteps
                ? __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(lds + (j * 32 + lr) * wp + 2 * (16 * t + 8 * lk)))
                : bf16x8_t{};

    // Geometry of unit u: output row q = n*OH + oh, first pixel ow0, and the
    // first element e_lo of the run of each input row it reads.
    struct Unit {
        int n, oh, ow0, q, e_lo;
    };
    auto unit_of = [&](int u) {
        Unit g;
        g.q = u / a.win_segs;
        const int seg = u - g.q * a.win_segs;
        g.n = g.q / a.OH;
        g.oh = g.q - g.n * a.OH;
        g.ow0 = seg * a.win_seg;
        g.e_lo = (g.ow0 * a.stride - a.pad) * IC - sh;      // even
        return g;
    };
    // Byte offset within the row buffer of the run's first element: the
    // copy starts at the 16-byte boundary below it.
    auto row_delta = [&](const Unit &g, int ih) {
        const long long gb = 2LL * (((long long)(g.n * a.H + ih) * a.W) * IC + g.e_lo);
        return (int)(gb & 15);
    };
    // Copy the KH input rows of unit u into buffer set `set`: per row
    // rb / 1024 instructions of 64 16-byte chunks, dealt round-robin over
    // the waves; rows outside the image and chunks outside x read zeros.
    const int bpr = rb >> 10;               // 1 KB copies per row
    auto issue_rows = [&](int u, int set) {
        const Unit g = unit_of(u);
        for (int idx = wave; idx < KH * bpr; idx += 4) {
            const int kh = idx / bpr, b = idx - kh * bpr;
            const int ih = g.oh * a.stride - a.pad + kh * a.dil;
            const long long gb = 2LL * (((long long)(g.n * a.H + ih) * a.W) * IC + g.e_lo);
            const long long src = (gb & ~15LL) + 16LL * (b * 64 + lane);
            // a chunk that runs past the end of x still brings its dwords
            // inside x (the buffer range check is per dword)
            const bool ok = (unsigned)ih < (unsigned)a.H && src >= 0 && src < (long long)a.x_bytes;
            dma16(rx, (u32x4_t *)(rows + (set * KH + kh) * rb) + b * 64, ok ? (unsigned)src : kOutOfRange);
        }
    };

    floatx16_t acc[2];
    issue_rows(u_begin, 0);
    for (int u = u_begin; u < u_end; ++u) {
        const int set = (u - u_begin) & 1;
        const Unit g = unit_of(u);
        // this unit's rows have landed (the previous unit's stores may not)
        if (u == u_begin)
            wait_vmcnt<0>();
        else
            wait_vmcnt<kWinStores>();
        __syncthreads();
        // zero the elements of each row run that lie outside the image row
        {
            const int left = min(max(-g.e_lo, 0), jcap);        // j < -e_lo
            const int right0 = max(min(WIC - g.e_lo, jcap), 0);  // j >= WIC - e_lo
            const int nfix = left + (jcap - right0);
            for (int kh = 0; kh < KH; ++kh) {
                const int ih = g.oh * a.stride - a.pad + kh * a.dil;
                char *const row = rows + (set * KH + kh) * rb + row_delta(g, ih);
                for (int f = tid; f < nfix; f += kWinThreads) {
                    const int j = f < left ? f : right0 + (f - left);
                    *(unsigned short *)(row + 2 * j) = 0;
                }
            }
        }
        __syncthreads();
        if (u + 1 < u_end)
            issue_rows(u + 1, set ^ 1);

        // A fragment of step t: row buffer t >> 1, bytes
        // delta + 2 * (pixel * sic + 16 (t & 1) + 8 lk), 4-byte aligned
        int abase[kWinMaxKH];
#pragma unroll
        for (int kh = 0; kh < kWinMaxKH; ++kh) {
            const int ih = g.oh * a.stride - a.pad + min(kh, KH - 1) * a.dil;
            abase[kh] = (set * KH + min(kh, KH - 1)) * rb + row_delta(g, ih)
                + 2 * ((32 * wave + lr) * sic + 8 * lk);
        }
        auto aload = [&](int t) {
            const unsigned *p = (const unsigned *)(rows + abase[t >> 1] + 32 * (t & 1));
            return __builtin_bit_cast(bf16x8_t, u32x4_t{p[0], p[1], p[2], p[3]});
        };
        acc[0] = floatx16_t{};
        acc[1] = floatx16_t{};
        bf16x8_t fa0 = aload(0), fa1;
#pragma unroll
        for (int t = 0; t < 2 * kWinMaxKH; t += 2) {
            if (t < nsteps) {
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
        }

        // ---- stores: value v of block j is pixel 32*wave + 8*(v >> 2) +
        // 4*lk + (v & 3), channel n0 + j*32 + lr; always kWinStores stores
        const int ow_end = min(g.ow0 + a.win_seg, a.OW);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int oc = n0 + j * 32 + lr;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int ow = g.ow0 + 32 * wave + 8 * (v >> 2) + 4 * lk + (v & 3);
                const int m = g.q * a.OW + ow;
                const unsigned off = (ow < ow_end && oc < a.OC) ? 4u * (unsigned)(m * a.OC + oc) : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, acc[j][v] + bv[j]), ro,
                                                      off, 0, 0);
            }
        }
    }
}

}  // namespace convimg
