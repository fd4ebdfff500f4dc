// igemm_dgrad.hpp -- the data-backward pass: the weight transform that maps
// it onto the forward kernels at stride 1, and the two kernels of the
// fallback route (by phases of the stride; element by element).
//
// For stride 1 the gradient with respect to the input is a forward
// convolution of the output gradient (burn-cubecl "kernel/conv/base.rs"
// listing, conv_data_backward: the implicit-GEMM route is taken for
// groups = 1 and stride 1, everything else goes to a fallback):
//
//   dx[n][ih][iw][ic] = sum_{kh,kw,oc} dY(n, ih + p - kh*d, iw + p - kw*d, oc) * w[oc][kh][kw][ic]
//                     = sum_{kh',kw',oc} dY(n, ih - p' + kh'*d, iw - p' + kw'*d, oc) * wt[ic][kh'][kw'][oc]
//
// with kh' = KH-1-kh, kw' = KW-1-kw, p' = d*(K-1) - p (K = KH = KW) and
//
//   wt[ic][kh'][kw'][oc] = w[oc][KH-1-kh'][KW-1-kw'][ic]
//
// -- the weights flipped in both spatial axes with the channel roles
// swapped, again in OHWI order for the forward kernels.  With taps numbered
// t = kh*KW + kw, the flip of both axes is t -> KK-1-t.
#pragma once

namespace convimg {

constexpr int kFlipTile = 64;   // channels per side of a transposed tile
constexpr int kFlipThreads = 256;

// One workgroup: a 64 (oc) x 64 (ic) tile of source tap t.  Rows of w are
// read along ic and rows of wt written along oc, 16 bytes per lane where
// the channel count and the buffer's alignment allow (vec_in: IC is a
// multiple of the 16-byte vector and w is 16-byte aligned; vec_out: the
// same for OC and wt), element by element otherwise; the transposition goes
// through LDS, stored [ic][oc] with rows padded by one vector.
// Grid: (ceil(IC/64), ceil(OC/64), KK).  T: 2- or 4-byte element.
template <typename T>
__global__ __launch_bounds__(kFlipThreads) void flip_transpose(const T *__restrict__ w, T *__restrict__ wt,
                                                              int OC, int KK, int IC, int vec_in,
                                                              int vec_out)
{
    constexpr int V = 16 / (int)sizeof(T);          // elements per 16-byte vector
    constexpr int kVecs = kFlipTile * kFlipTile / V;
    constexpr int kRowVecs = kFlipTile / V;
    union Vec {
        uint4 u;
        T e[V];
    };
    __shared__ __align__(16) T tile[kFlipTile][kFlipTile + V];
    const int ic0 = blockIdx.x * kFlipTile, oc0 = blockIdx.y * kFlipTile, t = blockIdx.z;
    for (int i = threadIdx.x; i < kVecs; i += kFlipThreads) {
        const int r = i / kRowVecs, c = (i % kRowVecs) * V;
        const int oc = oc0 + r, ic = ic0 + c;
        Vec v;
        v.u = make_uint4(0, 0, 0, 0);
        if (oc < OC && ic < IC) {
            const T *src = w + ((size_t)oc * KK + t) * IC + ic;
            if (vec_in)             // IC % V == 0: the whole vector is inside the row
                v.u = *(const uint4 *)src;
            else
                for (int j = 0; j < V; ++j)
                    if (ic + j < IC)
                        v.e[j] = src[j];
        }
        for (int j = 0; j < V; ++j)
            tile[c + j][r] = v.e[j];
    }
    __syncthreads();
    const int tp = KK - 1 - t;
    for (int i = threadIdx.x; i < kVecs; i += kFlipThreads) {
        const int r = i / kRowVecs, c = (i % kRowVecs) * V;
        const int ic = ic0 + r, oc = oc0 + c;
        if (ic >= IC || oc >= OC)
            continue;
        T *dst = wt + ((size_t)ic * KK + tp) * OC + oc;
        if (vec_out) {              // OC % V == 0: the whole vector is inside the row
            // streaming store: the GEMM that follows reads wt once, from
            // memory (measured 0.2-1.8 us faster per call than the default
            // policy on 64..512-channel 3x3 weights)
            __builtin_nontemporal_store(*(const u32x4_t *)&tile[r][c], (u32x4_t *)dst);
        } else {
            for (int j = 0; j < V && oc + j < OC; ++j)
                dst[j] = tile[r][c + j];
        }
    }
}

// Data backward for every problem the stride-1 mapping above does not serve
// (stride != 1, KH != KW, pad > dilation*(KH-1): the fallback route of the
// burn-cubecl listing's conv_data_backward), computed from its definition as
// a GEMM over the input pixels:
//
//   dx[m][ic] = sum_k A[m][k] B[k][ic],  m = (n, ih, iw),  k = (t, oc),
//   A[m][(t, oc)] = dy[n][oh][ow][oc] where oh = (ih + p - kh d) / s and
//                   ow = (iw + p - kw d) / s divide evenly and lie in the
//                   output, else 0;   B[(t, oc)][ic] = w[oc][t][ic].
//
// 64 (m) x 64 (ic) tiles, 64 k a step, both operands gathered element by
// element (buffer loads; masked lanes read zero past the end) and staged in
// LDS as fp32; v_mfma_f32_16x16x4_f32, four waves of 32 x 32.  The lanes of
// an A load take 64 consecutive k of one pixel (one tap's output channels:
// contiguous in dy), written to A's rows of 68 floats (pixel-major: the 16
// rows x 4 k of an operand read cover all 64 banks); the lanes of a B load
// take 64 consecutive input channels of one k (contiguous in w), written to
// B's rows of 80 floats (k-major: the four k rows of an operand read fall on
// disjoint bank quarters).  bf16 values convert to fp32 exactly and their
// products are exact in fp32, so the numerics are those of the other paths
// (exact products, fp32 sums).  The tile's pixel decodes and each step's k
// decodes (for B) are written to LDS by the first 64 threads; the loads of
// step st + 1 are in flight during step st's MFMAs.
struct DgArgs {
    const void *dy, *w;
    float *dx;
    int N, H, W, IC, OC, KH, KW, s, p, d, OH, OW, M, K, tiles_m;
    unsigned dy_bytes, w_bytes, dx_bytes;     // each below 2^31
    FastDiv div_oc, div_kw, div_hw, div_w;
};

constexpr int kDgAnyRow = 80;       // B rows (k-major)
constexpr int kDgAnyRowA = 68;      // A rows (pixel-major)

template <bool BF16>
__global__ __launch_bounds__(256) void igemm_dgrad_any(DgArgs a)
{
    __shared__ float sA[64 * kDgAnyRowA];     // [m - m0][k - k0]
    __shared__ float sB[64 * kDgAnyRow];      // [k - k0][ic - ic0]
    __shared__ int4 kinf[2][64];              // per k row of a step: kh d, kw d, oc, tap (-1: past K)
    __shared__ int4 minf[64];                 // per pixel of the tile: n OH, ih + p, iw + p, valid

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tm = blockIdx.x % a.tiles_m, tn = blockIdx.x / a.tiles_m;
    const int m0 = tm * 64, ic0 = tn * 64;
    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc((void *)a.dy, 0, a.dy_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)a.w, 0, a.w_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(a.dx, 0, a.dx_bytes, kRsrcWord3);
    constexpr unsigned ES = BF16 ? 2u : 4u;

    // this thread's column c: k = k0 + c (A) and input channel ic0 + c (B);
    // its rows (tid >> 6) + 4 q: pixels (A) and k (B)
    const int c = tid & 63;
    const int ic = ic0 + c;
    const bool icok = ic < a.IC;
    if (tid < 64) {
        const int m = m0 + tid;
        int4 mi = make_int4(0, 0, 0, 0);
        if (m < a.M) {
            const int n = fast_div(m, a.div_hw);
            const int r = m - n * (a.H * a.W);
            const int ih = fast_div(r, a.div_w);
            mi = make_int4(n * a.OH, ih + a.p, r - ih * a.W + a.p, 1);
        }
        minf[tid] = mi;
    }
    const float inv_s = __builtin_amdgcn_rcpf((float)a.s);
    const int KK = a.KH * a.KW;
    const int steps = (a.K + 63) / 64;

    // threads 0..63: k row `tid` of step st
    auto decode = [&](int st, int buf) {
        const int k = st * 64 + tid;
        int4 ki = make_int4(0, 0, 0, -1);
        if (k < a.K) {
            const int t = fast_div(k, a.div_oc);
            const int kh = fast_div(t, a.div_kw);
            ki = make_int4(kh * a.d, (t - kh * a.KW) * a.d, k - t * a.OC, t);
        }
        kinf[buf][tid] = ki;
    };
    float va[16], vb[16];
    auto elem = [&](__amdgpu_buffer_rsrc_t rs, unsigned off) {
        if constexpr (BF16)
            return __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0) << 16);
        else
            return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    };
    auto load = [&](int st, int buf) {
        // A: this thread's k = (t, oc) against 16 pixels
        const int k = st * 64 + c;
        const bool kok = k < a.K;
        int khd = 0, kwd = 0, oc = 0;
        if (kok) {
            const int t = fast_div(k, a.div_oc);
            const int kh = fast_div(t, a.div_kw);
            khd = kh * a.d;
            kwd = (t - kh * a.KW) * a.d;
            oc = k - t * a.OC;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            // dy at (oh, ow) = ((ih + p - kh d) / s, (iw + p - kw d) / s)
            const int4 mi = minf[(tid >> 6) + 4 * q];
            const int hn = mi.y - khd, wn = mi.z - kwd;
            const int oh = small_div(max(hn, 0), inv_s), ow = small_div(max(wn, 0), inv_s);
            const bool aok = kok && mi.w && hn >= 0 && wn >= 0 && oh * a.s == hn && ow * a.s == wn
                && oh < a.OH && ow < a.OW;
            const unsigned oa = aok ? ES * (unsigned)(((mi.x + oh) * a.OW + ow) * a.OC + oc) : kOutOfRange;
            va[q] = elem(rdy, oa);
        }
        // B: w[oc][t][ic] for 16 k rows
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int4 ki = kinf[buf][(tid >> 6) + 4 * q];
            const unsigned ob = (ki.w >= 0 && icok) ? ES * (unsigned)((ki.z * KK + ki.w) * a.IC + ic) : kOutOfRange;
            vb[q] = elem(rw, ob);
        }
    };

    const int wm = wave & 1, wn = wave >> 1;
    const int lrow = lane & 15, lk = lane >> 4;
    floatx4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
            acc[i][jb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    if (steps > 0) {
        if (tid < 64)
            decode(0, 0);
        __syncthreads();
        load(0, 0);
    }
    for (int st = 0; st < steps; ++st) {
        const int buf = st & 1;
        __syncthreads();            // the previous step's operand reads are done
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int r = (tid >> 6) + 4 * q;
            sA[r * kDgAnyRowA + c] = va[q];
            sB[r * kDgAnyRow + c] = vb[q];
        }
        if (tid < 64 && st + 1 < steps)
            decode(st + 1, buf ^ 1);
        __syncthreads();
        if (st + 1 < steps)
            load(st + 1, buf ^ 1);
#pragma unroll 4
        for (int kk = 0; kk < 16; ++kk) {
            const int row = (4 * kk + lk) * kDgAnyRow;
            float af[2], bfv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = sA[(32 * wm + 16 * i + lrow) * kDgAnyRowA + 4 * kk + lk];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
                bfv[jb] = sB[row + 32 * wn + 16 * jb + lrow];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfv[jb], acc[i][jb], 0, 0, 0);
        }
    }
    // acc[i][jb]: lane holds rows (pixels) m0 + 32 wm + 16 i + 4 lk + v of
    // column (channel) ic0 + 32 wn + 16 jb + lrow
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int icc = ic0 + 32 * wn + 16 * jb + lrow;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int mm = m0 + 32 * wm + 16 * i + 4 * lk + v;
                const unsigned off = (mm < a.M && icc < a.IC) ? 4u * (unsigned)(mm * a.IC + icc) : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][jb][v]), rx, off, 0, kOutAux);
            }
        }
}

// Data backward by phases (bf16 storage, OC % 8 == 0, dy 16-byte aligned;
// any stride, kernel shape and padding).  The same sum as the general
// kernel above, with the input pixels grouped by phase: the pixels with ih
// = rh + s i and iw = rw + s j for one (rh, rw) in [0, s)^2.  For such a
// pixel, oh = (ih + p - kh d) / s divides evenly exactly when kh d = rh + p
// (mod s), i.e. for kh = kh0, kh0 + s/g, kh0 + 2 s/g, ... (g = gcd(s, d)),
// and then oh = i + oh0 - a d/g for the a-th of those taps.  So the taps
// that reach a phase are the same for all of its pixels, and along a phase
// row they read consecutive dy pixels: a tile of 64 pixels of one phase
// (N x Hp x Wp of them, Hp = ceil(H / s) rows a phase, rows past H masked)
// loops over those taps only, nth x ntw of KH x KW (a quarter for a 3x3
// kernel at stride 2), 64 output channels a step, and each step's operands
// are 16-byte runs of dy (64 channels of one pixel) and of w (64 input
// channels of one (oc, tap)).  A phase no tap reaches has zero steps: its
// dx is 0.
//
// 64 (pixels) x 64 (input channels) tiles, four waves of 32 x 32 with
// v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 sums).  LDS stage: A
// (64 pixel rows of 64 dy channels) and B (64 output-channel rows of 64 w
// input channels), 128-byte rows, chunk c of row r at c ^ swz(r).  A is read
// as it lies (a lane's 8 consecutive k are one 16-byte chunk of its pixel's
// row: swz(r) = (r >> 1) & 7 puts the 16 rows of one 128-bit read pass on 16
// distinct bank groups); B is read with ds_read_b64_tr_b16 (lane r of a
// 16-lane group points at k row kb + (r >> 2), column n0 + 4 (r & 3); lane l
// then holds column n0 + l at k rows kb .. kb + 3, and two reads give the 8
// consecutive k of a B operand; swz(r) = 2 bit1(r) + 4 bit3(r) keeps those
// 4 rows x 32 bytes, and the next group's 8 rows on, on distinct banks).
// VB (IC % 8 == 0, w 16-byte aligned): A and B arrive by direct-to-LDS
// copies into a ring of three stages, two steps in flight; else A does and
// B is gathered element by element into registers one step ahead and
// written to LDS before the step's barrier.
constexpr int kDgPhRegion = 64 * 128;           // bytes: 64 rows x 64 bf16
constexpr int kDgPhStage = 2 * kDgPhRegion;     // A, then B
constexpr int kDgPhStages = 3;
constexpr int kDgPhCopies = 4;                  // copy instructions a wave issues per step (VB)

struct DgPhArgs {
    const void *dy, *w;
    float *dx;
    int N, H, W, IC, OC, KH, KW, s, p, d, OH, OW;
    int dk, dq;                  // tap step between the taps of a phase (s / g) and dy step per tap (d / g)
    int Hp, Wp, Mp;              // rows and columns a phase, pixels a phase (N Hp Wp)
    int tiles_p, tiles_m, ob;    // m tiles a phase, m tiles in all (s^2 tiles_p), 64-channel blocks of OC
    unsigned dy_bytes, w_bytes, dx_bytes;   // each below 2^31
    FastDiv div_tp, div_hwp, div_wp, div_s;
};

__device__ __forceinline__ int dg_swz_a(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int dg_swz_b(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }

template <bool VB>
__global__ __launch_bounds__(256) void igemm_dgrad_phase_bf16(DgPhArgs a)
{
    // one LDS variable per stage: the compiler can then tell a stage being
    // copied into from the one the fragments are read from
    __shared__ __align__(16) unsigned char lds0[kDgPhStage];
    __shared__ __align__(16) unsigned char lds1[kDgPhStage];
    __shared__ __align__(16) unsigned char lds2[VB ? kDgPhStage : 16];
    __shared__ int pix[64];                       // dx element offset of each tile pixel, -1 past the phase
    auto stage_base = [&](int stage) __attribute__((always_inline)) -> unsigned char * {
        return stage == 0 ? lds0 : stage == 1 ? lds1 : lds2;
    };
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int tn = bid / a.tiles_m, tmg = bid - tn * a.tiles_m;
    const int ph = fast_div(tmg, a.div_tp), tm = tmg - ph * a.tiles_p;
    const int rh = fast_div(ph, a.div_s), rw = ph - rh * a.s;
    const int ic0 = tn * 64;
    // the taps that reach this phase along h and along w (uniform)
    int kh0 = -1, kw0 = -1;
    for (int k = min(a.KH, a.dk) - 1; k >= 0; --k)
        if ((rh + a.p - k * a.d) % a.s == 0)
            kh0 = k;
    for (int k = min(a.KW, a.dk) - 1; k >= 0; --k)
        if ((rw + a.p - k * a.d) % a.s == 0)
            kw0 = k;
    const int nth = kh0 < 0 ? 0 : (a.KH - 1 - kh0) / a.dk + 1;
    const int ntw = kw0 < 0 ? 0 : (a.KW - 1 - kw0) / a.dk + 1;
    const int oh0 = kh0 < 0 ? 0 : (rh + a.p - kh0 * a.d) / a.s;
    const int ow0 = kw0 < 0 ? 0 : (rw + a.p - kw0 * a.d) / a.s;
    const int steps = nth * ntw * a.ob;

    // this lane's two A rows (pixels 16 w + 8 q + (lane >> 3) of the tile)
    // and, for the first 64 threads, the tile's dx offsets
    int yb[2], pi[2], pj[2];
    bool pv[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int m = tm * 64 + 16 * wave + 8 * q + (lane >> 3);
        const int n = fast_div(m, a.div_hwp);
        const int r = m - n * (a.Hp * a.Wp);
        const int i = fast_div(r, a.div_wp);
        pi[q] = i;
        pj[q] = r - i * a.Wp;
        yb[q] = n * a.OH;
        pv[q] = m < a.Mp && rh + a.s * i < a.H && rw + a.s * pj[q] < a.W;
    }
    if (tid < 64) {
        const int m = tm * 64 + tid;
        const int n = fast_div(m, a.div_hwp);
        const int r = m - n * (a.Hp * a.Wp);
        const int i = fast_div(r, a.div_wp);
        const int j = r - i * a.Wp;
        const int ih = rh + a.s * i, iw = rw + a.s * j;
        pix[tid] = (m < a.Mp && ih < a.H && iw < a.W) ? ((n * a.H + ih) * a.W + iw) * a.IC : -1;
    }

    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc((void *)a.dy, 0, a.dy_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw_ = __builtin_amdgcn_make_buffer_rsrc((void *)a.w, 0, a.w_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(a.dx, 0, a.dx_bytes, kRsrcWord3);
    // copy lanes: row (lane >> 3) of an 8-row block, physical chunk lane & 7
    const int pc = lane & 7;
    int ca[2], cb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = 16 * wave + 8 * q + (lane >> 3);
        ca[q] = pc ^ dg_swz_a(r);
        cb[q] = pc ^ dg_swz_b(r);
    }
    // step st = tap (ah, aw) x channel block ob, ob fastest; the running
    // position of the steps issued so far (issue() is called once per step,
    // in order, also for the steps past the last, which copy zeros)
    int nxt_ob = 0, nxt_aw = 0, nxt_ah = 0, nxt_st = 0;
    unsigned vb[16];                              // B gathers of the next step (not VB): raw bf16 bits
    auto issue = [&](unsigned char *sbase) __attribute__((always_inline)) {
        const bool live = nxt_st < steps;
        const int ob = nxt_ob, ah = nxt_ah, aw = nxt_aw;
        // A: dy at (oh, ow) = (i + oh0 - ah dq, j + ow0 - aw dq), channels 64 ob + 8 c
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int oh = pi[q] + oh0 - ah * a.dq, ow = pj[q] + ow0 - aw * a.dq;
            const int oc = 64 * ob + 8 * ca[q];
            const bool ok = live && pv[q] && (unsigned)oh < (unsigned)a.OH && (unsigned)ow < (unsigned)a.OW
                && oc < a.OC;
            const unsigned off = ok ? 2u * ((unsigned)((yb[q] + oh) * a.OW + ow) * (unsigned)a.OC + (unsigned)oc)
                                    : kOutOfRange;
            dma16(rdy, (u32x4_t *)(sbase + (16 * wave + 8 * q) * 128), off);
        }
        // B: w[64 ob + row][kh][kw][ic0 + 8 c]
        const int kh = kh0 + ah * a.dk, kw = kw0 + aw * a.dk;
        const int tap = kh * a.KW + kw;
        if constexpr (VB) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int oc = 64 * ob + 16 * wave + 8 * q + (lane >> 3);
                const int ic = ic0 + 8 * cb[q];
                const bool ok = live && oc < a.OC && ic < a.IC;
                const unsigned off = ok
                    ? 2u * ((unsigned)(oc * a.KH * a.KW + tap) * (unsigned)a.IC + (unsigned)ic) : kOutOfRange;
                dma16(rw_, (u32x4_t *)(sbase + kDgPhRegion + (16 * wave + 8 * q) * 128), off);
            }
        } else {
            // thread: column tid & 63, rows (tid >> 6) + 4 q
            const int ic = ic0 + (tid & 63);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int oc = 64 * ob + (tid >> 6) + 4 * q;
                const bool ok = live && oc < a.OC && ic < a.IC;
                const unsigned off = ok
                    ? 2u * ((unsigned)(oc * a.KH * a.KW + tap) * (unsigned)a.IC + (unsigned)ic) : kOutOfRange;
                vb[q] = (unsigned)__builtin_amdgcn_raw_buffer_load_b16(rw_, off, 0, 0);
            }
        }
        ++nxt_st;
        if (++nxt_ob == a.ob) {
            nxt_ob = 0;
            if (++nxt_aw == ntw) {
                nxt_aw = 0;
                ++nxt_ah;
            }
        }
    };
    auto put_b = [&](unsigned char *sbase) __attribute__((always_inline)) {
        const int c = tid & 63;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int r = (tid >> 6) + 4 * q;
            *(unsigned short *)(sbase + kDgPhRegion + r * 128 + 16 * ((c >> 3) ^ dg_swz_b(r)) + 2 * (c & 7)) =
                (unsigned short)vb[q];
        }
    };

    // fragments: wave (wm, wn) = pixels 32 wm .., input channels 32 wn ..
    const int wm = wave & 1, wn = wave >> 1;
    const int g16 = lane >> 4, r16 = lane & 15;
    int aoff[2][2], boff[2][2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int r = 32 * wm + 16 * i + r16;
            aoff[i][ks] = r * 128 + 16 * ((4 * ks + g16) ^ dg_swz_a(r));
        }
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 32 * ks + 8 * g16 + 4 * h + (r16 >> 2);
                const int n = 32 * wn + 16 * jb + 4 * (r16 & 3);
                boff[jb][ks][h] = kDgPhRegion + r * 128 + 16 * ((n >> 3) ^ dg_swz_b(r)) + 2 * (n & 7);
            }
    floatx4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
            acc[i][jb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    auto tr = [&](const unsigned char *p) __attribute__((always_inline)) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
    };
    auto compute = [&](const unsigned char *sbase) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8_t fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fa[i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(sbase + aoff[i][ks]));
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const v4i16 lo = tr(sbase + boff[jb][ks][0]), hi = tr(sbase + boff[jb][ks][1]);
                fb[jb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[jb], acc[i][jb], 0, 0, 0);
        }
    };

    if constexpr (VB) {
        // ring of three stages: step st's copies are issued after the
        // barrier of step st - 2, which certifies every wave is done with
        // step st - 3's stage.  The loop is unrolled by three so that every
        // stage is a constant and runs whole rounds of three steps with no
        // branch inside (a branch around each step made the compiler wait
        // for the copies of the step ahead before most fragment reads),
        // then the last partial round step by step.
        static_assert(kDgPhStages == 3, "the rounds below are written for three stages");
        auto step = [&](int q) __attribute__((always_inline)) {
            wait_vmcnt<(kDgPhStages - 2) * kDgPhCopies>();   // this step landed (this wave's part)
            lds_barrier();
            issue(stage_base((q + kDgPhStages - 1) % kDgPhStages));
            compute(stage_base(q));
        };
#pragma unroll
        for (int q = 0; q < kDgPhStages - 1; ++q)
            issue(stage_base(q));
        const int full = steps - steps % kDgPhStages;
        for (int st0 = 0; st0 < full; st0 += kDgPhStages) {
            step(0);
            step(1);
            step(2);
        }
        if (full < steps)
            step(0);
        if (full + 1 < steps)
            step(1);
        wait_vmcnt<0>();       // (the copies past the last step: done before the workgroup ends)
    } else {
        // two stages: step st + 1's copies and B gathers are issued after
        // step st's barrier (every wave is then done with step st - 1's
        // stage), the gathers written to LDS before step st + 1's barrier
        issue(stage_base(0));
        for (int st0 = 0; st0 < steps; st0 += 2) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (st0 + q < steps) {
                    wait_vmcnt<0>();
                    put_b(stage_base(q));
                    __syncthreads();
                    issue(stage_base(q ^ 1));
                    compute(stage_base(q));
                }
            }
        }
        wait_vmcnt<0>();
    }
    __syncthreads();       // (pix was written by the first wave; a zero-step tile meets no barrier before)
    // acc[i][jb]: lane holds pixels 32 wm + 16 i + 4 g16 + v of input channel
    // ic0 + 32 wn + 16 jb + r16
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int ic = ic0 + 32 * wn + 16 * jb + r16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int base = pix[32 * wm + 16 * i + 4 * g16 + v];
                const unsigned off = (base >= 0 && ic < a.IC) ? 4u * (unsigned)(base + ic) : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][jb][v]), rx, off, 0, kOutAux);
            }
        }
}

}  // namespace convimg
