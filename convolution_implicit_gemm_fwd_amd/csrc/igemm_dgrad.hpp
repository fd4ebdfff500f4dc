// igemm_dgrad.hpp -- weight transform for the data-backward pass.
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

}  // namespace convimg
