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

}  // namespace convimg
