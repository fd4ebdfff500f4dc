// igemm_layout.hpp -- layout conversions around the NHWC core, for callers
// whose tensors are NCHW (input), OIHW (weights) and NCHW (output) and
// whose problem the resident kernel's NCHW variant (which needs none of
// them) does not serve.
//
// burn-cubecl "kernel/conv/base.rs" listing: the NCHW entry points permute
// the input to channels-last and the weight to [OC][KH][KW][IC] before the
// NHWC convolution and permute the result back.  Here each permute is a
// transpose of the last two axes of a [B][R][C] array, 64 x 64 tiles through
// LDS: the input and weight permutes share one launch, and the output
// permute can also round the fp32 result to bf16.  The implicit GEMM itself always writes fp32 (its split-K
// reduction accumulates in the output buffer), into a workspace, so a bf16
// output never aliases the accumulation buffer.
#pragma once

namespace convimg {

constexpr int kPermTile = 64;
constexpr int kPermThreads = 256;

__device__ __forceinline__ float elem_to_float(unsigned short h) { return __uint_as_float((unsigned)h << 16); }
__device__ __forceinline__ float elem_to_float(float f) { return f; }

template <typename T>
__device__ __forceinline__ T float_to_elem(float f);
template <>
__device__ __forceinline__ unsigned short float_to_elem<unsigned short>(float f) { return bf16_rne(f); }
template <>
__device__ __forceinline__ float float_to_elem<float>(float f) { return f; }

// out[b][c][r] = in[b][r][c] for r < R, c < C, converted from Tin to Tout
// (exact between equal types and from bf16 to fp32; rounded to nearest even
// from fp32 to bf16), for the 64 x 64 tile (c0, r0) of batch b.  One
// workgroup moves the tile through LDS: reads along c, writes along r, both
// coalesced.
template <typename Tin, typename Tout>
__device__ __forceinline__ void transpose_tile(const Tin *__restrict__ in, Tout *__restrict__ out, int R, int C,
                                               int b, int r0, int c0)
{
    __shared__ float tile[kPermTile][kPermTile + 1];
    const size_t base = (size_t)b * R * C;
    const int tx = threadIdx.x % kPermTile, ty = threadIdx.x / kPermTile;
    constexpr int kRows = kPermThreads / kPermTile;
    // every lane loads (out-of-range lanes from the tile's first element,
    // then discard it): no branch around the loads, so all 16 are in flight
    // together instead of one round trip each
    float v[kPermTile / kRows];
#pragma unroll
    for (int k = 0; k < kPermTile / kRows; ++k) {
        const int r = ty + k * kRows;
        const bool ok = r0 + r < R && c0 + tx < C;
        v[k] = elem_to_float(in[base + (ok ? (size_t)(r0 + r) * C + c0 + tx : (size_t)r0 * C + c0)]);
        v[k] = ok ? v[k] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kPermTile / kRows; ++k)
        tile[ty + k * kRows][tx] = v[k];
    __syncthreads();
    for (int c = ty; c < kPermTile; c += kRows)
        if (c0 + c < C && r0 + tx < R)
            out[base + (size_t)(c0 + c) * R + r0 + tx] = float_to_elem<Tout>(tile[tx][c]);
}

// One batched transpose (above) per launch.  Grid: (ceil(C/64), ceil(R/64), B).
template <typename Tin, typename Tout>
__global__ __launch_bounds__(kPermThreads) void transpose_batched(const Tin *__restrict__ in,
                                                                 Tout *__restrict__ out, int R, int C)
{
    transpose_tile(in, out, R, C, blockIdx.z, blockIdx.y * kPermTile, blockIdx.x * kPermTile);
}

// Two batched transposes in one launch (x and w of the NCHW entry point):
// workgroup g < t1 takes tile g of the first (tiles numbered c fastest, then
// r, then batch: cx1 x ry1 per batch), the rest the second.  One launch
// instead of two: each costs a dependent launch on the stream, more than
// the small weight transpose's own work.  Grid: t1 + t2 workgroups.
struct TransposeJob {
    int R, C, cx, ry;        // extents; tiles along c and r
};

template <typename T>
__global__ __launch_bounds__(kPermThreads) void transpose_batched2(const T *__restrict__ in1, T *__restrict__ out1,
                                                                  TransposeJob j1, int t1,
                                                                  const T *__restrict__ in2, T *__restrict__ out2,
                                                                  TransposeJob j2)
{
    const bool first = (int)blockIdx.x < t1;
    const TransposeJob j = first ? j1 : j2;
    const int g = first ? (int)blockIdx.x : (int)blockIdx.x - t1;
    const int per = j.cx * j.ry;
    const int b = g / per, rem = g - b * per;
    const int ry = rem / j.cx, cx = rem - ry * j.cx;
    if (first)
        transpose_tile(in1, out1, j.R, j.C, b, ry * kPermTile, cx * kPermTile);
    else
        transpose_tile(in2, out2, j.R, j.C, b, ry * kPermTile, cx * kPermTile);
}

}  // namespace convimg
