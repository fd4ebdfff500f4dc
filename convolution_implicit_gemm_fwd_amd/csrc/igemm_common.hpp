// igemm_common.hpp -- pieces shared by the implicit-GEMM convolution kernels.
//
// GEMM view (burn PR "Introduce autotuning to conv2d and conv_transpose2d
// with a new im2col/GEMM algorithm", Changes): M = N*OH*OW output pixels,
// N = OC output channels, K = IC*KH*KW, ordered k = (kh*KW + kw)*IC + ic so
// that a row of the OHWI weight is a row of B (burn-cubecl
// "kernel/conv/base.rs" listing, conv_forward: the weight is permuted to
// channels-last before the NHWC kernel runs).
//
// Common to every bf16 kernel:
//   * LDS rows are 64 bf16 = 8 chunks of 16 bytes; logical chunk c of row r
//     is stored at position c ^ ((r >> 1) & 7).  A 128-bit LDS read serves
//     16 lanes a clock, and the MFMA fragment reads give those 16 lanes one
//     chunk column of 16 consecutive rows; a row covers half the banks (8
//     of the 16 4-bank groups, by the row's parity), so among the 8 rows of
//     each parity the positions must all differ, which (r >> 1) & 7 gives
//     (r & 7 repeats every 8 rows: a 2-way conflict on every read);
//   * MFMA, two shapes.  v_mfma_f32_16x16x32_bf16: lane l feeds row (l & 15)
//     of a 16x16 block with the 8 consecutive k of chunk (l >> 4) of each
//     32-wide k step; its 4 results are column (l & 15), rows 4*(l >> 4) + v.
//     v_mfma_f32_32x32x16_bf16: lane l feeds row (l & 31) of a 32x32 block
//     with the 8 k of chunk (l >> 5) of each 16-wide k step; its 16 results
//     are column (l & 31), rows 8*(v >> 2) + 4*(l >> 5) + (v & 3).  A and B
//     always take the same chunks, so every product pairs x and w at one k;
//   * epilogue: + fp32 bias, fp32 NHWC store; with split-K, the splits of one
//     tile take turns on a per-tile semaphore and accumulate in place into the
//     fp32 output, which is the reduction buffer (nvFuser issue "Split-K
//     matmul is slow even for few partitions", section "Eliminating the
//     workspace": blocks serialised by a semaphore, each waiting for its turn,
//     and the output tensor reused as the work buffer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convimg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

enum : int { kLoaderTap = 0, kLoaderVec8 = 1, kLoaderScalar = 2 };

constexpr int kBK = 64;              // K per tile (bf16 kernels)
constexpr int kChunks = kBK / 8;     // 16-byte chunks per LDS row
constexpr int kSpinLimit = 1 << 20;  // split-K wait bound (iterations of s_sleep), unless a test shortens it
constexpr unsigned kOutOfRange = 0x80000000u;  // buffer offset past every buffer addressed so
constexpr int kRsrcWord3 = 0x00020000;         // raw buffer, 32-bit data format
constexpr int kCoherent = 16;                  // cache policy sc1: agent-coherent access
// Cache policy of the final output stores: sc0 | nt | sc1, system scope and
// streaming.  The results then go out to memory as they are stored instead
// of staying dirty in the XCD's L2 until the end of the kernel; measured
// 5-9 % faster launches than the default policy on the fp32-output layers.
#ifndef CONVIMG_OUT_AUX
#define CONVIMG_OUT_AUX 19
#endif
constexpr int kOutAux = CONVIMG_OUT_AUX;

// Division by a run-time constant with one 64-bit multiply (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// for 0 <= n < 2^31 and divisor v >= 1, with l = ceil(log2 v),
// mul = ceil(2^(31+l) / v) < 2^32 gives n / v = (n * mul) >> (31 + l).
struct FastDiv {
    unsigned mul;
    int shift;
};

__device__ __forceinline__ int fast_div(int n, FastDiv f)
{
    return (int)(((unsigned long long)(unsigned)n * f.mul) >> f.shift);
}

// An 8 x 8 transpose of 16-bit elements held as eight 16-byte rows: v[e]
// holds elements (e, 0 .. 7) (element 2h in the low half of dword h);
// out[c] receives elements (0 .. 7, c) (element 2q in the low half of dword
// q).  In the kernels a row is 8 channels of one pixel and a column 8
// pixels of one channel, or the other way round.
__device__ __forceinline__ void transpose8x8(const u32x4_t (&v)[8], u32x4_t (&out)[8])
{
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // byte selects over {hi, lo}: lo bytes are 0-3, hi bytes 4-7
            const unsigned lo = v[2 * q][h], hi = v[2 * q + 1][h];
            out[2 * h][q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);       // low halves
            out[2 * h + 1][q] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);   // high halves
        }
    }
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN (quiet).
__device__ __forceinline__ unsigned short bf16_rne(float f)
{
    const unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (unsigned short)((u >> 16) | 0x40u);
    return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

struct ConvArgs {
    const void *x;
    const void *w;
    const float *bias;
    float *out;
    int *sem;        // split-K: one int per output tile, then one status word
    int spin_limit;  // split-K: iterations a workgroup waits for its turn before it gives up
    unsigned x_bytes, w_bytes;  // buffer extents for bounds-checked loads
    unsigned out_bytes;         // extent of out, at most kOutOfRange (buffer stores past it are dropped)
    int N, H, W, IC, OC, KH, KW, stride, pad, dil;
    int OH, OW, M, K;
    int tiles_m, tiles_n, ktiles, splits;
    int tiles_pad;   // workgroup slots per split: tiles rounded up to a multiple of 8
    int remap;       // 1: XCD-aware order of tiles (single split only)
    int nfast;       // 1: tiles numbered N-fastest (split-K with weights larger than x)
    int vec_out;     // 1: out is 16-byte aligned and OC % 4 == 0 (16-byte stores allowed)
    FastDiv div_ohw, div_ow;    // division by OH * OW and by OW
    // strip kernel only
    int strip_px;    // output pixels per workgroup
    int chunk_px;    // output pixels per patch load
    int lds_zero, lds_patch, lds_scratch, lds_flags;   // LDS: zero block size; offsets of patch, epilogue scratch, progress words
    // window kernel only
    int win_seg, win_segs;   // pixels per unit, units per output row
    int win_sh;              // k positions before a window (0 or 1)
    int win_wp, win_rb;      // LDS bytes per weight row, per input-row buffer
    int lds_rows;            // LDS offset of the input-row buffers
    int win_sets;            // input-row buffer sets (units in flight + 1)
    FastDiv win_div_g;       // division by tiles_m (the unit groups)
    FastDiv win_div_q, win_div_q1;  // by tiles_m / 8 and tiles_m / 8 + 1 (an XCD's groups)
    // resident kernel only (also lds_rows: LDS offset of the input rows)
    int res_zero;            // LDS offset of the zero pixel record
    int res_scr;             // LDS offset of the per-wave store scratch, or -1 (dword stores)
    int res_flipw;           // 1: w holds the forward weights of a data backward's mapped
                             // problem (64 x 64 channels, square kernel), flipped and
                             // transposed in LDS by the prologue
    // image kernel only
    int img_set, img_wofs;   // LDS bytes per buffer set; weights' offset within a set
    int img_ti, img_ts;      // workgroup blocks: images x channel slices (dividing N and tiles_n)
    int img_flipw;           // 1: w holds the forward weights of a data backward's mapped problem,
                             // copied as they are and flipped and transposed in LDS per chunk
};

// Workgroup IDs are dealt round-robin to the 8 XCDs (id % 8).  Renumber them
// so each XCD works through a contiguous range of tiles: neighbouring M tiles
// share input rows (the kernel's halo) and all M tiles of one N column share
// weights, so they should meet in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg)
{
    const int q = nwg >> 3, r = nwg & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

__device__ __forceinline__ int swz(int row, int chunk)
{
    return row * kChunks + (chunk ^ ((row >> 1) & 7));
}

struct TileCoord {
    int split, tile, m0, n0, kt_begin, kt_end;
    bool valid;
};

// Workgroup -> (split, tile, K range).  Split-major with a stride of
// tiles_pad (a multiple of 8): the predecessor of split s of a tile has an
// id lower by tiles_pad, so it sits on the same XCD and was dispatched there
// before this workgroup; a waiting workgroup never holds a slot its
// predecessor needs.
template <int BM, int BN>
__device__ __forceinline__ TileCoord tile_coord(const ConvArgs &a)
{
    TileCoord t;
    int bid = blockIdx.x;
    if (a.remap)
        bid = xcd_remap(bid, gridDim.x);
    t.split = bid / a.tiles_pad;
    t.tile = bid - t.split * a.tiles_pad;
    const int tiles = a.tiles_m * a.tiles_n;
    t.valid = t.tile < tiles;
    // Split-K keeps ids round-robin over the XCDs (tile t on XCD t % 8).
    // Numbering the tiles N-fastest then gives each XCD a fixed set of
    // output-channel columns, so its L2 holds only those columns' weights.
    const int tm = a.nfast ? t.tile / a.tiles_n : t.tile % a.tiles_m;
    const int tn = a.nfast ? t.tile - tm * a.tiles_n : t.tile / a.tiles_m;
    t.m0 = tm * BM;
    t.n0 = tn * BN;
    t.kt_begin = (int)(((long long)t.split * a.ktiles) / a.splits);
    t.kt_end = (int)(((long long)(t.split + 1) * a.ktiles) / a.splits);
    return t;
}

// Bits of a float for a dword store.  Takes the value, not a vector
// element: __builtin_bit_cast of an ext_vector element lvalue (v[e]) reads
// element 0 with this compiler, whatever e is.
__device__ __forceinline__ unsigned f32_bits(float f)
{
    return __builtin_bit_cast(unsigned, f);
}

// Buffer stores to out are used only while out ends at or below
// kOutOfRange: masked lanes store to that offset, which must then lie past
// the buffer (the host clamps out_bytes to it as well).
__device__ __forceinline__ bool out_fits_buffer(const ConvArgs &a)
{
    return (unsigned long long)a.M * (unsigned)a.OC * 4ull <= (unsigned long long)kOutOfRange;
}

// Row of value v of an S x S accumulator block, relative to the lane's row0.
template <int S>
__device__ __forceinline__ int acc_row(int v)
{
    return S == 16 ? v : 8 * (v >> 2) + (v & 3);
}

template <int S>
__device__ __forceinline__ int acc_row0(int lane)
{
    return S == 16 ? 4 * (lane >> 4) : 4 * (lane >> 5);
}

template <int S>
__device__ __forceinline__ int acc_col0(int lane)
{
    return S == 16 ? (lane & 15) : (lane & 31);
}

// Write the accumulators of one wave.  Block (i, j) of this lane covers rows
// row0 + i*16 + v (v = 0..3) and column col0 + j*16; bv[j] is that column's
// bias (0 without bias).
//
// Serial split-K: split s waits until the tile's semaphore reads s, then
// writes bias + partial (s = 0) or adds its partial to what is there, then
// hands the tile to s + 1 (the last split resets the semaphore to 0, so the
// array stays zeroed between calls).  The summation order is fixed:
// ((bias + p0) + p1) + ..., so repeated runs agree bit for bit.
//
// The hand-off needs no cache maintenance: the partial sums and the
// semaphore are read and written with sc1 (agent-coherent) accesses, the
// instructions the gfx950 memory model uses for relaxed agent-scope atomics,
// which are coherent across XCDs by themselves.  They are issued as plain
// buffer loads/stores with the sc1 policy so that a thread's loads go out as
// one batch.  A writer waits until all of its stores are acknowledged
// (vmcnt 0) before the barrier that precedes the semaphore store, and a
// reader loads only after the barrier that follows the semaphore load.
template <int S, int FM, int FN, typename AccT>
__device__ __forceinline__ void store_tile(const ConvArgs &a, const AccT (&acc)[FM][FN],
                                           const float (&bv)[FN], int row0, int col0,
                                           int split, int tile)
{
    constexpr int NV = S * S / 64;      // results per lane per block
    if (a.splits == 1) {
        // buffer stores (the output policy) while out ends at or below the
        // out-of-range offset that masked lanes store to, else plain 64-bit
        // addressed stores
        const bool small = out_fits_buffer(a);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.out_bytes, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int oc = col0 + j * S;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int m = row0 + i * S + acc_row<S>(v);
                    const float val = acc[i][j][v] + bv[j];
                    if (small) {
                        const unsigned off = (m < a.M && oc < a.OC) ? 4u * (unsigned)(m * a.OC + oc) : kOutOfRange;
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, val), ro, off, 0, kOutAux);
                    } else if (m < a.M && oc < a.OC) {
                        a.out[(long long)m * a.OC + oc] = val;
                    }
                }
            }
        return;
    }

    // Every wave waits for the turn itself (its first lane polls), so no
    // workgroup-wide vote is needed (__syncthreads_or takes static LDS,
    // which measured 4 % slower launches of the kernels that use this).
    int *sem = a.sem + tile;
    int late = 0;
    if ((threadIdx.x & 63) == 0) {
        int spins = 0;
        while (__hip_atomic_load(sem, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != split) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins >= a.spin_limit) {
                const int tiles = a.tiles_m * a.tiles_n;
                __hip_atomic_store(a.sem + tiles, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                late = 1;
                break;
            }
        }
    }
    late = __builtin_amdgcn_readfirstlane(late);
    // A wave whose wait gave up must not add its partial while the tile's
    // turn holder may be writing it: it poisons its part of the tile with
    // NaN instead (so the failure shows in out without a status poll), and
    // the semaphore is left as it is unless the first wave got the turn;
    // conv2d_fwd_status reports the timeout and resets the semaphores.
    if (late) {
        // (a rolled loop: this path never runs in practice, and unrolled it
        // would add a thousand instructions to every kernel that has it)
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.out_bytes, kRsrcWord3);
#pragma unroll 1
        for (int q = 0; q < FM * FN * NV; ++q) {
            const int i = q / (FN * NV), j = (q / NV) % FN, v = q % NV;
            const int m = row0 + i * S + acc_row<S>(v), oc = col0 + j * S;
            const unsigned off = (m < a.M && oc < a.OC) ? 4u * (unsigned)(m * a.OC + oc) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(0x7fc00000u, ro, off, 0, kCoherent);
        }
        __syncthreads();
        return;
    }
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.out_bytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        // one block row at a time: its loads go out as one batch
        unsigned off[FN][NV];
        float prev[FN][NV];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int m = row0 + i * S + acc_row<S>(v), oc = col0 + j * S;
                off[j][v] = (m < a.M && oc < a.OC) ? 4u * (unsigned)(m * a.OC + oc) : kOutOfRange;
                prev[j][v] = split == 0 ? bv[j]
                    : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ro, off[j][v], 0, kCoherent));
            }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < NV; ++v)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(unsigned, prev[j][v] + acc[i][j][v]), ro, off[j][v], 0,
                    kCoherent);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this thread's stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0)            // (the first wave got the turn: it did not give up)
        __hip_atomic_store(sem, (split + 1 == a.splits) ? 0 : split + 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Floats per row of the epilogue scratch for a block row of C columns: C
// plus a pad that puts the rows written by one store instruction into
// disjoint bank groups (rows 4 apart for 32x32 blocks: stride = 8 mod 16;
// rows 4, 8, 12 apart for 16x16 blocks: stride = 4 mod 16).
template <int S, int C>
struct EpiScratch {
    static constexpr int stride = C + (S == 32 ? 8 : 4);
    static constexpr int floats = S * stride;        // per wave
};

// Single-split epilogue with 16-byte stores: per block row i, each wave
// writes acc + bias of its S x WTN sub-tile into its own LDS scratch in
// row-major order, reads it back four consecutive output channels per lane
// and stores them with one 16-byte store.  A store instruction then covers
// whole row segments of WTN channels instead of 4-byte pieces.  The scratch
// is private to the wave, and LDS accesses of one wave are performed in
// order, so no barrier is needed between block rows.
template <int S, int FM, int FN, int WTN, typename AccT>
__device__ __forceinline__ void store_tile_vec(const ConvArgs &a, const AccT (&acc)[FM][FN],
                                               const float (&bv)[FN], int m_wave0, int n_wave0,
                                               float *scratch)
{
    constexpr int NV = S * S / 64;
    constexpr int STRIDE = EpiScratch<S, WTN>::stride;
    constexpr int C4 = WTN / 4;                      // float4 per scratch row
    constexpr int F = S * C4;                        // float4 per block row
    static_assert(F % 64 == 0, "whole float4 passes");
    const int lane = threadIdx.x & 63;
    const int r0 = acc_row0<S>(lane), c0 = acc_col0<S>(lane);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, a.out_bytes, kRsrcWord3);
    const bool small = out_fits_buffer(a);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < NV; ++v)
                scratch[(r0 + acc_row<S>(v)) * STRIDE + j * S + c0] = acc[i][j][v] + bv[j];
#pragma unroll
        for (int t = 0; t < F / 64; ++t) {
            const int f = t * 64 + lane;
            const int row = f / C4, c4 = (f % C4) * 4;
            const floatx4_t val = *(const floatx4_t *)(scratch + row * STRIDE + c4);
            const int m = m_wave0 + i * S + row, oc = n_wave0 + c4;
            if (m < a.M && small) {
                // (the output policy; out ends at or below kOutOfRange)
                const unsigned off = 4u * (unsigned)(m * a.OC + oc);
                if (oc + 3 < a.OC) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, val), ro, off, 0, kOutAux);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(f32_bits(val[e]), ro,
                                                              oc + e < a.OC ? off + 4u * e : kOutOfRange, 0, kOutAux);
                }
            } else if (m < a.M) {
                float *o = a.out + (long long)m * a.OC + oc;
                if (oc + 3 < a.OC) {
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
}

// Zero an int array (semaphores); a plain kernel, so the call is an ordinary
// kernel node if the caller captures the stream in a graph.
__global__ void fill_zero_i32(int *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0;
}

}  // namespace convimg
