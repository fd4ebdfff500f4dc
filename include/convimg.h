/*
 * convimg.h -- C ABI of libconvimg: 2-D convolution forward computed as an
 * implicit GEMM on AMD Instinct MI355X (gfx950).
 *
 * The operation is the forward convolution of the burn conv pages
 * (burn-cubecl "kernel/conv/base.rs" listing, conv_forward_nhwc: NHWC input,
 * weight permuted to [OC][KH][KW][IC], optional bias "added to each
 * channel", groups = 1 on the implicit-GEMM route):
 *
 *   out[n][oh][ow][oc] = bias[oc] + sum_{kh,kw,ic}
 *       X(n, oh*stride - pad + kh*dilation, ow*stride - pad + kw*dilation, ic)
 *       * w[oc][kh][kw][ic]
 *
 * with X = x inside the image and 0 in the padding.  It is evaluated as a
 * GEMM with M = N*OH*OW, N = OC, K = IC*KH*KW (burn PR "Introduce
 * autotuning to conv2d and conv_transpose2d with a new im2col/GEMM
 * algorithm", Changes: the implicit-GEMM dimensions batch*out_h*out_w,
 * out_channels, in_channels*kernel_h*kernel_w).  The A operand is gathered
 * from x on the fly; no im2col buffer is ever written.
 *
 * Every entry point is extern "C", takes plain pointers and sizes, and never
 * throws.  Nothing is printed unless the environment sets CONVIMG_LOG=1.
 */
#ifndef CONVIMG_H
#define CONVIMG_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of x and w.  The output and the bias are always fp32. */
#define CONVIMG_BF16 0   /* bf16 inputs, bf16 MFMA products, fp32 accumulation */
#define CONVIMG_FP32 1   /* fp32 inputs, fp32 MFMA products, fp32 accumulation */

/* Status codes.  0 is success; every error is returned before any work is
 * queued, and then `out` is untouched, except CONVIMG_ERR_LAUNCH. */
#define CONVIMG_OK          0
#define CONVIMG_ERR_NULL    1  /* x, w or out is NULL, or plan is NULL */
#define CONVIMG_ERR_SHAPE   2  /* a size <= 0, stride/dilation < 1, pad < 0, or no output pixel */
#define CONVIMG_ERR_DTYPE   3  /* dtype is neither CONVIMG_BF16 nor CONVIMG_FP32 */
#define CONVIMG_ERR_RANGE   4  /* an element count of x, w or out reaches 2^31 */
#define CONVIMG_ERR_ALIAS   5  /* out overlaps x, w or bias */
#define CONVIMG_ERR_ALLOC   6  /* the library could not allocate its semaphores */
#define CONVIMG_ERR_LAUNCH  7  /* the HIP runtime refused the launch */
#define CONVIMG_ERR_DEVICE  8  /* no usable HIP device, or a device query failed */
#define CONVIMG_ERR_TIMEOUT 9  /* a split-K wait gave up (reported by conv2d_fwd_status) */
#define CONVIMG_ERR_UNSUPPORTED 10 /* no entry point returns it now: conv2d_bwd_data serves every
                                      stride, window and padding, conv2d_bwd_weight fp32 storage */
#define CONVIMG_ERR_WORKSPACE 11   /* conv2d_bwd_weight: ws_bytes below what it needs */
#define CONVIMG_ERR_SCRATCH 12     /* conv2d_fwd_noalloc: the plan needs more semaphores than its scratch holds */

/* Loader variants used by the plan. */
#define CONVIMG_LOADER_TAP    0  /* IC % 64 == 0: one 64-channel slice of one tap per K tile, 16-byte loads */
#define CONVIMG_LOADER_VEC8   1  /* IC % 8 == 0: 16-byte loads of 8 channels, tap decoded per vector */
#define CONVIMG_LOADER_SCALAR 2  /* any IC (the masked edge path): element-wise gather */
#define CONVIMG_LOADER_FP32   3  /* fp32 storage: element-wise gather into fp32 tiles */

/* What conv2d_fwd will launch for a problem (filled by conv2d_fwd_plan). */
typedef struct convimg_plan {
    int OH, OW;          /* output extent */
    long long M;         /* N*OH*OW */
    int Ngemm;           /* OC */
    int K;               /* IC*KH*KW */
    int tile_id;         /* index into the tile table */
    int BM, BN, BK;      /* workgroup tile */
    int loader;          /* CONVIMG_LOADER_* */
    int splits;          /* split-K factor S (1 = no split) */
    int tiles_m, tiles_n, ktiles;
    int grid;            /* workgroups launched = tiles_m*tiles_n*splits */
    int threads;         /* threads per workgroup */
    int lds_bytes;       /* LDS per workgroup */
} convimg_plan;

/*
 * conv2d_fwd -- out = conv2d(x, w) + bias, asynchronously on `stream`.
 *
 *   x     device pointer, [N][H][W][IC] contiguous (NHWC), bf16 or fp32 per dtype
 *   w     device pointer, [OC][KH][KW][IC] contiguous (OHWI), same type as x
 *   bias  device pointer to OC fp32 values, or NULL for zeros
 *   out   device pointer, [N][OH][OW][OC] fp32 contiguous (NHWC); every element
 *         is overwritten (nothing is accumulated into its previous contents)
 *   stride >= 1, pad >= 0, dilation >= 1: the same for both spatial axes
 *   OH = floor((H + 2*pad - dilation*(KH-1) - 1)/stride) + 1, likewise OW
 *   stream  HIP stream on the device that owns all four buffers (0 = null stream)
 *
 * Ownership: the caller owns x, w, bias and out and keeps them alive until
 * the stream has run the call.  The library owns only a small array of int32
 * split-K semaphores per (device, stream), allocated on first need (that
 * first call may block while it allocates) and freed by conv2d_release().
 *
 * Errors: CONVIMG_ERR_* as listed above; argument errors leave `out`
 * untouched and queue nothing.  A fault inside the kernel surfaces at the
 * caller's next synchronisation, as for any HIP kernel.  Calls on different
 * streams may run concurrently; calls on one stream run in order.
 *
 * Split-K (plans with splits > 1): the splits of an output tile take turns
 * on a semaphore, with a bounded wait.  The plan keeps every split of every
 * tile resident at once, so the wait always ends in practice; if it ever
 * gives up, that split writes NaN over (its part of) its tile instead of adding its
 * partial sums, so `out` is invalid and visibly so, and the stream's
 * semaphores stay out of step until conv2d_fwd_status() is called, which
 * reports CONVIMG_ERR_TIMEOUT and resets them.
 */
int conv2d_fwd(const void *x, const void *w, const float *bias,
               int N, int H, int W, int IC, int OC, int KH, int KW,
               int stride, int pad, int dilation, int dtype,
               float *out, hipStream_t stream);

/* conv2d_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, plan, kernels and result as conv2d_fwd; it calls no
 * hipMalloc, hipFree or other allocating routine.  Its only scratch, the
 * split-K semaphores, lives in a fixed array of 4096 int32 in each device's
 * memory (held until the process ends), cleared by a small kernel on
 * `stream` at the start of every split-K call.  Every call on one device
 * shares that array: calls that overlap on one device (different streams
 * running at once) race and must not be made.  A split-K wait that gives
 * up shows only as NaN tiles in `out` (conv2d_fwd_status does not cover
 * this entry point).  Errors: those of conv2d_fwd, and CONVIMG_ERR_SCRATCH
 * (before any work is queued) if the plan would need more than 4095
 * semaphores, which the plan's residency cap keeps from happening on
 * MI355X. */
int conv2d_fwd_noalloc(const void *x, const void *w, const float *bias,
                       int N, int H, int W, int IC, int OC, int KH, int KW,
                       int stride, int pad, int dilation, int dtype,
                       float *out, hipStream_t stream);

/* Output extent along one axis, or -1 when an argument is out of range or no
 * window fits.  Host only.  The pages give no formula for it: this is the
 * floor formula quoted under conv2d_fwd (a trailing input row or column that
 * does not complete a window is not used), the usual reading of the burn
 * conv options' stride, padding and dilation (burn-cubecl
 * "kernel/conv/base.rs" listing, ConvOptions). */
int conv2d_fwd_out_dim(int in, int k, int stride, int pad, int dilation);

/* The plan conv2d_fwd would use for this problem with 16-byte aligned
 * buffers, on a device with `num_cus` compute units (num_cus <= 0: query the
 * current device).  Host only when num_cus > 0.  Returns a status code.
 * The pages choose among their kernels by shape (burn PR "[Optimization]
 * Implicit gemm rewrite", Changes: small and large K behave differently;
 * burn PR "Introduce autotuning to conv2d and conv_transpose2d with a new
 * im2col/GEMM algorithm", Changes: the implicit GEMM only where its
 * divisibility conditions hold); this reports this library's own choice. */
int conv2d_fwd_plan(int N, int H, int W, int IC, int OC, int KH, int KW,
                    int stride, int pad, int dilation, int dtype, int num_cus,
                    convimg_plan *plan);

/* Static description of a status code (never NULL).  Library plumbing: the
 * pages define no status codes (burn-cubecl "kernel/conv/base.rs" listing
 * returns a ConvSetupError for setups it cannot run, the role these codes
 * play here). */
const char *conv2d_strerror(int status);

/* Test knob: force the tile (-1 = automatic), the split-K factor (-1 =
 * automatic) and the loader (-1 = automatic) of later calls in this process.
 * A forced loader is honoured only when the shape allows it (the vector
 * loaders need IC % 64 or IC % 8 and aligned buffers); a forced split is
 * clipped to the number of K tiles.  Returns CONVIMG_OK or
 * CONVIMG_ERR_SHAPE for an unknown tile or loader. */
int conv2d_fwd_force(int tile_id, int splits, int loader);

/* Number of entries in the tile table (valid tile_id values are 0..n-1).
 * The table is this library's tile/occupancy table per shape class; the
 * pages' kernels pick tile sizes per problem the same way (burn PR
 * "[Optimization] Implicit gemm rewrite", Changes). */
int conv2d_fwd_num_tiles(void);

/* Kernel family of a tile table entry, or -1 for an unknown tile_id:
 *   CONVIMG_KIND_REGS  register-staged gather (every loader, incl. the edge path)
 *   CONVIMG_KIND_PIPE  multi-stage direct-to-LDS pipeline (vector loaders)
 *   CONVIMG_KIND_PATCH pipeline with an LDS patch of input rows (IC % 64 == 0)
 *   CONVIMG_KIND_STRIP one workgroup per CU per 64 output channels: the
 *                      weight slice for all of K and the input rows of a strip
 *                      of output pixels held in LDS (IC % 64 == 0, when
 *                      they fit).  Forcing any strip entry selects this
 *                      kernel with the chunk size the plan derives; a problem
 *                      it cannot take falls back to the pipelined kernel.
 *   CONVIMG_KIND_WINDOW few input channels (the fast edge path, e.g. IC = 3):
 *                      one kernel row of the receptive field, ((KW-1)*d+1)*IC
 *                      elements, fits in 32 k values; input rows copied to
 *                      LDS, weights in registers.  Chosen automatically where
 *                      the element-wise gather would run and it applies.
 *   CONVIMG_KIND_RESIDENT one workgroup per CU per 64 output channels holds the
 *                      weight slice and every input row of its share of the
 *                      output pixels in LDS, then its waves work through
 *                      32-pixel units with no further copies (3x3, IC = 16,
 *                      32, 64 or 128, when they fit).
 *   CONVIMG_KIND_IMAGE deep layers on small images: one workgroup per image
 *                      and 32 output channels over all of K, K in chunks of
 *                      64 input channels with the zero-padded image and the
 *                      chunk's weights double-buffered in LDS (3x3,
 *                      IC % 64 == 0, at most 256 output pixels per image).
 * Host only. */
#define CONVIMG_KIND_REGS   0
#define CONVIMG_KIND_PIPE   1
#define CONVIMG_KIND_PATCH  2
#define CONVIMG_KIND_STRIP  3
#define CONVIMG_KIND_WINDOW 4
#define CONVIMG_KIND_RESIDENT 5
#define CONVIMG_KIND_IMAGE 6
int conv2d_fwd_tile_kind(int tile_id);

/* Split-K health on `stream` (conv2d_fwd's splits and conv2d_bwd_weight's
 * in-place pixel ranges): CONVIMG_OK, or CONVIMG_ERR_TIMEOUT if a
 * workgroup gave up waiting for its turn since the last call of this
 * function (the flag and the stream's semaphores are then reset).
 * Synchronises the stream.  The turn-taking is that of nvFuser issue
 * "Split-K matmul is slow even for few partitions", section "Eliminating
 * the workspace" (blocks serialised by a semaphore); the bounded wait and
 * this report are this library's own. */
int conv2d_fwd_status(hipStream_t stream);

/* Test knob: the number of sleep iterations a split-K workgroup (of
 * conv2d_fwd, or a pixel range of conv2d_bwd_weight adding into dw) waits
 * for its turn before it gives up (iterations < 1: the default, 2^20), for
 * later calls in this process.  Lets tests force the timeout path from the
 * host.  Returns the previous bound. */
int conv2d_fwd_test_spin_limit(int iterations);

/* NCHW tensors (burn-cubecl "kernel/conv/base.rs" listing: its NCHW entry
 * points permute the input to channels-last and the weights to
 * [OC][KH][KW][IC], run the NHWC convolution and permute the result back).
 * Here bf16 problems that conv2d_fwd runs on its resident kernel (3x3),
 * with W % 8 == 0 and x and out 16-byte aligned, take one launch of that
 * kernel's NCHW variant instead, which reads x and w and writes out in
 * these layouts itself (the workspace is then not used); every other
 * problem takes the permutes around conv2d_fwd.
 *
 *   x     device, N x IC x H x W (NCHW) in `dtype`
 *   w     device, OC x IC x KH x KW (OIHW) in `dtype`
 *   bias  device, OC fp32 values, or NULL
 *   out   device, N x OC x OH x OW (NCHW) in `out_dtype` (CONVIMG_FP32, or
 *         CONVIMG_BF16: the fp32 result rounded to nearest even), fully
 *         overwritten
 *   ws    device workspace of ws_bytes >= conv2d_fwd_nchw_workspace bytes,
 *         caller-owned: on the permute route receives the NHWC copy of x,
 *         the OHWI copy of w and the fp32 NHWC result, which conv2d_fwd
 *         computes (so a bf16 output never serves as the split-K
 *         accumulation buffer); required on both routes
 *   other arguments and the output extent as for conv2d_fwd
 *
 * Errors (before any work is queued): those of conv2d_fwd;
 * CONVIMG_ERR_NULL for a NULL ws; CONVIMG_ERR_DTYPE for another out_dtype;
 * CONVIMG_ERR_WORKSPACE if ws_bytes is too small; CONVIMG_ERR_ALIAS if out
 * or ws overlaps another buffer; CONVIMG_ERR_RANGE for N or OC above 65535
 * or more than 65535 64-wide tiles of IC or OH*OW.  Asynchronous on
 * `stream`; the workspace is in use until the stream has run the call. */
int conv2d_fwd_nchw(const void *x, const void *w, const float *bias, int N, int H, int W, int IC, int OC,
                    int KH, int KW, int stride, int pad, int dilation, int dtype, int out_dtype, void *out,
                    void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes conv2d_fwd_nchw needs for this problem, in *bytes.
 * Errors: CONVIMG_ERR_NULL for a NULL bytes, the argument errors of
 * conv2d_fwd. */
int conv2d_fwd_nchw_workspace(int N, int H, int W, int IC, int OC, int KH, int KW, int stride, int pad,
                              int dilation, int dtype, size_t *bytes);

/* Run-time selection over the tile table (burn PR "Introduce autotuning to
 * conv2d and conv_transpose2d with a new im2col/GEMM algorithm", Changes:
 * the fastest of the candidate algorithms is picked by timing them on the
 * problem and the choice is cached per problem).
 *
 * Times, on `stream` with the caller's buffers, the plan conv2d_fwd would
 * use and the plans the planner makes of every other tile of the table
 * (with its split-K factor, half of it and none), 2 warm-up and 5 timed
 * launches each, and records the fastest for this problem: later
 * conv2d_fwd and conv2d_fwd_plan calls (any thread) on the same shape,
 * dtype, device CU count and 16-byte alignment of x and w use it.  `out`
 * is overwritten many times and finally holds the chosen plan's result.
 * Arguments as for conv2d_fwd; tile_out / splits_out receive the choice
 * and us_best / us_default the mean microseconds per launch of it and of
 * the static plan (each of the four may be NULL).  Synchronises `stream`.
 * Errors: those of conv2d_fwd (nothing is recorded then). */
int conv2d_fwd_autotune(const void *x, const void *w, const float *bias, int N, int H, int W, int IC, int OC,
                        int KH, int KW, int stride, int pad, int dilation, int dtype, float *out,
                        hipStream_t stream, int *tile_out, int *splits_out, float *us_best, float *us_default);

/* Forget every choice conv2d_fwd_autotune recorded (the static plans apply
 * again). */
void conv2d_fwd_autotune_clear(void);

/* Data backward: the gradient of conv2d_fwd's output with respect to its
 * input x (burn-cubecl "kernel/conv/base.rs" listing, conv_data_backward,
 * whose implicit-GEMM route serves groups = 1 and stride 1):
 *
 *   dx[n][ih][iw][ic] = sum_{kh,kw,oc} dY(n, ih + pad - kh*dilation,
 *                                         iw + pad - kw*dilation, oc)
 *                       * w[oc][kh][kw][ic]
 *
 * with dY = dy inside [0,OH) x [0,OW) and 0 outside.  For stride 1 this is
 * the forward convolution of dy with the weights flipped in both spatial
 * axes and transposed OC <-> IC, padding dilation*(KH-1) - pad: the call
 * writes those weights to `wt` (conv2d_bwd_data_weights), then runs
 * conv2d_fwd(dy, wt, NULL, N, OH, OW, OC, IC, KH, KW, 1,
 * dilation*(KH-1) - pad, dilation, dtype, dx, stream) -- same plans, same
 * kernels, no bias.  Where that forward runs (bf16) on the resident kernel
 * with 64 -> 64 channels or on the image kernel, the kernel instead copies
 * w itself and flips and transposes it in LDS: one launch, and `wt` is
 * left as it was.  A
 * caller whose weights do not change between calls may transform them once
 * and make that conv2d_fwd call itself.  Every other problem (stride above
 * 1, KH != KW, pad > dilation*(KH-1): the listing's fallback route)
 * computes dx from the definition above as a GEMM over the input pixels,
 * K = (tap, oc), and leaves `wt` as it was: in bf16 with OC % 8 == 0 and a
 * 16-byte aligned dy, a kernel that takes the input pixels by phase of the
 * stride (ih % stride, iw % stride), so that each tile runs only the taps
 * whose (ih + pad - kh*dilation) / stride divides evenly (bf16 MFMA, exact
 * products, fp32 sums); otherwise a kernel that gathers dY element by
 * element with the divisibility test (fp32 products and sums; bf16
 * products are exact in fp32).
 *
 *   dy    device, N x OH x OW x OC (NHWC) in `dtype`, OH/OW the forward
 *         output extents of H/W (the formula under conv2d_fwd)
 *   w     device, OC x KH x KW x IC (OHWI) in `dtype`: the forward weights
 *   wt    device, OC*KH*KW*IC elements of `dtype`, caller-owned workspace;
 *         receives IC x KH x KW x OC, the flipped and transposed weights,
 *         except on the in-LDS path and the fallback route (then untouched)
 *   dx    device, fp32 N x H x W x IC (NHWC), fully overwritten
 *   N, H, W, IC, OC, KH, KW, stride, pad, dilation, dtype: the forward
 *         problem's arguments
 *
 * Errors: the argument errors of conv2d_fwd for the forward problem and
 * (stride 1) for the one it maps to; CONVIMG_ERR_ALIAS if wt or dx overlaps
 * another buffer; CONVIMG_ERR_RANGE (fallback route) for dy, w or dx of
 * 2^31 bytes or more; CONVIMG_ERR_DEVICE without a usable device.  These are returned before any work is queued.  After the
 * transform is queued, CONVIMG_ERR_LAUNCH / CONVIMG_ERR_ALLOC may still come
 * back (wt then holds the transform).  Asynchronous on `stream`. */
int conv2d_bwd_data(const void *dy, const void *w, int N, int H, int W, int IC, int OC, int KH, int KW,
                    int stride, int pad, int dilation, int dtype, void *wt, float *dx, hipStream_t stream);

/* The weight transform of conv2d_bwd_data alone (same passage):
 *
 *   wt[ic][KH-1-kh][KW-1-kw][oc] = w[oc][kh][kw][ic]
 *
 * for any KH, KW.  w: device, OC x KH x KW x IC in `dtype`; wt: device,
 * the same number of elements, caller-owned, must not overlap w.  Errors
 * (returned before any work is queued): CONVIMG_ERR_NULL, _SHAPE (a size
 * <= 0), _DTYPE, _RANGE (2^31 elements or more, or more than 65535
 * 64-channel tiles of OC or kernel taps), _ALIAS; _LAUNCH if the launch
 * fails.  Asynchronous on `stream`. */
int conv2d_bwd_data_weights(const void *w, int OC, int KH, int KW, int IC, int dtype, void *wt,
                            hipStream_t stream);

/* Weight backward: the gradient of conv2d_fwd's output with respect to its
 * weights w (burn-cubecl "kernel/conv/base.rs" listing, conv_weight_backward,
 * whose implicit-GEMM route serves every groups = 1 problem):
 *
 *   dw[oc][kh][kw][ic] = sum_{n,oh,ow} dy[n][oh][ow][oc]
 *                        * X(n, oh*stride - pad + kh*dilation, ow*stride - pad + kw*dilation, ic)
 *
 * with X = x inside the image and 0 in the padding; any stride, padding and
 * dilation.  An implicit GEMM with M = OC, N = KH*KW*IC and the reduction
 * over the N*OH*OW pixels, split into contiguous pixel ranges.  Up to four
 * ranges add into dw in range order, taking turns on the library's split-K
 * semaphores (the forward's serial split-K; no workspace); more ranges
 * write partial sums to `ws`, which a second kernel adds in a fixed order.
 * Either way the result is the same on every call.  A range whose wait for
 * its turn gives up (a bound of many milliseconds) writes NaN over its part
 * of dw and sets the status that conv2d_fwd_status reports.  fp32 storage
 * runs a kernel of its own with fp32 products and sums (v_mfma_f32_16x16x4
 * _f32), its ranges at most 8192 pixels each and always through `ws` when
 * there are several.
 *
 *   x     device, N x H x W x IC (NHWC) in `dtype`
 *   dy    device, N x OH x OW x OC (NHWC) in `dtype`, OH/OW the forward
 *         output extents of H/W (the formula under conv2d_fwd)
 *   dw    device, fp32 OC x KH x KW x IC (OHWI, the layout of w), fully
 *         overwritten
 *   ws    device workspace of ws_bytes bytes, caller-owned; at least what
 *         conv2d_bwd_weight_workspace reports for the same problem on the
 *         current device (NULL allowed when that is 0)
 *   N, H, W, IC, OC, KH, KW, stride, pad, dilation: the forward problem
 *   dtype CONVIMG_BF16 or CONVIMG_FP32
 *
 * Errors (returned before any work is queued): the argument errors of
 * conv2d_fwd for the forward problem; CONVIMG_ERR_RANGE (fp32) when the
 * ranges' partial sums would need more than 1 GiB of workspace;
 * CONVIMG_ERR_NULL for a NULL x, dy or dw, or a NULL ws when one is
 * needed; CONVIMG_ERR_WORKSPACE if ws_bytes is too small; CONVIMG_ERR_ALIAS
 * if dw or the used part of ws overlaps another buffer.  CONVIMG_ERR_LAUNCH
 * if a launch fails.  Asynchronous on `stream`; the workspace is in use
 * until the stream has run the call. */
int conv2d_bwd_weight(const void *x, const void *dy, int N, int H, int W, int IC, int OC, int KH, int KW,
                      int stride, int pad, int dilation, int dtype, float *dw, void *ws, size_t ws_bytes,
                      hipStream_t stream);

/* Bytes of workspace conv2d_bwd_weight needs for this problem on the current
 * device (0: none), in *bytes.  Errors: CONVIMG_ERR_NULL for a NULL bytes,
 * the argument errors of conv2d_bwd_weight, CONVIMG_ERR_DEVICE. */
int conv2d_bwd_weight_workspace(int N, int H, int W, int IC, int OC, int KH, int KW, int stride, int pad,
                                int dilation, int dtype, size_t *bytes);

/* Free every library-owned buffer (synchronising each device that has
 * one).  Later calls allocate again as needed.  Library plumbing with no
 * counterpart on the pages: the only library-owned buffers are the split-K
 * semaphores of conv2d_fwd and conv2d_bwd_weight. */
void conv2d_release(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVIMG_H */
