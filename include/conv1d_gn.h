/*
 * conv1d_gn.h - C ABI of the MI355X (gfx950) conv1d -> GroupNorm library.
 *
 * A 1-D convolution computed as an implicit GEMM (rows m = (n, t_out),
 * columns = output channels, reduction over (input channel, tap)), feeding a
 * GroupNorm, a LayerNorm over channels, or nothing, with an optional per-row
 * min plus broadcast bias.
 *
 * Operation sources (web pages, cited by title and passage):
 *   "Kimi-K2.6 l2_p35"  POPCORNBENCH trace, Conv1d -> GroupNorm: the problem
 *                       statement (x [N,C_in,T], weight [C_out,C_in,K],
 *                       gamma/beta [C_out]), the output-length formula, the
 *                       conv input index with zero padding, GroupNorm over
 *                       (C_out/G channels x T_out) per (n, group) with
 *                       population variance and eps inside the square root.
 *   "Kimi-K2.6 l1_p5"   POPCORNBENCH trace, causal Conv1d: left padding of
 *                       (K-1)*dilation zeros, no right padding, tap 0 oldest.
 *   "Kimi-K2.6 l2_p75"  POPCORNBENCH trace, Linear -> GroupNorm -> min ->
 *                       +bias: the K=1, T=1 case, min over channels after
 *                       the GroupNorm affine, bias broadcast over channels.
 *   "Kimi-K2.6 l2_p3"   POPCORNBENCH trace: the stats-then-apply split of a
 *                       normalisation (statistics first, one affine pass after).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, contiguous, in device memory (HBM of the
 *     current HIP device).  x and w are fp32 or bf16 (c1g_dtype); y / out are
 *     fp32 or bf16 (c1g_conv_desc.out_dtype); every other tensor (bias,
 *     gamma, beta, bias2, mean, rstd) is fp32.  bf16 tensors hold the raw
 *     16-bit patterns; bf16 outputs are the fp32 results rounded to nearest
 *     even (accumulation, statistics and the affine always run in fp32).
 *   - Ownership: the caller allocates and frees every buffer, including the
 *     workspace; the library never allocates, frees or synchronises.  Outputs
 *     must not overlap inputs unless an entry point says so.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  All work
 *     is enqueued on it in order and returns immediately; results are ready
 *     when the stream is synchronised.
 *   - Errors: arguments are validated before anything is launched; on any
 *     error nothing is launched, outputs are untouched and a non-zero
 *     c1g_status is returned.  A launch failure reported by the HIP runtime
 *     returns C1G_ERR_HIP.  Device faults surface at the caller's next
 *     synchronisation, like any stream work.
 *   - Determinism: for a given device, shape and inputs the outputs are bit
 *     identical from run to run (no atomics; fixed reduction orders).
 *   - Thread safety: entry points may be called concurrently from several
 *     host threads; calls on one stream execute in order.
 *   - Empty batch: N = 0 is valid everywhere.  The call checks the other
 *     arguments, then returns C1G_OK without reading a pointer or launching
 *     anything (tensor pointers may be NULL); its workspace size is 0.
 *   - Sizes: conv1d_forward / conv1d_gn_forward take N up to 65535, C_in and
 *     C_out up to 2^30, T up to 2^40, x and w below 2^46 elements each and
 *     N*C_out*T_out below 2^32 (C1G_ERR_UNSUPPORTED beyond); every size check
 *     is made without a product that could wrap, so no oversized argument is
 *     accepted as a small one.  Taps K up to 8, and the input window of a
 *     tile must fit on chip: fp32 (split path), (128 - 1)*stride +
 *     (K - 1)*dilation + 1 <= 541 rows; bf16, the same window <= 544 rows
 *     (224 for K = 6..8), or, for strides 2 to 5, 512 + (ceil(K/stride) -
 *     1)*dilation <= 544 rows (passes over every stride-th row).  c1g_check
 *     reports whether a shape is built.
 *   - Environment variables (read at each call; none is needed):
 *       C1G_LOG=1             every entry-point call writes one line to stderr:
 *                             its sizes, the plan (route, tiles, workspace;
 *                             for the bf16 convolution its tile positions
 *                             and passes over the input channels),
 *                             the status and, for a refusal or a fallback taken
 *                             at run time, its cause.  Host only.
 *       C1G_FORCE_PATH=split  for tests: problems planned on a single-kernel
 *                             route (fused_single_pass, fused_persistent) take
 *                             the split route, so one problem runs down both.
 *       C1G_BARRIER_SPINS, C1G_RESIDENT_LIMIT  for tests of the routes whose
 *                             workgroups wait on each other (see c1g_route).
 */
#ifndef CONV1D_GN_H
#define CONV1D_GN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of x and w, and of y / out */
enum c1g_dtype { C1G_F32 = 0, C1G_BF16 = 1 };

/* memory layout of x */
enum c1g_layout {
  C1G_LAYOUT_NCL = 0,          /* x [N, C_in, T]: positions contiguous (default)      */
  C1G_LAYOUT_NLC = 1           /* x [N, T, C_in]: channels contiguous (channels-last)  */
};

/* normalisation applied to the convolution output y */
enum c1g_norm {
  C1G_NORM_NONE = 0,           /* out = y                                            */
  C1G_NORM_GROUP = 1,          /* GroupNorm over (C_out/G x T_out) per (n, group)     */
  C1G_NORM_LAYER_CHANNELS = 2  /* LayerNorm over the C_out values at each (n, t_out)  */
};

/* epilogue after the normalisation */
enum c1g_epilogue {
  C1G_EPI_NONE = 0,
  C1G_EPI_ROWMIN_BIAS = 1      /* out[n,c,t] = min_c' z[n,c',t] + bias2[c]             */
};

enum c1g_status {
  C1G_OK = 0,
  C1G_ERR_INVALID_ARG = 1,     /* bad size, NULL required pointer, C_out % G != 0 ...  */
  C1G_ERR_UNSUPPORTED = 2,     /* valid but not built (e.g. window wider than a tile)  */
  C1G_ERR_WORKSPACE = 3,       /* workspace NULL or smaller than the size query       */
  C1G_ERR_MISALIGNED = 4,      /* a tensor pointer not aligned to its element size,   */
                               /* x / w not 16-byte aligned on the gemm_rows route,   */
                               /* or a workspace not 256-byte aligned                 */
  C1G_ERR_HIP = 5              /* the HIP runtime reported an error at launch         */
};

/* Geometry of the convolution.
 *   x [N, C_in, T] (or [N, T, C_in] with x_layout = C1G_LAYOUT_NLC),
 *   w [C_out, C_in, K], y/out [N, C_out, T_out] with
 *   T_out = floor((T + pad_left + pad_right - dilation*(K-1) - 1) / stride) + 1
 *   ("Kimi-K2.6 l2_p35", output-length formula; symmetric padding p is
 *   pad_left = pad_right = p; causal per "Kimi-K2.6 l1_p5" is
 *   pad_left = (K-1)*dilation, pad_right = 0).
 *   y[n,c,t] = bias[c] + sum_{ci<C_in} sum_{j<K} w[c,ci,j] * x[n,ci,t*stride+j*dilation-pad_left],
 *   with x read as 0 outside [0, T): a cross-correlation, no kernel flip. */
typedef struct c1g_conv_desc {
  int64_t N, C_in, C_out, T;
  int32_t K, stride, dilation;
  int32_t pad_left, pad_right;
  int32_t dtype;               /* enum c1g_dtype of x and w */
  int32_t out_dtype;           /* enum c1g_dtype of y (conv1d_forward) and out
                                  (conv1d_gn_forward); 0 = fp32 */
  int32_t x_layout;            /* enum c1g_layout of x; 0 = [N, C_in, T].  The
                                  result is the same, bit for bit, in either layout:
                                  bf16 routes build their channels-last input image
                                  from it directly, fp32 routes transpose it once
                                  into the workspace (counted by the size queries);
                                  with T = 1 the two layouts are the same bytes */
} c1g_conv_desc;

/* What follows the convolution in conv1d_gn_forward. */
typedef struct c1g_norm_desc {
  int32_t norm;                /* enum c1g_norm                                        */
  int32_t G;                   /* groups for C1G_NORM_GROUP (C_out % G == 0); else 0   */
  float eps;                   /* added to the variance inside the square root (> 0)   */
  int32_t epilogue;            /* enum c1g_epilogue                                    */
  int32_t flags;               /* C1G_FLAG_* bits; 0 = defaults                        */
} c1g_norm_desc;

/* c1g_norm_desc.flags */
enum c1g_flags {
  C1G_FLAG_NO_PERSISTENT = 1,  /* no kernel whose workgroups wait on each other:
                                  never take the "fused_persistent" route, and ignore
                                  C1G_FLAG_ROWMIN_ONE_LAUNCH (both need every
                                  workgroup of a round resident at once) */
  C1G_FLAG_ROWMIN_ONE_LAUNCH = 2, /* "gemm_rows" with GroupNorm + row-min: one
                                  launch whose workgroups wait on each other instead of
                                  a GEMM and a broadcast kernel (same result, bit for
                                  bit) */
  C1G_FLAG_COOPERATIVE = 4     /* launch the kernels whose workgroups wait on each
                                  other ("fused_persistent", the one-launch row-min)
                                  through hipLaunchCooperativeKernel.  By default they
                                  are ordinary launches whose grid fits the device's
                                  resident capacity, which keeps every workgroup
                                  resident as long as no other work runs on the device
                                  at the same time; callers that share the device with
                                  concurrent work set this flag, and the runtime then
                                  guarantees co-residency (at the cost of a queue
                                  synchronisation on each side of the launch, ~11 us
                                  each on MI355X).  Either way every wait is bounded: a
                                  workgroup denied co-residency gives up and writes NaN,
                                  it never hangs */
};

/* T_out of the geometry, or -1 if the geometry is invalid or has no output.
 * Pure host function; touches no device. */
int64_t c1g_out_len(const c1g_conv_desc* d);

/* Validation only: the status conv1d_gn_forward would return for this
 * geometry, normalisation and workspace size before any pointer checks.
 * norm may be NULL (plain convolution).  Pure host function. */
int c1g_check(const c1g_conv_desc* d, const c1g_norm_desc* norm, size_t ws_bytes);

/* Workspace bytes conv1d_forward needs for this geometry (0 for fp32). */
size_t c1g_conv1d_workspace_size(const c1g_conv_desc* d);

/* Plain convolution ("Kimi-K2.6 l1_p5" causal Conv1d; "Kimi-K2.6 l2_p35"
 * conv index rule): y = conv(x, w) + bias.
 *   x    [N, C_in, T]        fp32 or bf16, device
 *   w    [C_out, C_in, K]    same type as x, device
 *   bias [C_out] fp32 or NULL (no bias)
 *   y    [N, C_out, T_out] of d->out_dtype, device, written completely
 *   ws   device scratch of ws_bytes >= c1g_conv1d_workspace_size(d), 256-byte
 *        aligned (C1G_ERR_MISALIGNED otherwise; may be NULL when that size is
 *        0); contents are clobbered. */
int conv1d_forward(const c1g_conv_desc* d, const void* x, const void* w, const float* bias,
                   void* y, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes gn_stats needs: 0 when every group holds at most 32768
 * values (C/G * L), else 8 bytes per slice of 32768 values of every group
 * (rounded up to 256 bytes).  0 for invalid arguments. */
size_t c1g_gn_stats_workspace_size(int64_t N, int64_t C, int64_t L, int32_t G);

/* GroupNorm statistics of an existing y ("Kimi-K2.6 l2_p35", the GroupNorm
 * definition: mean and population variance over the C/G channels x L
 * positions of (n, g), eps inside the square root; "Kimi-K2.6 l2_p3", the
 * statistics kernel of its stats-then-apply split):
 *   y    [N, C, L] fp32 device, C % G == 0
 *   mean [N, G]  fp32 device: mean of the C/G x L values of (n, g)
 *   rstd [N, G]  fp32 device: 1/sqrt(population variance + eps)
 *   ws   device scratch of ws_bytes >= c1g_gn_stats_workspace_size(...),
 *        256-byte aligned (C1G_ERR_MISALIGNED otherwise); may be NULL when
 *        that size is 0 (C1G_ERR_WORKSPACE when needed and missing or short).
 * Two stages: every slice of 32768 values of a group is reduced by its own
 * workgroup to (mean, M2) in ws, then the slices of each group are merged in
 * a fixed order (bit-identical results from run to run).  eps must be finite
 * and > 0 (C1G_ERR_INVALID_ARG). */
int gn_stats(int64_t N, int64_t C, int64_t L, int32_t G, float eps, const float* y,
             float* mean, float* rstd, void* ws, size_t ws_bytes, void* stream);

/* GroupNorm normalise + affine ("Kimi-K2.6 l2_p35", GroupNorm: normalise
 * each value with its group's mean and rstd, then the per-channel affine;
 * "Kimi-K2.6 l2_p3", the apply kernel of its stats-then-apply split):
 *   out[n,c,l] = (y[n,c,l] - mean[n,g]) * rstd[n,g] * gamma[c] + beta[c],  g = c / (C/G)
 *   y, out [N, C, L] fp32 device; out may equal y (in place), no other overlap
 *   mean, rstd [N, G] fp32 device
 *   gamma, beta [C] fp32 device, or NULL (1 and 0)
 * N*C*L < 2^32 (C1G_ERR_UNSUPPORTED otherwise). */
int gn_apply(int64_t N, int64_t C, int64_t L, int32_t G, const float* y, const float* mean,
             const float* rstd, const float* gamma, const float* beta, float* out,
             void* stream);

/* gn_apply on bf16 tensors (the same definition and passages as gn_apply):
 * y, out [N, C, L] bf16
 * device (out may equal y), everything else as gn_apply; computed in fp32,
 * out rounded to nearest even.  The apply pass of a bf16 output moves half
 * the bytes of the fp32 one. */
int gn_apply_bf16(int64_t N, int64_t C, int64_t L, int32_t G, const uint16_t* y,
                  const float* mean, const float* rstd, const float* gamma, const float* beta,
                  uint16_t* out, void* stream);

/* Workspace bytes conv1d_gn_forward needs. */
size_t c1g_conv1d_gn_workspace_size(const c1g_conv_desc* d, const c1g_norm_desc* norm);

/* The whole path: conv -> normalisation -> optional row-min epilogue.
 *   x, w, bias     as conv1d_forward
 *   gamma, beta    [C_out] fp32 or NULL (1 and 0): the normalisation's affine
 *                  (ignored when norm == C1G_NORM_NONE)
 *   bias2          [C_out] fp32, required iff epilogue == C1G_EPI_ROWMIN_BIAS
 *   out            [N, C_out, T_out] of d->out_dtype, device, written completely
 *   mean_out, rstd_out  optional fp32 device outputs ([N,G] for GroupNorm,
 *                  [N,T_out] for LayerNorm over channels), or NULL
 *   ws             device scratch of ws_bytes >= c1g_conv1d_gn_workspace_size,
 *                  256-byte aligned (C1G_ERR_MISALIGNED otherwise)
 * A bf16 out: on the "split" route the conv stores y already rounded to bf16
 * (its statistics come from the fp32 accumulators) and the normalisation
 * runs in place on those values; the other routes round only the final
 * value.
 * GroupNorm: z = (y - mean[n,g]) * rstd[n,g] * gamma[c] + beta[c]
 *   ("Kimi-K2.6 l2_p35"); LayerNorm over channels: the same formula with the
 *   statistics of y[n,:,t]; row-min: out = min over channels of z at (n,t)
 *   plus bias2[c] ("Kimi-K2.6 l2_p75"). */
int conv1d_gn_forward(const c1g_conv_desc* d, const c1g_norm_desc* norm, const void* x,
                      const void* w, const float* bias, const float* gamma, const float* beta,
                      const float* bias2, void* out, float* mean_out, float* rstd_out,
                      void* ws, size_t ws_bytes, void* stream);

/* Device scratch conv1d_gn_forward_noalloc holds on each device it runs on
 * (until the process ends): the largest workspace it can serve. */
#define C1G_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* conv1d_gn_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation, arguments and results, without the
 * workspace: the library uses its own static device scratch of
 * C1G_NOALLOC_SCRATCH_BYTES per device (its address is looked up on the first
 * call on each device).  The caller still allocates x, w, the parameters and
 * the outputs.  Returns C1G_ERR_WORKSPACE, launching nothing, when
 * c1g_conv1d_gn_workspace_size for these arguments exceeds the scratch.
 * Allocates and frees nothing.  Every call on a device shares that device's
 * scratch, which keeps the last call's contents (each call initialises what
 * it reads): calls that may overlap in time on one device (other streams,
 * other host threads) race on it and must be serialised by the caller; calls
 * on one stream are ordered. */
int conv1d_gn_forward_noalloc(const c1g_conv_desc* d, const c1g_norm_desc* norm, const void* x,
                              const void* w, const float* bias, const float* gamma,
                              const float* beta, const float* bias2, void* out,
                              float* mean_out, float* rstd_out, void* stream);

/* Name of the kernel route conv1d_gn_forward takes for these arguments, or
 * "invalid".  Pure host function.  Routes:
 *   "conv_only"          norm == C1G_NORM_NONE and no epilogue: the convolution
 *   "fused_single_pass"  fp32, stride 1, GroupNorm with C_out/G dividing 16,
 *                        T_out <= 1024, (K-1)*dilation <= 28: one launch, the
 *                        output slab of a group never leaves the chip
 *   "gemm_rows"          bf16, K = 1, T = 1, no padding, C_in % 8 == 0 (a Linear
 *                        layer): an MFMA GEMM whose epilogue applies GroupNorm
 *                        and the row-min when C_out/G == 16; needs x and w
 *                        16-byte aligned (C1G_ERR_MISALIGNED otherwise).  The
 *                        row-min epilogue runs as the GEMM plus a broadcast
 *                        kernel, or with C1G_FLAG_ROWMIN_ONE_LAUNCH (and the
 *                        device able to keep every GEMM tile resident at once)
 *                        as one launch (C1G_FLAG_COOPERATIVE: cooperative)
 *                        whose workgroups wait on each other: each publishes
 *                        its rows' partial minima, waits for the other channel
 *                        tiles of those rows and writes its block of the
 *                        broadcast output (same result, bit for bit)
 *   "fused_persistent"   bf16, GroupNorm (any G) or LayerNorm
 *                        over channels, no epilogue, at most 256 tiles per
 *                        sample, flags without C1G_FLAG_NO_PERSISTENT: one
 *                        launch (C1G_FLAG_COOPERATIVE: cooperative) in rounds
 *                        of whole samples; each
 *                        workgroup publishes partial statistics, waits for
 *                        the other workgroups of its sample, merges them in a
 *                        fixed order, normalises its tile in registers and
 *                        writes out once (y never reaches memory).  On a
 *                        device that cannot keep a sample's tiles resident
 *                        together, the call runs the split route instead
 *                        (the environment variable C1G_RESIDENT_LIMIT, a
 *                        positive integer, caps the resident workgroups the
 *                        library assumes, so these paths, and rounds of fewer
 *                        samples, can be exercised on any device).
 *                        The waits are bounded (environment variable
 *                        C1G_BARRIER_SPINS, default 4194304 polls); a wait
 *                        that gives up makes that workgroup's output NaN.
 *   "split"              everything else: conv with a partial-statistics
 *                        epilogue, a fixed-order merge, then the apply pass
 *   "empty"              N = 0: nothing to do */
const char* c1g_route(const c1g_conv_desc* d, const c1g_norm_desc* norm);

/* Static string describing a status code. */
const char* c1g_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CONV1D_GN_H */
