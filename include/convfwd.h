/*
 * convfwd -- forward convolution as implicit im2col + tiled MFMA GEMM on
 * MI355X (gfx950).  C ABI.
 *
 * The operation (the ExecuTorch conv1d issue, sections "Describe the bug"
 * and "Suggested fix": nn.Conv1d / nn.Conv2d / aten.convolution semantics,
 * conv1d re-expressed as conv2d with a singleton height and run as im2col +
 * GEMM; the Composable Kernel grouped-conv note, intro and section 2: grouped
 * forward conv NHWGC x GKYXC -> NHWGK in 2-D and 3-D with per-dimension
 * dilation):
 *
 *   y[n,od,oh,ow,g,k] = act( b[g,k] + sum_{z,y,x,c} x[n, od*sd-pd+z*dd,
 *                              oh*sh-ph+y*dh, ow*sw-pw+x*dw, g, c] * w[g,k,z,y,x,c] )
 *
 * cross-correlation (no kernel flip), symmetric zero padding (out-of-range
 * input positions contribute nothing), act = identity or the exact erf-GELU
 * 0.5*v*erfc(-v/sqrt(2)).  Output extent per spatial dim:
 *   O = floor((I + 2*p - d*(F-1) - 1) / s) + 1.
 *
 * Every problem is handled as a 3-D one: a 1-D conv is ndim = 1 with
 * D = H = 1 (and Z = Y = 1), a 2-D conv is ndim = 2 with D = 1 (Z = 1).
 *
 * Layouts (row-major, last index fastest; C and K are PER GROUP):
 *   x    : N x Di x Hi x Wi x G x C     (for 1-D: N x W x C when G = 1)
 *   w    : G x K  x Z  x Y  x X x C     (for 1-D: K x X x C)
 *   bias : G x K
 *   y    : N x Do x Ho x Wo x G x K
 * dtype CONV_DT_F32: x, w, bias, y are float32; products and sums in fp32
 *                    (full-precision f32 MFMA).
 * dtype CONV_DT_BF16: x, w, bias, y are bfloat16; products exact, sums in
 *                    fp32, bias and GELU applied in fp32, the result rounded
 *                    to bfloat16 nearest-even.
 *
 * Ownership: the caller owns every device buffer and the stream.  A plan
 * holds host memory only, is immutable after creation and may be used from
 * several threads and streams at once.  conv_fwd_run allocates nothing,
 * does not synchronise and only enqueues work on the given stream.
 *
 * Errors: every call returns a status and never throws.  A thread-local
 * message describing the last failure is returned by conv_fwd_last_error().
 * Failures inside an already-enqueued kernel surface at the caller's next
 * synchronisation of that stream.
 */
#ifndef CONVFWD_H
#define CONVFWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONV_DT_F32 = 0,
    CONV_DT_BF16 = 1
} conv_dtype_t;

typedef enum {
    CONV_OK = 0,
    CONV_ERR_INVALID_ARG = 1,  /* a value outside its documented range        */
    CONV_ERR_UNSUPPORTED = 2,  /* valid, but beyond this library's limits      */
    CONV_ERR_HIP = 3,          /* the HIP runtime reported an error            */
    CONV_ERR_NOMEM = 4         /* host allocation of the plan failed           */
} conv_status_t;

/* Problem descriptor.  For ndim < 3 the unused leading spatial dims must be
 * trivial: in = filt = stride = dilation = 1 and pad = 0. */
typedef struct {
    int32_t ndim;          /* 1, 2 or 3 spatial dims                          */
    int32_t dtype;         /* conv_dtype_t                                     */
    int64_t N;             /* batch, >= 0 (N = 0 is an empty, valid problem)   */
    int64_t G;             /* groups, >= 1                                     */
    int64_t C;             /* input channels per group, >= 1                   */
    int64_t K;             /* output channels per group, >= 1                  */
    int64_t in[3];         /* Di, Hi, Wi, >= 1                                 */
    int64_t filt[3];       /* Z, Y, X, >= 1                                    */
    int64_t stride[3];     /* >= 1                                             */
    int64_t pad[3];        /* >= 0, same amount before and after               */
    int64_t dilation[3];   /* >= 1                                             */
    int32_t has_bias;      /* 0 or 1                                           */
    int32_t gelu;          /* 0 or 1: apply exact erf-GELU after the bias      */
} conv_fwd_desc_t;

typedef struct conv_fwd_plan conv_fwd_plan_t;   /* opaque */

/* Validates the descriptor on the host, computes the output extents, picks a
 * tile configuration for the shape (per-shape selector) and returns an
 * immutable plan in *plan.  Needs no GPU work; reads the current device's
 * compute-unit count if a device is present.
 *   CONV_ERR_INVALID_ARG : NULL pointer, ndim not 1..3, N < 0, G/C/K < 1,
 *                          in/filt/stride/dilation < 1, pad < 0, a
 *                          non-trivial unused dim, unknown dtype, has_bias or
 *                          gelu not 0/1, or an empty output extent.
 *   CONV_ERR_UNSUPPORTED : a tensor (x including its padding halo, w, y) of
 *                          2^31 elements or more.
 *   CONV_ERR_NOMEM       : plan allocation failed. */
conv_status_t conv_fwd_create(const conv_fwd_desc_t *desc, conv_fwd_plan_t **plan);

/* As conv_fwd_create, but forces tile configuration `config` (an index below
 * conv_fwd_num_configs()).  CONV_ERR_UNSUPPORTED if that configuration is
 * for the other dtype.  For sweeps and for testing every kernel variant. */
conv_status_t conv_fwd_create_with_config(const conv_fwd_desc_t *desc, int32_t config,
                                          conv_fwd_plan_t **plan);

/* Writes (Do, Ho, Wo) of the plan's problem to out[3]. */
conv_status_t conv_fwd_out_dims(const conv_fwd_plan_t *plan, int64_t out[3]);

/* Writes the plan's useful work to *flop: 2 x the multiply-adds of the sum
 * above, taps that fall in the zero padding included (the ExecuTorch conv1d
 * issue, section "Measurements", turns dispatch times into GFLOP/s this way):
 * 2 * N * G * K * C * Do*Ho*Wo * Z*Y*X.  INVALID_ARG for NULL arguments. */
conv_status_t conv_fwd_useful_flop(const conv_fwd_plan_t *plan, int64_t *flop);

/* Enqueues y = conv(x, w) (+ bias) (then GELU) on `stream` (a hipStream_t;
 * NULL = the null stream).  x, w, y: device pointers in the layouts above,
 * 16-byte aligned; bias: device pointer, must be NULL iff the plan has no
 * bias.  y must not overlap x, w or bias.
 *   CONV_ERR_INVALID_ARG : NULL plan, a required NULL pointer, bias given or
 *                          missing against has_bias, misalignment, overlap.
 *   CONV_ERR_HIP         : the launch failed (message has the HIP text). */
conv_status_t conv_fwd_run(const conv_fwd_plan_t *plan, const void *x, const void *w,
                           const void *bias, void *y, void *stream);

/* As conv_fwd_run, and additionally records start_event when the kernel
 * starts executing and stop_event when it ends (hipEvent_t handles created
 * by the caller, either may be NULL), so hipEventElapsedTime gives the
 * kernel's own duration without the launch gap before it.  For measuring the
 * kernels' throughput; errors as conv_fwd_run. */
conv_status_t conv_fwd_run_events(const conv_fwd_plan_t *plan, const void *x, const void *w,
                                  const void *bias, void *y, void *stream,
                                  void *start_event, void *stop_event);

/* ---- Prepacked weights ----------------------------------------------------
 * The ExecuTorch conv1d issue's conv2d path (section "The conv2d path
 * already solves this") prepacks its weights once, ahead of the runs.  The
 * packed form of a plan's weights is the weight part of every LDS stage of
 * the plan's kernel, in the order the kernel consumes it: one image per
 * (group, output-channel tile, K-step), zeros wherever the kernel would
 * load nothing.  Each K-step then fetches its weights as contiguous
 * kilobytes.  It depends on the plan (its tile configuration), not only on
 * the problem: pack with the plan that runs.
 *
 * The prepacked entry points of a plan may run another tile configuration
 * than conv_fwd_run: where a tuning record names a faster one for prepacked
 * weights (cheaper weight loads can favour, say, smaller boxes with two
 * workgroups per compute unit), the plan holds both, and
 * conv_fwd_packed_config says which the prepacked calls use.  Their
 * results are those of conv_fwd_run with that configuration
 * (conv_fwd_create_with_config), bit for bit (same kernel, same summation
 * order), and meet the same error bound against the exact convolution.
 *
 * conv_fwd_packed_config: index of the configuration the prepacked entry
 *   points run (the plan's own unless a tuning record names another);
 *   INVALID_ARG for NULL arguments.
 * conv_fwd_packed_bytes: size of the packed weights (a multiple of 16).
 *   CONV_ERR_UNSUPPORTED if the plan's kernel reads natural weights only
 *   (the register-staged and the runtime-filter patch kernels), or the image
 *   would reach 2 GiB; INVALID_ARG for NULL arguments.
 * conv_fwd_pack_weights: enqueues the rearrangement of w (GKZYXC, the
 *   plan's dtype) into `packed`, a caller-owned device buffer of
 *   conv_fwd_packed_bytes bytes, on `stream`.  Both 16-byte aligned, not
 *   overlapping.  Allocates nothing.
 * conv_fwd_run_packed(_events): as conv_fwd_run(_events) with the packed
 *   weights in place of w (16-byte aligned; y must not overlap it). */
conv_status_t conv_fwd_packed_config(const conv_fwd_plan_t *plan, int32_t *config);
conv_status_t conv_fwd_packed_bytes(const conv_fwd_plan_t *plan, int64_t *bytes);
conv_status_t conv_fwd_pack_weights(const conv_fwd_plan_t *plan, const void *w, void *packed, void *stream);
conv_status_t conv_fwd_run_packed(const conv_fwd_plan_t *plan, const void *x, const void *packed,
                                  const void *bias, void *y, void *stream);
conv_status_t conv_fwd_run_packed_events(const conv_fwd_plan_t *plan, const void *x, const void *packed,
                                         const void *bias, void *y, void *stream, void *start_event,
                                         void *stop_event);

/* Frees a plan.  NULL is a no-op. */
void conv_fwd_destroy(conv_fwd_plan_t *plan);

/* Human-readable description of the plan's chosen kernel and grid; owned by
 * the plan, valid until conv_fwd_destroy.  "" for NULL. */
const char *conv_fwd_describe(const conv_fwd_plan_t *plan);

/* Number of tile configurations compiled into the library, and the name and
 * dtype of one (NULL / -1 for an index out of range). */
int32_t conv_fwd_num_configs(void);
const char *conv_fwd_config_name(int32_t config);
int32_t conv_fwd_config_dtype(int32_t config);

/* ---- Fused two-conv 1-D frontend -----------------------------------------
 * The conv frontend of the ExecuTorch conv1d issue (section "Describe the
 * bug", the table that splits it into conv1 + GELU + conv2 + GELU), run as
 * one kernel whose intermediate never leaves the chip:
 *
 *   h = round_bf16(act(conv1(x) + b1)),   y = act(conv2(h) + b2)
 *
 * conv1 and conv2 follow conv_fwd (cross-correlation, zero padding, act =
 * identity or erf-GELU, bf16 in and out, fp32 sums); h has the call's dtype
 * (bf16), as the unfused chain would store it.  Supported: both 1-D, bf16,
 * G = 1; conv1 C1 -> 384 channels, kernel 3, stride 1, pad 1, C1 a
 * multiple of 16 and at most 352; conv2 384 -> 384, kernel 3, stride 2,
 * pad 1; no dilation; both with the same bias and GELU flags; x and y below
 * 2 GiB.  Layouts as conv_fwd with ndim = 1: x N x L x C1, w1 384 x 3 x C1,
 * w2 384 x 3 x 384, b1 and b2 384, y N x Lo x 384 (Lo = (L - 1) / 2 + 1).
 * Ownership, threading and asynchrony as conv_fwd. */
typedef struct conv_chain_plan conv_chain_plan_t;   /* opaque */

/* Validates both descriptors (each as conv_fwd_create would) and checks that
 * they form a supported chain.
 *   CONV_ERR_INVALID_ARG : NULL pointers, an invalid descriptor, or a second
 *                          conv that does not read the first one's output
 *                          (N, C2 == K1, input length == first output length).
 *   CONV_ERR_UNSUPPORTED : a valid chain outside the supported set above.
 *   CONV_ERR_NOMEM       : plan allocation failed. */
conv_status_t conv_chain_create(const conv_fwd_desc_t *first, const conv_fwd_desc_t *second,
                                conv_chain_plan_t **plan);

/* Enqueues the fused chain on `stream`.  x, w1, w2, y: device pointers,
 * 16-byte aligned; b1, b2: device pointers (NULL iff the plan has no bias).
 * y must not overlap an input.  Errors as conv_fwd_run. */
conv_status_t conv_chain_run(const conv_chain_plan_t *plan, const void *x, const void *w1, const void *b1,
                             const void *w2, const void *b2, void *y, void *stream);

/* As conv_chain_run, recording start_event / stop_event (may be NULL) when
 * the kernel starts and ends, as conv_fwd_run_events does. */
conv_status_t conv_chain_run_events(const conv_chain_plan_t *plan, const void *x, const void *w1,
                                    const void *b1, const void *w2, const void *b2, void *y, void *stream,
                                    void *start_event, void *stop_event);

/* ---- The same chain with prepacked weights -------------------------------
 * The ExecuTorch conv1d issue's conv2d path (section "The conv2d path
 * already solves this") prepacks its weights once, ahead of the runs.  Here
 * the prepacked form puts every 16-element slice of 32 output channels'
 * weights that one MFMA step consumes in one contiguous kilobyte, so the
 * kernel streams the weights from L2 with whole-line loads and without
 * staging them in LDS.  Same results as conv_chain_run for the same inputs
 * (any summation order within the fp32 bound; bit-identical for
 * integer-valued inputs).
 *
 * conv_chain_packed_bytes: size of the packed weights (a multiple of 16);
 *   INVALID_ARG for NULL arguments.
 * conv_chain_pack_weights: enqueues the rearrangement of w1 and w2 (layouts
 *   as conv_chain_run) into `packed`, a caller-owned device buffer of
 *   conv_chain_packed_bytes bytes, on `stream`.  All three 16-byte aligned,
 *   packed not overlapping w1 or w2.  Allocates nothing.  The packed buffer
 *   stays valid for any run of a plan with the same C1.
 * conv_chain_run_packed(_events): as conv_chain_run(_events) with the packed
 *   weights in place of w1 and w2 (16-byte aligned; y must not overlap it). */
conv_status_t conv_chain_packed_bytes(const conv_chain_plan_t *plan, int64_t *bytes);
conv_status_t conv_chain_pack_weights(const conv_chain_plan_t *plan, const void *w1, const void *w2, void *packed,
                                      void *stream);
conv_status_t conv_chain_run_packed(const conv_chain_plan_t *plan, const void *x, const void *packed,
                                    const void *b1, const void *b2, void *y, void *stream);
conv_status_t conv_chain_run_packed_events(const conv_chain_plan_t *plan, const void *x, const void *packed,
                                           const void *b1, const void *b2, void *y, void *stream,
                                           void *start_event, void *stop_event);

/* Writes (1, 1, Lo) -- the extents of y, the second conv's output -- to
 * out[3], and the useful work of both convs (2 x multiply-adds each, padded
 * taps included, as conv_fwd_useful_flop) to *flop.  INVALID_ARG for NULL
 * arguments. */
conv_status_t conv_chain_out_dims(const conv_chain_plan_t *plan, int64_t out[3]);
conv_status_t conv_chain_useful_flop(const conv_chain_plan_t *plan, int64_t *flop);

/* Frees a chain plan (NULL is a no-op). */
void conv_chain_destroy(conv_chain_plan_t *plan);

/* Description of the chain plan; owned by the plan.  "" for NULL. */
const char *conv_chain_describe(const conv_chain_plan_t *plan);

/* ---- Backward-data (input gradient) --------------------------------------
 * The grouped bwd_data convolution that the Composable Kernel grouped-conv
 * note (section 6) names beside the forward one, same layouts:
 *
 *   dx[n,i,g,c] = sum over taps t and k of dy[n,o,g,k] * w[g,k,t,c]
 *                 for every output o with o*s - p + t*d = i (per spatial dim)
 *
 * i.e. the gradient of the forward sum with respect to x (no bias, no GELU:
 * the backward of the linear convolution).  `desc` describes the FORWARD
 * problem; has_bias and gelu must be 0 (else CONV_ERR_UNSUPPORTED).  Layouts:
 * dy as the forward y (N x Do x Ho x Wo x G x K), w as the forward w
 * (G x K x Z x Y x X x C), dx as the forward x (N x Di x Hi x Wi x G x C);
 * all in the descriptor's dtype, fp32 sums.
 *
 * It runs as a forward convolution (same tile kernels and selector) of dy
 * spread onto a grid of Di + dd(Z-1) (etc.) positions with tap-flipped,
 * channel-swapped weights, both written to a caller-owned device workspace
 * of conv_bwd_data_workspace_bytes bytes (16-byte aligned; with unit strides
 * and pad <= d(F-1) only the weights).  A 1-D problem with stride s > 1 runs
 * instead as s forward convolutions of dy itself, one per stride phase (dx
 * positions i = s j + f take the taps t with f + p - t d divisible by s),
 * each writing every s-th row of dx, with only the phases' filters in the
 * workspace -- where every phase has taps, N = 1 or the length is a
 * multiple of s, and a group's row of dx is whole 16-byte vectors; the
 * result is the same sum in another order.  The library allocates nothing.
 * Ownership, threading and asynchrony as conv_fwd; errors as conv_fwd_create
 * and conv_fwd_run, plus INVALID_ARG for a workspace that is NULL, too small
 * or overlapping dy, w or dx. */
typedef struct conv_bwd_data_plan conv_bwd_data_plan_t;   /* opaque */
conv_status_t conv_bwd_data_create(const conv_fwd_desc_t *desc, conv_bwd_data_plan_t **plan);
conv_status_t conv_bwd_data_workspace_bytes(const conv_bwd_data_plan_t *plan, int64_t *bytes);
conv_status_t conv_bwd_data_run(const conv_bwd_data_plan_t *plan, const void *dy, const void *w, void *dx,
                                void *workspace, int64_t workspace_bytes, void *stream);
void conv_bwd_data_destroy(conv_bwd_data_plan_t *plan);

/* Backward-data for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * as conv_bwd_data_run, with the workspace taken from a static device array
 * of CONV_BWD_DATA_SCRATCH_BYTES (64 MiB) that the library holds on each GPU
 * it runs on until the process ends.  It calls no allocating routine.  The
 * caller still passes dy, w and dx.
 *   CONV_ERR_UNSUPPORTED : the plan needs more workspace than the array holds
 *                          (conv_bwd_data_workspace_bytes > 64 MiB).
 *   CONV_ERR_HIP         : the array's device address could not be obtained
 *                          (first call on a device), or a launch failed.
 *   other errors as conv_bwd_data_run.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams, threads or processes sharing the context)
 * race on it.  Each call writes every workspace byte it reads, so nothing
 * carries over from the previous call. */
#define CONV_BWD_DATA_SCRATCH_BYTES (64ll << 20)
conv_status_t conv_bwd_data_run_noalloc(const conv_bwd_data_plan_t *plan, const void *dy, const void *w, void *dx,
                                        void *stream);
const char *conv_bwd_data_describe(const conv_bwd_data_plan_t *plan);

/* ---- Backward-weight (weight gradient) ------------------------------------
 * The grouped bwd_weight convolution of the same note (section 6):
 *
 *   dw[g,k,z,y,x,c] = sum over output pixels (n,od,oh,ow) whose tap (z,y,x)
 *                     lies inside the input of
 *                     dy[n,od,oh,ow,g,k] * x[n, od*sd-pd+z*dd, oh*sh-ph+y*dh, ow*sw-pw+x*dw, g, c]
 *
 * the gradient of the forward sum with respect to w.  `desc` describes the
 * FORWARD problem; dtype must be bf16, has_bias and gelu 0, C and K per group
 * multiples of 8 (else CONV_ERR_UNSUPPORTED).  x, dy, dw in the forward x, y
 * and w layouts, bf16; sums in fp32 (split over the pixels into fp32
 * partials in a caller-owned device workspace of
 * conv_bwd_weight_workspace_bytes bytes, then added in a fixed order, so
 * results are deterministic) and rounded to bf16 nearest-even.  An empty
 * batch gives dw = 0.  The library allocates nothing; ownership, threading,
 * asynchrony and errors as conv_bwd_data. */
typedef struct conv_bwd_weight_plan conv_bwd_weight_plan_t;   /* opaque */
conv_status_t conv_bwd_weight_create(const conv_fwd_desc_t *desc, conv_bwd_weight_plan_t **plan);
conv_status_t conv_bwd_weight_workspace_bytes(const conv_bwd_weight_plan_t *plan, int64_t *bytes);
conv_status_t conv_bwd_weight_run(const conv_bwd_weight_plan_t *plan, const void *x, const void *dy, void *dw,
                                  void *workspace, int64_t workspace_bytes, void *stream);
void conv_bwd_weight_destroy(conv_bwd_weight_plan_t *plan);
const char *conv_bwd_weight_describe(const conv_bwd_weight_plan_t *plan);

/* Message of the last failed call on this thread ("" if none). */
const char *conv_fwd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVFWD_H */
