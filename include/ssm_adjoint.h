/*
 * ssm_adjoint.h -- C ABI of the MI355X (gfx950) selective-SSM adjoint-gradient library.
 *
 * The library computes the gradient of one diagonal selective state-space
 * layer, and of a residual stack of such layers, as the sum of per-token
 * vector-Jacobian products driven by adjoint states, optionally truncated to
 * a window of the last T-bar tokens.
 *
 * Source of the method: Pith review of "Adjoint sharding for very long
 * context training of state space models" (arXiv 2501.00692):
 *   - "Assumptions", Section 3.1: the recurrence h_t = A_t h_{t-1} + B_t x_t,
 *     y_t = C_t h_t;  Section 3.2: the residual identity of the stack.
 *   - "What carries the argument": the adjoint state
 *     lambda_{t,tau} = C_t A_t ... A_{tau+1} and Proposition 1 (the adjoint
 *     method for recurrences); a VJP seeded with the vector v.
 *   - "Core claim": Proposition 2 (one layer's gradient as sums of
 *     vjp^{A_i}, vjp^{B_i} and vjp^{C_t} terms), Proposition 3 (the sum over
 *     layers) and truncated adjoint sharding (only the last T-bar states).
 * Recompute-from-checkpoint follows the Pith review of "Training Deep Nets
 * with Sublinear Memory Cost" (arXiv 1604.06174), "What carries the argument":
 * store states at segment boundaries and recompute inside each segment.
 *
 * Layer (per token t, channel p, state n; all index spaces 0-based):
 *   Delta_t[p] = sum_q W_delta[p][q] x_t[q] + delta_bias[p]
 *   s_t[p]     = softplus(Delta_t[p])
 *   a_t[p][n]  = exp(-s_t[p] * alpha[p][n])
 *   b_t[n]     = sum_q W_B[n][q] x_t[q],   c_t[n] = sum_q W_C[n][q] x_t[q]
 *   h_t[p][n]  = a_t[p][n] h_{t-1}[p][n] + b_t[n] x_t[p],   h_{-1} = 0
 *   y_t[p]     = sum_n c_t[n] h_t[p][n]
 * Loss seen by the gradient calls: L = sum_t <g_t, y_t>, i.e. g is the
 * cotangent dL/dy that seeds the VJPs.
 *
 * Window W (T-bar): token pair (t, i) contributes iff 0 <= t - i < W.
 * W >= T is the exact gradient (equal to backpropagation); W < T is the
 * truncated sum, which is not the gradient of any loss.  The forward state h
 * is always exact.
 *
 * Conventions for every call:
 *   - All pointers are DEVICE pointers owned by the caller, row-major, 16-byte
 *     aligned, on the device current when the call is made.  The library
 *     never allocates, frees or synchronises; all work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the default stream).
 *   - "io" arrays (x and the three weight matrices) have the dtype dims.io:
 *     SSM_F32 (float) or SSM_BF16 (bfloat16 bits, uint16).  Everything else
 *     is float32 unless stated.
 *   - Outputs are overwritten, never accumulated.
 *   - Validation happens before anything is enqueued: on SSM_ERR_ARG,
 *     SSM_ERR_WORKSPACE or SSM_ERR_UNSUPPORTED nothing has been launched.
 *     SSM_ERR_HIP reports a failed launch; faults inside kernels surface at
 *     the caller's next synchronisation.
 *   - The library keeps no mutable global state except for
 *     ssm_adjoint_grad_noalloc's device array (see there): calls on
 *     different workspaces are independent; calls sharing a workspace must be
 *     ordered (same stream).
 *   - Results are bitwise repeatable for identical inputs, dims and window.
 *
 * Supported shapes: T >= 1, P >= 1, N in {1, 2, 4, 8, 16, 32, 64},
 * 1 <= chunk <= 512.  Other values return SSM_ERR_UNSUPPORTED.
 */
#ifndef SSM_ADJOINT_H
#define SSM_ADJOINT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_OK = 0,
  SSM_ERR_ARG = 1,         /* null required pointer, non-positive size, bad window/K, misalignment */
  SSM_ERR_WORKSPACE = 2,   /* workspace pointer NULL with ws_bytes > 0, or ws_bytes too small */
  SSM_ERR_HIP = 3,         /* a kernel launch failed */
  SSM_ERR_UNSUPPORTED = 4  /* valid arguments outside the supported shapes or dtypes */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* Problem sizes.  chunk = C is the checkpoint interval of the forward state:
 * h is stored only for tokens kC - 1 (the state entering chunk k). */
typedef struct {
  int64_t T;      /* tokens */
  int64_t P;      /* channels (model width) */
  int64_t N;      /* state size per channel */
  int32_t chunk;  /* C */
  int32_t io;     /* ssm_dtype of x and the weights */
} ssm_dims;

/* Parameters of one layer (inputs; not modified). */
typedef struct {
  const void *W_delta;      /* [P][P] io */
  const void *W_B;          /* [N][P] io */
  const void *W_C;          /* [N][P] io */
  const float *alpha;       /* [P][N]  decay rates, a = exp(-softplus(Delta) alpha) */
  const float *delta_bias;  /* [P] or NULL (zero bias) */
  const float *norm_scale;  /* [P] or NULL.  Stack only: the layer reads the RMS-normalised
                             * residual stream (see ssm_stack_grad).  The single-layer calls
                             * take x as given and reject a non-NULL norm_scale. */
} ssm_layer;

/* State saved by ssm_forward for ssm_adjoint_grad (caller-owned buffers).
 * Instead of the whole state sequence h (T*P*N) only the checkpoints are
 * kept; the gradient call recomputes h inside each chunk (the segment
 * recomputation of "Training Deep Nets with Sublinear Memory Cost").
 *
 * h_sub is optional (NULL: not kept).  When set, ssm_forward also stores the
 * state entering every 8th token of each chunk there, in a layout private to
 * this library (ssm_sub_state_bytes(dims) bytes, 16-byte aligned), and
 * ssm_adjoint_grad reads it instead of re-walking each chunk to rebuild it:
 * more saved memory (T*P*N/8 floats, 16 GiB at T = 2^20, P = 2048, N = 16,
 * against 0.5 GiB of chunk checkpoints) for one pass less in the gradient,
 * whose workspace then drops the region in which it would rebuild them
 * (ssm_grad_workspace_bytes_sub).
 * h_sub must be NULL in both calls or, in the gradient call, hold what
 * ssm_forward wrote for the same dims, x and layer.
 *
 * h_all is optional too (NULL: not kept) and is the store-everything
 * baseline of backpropagation through time, kept for comparison: when set,
 * ssm_forward stores the state after every token (ssm_all_state_bytes(dims)
 * bytes, T*P*N floats in a private layout: 128 GiB at T = 2^20, P = 2048,
 * N = 16) and ssm_adjoint_grad reads those states instead of rebuilding any,
 * with the same reverse kernel otherwise.  At most one of h_sub and h_all may
 * be set (SSM_ERR_ARG otherwise); with either set, the gradient's workspace
 * is ssm_grad_workspace_bytes_sub(dims, window). */
typedef struct {
  float *s;        /* [T][P]  softplus(Delta) */
  float *b;        /* [T][N] */
  float *c;        /* [T][N] */
  float *h_ckpt;   /* [ceil(T/C)][P][N]  h_{kC-1}; entry 0 is the zero state */
  double *s_sum;   /* [ceil(T/C)][P]  sum of s over each chunk, in fp64 */
  float *h_sub;    /* optional sub-chunk states (see above), or NULL */
  float *h_all;    /* optional: every state, the store-everything baseline (see above), or NULL */
} ssm_saved;

/* Gradient outputs of one layer.  The three weight gradients are required;
 * the others are optional (NULL = not computed). */
typedef struct {
  float *dW_delta;  /* [P][P] */
  float *dW_B;      /* [N][P] */
  float *dW_C;      /* [N][P] */
  float *dalpha;    /* [P][N] or NULL */
  float *dbias;     /* [P] or NULL */
  float *dx;        /* [T][P] or NULL: cotangent of the layer input x */
  float *dnorm_scale; /* [P] or NULL: gradient of norm_scale (stack layers that normalise) */
} ssm_grads;

/* Library version (major*10000 + minor*100 + patch). */
int32_t ssm_version(void);

/* Human-readable name of a status code (static string, never NULL; any
 * value, including ones outside ssm_status, is accepted). */
const char *ssm_status_str(int32_t status);

/* Bytes of the five required ssm_saved buffers together (informational; the
 * caller may allocate them separately; h_sub not included).  0 if dims are
 * invalid. */
size_t ssm_saved_bytes(const ssm_dims *dims);

/* Bytes of the optional ssm_saved.h_sub buffer.  0 if dims are invalid. */
size_t ssm_sub_state_bytes(const ssm_dims *dims);

/* Bytes of the optional ssm_saved.h_all buffer (every state, the
 * store-everything baseline).  0 if dims are invalid. */
size_t ssm_all_state_bytes(const ssm_dims *dims);

/* Workspace bytes needed by ssm_forward (window = 0, K = 0), by
 * ssm_adjoint_grad (window >= 1, K = 0) or by ssm_stack_grad (K >= 1) for a
 * stack in which no layer normalises its input (for other stacks see
 * ssm_stack_workspace_bytes).  0 if the arguments are invalid or unsupported.
 *
 * The gradient's workspace does not hold the state sequence: when the
 * forward kept no sub-chunk states (saved->h_sub NULL), the gradient rebuilds
 * them from the chunk checkpoints slab by slab of chunks into a region of at
 * most 1 GiB (the segment recomputation of "Training Deep Nets with
 * Sublinear Memory Cost"), so apart from that region the workspace is
 * O(T (P + 2N)) for the GEMM operand and the channel partials plus
 * O((T / C) P N) for the chunk aggregates. */
size_t ssm_workspace_bytes(const ssm_dims *dims, int64_t window, int32_t K);

/* Workspace bytes of ssm_stack_grad for these K layers (host array of
 * structs): like ssm_workspace_bytes(dims, window, K), plus the buffers of
 * the layers that normalise their input (norm_scale set): the residual
 * stream r^k (T*P floats) and 1/rms (T floats) per such layer, and one dx
 * and row scratch.  0 if the arguments are invalid. */
size_t ssm_stack_workspace_bytes(int32_t K, const ssm_dims *dims, const ssm_layer *layers, int64_t window);

/* Workspace bytes of ssm_adjoint_grad (window >= 1) when saved->h_sub or saved->h_all is set:
 * smaller than ssm_workspace_bytes(dims, window, 0) by the region that would
 * otherwise hold a slab of sub-chunk states.  0 if the arguments are invalid. */
size_t ssm_grad_workspace_bytes_sub(const ssm_dims *dims, int64_t window);

/* Number of slabs of chunks ssm_adjoint_grad processes (each slab: the
 * rebuild of its sub-chunk states, then the fused reverse adjoint + VJP
 * kernel over it): 1 when the forward kept sub-chunk states or every state
 * (sub_states_given != 0: saved->h_sub or saved->h_all set).  Instrumentation (see ssm_adjoint_grad_timed);
 * 0 if the arguments are invalid. */
int32_t ssm_grad_slab_count(const ssm_dims *dims, int64_t window, int32_t sub_states_given);

/*
 * Forward pass of one layer: the projections, the chunked scan of the
 * recurrence (Section 3.1) with checkpoints every C tokens, and y.
 *   x   [T][P] io (input), y [T][P] float32 (output)
 *   saved: the five required buffers written, and h_sub when it is set.
 *   ws: at least ssm_workspace_bytes(dims, 0, 0) bytes (256-byte aligned).
 */
ssm_status ssm_forward(const ssm_dims *dims, const ssm_layer *layer, const void *x, float *y,
                       const ssm_saved *saved, void *ws, size_t ws_bytes, void *stream);

/*
 * Gradient of L = sum_t <g_t, y_t> for one layer, as the sum over tokens of
 * the per-token VJPs of Proposition 2 driven by the adjoint states, limited
 * to the window W (truncated adjoint sharding).  Needs the saved state of
 * ssm_forward for the same x and layer.
 *   g [T][P] float32 cotangent of y; window >= 1 (>= T means exact).
 *   grads: outputs (see ssm_grads).  grads->dx, when set, also serves as
 *   the buffer of the direct term sum_n mu b before the input-cotangent GEMM
 *   adds the projections' part in place, so it must not overlap any input.
 *   ws: at least ssm_workspace_bytes(dims, window, 0) bytes, or, when
 *       saved->h_sub is set, ssm_grad_workspace_bytes_sub(dims, window).
 */
ssm_status ssm_adjoint_grad(const ssm_dims *dims, const ssm_layer *layer, const void *x,
                            const ssm_saved *saved, const float *g, int64_t window,
                            const ssm_grads *grads, void *ws, size_t ws_bytes, void *stream);

/*
 * ssm_adjoint_grad without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc).  It computes the same
 * gradient with the same kernels and calls no hipMalloc, hipFree or other
 * allocating routine.  The result is bitwise equal to ssm_adjoint_grad's
 * whenever its slab (below) holds at least 16 chunks, since the carry between
 * chunks is then grouped the same way; a smaller slab rounds the carries
 * differently, within fp32 rounding.  Its workspace is a
 * device array of SSM_NOALLOC_SCRATCH_BYTES bytes inside the library, one per
 * device, held until the process ends.  Whatever the gradient's fixed buffers
 * leave of it holds the slab of rebuilt sub-chunk states, so a larger problem
 * runs more, smaller slabs.  Returns SSM_ERR_WORKSPACE (nothing launched) when
 * the fixed buffers -- the GEMM operand dY (T (P + 2N) io elements), the
 * channel partials, the chunk aggregates and the split-K partials -- plus one
 * chunk of sub-chunk states exceed the array.  Every call on a device shares
 * that device's array: calls that may overlap in time on one device (other
 * streams, other threads) race and must be ordered by the caller.  No part of
 * the array needs to start at zero.
 */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
ssm_status ssm_adjoint_grad_noalloc(const ssm_dims *dims, const ssm_layer *layer, const void *x,
                                    const ssm_saved *saved, const float *g, int64_t window,
                                    const ssm_grads *grads, void *stream);

/*
 * Residual stack of K layers (Section 3.2, Proposition 3):
 *   r^0 = x0,  x^k = io(r^k),  r^{k+1} = r^k + y^k(x^k),  L = sum_t <g_t, r^K_t>
 * where io() stores the float32 residual stream in the io dtype (bf16: round
 * to nearest even).  Runs the K forwards, then the layers in reverse: layer k
 * is driven by the total cotangent delta^{k+1} = dL/dr^{k+1}, and
 * delta^k = delta^{k+1} + dx^k (the io cast is treated as the identity).
 * Every layer uses the same window.
 * A layer with norm_scale = gamma reads the normalised stream instead (the
 * review's Algorithm 1 "normalised input"; the norm is RMS normalisation):
 *   x^k = io(gamma r^k / sqrt(mean_p (r^k)^2 + 1e-5))  per token,
 * and delta^k = delta^{k+1} + (the normalisation's VJP of dx^k); its
 * gradient goes to grads[k].dnorm_scale when that is non-NULL.
 *   layers [K], grads [K] (host arrays of structs with device pointers)
 *   x0 [T][P] io; g [T][P] float32
 *   dx0 [T][P] float32 or NULL: dL/dx0
 *   xK  [T][P] float32 or NULL: the final residual stream r^K
 *   ws: at least ssm_stack_workspace_bytes(K, dims, layers, window) bytes
 *   (= ssm_workspace_bytes(dims, window, K) when no layer normalises); it
 *   also holds the saved states of all K layers.  SSM_ERR_WORKSPACE if it is
 *   smaller.
 */
ssm_status ssm_stack_grad(int32_t K, const ssm_dims *dims, const ssm_layer *layers, const void *x0,
                          const float *g, int64_t window, const ssm_grads *grads, float *dx0,
                          float *xK, void *ws, size_t ws_bytes, void *stream);

/*
 * Instrumented variants for timing: identical to ssm_forward and
 * ssm_adjoint_grad, and additionally record the caller's HIP events
 * (hipEvent_t handles passed as void*; NULL entries and indices >= n_events
 * are skipped) on `stream` at the phase boundaries:
 *   forward : [0] start  [1] after the projection GEMM  [2] after the
 *             chunk-local scan  [3] after the chunk carry  [4] after the final scan
 *   gradient: [0] start  [1] after the chunk-local adjoint aggregates
 *             [2] after the adjoint carry  [3] after the last slab's fused
 *             adjoint + VJP kernel  [4] after the channel / chunk reductions
 *             [5] after the weight-gradient GEMM  [6] after the input-cotangent
 *             GEMM (or its absence); then [7 + 2 s] and [8 + 2 s] just before
 *             and just after the fused kernel's launch over slab s
 *             (s < ssm_grad_slab_count), so that [2]..[3] less those launches
 *             is the time of the sub-chunk-state rebuild passes.
 * events may be NULL only when n_events == 0.
 */
ssm_status ssm_forward_timed(const ssm_dims *dims, const ssm_layer *layer, const void *x, float *y,
                             const ssm_saved *saved, void *ws, size_t ws_bytes, void *stream,
                             void *const *events, int32_t n_events);
ssm_status ssm_adjoint_grad_timed(const ssm_dims *dims, const ssm_layer *layer, const void *x,
                                  const ssm_saved *saved, const float *g, int64_t window,
                                  const ssm_grads *grads, void *ws, size_t ws_bytes, void *stream,
                                  void *const *events, int32_t n_events);

#ifdef __cplusplus
}
#endif

#endif /* SSM_ADJOINT_H */
