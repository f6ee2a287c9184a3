/*
 * instant.h - C ABI of the INSTANT low-rank backward for a linear layer y = x . w^T
 *
 * Method: the notes "INSTANT: Compressing Gradients and Activations for
 * Resource-Efficient Training" (papernotes.org, ICLR 2026). Section keys used below:
 *   [Framework] 整体框架   forward unchanged; x_hat = P x is stored instead of x;
 *                           P and Q are refreshed every N_t steps
 *   [KD1]       关键设计 1 per-tensor token autocorrelations C_X = E[x x^T], C_G = E[g_y g_y^T],
 *                           batch not folded into the decomposition; only the statistics are kept
 *   [KD2]       关键设计 2 energy threshold k, p oversampled bases, the compensation in the
 *                           Q equation; P in R^{Rx x L}, Q in R^{Ry x L}
 *   [KD3]       关键设计 3 reordered products g_w ~ (g_y^T P^T)(P x),
 *                           g_x ~ Q^T ((Q g_y) w)
 *
 * Shapes and layouts (all row-major, channels contiguous):
 *   x     [B, L, Cx]      activations of the linear layer's input
 *   gy    [B, L, Cy]      gradient of the layer output
 *   w     [Cy, Cx]        weight (y = x . w^T)
 *   xhat  [B, Rx, Cx]     compressed activation (rows packed with the current Rx)
 *   gw    [Cy, Cx]        weight gradient (overwritten)
 *   gx    [B, L, Cx]      input gradient (overwritten)
 *   P     [Rx, L], Q [Ry, L]  projections, float32 masters
 *
 * Conventions
 *   - Every pointer named as "device" is owned by the caller. The library never
 *     allocates device memory: all device state lives in the caller's workspace
 *     (instant_workspace_bytes). The host handle is the library's own.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream). The exception is a synchronous finalize (instant_calibrate with
 *     INSTANT_FINALIZE_SYNC), which returns only when the new projections (or the
 *     failure) are known: the ranks Rx, Ry it decides size every later launch. An
 *     asynchronous finalize (INSTANT_FINALIZE_ASYNC) returns at once; its outcome is
 *     applied later (see instant_calibrate). A finalize happens once per N_t steps
 *     ([Framework]).
 *   - Host-detectable errors return at once with no side effect.
 *     Calibration failures found on the device (and a finalize whose launch failed or
 *     whose bounded eigensolver wait gave up, E_HIP) are latched: the previous
 *     projections stay active and instant_query reports the failure.
 *   - The I/O dtype (x, gy, w, xhat, gw, gx) is fixed per handle: float32 or
 *     bfloat16. Accumulation is float32; statistics are summed in float64 across
 *     batches.
 *   - Cx and Cy must be multiples of 8; 1 <= L <= 2048; 1 <= R_max <= 64 and R_max <= L.
 *   - Calls on one handle are not re-entrant (one host thread at a time). They are
 *     ordered by their streams: the caller gives every call its inputs on that call's
 *     stream. One overlap is allowed: statistics calls (instant_calibrate) may run on a
 *     second stream while instant_compress_fwd / instant_backward run on another, since
 *     they use disjoint parts of the workspace. A finalizing call rewrites the inactive
 *     projection buffer, the one the calls before the previous finalize used: order it
 *     after the hot-path calls already enqueued on the other stream (an event).
 */
#ifndef INSTANT_H_
#define INSTANT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  INSTANT_OK = 0,
  INSTANT_E_ARG = 1,        /* null pointer, bad enum, non-positive size */
  INSTANT_E_SHAPE = 2,      /* sizes outside what the handle was created for */
  INSTANT_E_STATE = 3,      /* compress/backward before any projection exists */
  INSTANT_E_RANK = 4,       /* k + p exceeds R_max ([KD2]) */
  INSTANT_E_ENERGY = 5,     /* statistics with zero energy ([KD2]: E = 0) */
  INSTANT_E_NONFINITE = 6,  /* NaN or Inf in the statistics */
  INSTANT_E_NOCONV = 7,     /* eigensolver did not converge within max_sweeps */
  INSTANT_E_HIP = 8         /* a HIP runtime call or kernel launch failed */
} instant_status;

typedef enum { INSTANT_FP32 = 0, INSTANT_BF16 = 1 } instant_dtype;

/* Energy compensation applied to the kept bases ([KD2], the Q equation):
 *   PAPER: c = (sum_{i<=R} sigma_i^2)^(-1/2), as printed
 *   NONE : c = 1 (orthonormal rows)
 *   RATIO: c = (E / sum_{i<=R} sigma_i^2)^(1/2), E = sum_i sigma_i^2
 * with P = c * U_R^T. */
typedef enum { INSTANT_COMP_PAPER = 0, INSTANT_COMP_NONE = 1, INSTANT_COMP_RATIO = 2 } instant_comp;

/* Eigensolver of the finalize ([KD1]: "SVD of C"; [KD2]: only the top k + p directions
 * and E = sum_i sigma_i^2 = ||C||_F^2 are needed).
 *   JACOBI    the full decomposition: blocked one-sided Jacobi on all L columns, warm
 *             started from the previous finalize's rotation.
 *   SUBSPACE  the top m = R_max + 16 (rounded up to 16) eigenpairs by at most sub_iters
 *             steps of block subspace iteration with Rayleigh-Ritz (W = C V on the matrix
 *             cores, one-sided Jacobi on the m columns), warm started from the previous
 *             finalize's basis, stopping after the first step whose R_max largest Ritz
 *             pairs all pass the residual test below; E is taken from C. Status E_RANK when eps * E lies beyond
 *             the m directions, E_NOCONV when a kept direction's Ritz residual exceeds
 *             3e-5 * sigma_0. When m >= L it is the JACOBI solver. sigma_x / sigma_g
 *             then hold the m leading values followed by zeros. */
typedef enum { INSTANT_SOLVER_JACOBI = 0, INSTANT_SOLVER_SUBSPACE = 1 } instant_solver;

/* The finalize argument of instant_calibrate. */
typedef enum { INSTANT_FINALIZE_NONE = 0, INSTANT_FINALIZE_SYNC = 1, INSTANT_FINALIZE_ASYNC = 2 } instant_finalize;

typedef struct {
  int32_t L;          /* tokens per sample */
  int32_t Cx, Cy;     /* input / output channels */
  int32_t B_max;      /* largest batch any call will pass */
  int32_t R_max;      /* largest Rx or Ry the handle accepts (<= 64, <= L) */
  int32_t p;          /* oversampled bases added to k ([KD2]) */
  int32_t N_t;        /* recalibration period, kept for bookkeeping ([Framework]) */
  float eps;          /* energy threshold, 0 < eps <= 1 ([KD2]) */
  int32_t dtype;      /* instant_dtype of x, gy, w, xhat, gw, gx */
  int32_t comp;       /* instant_comp */
  int32_t max_sweeps; /* Jacobi sweep limit (e.g. 30); per subspace step for SUBSPACE */
  int32_t solver;     /* instant_solver */
  int32_t sub_iters;  /* most subspace steps per finalize (SUBSPACE; >= 1) */
} instant_config;

typedef struct {
  int32_t kx, ky;           /* truncation indices ([KD2]) */
  int32_t Rx, Ry;           /* ranks in use = min(k + p, L) */
  int32_t sweeps_x, sweeps_g;
  int32_t status;           /* instant_status of the last finalize */
  float cP, cQ;             /* compensation scalars */
  double kept_x, kept_g;    /* sum_{i<=R} sigma_i^2 / E */
  int64_t n_samples_x, n_samples_g; /* samples in the statistics of the last finalize */
  uint32_t generation;      /* bumped each time new projections become active */
} instant_info;

typedef struct instant_layer instant_layer;

/* Bytes of device workspace the handle needs for `cfg` (0 if cfg is invalid). */
size_t instant_workspace_bytes(const instant_config* cfg);

/* Create a handle over the caller's device workspace (instant_workspace_bytes(cfg)
 * bytes, 256-byte aligned). Clears the statistics on `stream`. The workspace must
 * outlive the handle. Errors: E_ARG (null, invalid cfg), E_HIP. */
instant_status instant_create(instant_layer** h, const instant_config* cfg, void* workspace, void* stream);

/* Release the host handle (not the workspace). */
instant_status instant_destroy(instant_layer* h);

/* [KD1] calibration statistics. Adds sum_b x_b x_b^T to the C_X sum (x may be NULL)
 * and sum_b gy_b gy_b^T to the C_G sum (gy may be NULL); B <= B_max.
 * finalize != 0 then turns both sums into means over the samples seen, takes the
 * eigen-decomposition of each, truncates at the energy threshold with p extra
 * bases, applies the compensation ([KD2]), publishes the new P and Q and clears
 * the sums. A finalize needs samples on both sides (else E_STATE).
 *   INSTANT_FINALIZE_SYNC (1): returns once done, with the finalize's status:
 *     E_ENERGY, E_NONFINITE, E_NOCONV or E_RANK leave the previous projections active.
 *   INSTANT_FINALIZE_ASYNC (2): queues the same work on `stream` and returns E_OK at
 *     once; the host does not wait. The outcome is applied by the first
 *     instant_compress_fwd after the device has finished it (that call then uses the new
 *     projections; instant_backward never switches them, so a compress / backward pair
 *     uses one set), or by instant_query, instant_get_projections,
 *     instant_set_projections, the next finalize, which wait for it. Until then the
 *     previous projections stay active and the status is read by instant_query. The
 *     decomposition runs on the handle's workspace alongside calls on other streams;
 *     it rewrites the inactive projection buffer, so it must be ordered after earlier
 *     calls that read that buffer while it was active (as for a synchronous finalize).
 * The finalize's outcome reaches the host through a small pinned host buffer that the
 * handle allocates at creation. B may be 0 when x and gy are both NULL. */
instant_status instant_calibrate(instant_layer* h, const void* x, const void* gy, int32_t B,
                                 int32_t finalize, void* stream);

/* [Framework] forward compression: xhat_b = P x_b for b < B. xhat holds B*Rx*Cx
 * elements (allocate with R_max to be safe). Errors: E_ARG, E_SHAPE, E_STATE, E_HIP. */
instant_status instant_compress_fwd(instant_layer* h, const void* x, int32_t B, void* xhat, void* stream);

/* [KD3] low-rank backward:
 *   gw     = sum_b (P gy_b)^T xhat_b                        [Cy, Cx]
 *   gx_b   = Q^T ((Q gy_b) w)                               [L, Cx]
 * gy is read once for both projections. xhat must come from instant_compress_fwd
 * under the same projections. Errors: E_ARG, E_SHAPE, E_STATE, E_HIP. */
instant_status instant_backward(instant_layer* h, const void* xhat, const void* gy, const void* w,
                                int32_t B, void* gw, void* gx, void* stream);

/* For callers that cannot allocate device memory at the time of the call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): instant_backward
 * with its per-call intermediates (P gy, Q gy, g_hat_x and the float32 K-slice partials of
 * the g_w and g_hat_x products, which instant_backward keeps in the handle's workspace) in a
 * static device array of INSTANT_STATIC_SCRATCH_BYTES that the library holds on every device
 * it runs on until the process ends. Same arguments, same kernels and the same results, bit
 * for bit, as instant_backward; no allocation of any kind.
 * The call needs align256(B*Rx*Cy*s) + align256(B*Ry*Cy*s) + align256(B*Ry*Cx*s) bytes
 * (s = bytes per I/O element, align256 = rounded up to 256), plus, when w does not stay in
 * L2 for the fused g_x path, 4 bytes per float32 partial of whichever of the two products is
 * split over K (S slices of its M x N output: g_hat_x's B*Ry x Cx when w is read once in
 * slices, g_w's Cy x Cx or g_hat_x's on the LDS-tiled GEMM), and returns E_SHAPE when that exceeds
 * INSTANT_STATIC_SCRATCH_BYTES (64 MiB covers B=8, L=2048, Cx=4096, Cy=11008 at Rx=Ry=34).
 * Nothing in the scratch needs to start at zero: every byte read is written earlier in the
 * same call. All calls on one GPU share its array, so calls that overlap on one GPU (other
 * streams, other handles, other threads) race; order them. Errors: E_ARG, E_SHAPE, E_STATE,
 * E_HIP (also when the array's device address could not be looked up at instant_create). */
#define INSTANT_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
instant_status instant_backward_static(instant_layer* h, const void* xhat, const void* gy, const void* w,
                                       int32_t B, void* gw, void* gx, void* stream);

/* Report the result of the last finalize (ranks, compensation, sweeps, status).
 * Returns that finalize's status (INSTANT_OK if none has failed). Host only. */
instant_status instant_query(instant_layer* h, instant_info* out);

/* Install projections directly (float32 device arrays P [Rx, L], Q [Ry, L]) with
 * no calibration; for checkpoint resume and for testing the hot path alone.
 * 1 <= Rx, Ry <= R_max. The data are copied into the workspace on `stream`. */
instant_status instant_set_projections(instant_layer* h, const float* P, int32_t Rx, const float* Q,
                                       int32_t Ry, void* stream);

/* Copy out the active projections and the last spectra (any pointer may be NULL):
 * P [Rx, L], Q [Ry, L] float32; sigma_x, sigma_g [L] float32 in descending order
 * (the singular values of C_X and C_G from the last finalize). Device pointers. */
instant_status instant_get_projections(instant_layer* h, float* P, float* Q, float* sigma_x,
                                       float* sigma_g, void* stream);

/* Copy out the current statistic means C_X, C_G [L, L] float64 (device pointers,
 * either may be NULL), i.e. the running sums divided by the samples seen so far.
 * Errors: E_ARG, E_STATE (a requested side has no samples in the current window), E_HIP. */
instant_status instant_get_statistics(instant_layer* h, double* C_X, double* C_G, void* stream);

/* Name of a status code. */
const char* instant_status_str(instant_status s);

#ifdef __cplusplus
}
#endif

#endif /* INSTANT_H_ */
