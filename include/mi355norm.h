/*
 * mi355norm.h -- C ABI of the MI355X (gfx950) normalization library
 * (libmi355norm.so): LayerNorm, RMSNorm and BatchNorm forward/backward.
 *
 * Operations follow three pages describing the attorch Triton kernels:
 *   [NormPage] "How attorch implements LayerNorm, BatchNorm and RMSNorm:
 *               the three normalization Triton kernels explained"
 *   [MathPage] "Building custom GPU operators quickly with attorch.math:
 *               an operator-fusion guide for advanced developers"
 *   [ActPage]  "Operator fusion in practice: attorch's activation and
 *               dropout fusion kernels"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer (memory from hipMalloc
 *   or a torch CUDA tensor), to dense, contiguous, row-major storage:
 *     row-wise ops:  x, y, dy, dx are [M][N]; w, b, dw, db are [N];
 *                    mean, rstd are [M];
 *     BatchNorm:     x, y, res, dy, dx, dres are NCHW, seen as [Nb][C][HW]
 *                    (HW = H*W; HW = 1 or L gives BatchNorm1d shapes);
 *                    w, b, dw, db, running/saved statistics are [C].
 *   Tensors may have any alignment; 16-byte aligned tensors whose rows (or
 *   planes) are a multiple of 16 bytes take the 128-bit vector path.
 * Dtypes.  `dt` is the I/O dtype of x, y, dy, dx, res, dres, w, b, dw, db:
 *   NORM_F32 (float), NORM_BF16 (bfloat16 bit patterns) or NORM_F16 (IEEE
 *   binary16 bit patterns).  Statistics (mean, rstd, save_*, running_*) are
 *   always float32.  All arithmetic is float32 with float64 for
 *   cross-workgroup merges; 16-bit results are rounded to nearest-even
 *   once, at the store (fp16 results beyond its range become +-inf).
 * Streams.  `stream` is a hipStream_t (NULL = the legacy default stream).
 *   Kernels are enqueued on it and the call returns without synchronizing.
 *   Launch geometry is planned from the current device's compute-unit
 *   count, so the stream should belong to the current device.
 * Ownership.  The caller allocates and owns every buffer, including the
 *   workspace; the library never allocates, frees or synchronizes, and keeps
 *   no state between calls (apart from the process-wide test hook
 *   norm_bn_force_path, the per-thread timing hook below and the static
 *   per-GPU scratch of rms_bwd_noalloc).  Concurrent
 *   calls are safe if they use distinct output and workspace buffers.
 *   Outputs must not alias inputs.
 * Capture.  A call enqueues kernels only (no memset, copy or host wait), so
 *   it can be recorded into a HIP graph by stream capture and replayed; the
 *   pointers and sizes are fixed at capture, as for any captured launch.
 * Errors.  Every entry point returns a norm_status.  Arguments are checked
 *   on the host before anything is enqueued; on an error nothing is
 *   launched and no output is touched.  A zero-sized problem (M == 0, or
 *   C == 0 / Nb*HW == 0 for BatchNorm eval) is a successful no-op.  A
 *   launch the HIP runtime rejects returns NORM_ERR_HIP; the status comes
 *   from the call's own launches (the thread's sticky HIP error, which may
 *   hold an earlier failure of the caller's, is neither read nor cleared).
 *   Faults inside a kernel surface at the caller's next synchronization, as
 *   for any stream operation.
 */
#ifndef MI355NORM_H
#define MI355NORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NORM_OK = 0,
    NORM_ERR_NULL = -1,      /* a required pointer is NULL                  */
    NORM_ERR_SHAPE = -2,     /* a size is negative, zero where it must not  */
                             /* be, or beyond the supported range           */
    NORM_ERR_DTYPE = -3,     /* unknown dtype                               */
    NORM_ERR_ACT = -4,       /* unknown activation                          */
    NORM_ERR_ARG = -5,       /* eps < 0, momentum outside [0,1], or a       */
                             /* BatchNorm batch of fewer than 2 values      */
    NORM_ERR_WORKSPACE = -6, /* workspace NULL or smaller than required     */
    NORM_ERR_HIP = -7        /* the HIP runtime rejected a launch           */
} norm_status;

typedef enum { NORM_F32 = 0, NORM_BF16 = 1, NORM_F16 = 2 } norm_dtype;

/* Activation fused after BatchNorm ([NormPage] "BatchNorm" section: relu,
 * gelu, silu, mish, leaky_relu and a dozen more; [ActPage] sections 5-6).
 * Definitions and derivative conventions at kinks are PyTorch's:
 *   RELU        max(z,0), derivative 0 at z <= 0
 *   GELU        exact error-function form z * Phi(z)
 *   SIGMOID, TANH, SILU (z * sigmoid z), MISH (z * tanh(softplus z)),
 *   LEAKY_RELU  z > 0 ? z : p * z                 (p = negative slope)
 *   ELU         z > 0 ? z : p * (e^z - 1)          (p = alpha)
 *   SELU        1.0507 * (z > 0 ? z : 1.6733 (e^z - 1))
 *   CELU        z > 0 ? z : p * (e^(z/p) - 1)      (p = alpha, nonzero)
 *   SOFTPLUS    log(1 + e^z), z above 20 passes through
 *   RELU6       min(max(z,0),6); HARDSIGMOID relu6(z+3)/6;
 *   HARDSWISH   z * relu6(z+3)/6
 * `act_param` (the p above) is ignored by the others.  NONE, RELU and GELU
 * have specialized kernels; the rest share a run-time-dispatched one. */
typedef enum {
    NORM_ACT_NONE = 0, NORM_ACT_RELU = 1, NORM_ACT_GELU = 2, NORM_ACT_SIGMOID = 3,
    NORM_ACT_TANH = 4, NORM_ACT_SILU = 5, NORM_ACT_MISH = 6, NORM_ACT_LEAKY_RELU = 7,
    NORM_ACT_ELU = 8, NORM_ACT_SELU = 9, NORM_ACT_CELU = 10, NORM_ACT_SOFTPLUS = 11,
    NORM_ACT_RELU6 = 12, NORM_ACT_HARDSIGMOID = 13, NORM_ACT_HARDSWISH = 14
} norm_act;

/* Largest row width the row-wise kernels accept (rows are held in
 * registers): 65536 features for the 16-bit dtypes, 32768 for float32. */
#define NORM_MAX_N_16 65536
#define NORM_MAX_N_BF16 NORM_MAX_N_16
#define NORM_MAX_N_F32 32768

/* ------------------------------------------------------------- LayerNorm
 * Forward, [NormPage] "LayerNorm: one program normalizes a batch of rows":
 * per row i, mean_i = sum_j x_ij / N, var_i = sum_j (x_ij - mean_i)^2 / N,
 * rstd_i = 1/sqrt(var_i + eps), y_ij = (x_ij - mean_i) * rstd_i * w_j + b_j.
 *   w, b      nullable (w = 1, b = 0 when NULL)
 *   mean,rstd nullable float32 [M] outputs (the statistics saved for the
 *             backward when training)
 *   Requires M >= 0, 1 <= N <= NORM_MAX_N_*, eps >= 0.                   */
norm_status ln_fwd(norm_dtype dt, int64_t M, int64_t N, float eps,
                   const void *x, const void *w, const void *b, void *y,
                   float *mean, float *rstd, void *stream);

/* Workspace bytes ln_bwd needs for (dt, M, N) (0 when dw and db are not
 * requested is also accepted by ln_bwd; this returns the size for both). */
size_t ln_bwd_workspace_bytes(norm_dtype dt, int64_t M, int64_t N);

/* Backward, [NormPage] "LayerNorm" section (two row sums along the feature
 * axis, one launch for the whole row gradient) and "Engineering tricks"
 * (weight/bias gradients as per-row-block partial sums, then a sum over
 * the blocks).  With g = dy * w and xhat = (x - mean) * rstd:
 *   dx = rstd * (g - mean_j(g) - xhat * mean_j(g * xhat)),
 *   dw = sum_i dy * xhat,  db = sum_i dy.
 *   mean, rstd  required float32 [M], as written by ln_fwd
 *   w           nullable (treated as 1)
 *   dw, db      nullable outputs [N] in dt; when either is non-NULL,
 *               ws must hold ln_bwd_workspace_bytes(dt, M, N) bytes of
 *               device memory (contents on entry are ignored).
 * The partial sums are reduced in a fixed order: results are bitwise
 * reproducible from run to run.                                         */
norm_status ln_bwd(norm_dtype dt, int64_t M, int64_t N, const void *dy,
                   const void *x, const void *w, const float *mean,
                   const float *rstd, void *dx, void *dw, void *db, void *ws,
                   size_t ws_bytes, void *stream);

/* --------------------------------------------------------------- RMSNorm
 * Forward, [NormPage] "RMSNorm: LayerNorm stripped of the mean":
 * rstd_i = 1/sqrt(sum_j x_ij^2 / N + eps), y_ij = x_ij * rstd_i * w_j.
 *   w nullable (1); rstd nullable float32 [M] output.                     */
norm_status rms_fwd(norm_dtype dt, int64_t M, int64_t N, float eps,
                    const void *x, const void *w, void *y, float *rstd,
                    void *stream);

size_t rms_bwd_workspace_bytes(norm_dtype dt, int64_t M, int64_t N);

/* Backward, [NormPage] "RMSNorm" section (one row sum of x * dy * w):
 * with g = dy * w,  dx = rstd * (g - x * rstd^2 * mean_j(g * x)),
 * dw = sum_i dy * x * rstd.  rstd required (from rms_fwd); w nullable;
 * dw nullable, and when given ws must hold rms_bwd_workspace_bytes.      */
norm_status rms_bwd(norm_dtype dt, int64_t M, int64_t N, const void *dy,
                    const void *x, const void *w, const float *rstd,
                    void *dx, void *dw, void *ws, size_t ws_bytes,
                    void *stream);

/* No-allocation variant of rms_bwd, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, results and
 * kernels as rms_bwd without (ws, ws_bytes): the dw partial rows live in a
 * static device array of NORM_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends.  The call allocates and
 * frees nothing.  It needs (partial rows of the launch plan) * N * 4 bytes
 * of that array -- at most 512 partial rows on a 256-CU part, so N up to
 * 8192 always fits, and M * N * 4 bytes whenever M is smaller than that --
 * and returns NORM_ERR_WORKSPACE, before anything is launched, for a shape
 * that needs more.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (different streams, or host threads) race and
 * must be serialized by the caller.  Nothing in the array needs to start at
 * zero (every partial row is written before it is read); it keeps the last
 * call's contents.  NORM_ERR_HIP if the runtime cannot resolve the array's
 * address on the stream's device (the current device for the null
 * stream).                                                                */
#define NORM_NOALLOC_SCRATCH_BYTES (16u << 20)
norm_status rms_bwd_noalloc(norm_dtype dt, int64_t M, int64_t N, const void *dy,
                            const void *x, const void *w, const float *rstd,
                            void *dx, void *dw, void *stream);

/* ------------------------------------------------------------- BatchNorm
 * Workspace bytes for bn_fwd_train and bn_bwd at this shape (the same
 * buffer serves both; its contents on entry are ignored).               */
size_t bn_workspace_bytes(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW);

/* Training forward, [NormPage] "BatchNorm: parallel over features +
 * activation fusion" and [MathPage] "Practice 2: Welford + EMA".  Per
 * channel c over its n = Nb*HW values: one-pass (Welford) statistics
 * merged across workgroups, mean_c and biased var_c,
 * rstd_c = 1/sqrt(var_c + eps);
 *   z = (x - mean_c) * rstd_c * w_c + b_c (+ res),  y = act(z);
 *   running_mean = (1 - momentum) * running_mean + momentum * mean_c,
 *   running_var  = (1 - momentum) * running_var
 *                  + momentum * var_c * n / (n - 1)   (unbiased, PyTorch).
 *   res                   nullable residual, added before the activation
 *   w, b                  nullable (1, 0)
 *   running_mean/var      nullable float32 [C], updated in place
 *   save_mean, save_rstd  required float32 [C] outputs (for bn_bwd)
 *   ws                    bn_workspace_bytes(dt, Nb, C, HW) bytes
 * Requires Nb*HW >= 2, eps >= 0, 0 <= momentum <= 1, a finite act_param
 * (nonzero for CELU).                                                     */
norm_status bn_fwd_train(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW,
                         float eps, float momentum, norm_act act,
                         float act_param, const void *x, const void *res, const void *w,
                         const void *b, float *running_mean,
                         float *running_var, float *save_mean,
                         float *save_rstd, void *y, void *ws,
                         size_t ws_bytes, void *stream);

/* Eval forward ([NormPage] "BatchNorm" section: inference reads the
 * running statistics): z = (x - rm_c) / sqrt(rv_c + eps) * w_c + b_c
 * (+ res), y = act(z).  running_mean/var required; res, w, b nullable.   */
norm_status bn_fwd_eval(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW,
                        float eps, norm_act act, float act_param, const void *x,
                        const void *res, const void *w, const void *b,
                        const float *running_mean, const float *running_var,
                        void *y, void *stream);

/* Backward of bn_fwd_train ([NormPage] "BatchNorm" section: the activation
 * backward first recovers the pre-activation gradient, then the BatchNorm
 * gradient; [ActPage] section 5 for the derivatives).  z is recomputed from
 * x, res and the saved statistics exactly as the forward computed it;
 *   dz = dy * act'(z);  dres = dz;  db = sum dz;  dw = sum dz * xhat;
 *   dx = (w * rstd / n) * (n * dz - db - xhat * dw),  xhat = (x-mean)*rstd.
 *   res, w, b      nullable, as passed to the forward
 *   dres           required iff res is non-NULL
 *   dw, db         nullable outputs [C]
 *   save_mean/rstd required (from bn_fwd_train)
 *   ws             bn_workspace_bytes(dt, Nb, C, HW) bytes.              */
norm_status bn_bwd(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW,
                   norm_act act, float act_param, const void *dy, const void *x,
                   const void *res, const void *w, const void *b,
                   const float *save_mean, const float *save_rstd, void *dx,
                   void *dres, void *dw, void *db, void *ws, size_t ws_bytes,
                   void *stream);

/* ------------------------------------------------------------- utilities */

/* Static description of a status code (never NULL). */
/* ------------------------------------------------- activation + dropout
 * [ActPage] sections 3-5: y = act(x), then inverted dropout -- an element
 * is dropped (y = 0) with probability p, a kept one is scaled by 1/(1-p)
 * -- in one pass over x; the backward recomputes the same mask from (seed,
 * offset) and returns dx = keep ? dy * act'(x) / (1-p) : 0.  Element-wise
 * over n contiguous elements of x, y, dy, dx (dtype dt).
 * Mask: element e = offset + i takes 16 bits of Philox4x32-10 (Salmon et
 * al., SC 2011) with key (seed mod 2^32, seed / 2^32) and counter
 * ((e/8) mod 2^32, (e/8) / 2^32, 0, 0): word (e mod 8)/2, its low half for
 * even e, its high half for odd e; it is dropped iff those 16 bits are
 * below round(p * 2^16) (p on a grid of 2^-16).  Calls with the same (seed, offset, n)
 * give the same mask; splitting a tensor across calls with offsets keeps
 * the whole-tensor mask.
 *   act, act_param  as for BatchNorm (the activation and its parameter)
 *   drop_p          in [0, 1]; 0 gives the plain activation, 1 all zeros
 *   offset          a multiple of 8 (NORM_ERR_ARG otherwise), offset + n
 *                   must not overflow 64 bits
 * n = 0 is a no-op. */
norm_status act_dropout_fwd(norm_dtype dt, int64_t n, norm_act act, float act_param,
                            float drop_p, uint64_t seed, uint64_t offset, const void *x,
                            void *y, void *stream);
norm_status act_dropout_bwd(norm_dtype dt, int64_t n, norm_act act, float act_param,
                            float drop_p, uint64_t seed, uint64_t offset, const void *dy,
                            const void *x, void *dx, void *stream);

const char *norm_status_str(norm_status s);

/* Timing hook for profilers and benchmarks.  `events` holds 2*n_pairs
 * caller-created hipEvent_t handles.  The NEXT entry-point call made by this
 * host thread launches its i-th kernel (i < n_pairs) with events[2i] and
 * events[2i+1] attached to that kernel's own dispatch (hipExtLaunchKernel),
 * so hipEventElapsedTime(events[2i], events[2i+1]) is the kernel's device
 * time, and (events[0], events[2k-1]) spans a k-kernel call from the first
 * kernel's start to the last kernel's end.  Either event of a pair may be
 * NULL (that side is not recorded; a kernel whose pair is all NULL is
 * launched plainly): an attached event delays the next dispatch by several
 * microseconds, so a call's span is best taken with only events[0] and
 * events[2k-1] set.  The call disarms the hook when it returns.  Costs
 * nothing when not armed.  n_pairs <= 0 disarms.                          */
void norm_arm_kernel_events(void *const *events, int n_pairs);

/* Kernels launched by the last entry-point call on this host thread: their
 * count, the name of the i-th (for matching profiler traces; "" when out of
 * range), and the index of the main streaming kernel (-1 if none).       */
int norm_last_kernel_count(void);
const char *norm_last_kernel_name(int i);
int norm_last_main_kernel(void);

/* Test hook: pins BatchNorm's data path for every later call in this
 * process.  0 = automatic (chosen from dt, C and HW), 1 = the plane path
 * (workgroups stream whole (n, c) planes), 2 = the column path (workgroups
 * stream a band of columns down the samples).  Both paths compute the same
 * results; the hook lets a test run either on any shape.
 * bn_workspace_bytes follows the setting, so set it before querying the
 * workspace and keep it until the calls that use that workspace have been
 * enqueued (a call given a workspace sized for the other path returns
 * NORM_ERR_WORKSPACE if it is too small).  Returns the previous setting,
 * or -1 (and changes nothing) for any other value.                       */
int norm_bn_force_path(int path);

#ifdef __cplusplus
}
#endif
#endif /* MI355NORM_H */
