/*
 * norm_oracle.h -- float64 CPU oracle for the normalization family.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, includes
 * or calls this code; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or helper with
 * the HIP kernels.
 *
 * Every function computes the plain mathematical definition of an operation,
 * in double precision, with straightforward loops.  Inputs are double arrays
 * holding the exact values the GPU path consumes (bf16 inputs are widened
 * exactly by the caller).  All tensors are dense and contiguous:
 *   row-wise ops:  x[M][N], normalized along the last axis;
 *   BatchNorm:     x[Nb][C][HW] (NCHW viewed as batch, channel, spatial).
 * Optional pointers may be NULL (weight -> 1, bias -> 0, residual -> 0,
 * running statistics -> not updated, statistic outputs -> not written).
 *
 * Sources (pages, by title):
 *   [NormPage]  "How attorch implements LayerNorm, BatchNorm and RMSNorm:
 *                the three normalization Triton kernels explained"
 *   [MathPage]  "Building custom GPU operators quickly with attorch.math:
 *                an operator-fusion guide for advanced developers"
 *   [ActPage]   "Operator fusion in practice: attorch's activation and
 *                dropout fusion kernels"
 */
#ifndef NORM_ORACLE_H
#define NORM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORC_ACT_NONE = 0, ORC_ACT_RELU = 1, ORC_ACT_GELU = 2, ORC_ACT_SIGMOID = 3,
    ORC_ACT_TANH = 4, ORC_ACT_SILU = 5, ORC_ACT_MISH = 6, ORC_ACT_LEAKY_RELU = 7,
    ORC_ACT_ELU = 8, ORC_ACT_SELU = 9, ORC_ACT_CELU = 10, ORC_ACT_SOFTPLUS = 11,
    ORC_ACT_RELU6 = 12, ORC_ACT_HARDSIGMOID = 13, ORC_ACT_HARDSWISH = 14
};

/* Activations and their derivatives ([ActPage] sections 5 and 6).  `p` is
 * the activation's parameter: the negative slope of leaky_relu, alpha of
 * elu and celu; ignored otherwise. */
double orc_act(int act, double p, double z);
double orc_act_grad(int act, double p, double z);
/* Element-wise over an array: out = act(z), or act'(z) when grad != 0. */
void orc_act_vec(int act, double p, int grad, int64_t n, const double *z, double *out);

/* LayerNorm ([NormPage] "LayerNorm" section). */
void orc_ln_fwd(int64_t M, int64_t N, double eps, const double *x,
                const double *w, const double *b, double *y, double *mean,
                double *rstd);
void orc_ln_bwd(int64_t M, int64_t N, double eps, const double *dy,
                const double *x, const double *w, double *dx, double *dw,
                double *db);

/* RMSNorm ([NormPage] "RMSNorm" section). */
void orc_rms_fwd(int64_t M, int64_t N, double eps, const double *x,
                 const double *w, double *y, double *rstd);
void orc_rms_bwd(int64_t M, int64_t N, double eps, const double *dy,
                 const double *x, const double *w, double *dx, double *dw);

/* BatchNorm ([NormPage] "BatchNorm" section; [MathPage] Welford + EMA). */
void orc_bn_stats(int64_t Nb, int64_t C, int64_t HW, const double *x,
                  double *mean, double *var_biased);
void orc_bn_fwd_train(int64_t Nb, int64_t C, int64_t HW, double eps,
                      double momentum, int act, double act_p, const double *x,
                      const double *res, const double *w, const double *b,
                      double *running_mean, double *running_var, double *y,
                      double *save_mean, double *save_rstd);
void orc_bn_fwd_eval(int64_t Nb, int64_t C, int64_t HW, double eps, int act,
                     double act_p, const double *x, const double *res, const double *w,
                     const double *b, const double *running_mean,
                     const double *running_var, double *y);
/* grad_at (nullable, [Nb][C][HW]): where it holds a number rather than NaN,
 * the activation's derivative for that element is taken at that point
 * instead of at z.  At a kink, where both one-sided derivatives are valid
 * answers and a pre-activation within rounding of the kink may be rounded
 * to either side, a caller passes a point just left or right of the kink to
 * select one side. */
void orc_bn_bwd(int64_t Nb, int64_t C, int64_t HW, double eps, int act,
                double act_p, const double *dy, const double *x, const double *res,
                const double *w, const double *b, const double *grad_at, double *dx,
                double *dres, double *dw, double *db);

/* The one-pass statistics the BatchNorm page describes, used only to show
 * that they reach the two-pass result: Welford's per-value update, and the
 * pairwise merge of two partial (count, mean, M2) triples. */
/* Activation + dropout ([ActPage] sections 3-5: inverted dropout fused
 * after the activation; the mask is a function of (seed, element offset)
 * from a counter-based generator and is recomputed in the backward).
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror & Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011).  Element e (the caller's offset
 * plus its index) takes 16 bits of Philox4x32-10 with
 *   key     = (seed mod 2^32, seed / 2^32)
 *   counter = ((e / 8) mod 2^32, (e / 8) / 2^32, 0, 0):
 * word (e mod 8) / 2, its low half for even e, its high half for odd e.
 * The element is dropped when that 16-bit value u < T with
 * T = round(p * 2^16) (ties away from zero), i.e. with probability
 * T / 2^16; a kept element is scaled by 1 / (1 - p). */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t orc_dropout_threshold(double p);
/* keep[i] = 1 if element offset + i is kept, else 0. */
void orc_dropout_keep(int64_t n, double p, uint64_t seed, uint64_t offset, uint8_t *keep);
/* y = keep ? act(x) / (1 - p) : 0. */
void orc_act_dropout_fwd(int64_t n, int act, double act_p, double p, uint64_t seed,
                         uint64_t offset, const double *x, double *y);
/* dx = keep ? dy * act'(x) / (1 - p) : 0. */
void orc_act_dropout_bwd(int64_t n, int act, double act_p, double p, uint64_t seed,
                         uint64_t offset, const double *dy, const double *x, double *dx);

void orc_welford(int64_t n, const double *x, double out[3]);
void orc_chan_merge(const double a[3], const double b[3], double out[3]);

int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
