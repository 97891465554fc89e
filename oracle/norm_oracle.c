/*
 * norm_oracle.c -- float64 CPU oracle for LayerNorm, RMSNorm and BatchNorm.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  See
 * norm_oracle.h for the conventions and the page titles cited below.
 *
 * Each routine writes out the definition of its operation with plain loops
 * and double accumulators.  Rows (or channels) are independent, so the outer
 * loop is split across OpenMP threads; nothing else is reordered or fused.
 */
#include "norm_oracle.h"

#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Activations and their derivatives.  [ActPage] section 5: the backward
 * multiplies the incoming gradient by the analytic derivative evaluated at
 * the saved pre-activation input; ReLU's derivative is 0 where the input is
 * <= 0 and 1 elsewhere; GELU uses the error-function form.  Section 6 lists
 * the activation family (sigmoid, GELU, SiLU, Mish, LeakyReLU, ELU, CELU,
 * ... with parameters such as a leaky slope or an ELU alpha).  The
 * definitions and the conventions at kinks are PyTorch's (the pages' layers
 * are PyTorch drop-ins):
 *   relu      max(z, 0);                      ' = [z > 0]
 *   gelu      z Phi(z);                       ' = Phi(z) + z phi(z)
 *   sigmoid   s = 1 / (1 + e^-z);             ' = s (1 - s)
 *   tanh      t = tanh z;                     ' = 1 - t^2
 *   silu      z s;                            ' = s (1 + z (1 - s))
 *   softplus  log(1 + e^z) (z if z > 20);     ' = s (1 if z > 20)
 *   mish      z tanh(log(1 + e^z));           ' = T + z s (1 - T^2), T = tanh(log(1+e^z))
 *   leaky     z if z > 0 else p z;            ' = 1 if z > 0 else p
 *   elu       z if z > 0 else p (e^z - 1);    ' = 1 if z > 0 else p e^z
 *   selu      S (z if z > 0 else A (e^z - 1)); ' = S (1 if z > 0 else A e^z)
 *   celu      z if z > 0 else p (e^(z/p) - 1); ' = 1 if z > 0 else e^(z/p)
 *   relu6     min(max(z, 0), 6);              ' = [0 < z < 6]
 *   hardsigmoid min(max(z + 3, 0), 6) / 6;    ' = 1/6 on (-3, 3), else 0
 *   hardswish z min(max(z + 3, 0), 6) / 6;    ' = 0 (z <= -3), z/3 + 1/2 (z < 3), 1
 * with S = 1.0507009873554804934, A = 1.6732632423543772848 (the SELU
 * constants). */
static const double kSeluScale = 1.0507009873554804934193349852946;
static const double kSeluAlpha = 1.6732632423543772848170429916717;

static double sigm(double z) { return 1.0 / (1.0 + exp(-z)); }

double orc_act(int act, double p, double z) {
    switch (act) {
    case ORC_ACT_RELU: return z > 0.0 ? z : 0.0;
    case ORC_ACT_GELU: return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
    case ORC_ACT_SIGMOID: return sigm(z);
    case ORC_ACT_TANH: return tanh(z);
    case ORC_ACT_SILU: return z * sigm(z);
    case ORC_ACT_SOFTPLUS: return z > 20.0 ? z : log1p(exp(z));
    case ORC_ACT_MISH: return z * tanh(log1p(exp(z)));
    case ORC_ACT_LEAKY_RELU: return z > 0.0 ? z : p * z;
    case ORC_ACT_ELU: return z > 0.0 ? z : p * expm1(z);
    case ORC_ACT_SELU: return kSeluScale * (z > 0.0 ? z : kSeluAlpha * expm1(z));
    case ORC_ACT_CELU: return z > 0.0 ? z : p * expm1(z / p);
    case ORC_ACT_RELU6: return z < 0.0 ? 0.0 : (z > 6.0 ? 6.0 : z);
    case ORC_ACT_HARDSIGMOID: return z <= -3.0 ? 0.0 : (z >= 3.0 ? 1.0 : z / 6.0 + 0.5);
    case ORC_ACT_HARDSWISH: return z <= -3.0 ? 0.0 : (z >= 3.0 ? z : z * (z + 3.0) / 6.0);
    default: return z;
    }
}

double orc_act_grad(int act, double p, double z) {
    switch (act) {
    case ORC_ACT_RELU: return z > 0.0 ? 1.0 : 0.0;
    case ORC_ACT_GELU: {
        double Phi = 0.5 * (1.0 + erf(z / sqrt(2.0)));
        double phi = exp(-0.5 * z * z) / sqrt(2.0 * M_PI);
        return Phi + z * phi;
    }
    case ORC_ACT_SIGMOID: { double s = sigm(z); return s * (1.0 - s); }
    case ORC_ACT_TANH: { double t = tanh(z); return 1.0 - t * t; }
    case ORC_ACT_SILU: { double s = sigm(z); return s * (1.0 + z * (1.0 - s)); }
    case ORC_ACT_SOFTPLUS: return z > 20.0 ? 1.0 : sigm(z);
    case ORC_ACT_MISH: {
        double t = tanh(log1p(exp(z)));
        return t + z * sigm(z) * (1.0 - t * t);
    }
    case ORC_ACT_LEAKY_RELU: return z > 0.0 ? 1.0 : p;
    case ORC_ACT_ELU: return z > 0.0 ? 1.0 : p * exp(z);
    case ORC_ACT_SELU: return kSeluScale * (z > 0.0 ? 1.0 : kSeluAlpha * exp(z));
    case ORC_ACT_CELU: return z > 0.0 ? 1.0 : exp(z / p);
    case ORC_ACT_RELU6: return (z > 0.0 && z < 6.0) ? 1.0 : 0.0;
    case ORC_ACT_HARDSIGMOID: return (z > -3.0 && z < 3.0) ? 1.0 / 6.0 : 0.0;
    case ORC_ACT_HARDSWISH: return z <= -3.0 ? 0.0 : (z < 3.0 ? z / 3.0 + 0.5 : 1.0);
    default: return 1.0;
    }
}

void orc_act_vec(int act, double p, int grad, int64_t n, const double *z, double *out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = grad ? orc_act_grad(act, p, z[i]) : orc_act(act, p, z[i]);
}

/* ---------------------------------------------------------------- LayerNorm
 * [NormPage] "LayerNorm: one program normalizes a batch of rows", steps 2-4:
 * per row, mean = sum(x) / N; variance from the sum of (x - mean)^2 (the
 * biased estimator, divided by N); inv_std = 1 / sqrt(var + eps); the output
 * is the standardized row times weight plus bias.  mean and inv_std are the
 * saved statistics. */
void orc_ln_fwd(int64_t M, int64_t N, double eps, const double *x,
                const double *w, const double *b, double *y, double *mean,
                double *rstd) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double *xr = x + i * N;
        double s = 0.0;
        for (int64_t j = 0; j < N; ++j) s += xr[j];
        double mu = s / (double)N;
        double ss = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double d = xr[j] - mu;
            ss += d * d;
        }
        double var = ss / (double)N;
        double r = 1.0 / sqrt(var + eps);
        for (int64_t j = 0; j < N; ++j) {
            double xhat = (xr[j] - mu) * r;
            double wj = w ? w[j] : 1.0;
            double bj = b ? b[j] : 0.0;
            y[i * N + j] = xhat * wj + bj;
        }
        if (mean) mean[i] = mu;
        if (rstd) rstd[i] = r;
    }
}

/* Row statistics shared by the backward routines below (mean and 1/std of
 * each row, recomputed from x by the same definition as the forward). */
static void ln_row_stats(int64_t M, int64_t N, double eps, const double *x,
                         double *mean, double *rstd) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double *xr = x + i * N;
        double s = 0.0;
        for (int64_t j = 0; j < N; ++j) s += xr[j];
        double mu = s / (double)N;
        double ss = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double d = xr[j] - mu;
            ss += d * d;
        }
        mean[i] = mu;
        rstd[i] = 1.0 / sqrt(ss / (double)N + eps);
    }
}

/* [NormPage] "LayerNorm" section, backward paragraph: the input gradient
 * needs two sums along the feature axis.  With g = dy * w and
 * xhat = (x - mean) * rstd, differentiating y = xhat * w + b gives
 *   dx = rstd * (g - mean_j(g) - xhat * mean_j(g * xhat)).
 * The parameter gradients are sums over rows ([NormPage] "Engineering
 * tricks", blocked gradient aggregation): dw = sum_i dy * xhat, db = sum_i dy.
 */
void orc_ln_bwd(int64_t M, int64_t N, double eps, const double *dy,
                const double *x, const double *w, double *dx, double *dw,
                double *db) {
    double *mean = (double *)malloc(sizeof(double) * (M > 0 ? M : 1));
    double *rstd = (double *)malloc(sizeof(double) * (M > 0 ? M : 1));
    ln_row_stats(M, N, eps, x, mean, rstd);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double *xr = x + i * N, *dyr = dy + i * N;
        double sum_g = 0.0, sum_gxhat = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double g = dyr[j] * (w ? w[j] : 1.0);
            double xhat = (xr[j] - mean[i]) * rstd[i];
            sum_g += g;
            sum_gxhat += g * xhat;
        }
        double c_g = sum_g / (double)N;          /* mean_j(g)        */
        double c_gx = sum_gxhat / (double)N;     /* mean_j(g * xhat) */
        for (int64_t j = 0; j < N; ++j) {
            double g = dyr[j] * (w ? w[j] : 1.0);
            double xhat = (xr[j] - mean[i]) * rstd[i];
            dx[i * N + j] = rstd[i] * (g - c_g - xhat * c_gx);
        }
    }
    if (dw || db) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < N; ++j) {
            double sw = 0.0, sb = 0.0;
            for (int64_t i = 0; i < M; ++i) {
                double xhat = (x[i * N + j] - mean[i]) * rstd[i];
                sw += dy[i * N + j] * xhat;
                sb += dy[i * N + j];
            }
            if (dw) dw[j] = sw;
            if (db) db[j] = sb;
        }
    }
    free(mean);
    free(rstd);
}

/* ------------------------------------------------------------------ RMSNorm
 * [NormPage] "RMSNorm: LayerNorm stripped of the mean": no mean is
 * subtracted; the row is scaled by its inverse root mean square,
 * output = x * inv_rms * weight, with inv_rms = 1 / sqrt(mean_j(x^2) + eps).
 * Only inv_rms is saved. */
void orc_rms_fwd(int64_t M, int64_t N, double eps, const double *x,
                 const double *w, double *y, double *rstd) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double *xr = x + i * N;
        double ss = 0.0;
        for (int64_t j = 0; j < N; ++j) ss += xr[j] * xr[j];
        double r = 1.0 / sqrt(ss / (double)N + eps);
        for (int64_t j = 0; j < N; ++j)
            y[i * N + j] = xr[j] * r * (w ? w[j] : 1.0);
        if (rstd) rstd[i] = r;
    }
}

/* [NormPage] "RMSNorm" section, backward: one row sum, of x * dy * w.
 * With g = dy * w, differentiating y = x * r * w, r = (mean_j(x^2)+eps)^-1/2:
 *   dx = r * (g - x * r^2 * mean_j(g * x)),   dw = sum_i dy * x * r. */
void orc_rms_bwd(int64_t M, int64_t N, double eps, const double *dy,
                 const double *x, const double *w, double *dx, double *dw) {
    double *rstd = (double *)malloc(sizeof(double) * (M > 0 ? M : 1));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double *xr = x + i * N, *dyr = dy + i * N;
        double ss = 0.0;
        for (int64_t j = 0; j < N; ++j) ss += xr[j] * xr[j];
        double r = 1.0 / sqrt(ss / (double)N + eps);
        rstd[i] = r;
        double sum_gx = 0.0;
        for (int64_t j = 0; j < N; ++j)
            sum_gx += dyr[j] * (w ? w[j] : 1.0) * xr[j];
        double c = sum_gx / (double)N;
        for (int64_t j = 0; j < N; ++j) {
            double g = dyr[j] * (w ? w[j] : 1.0);
            dx[i * N + j] = r * (g - xr[j] * r * r * c);
        }
    }
    if (dw) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t i = 0; i < M; ++i)
                s += dy[i * N + j] * x[i * N + j] * rstd[i];
            dw[j] = s;
        }
    }
    free(rstd);
}

/* ---------------------------------------------------------------- BatchNorm
 * [NormPage] "BatchNorm: parallel over features + activation fusion": the
 * statistics run over the batch and spatial axes, one set per channel.
 * Mean and biased variance over the n = Nb * HW values of channel c, by the
 * two-pass definition. */
void orc_bn_stats(int64_t Nb, int64_t C, int64_t HW, const double *x,
                  double *mean, double *var_biased) {
    const double n = (double)(Nb * HW);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < C; ++c) {
        double s = 0.0;
        for (int64_t b = 0; b < Nb; ++b)
            for (int64_t k = 0; k < HW; ++k) s += x[(b * C + c) * HW + k];
        double mu = s / n;
        double ss = 0.0;
        for (int64_t b = 0; b < Nb; ++b)
            for (int64_t k = 0; k < HW; ++k) {
                double d = x[(b * C + c) * HW + k] - mu;
                ss += d * d;
            }
        mean[c] = mu;
        var_biased[c] = ss / n;
    }
}

/* Training forward.  Per channel: standardize with the batch mean and
 * 1/sqrt(var + eps), apply the affine weight and bias, add the residual
 * before the activation (the fused "pre_act_add"), then apply the
 * activation.  [NormPage] "BatchNorm" section: in training the running
 * statistics follow the momentum update with PyTorch semantics;
 * [MathPage] "Practice 2: Welford + EMA" gives the update
 *   new_running = (1 - momentum) * old_running + momentum * batch_value,
 * where the variance fed to the running estimate is the unbiased one
 * (var * n / (n - 1)), as PyTorch does. */
void orc_bn_fwd_train(int64_t Nb, int64_t C, int64_t HW, double eps,
                      double momentum, int act, double act_p, const double *x,
                      const double *res, const double *w, const double *b,
                      double *running_mean, double *running_var, double *y,
                      double *save_mean, double *save_rstd) {
    double *mu = (double *)malloc(sizeof(double) * (C > 0 ? C : 1));
    double *var = (double *)malloc(sizeof(double) * (C > 0 ? C : 1));
    orc_bn_stats(Nb, C, HW, x, mu, var);
    const double n = (double)(Nb * HW);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < C; ++c) {
        double r = 1.0 / sqrt(var[c] + eps);
        double wc = w ? w[c] : 1.0, bc = b ? b[c] : 0.0;
        for (int64_t bi = 0; bi < Nb; ++bi)
            for (int64_t k = 0; k < HW; ++k) {
                int64_t idx = (bi * C + c) * HW + k;
                double z = (x[idx] - mu[c]) * r * wc + bc;
                if (res) z += res[idx];
                y[idx] = orc_act(act, act_p, z);
            }
        if (save_mean) save_mean[c] = mu[c];
        if (save_rstd) save_rstd[c] = r;
        if (running_mean)
            running_mean[c] = (1.0 - momentum) * running_mean[c] + momentum * mu[c];
        if (running_var)
            running_var[c] = (1.0 - momentum) * running_var[c] +
                             momentum * var[c] * n / (n - 1.0);
    }
    free(mu);
    free(var);
}

/* Eval forward: [NormPage] "BatchNorm" section -- inference reads the
 * running statistics in place of the batch statistics. */
void orc_bn_fwd_eval(int64_t Nb, int64_t C, int64_t HW, double eps, int act,
                     double act_p, const double *x, const double *res, const double *w,
                     const double *b, const double *running_mean,
                     const double *running_var, double *y) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < C; ++c) {
        double r = 1.0 / sqrt(running_var[c] + eps);
        double wc = w ? w[c] : 1.0, bc = b ? b[c] : 0.0;
        for (int64_t bi = 0; bi < Nb; ++bi)
            for (int64_t k = 0; k < HW; ++k) {
                int64_t idx = (bi * C + c) * HW + k;
                double z = (x[idx] - running_mean[c]) * r * wc + bc;
                if (res) z += res[idx];
                y[idx] = orc_act(act, act_p, z);
            }
    }
}

/* Backward of the training forward.  [NormPage] "BatchNorm" section: with a
 * fused activation, the activation backward first recovers the gradient at
 * the pre-activation z, then the BatchNorm gradient follows.  Per channel,
 * with n values, xhat = (x - mean) * rstd and dz = dy * act'(z):
 *   dres = dz                          (the residual enters z additively)
 *   db   = sum dz,   dw = sum dz * xhat
 *   dx   = (w * rstd / n) * (n * dz - db - xhat * dw).                    */
void orc_bn_bwd(int64_t Nb, int64_t C, int64_t HW, double eps, int act,
                double act_p, const double *dy, const double *x, const double *res,
                const double *w, const double *b, const double *grad_at, double *dx,
                double *dres, double *dw, double *db) {
    double *mu = (double *)malloc(sizeof(double) * (C > 0 ? C : 1));
    double *var = (double *)malloc(sizeof(double) * (C > 0 ? C : 1));
    orc_bn_stats(Nb, C, HW, x, mu, var);
    const double n = (double)(Nb * HW);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < C; ++c) {
        double r = 1.0 / sqrt(var[c] + eps);
        double wc = w ? w[c] : 1.0, bc = b ? b[c] : 0.0;
        double sum_dz = 0.0, sum_dz_xhat = 0.0;
        for (int64_t bi = 0; bi < Nb; ++bi)
            for (int64_t k = 0; k < HW; ++k) {
                int64_t idx = (bi * C + c) * HW + k;
                double xhat = (x[idx] - mu[c]) * r;
                double z = xhat * wc + bc + (res ? res[idx] : 0.0);
                if (grad_at && !isnan(grad_at[idx])) z = grad_at[idx];
                double dz = dy[idx] * orc_act_grad(act, act_p, z);
                if (dres) dres[idx] = dz;
                sum_dz += dz;
                sum_dz_xhat += dz * xhat;
            }
        for (int64_t bi = 0; bi < Nb; ++bi)
            for (int64_t k = 0; k < HW; ++k) {
                int64_t idx = (bi * C + c) * HW + k;
                double xhat = (x[idx] - mu[c]) * r;
                double z = xhat * wc + bc + (res ? res[idx] : 0.0);
                if (grad_at && !isnan(grad_at[idx])) z = grad_at[idx];
                double dz = dy[idx] * orc_act_grad(act, act_p, z);
                dx[idx] = (wc * r / n) * (n * dz - sum_dz - xhat * sum_dz_xhat);
            }
        if (db) db[c] = sum_dz;
        if (dw) dw[c] = sum_dz_xhat;
    }
    free(mu);
    free(var);
}

/* ------------------------------------------------------ one-pass statistics
 * [NormPage] "BatchNorm" section and [MathPage] "Practice 2": the
 * statistics are accumulated online, each new piece correcting the running
 * variance through its difference from the previous mean, so no second
 * traversal is needed.  Welford (1962): for each value, n += 1,
 * delta = x - mean, mean += delta / n, M2 += delta * (x - mean). */
void orc_welford(int64_t n, const double *x, double out[3]) {
    double cnt = 0.0, mean = 0.0, m2 = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        cnt += 1.0;
        double delta = x[i] - mean;
        mean += delta / cnt;
        m2 += delta * (x[i] - mean);
    }
    out[0] = cnt;
    out[1] = mean;
    out[2] = m2;
}

/* Chan, Golub & LeVeque: merge two partial (count, mean, M2) triples,
 * n = na + nb, delta = mean_b - mean_a, mean = mean_a + delta * nb / n,
 * M2 = M2_a + M2_b + delta^2 * na * nb / n. */
void orc_chan_merge(const double a[3], const double b[3], double out[3]) {
    double n = a[0] + b[0];
    if (n == 0.0) {
        out[0] = out[1] = out[2] = 0.0;
        return;
    }
    double delta = b[1] - a[1];
    double mean = a[1] + delta * b[0] / n;
    double m2 = a[2] + b[2] + delta * delta * a[0] * b[0] / n;
    out[0] = n;
    out[1] = mean;
    out[2] = m2;
}

/* ---------------------------------------------------- activation + dropout
 * Philox4x32-10 as published by Salmon et al. (SC 2011): ten rounds of
 *   (c0, c1, c2, c3) <- (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
 * with M0 = 0xD2511F53, M1 = 0xCD9E8D57, the key bumped by the Weyl
 * constants (0x9E3779B9, 0xBB67AE85) between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The drop threshold on a 16-bit uniform: round(p * 2^16); 0 keeps every
 * element, 2^16 drops every element. */
uint32_t orc_dropout_threshold(double p) {
    if (!(p > 0.0)) return 0;
    if (p >= 1.0) return 1u << 16;
    return (uint32_t)floor(p * 65536.0 + 0.5);
}

/* Element e reads 16 bits of the generator: counter e / 8 yields the four
 * words of eight consecutive elements; element e takes word (e mod 8) / 2,
 * its low half for even e and its high half for odd e. */
static int orc_kept(uint64_t e, uint64_t seed, uint32_t thresh) {
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    const uint64_t blk = e / 8;
    const uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    const uint32_t word = w[(e % 8) / 2];
    const uint32_t u16 = (e % 2 == 0) ? (word & 0xFFFFu) : (word >> 16);
    return u16 >= thresh;
}

void orc_dropout_keep(int64_t n, double p, uint64_t seed, uint64_t offset, uint8_t *keep) {
    const uint32_t t = orc_dropout_threshold(p);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) keep[i] = (uint8_t)orc_kept(offset + (uint64_t)i, seed, t);
}

void orc_act_dropout_fwd(int64_t n, int act, double act_p, double p, uint64_t seed,
                         uint64_t offset, const double *x, double *y) {
    const uint32_t t = orc_dropout_threshold(p);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        y[i] = orc_kept(offset + (uint64_t)i, seed, t) ? orc_act(act, act_p, x[i]) / (1.0 - p) : 0.0;
}

void orc_act_dropout_bwd(int64_t n, int act, double act_p, double p, uint64_t seed,
                         uint64_t offset, const double *dy, const double *x, double *dx) {
    const uint32_t t = orc_dropout_threshold(p);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        dx[i] = orc_kept(offset + (uint64_t)i, seed, t)
                    ? dy[i] * orc_act_grad(act, act_p, x[i]) / (1.0 - p) : 0.0;
}
