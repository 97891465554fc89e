// bn_common.hpp -- pieces shared by the two BatchNorm data paths (the
// plane path of bn_plane.hpp and the column path of bn_cols.hpp) and by the
// entry points in batchnorm.hip: launch constants, the per-channel affine
// coefficients, one-pass statistics (Welford / Chan), the backward's dx
// coefficients, both geometries, and the launcher declarations.  The
// launchers are instantiated once per I/O dtype in bn_inst.hip.
//
// Pages (by title):
//   [NormPage] "How attorch implements LayerNorm, BatchNorm and RMSNorm:
//               the three normalization Triton kernels explained"
//   [MathPage] "Building custom GPU operators quickly with attorch.math:
//               an operator-fusion guide for advanced developers"
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "norm_device.hpp"
#include "norm_host.hpp"

namespace mi355norm {

constexpr int kBnBlock = 256;
constexpr int kBnWaves = kBnBlock / kWave;
constexpr int kBnUnroll = 4;             // vectors in flight per thread per step: statistics,
                                         // backward reduction and the column path
constexpr int kBnUnrollStream = 8;       // the same for the plane apply and dx passes, which
                                         // stream with little arithmetic (measured: 4 -> 8 took
                                         // the bf16 GELU dx pass 204.6 -> 199.8 us and apply
                                         // 143.9 -> 141.0 us; the VALU-bound reduction, 143 ->
                                         // 147 us, keeps 4)
constexpr int64_t kBnStatsChunk = (int64_t)kBnBlock * kBnUnroll * 64;  // vectors of a plane
                                         // after which a thread's float32 statistics state
                                         // moves into float64 (64 x 4 vectors per thread:
                                         // 1024 float32 or 2048 16-bit values)

// Which activations take the fast (published-approximation) forms of GELU:
// the forward only for bf16 (fp16's 11-bit significand resolves the
// approximation error of small negative outputs), the derivative for both
// 16-bit types (its ~1e-7 absolute error stays under the fp16 tolerance).
template <typename T>
constexpr bool kFastGrad = sizeof(T) == 2;

// The backward passes of a GELU without a residual, for 16-bit I/O, scale
// the per-channel a, s by kGeluWScale and evaluate gelu_grad_fast_w on
// x a + s (with a residual, z = x a + s + res would need res scaled too).
template <typename T, int ACT, bool RES>
constexpr bool kGeluPrescale = ACT == kActGelu && kFastGrad<T> && !RES;


// Per-channel scale and shift shared by the forward apply and the backward
// recompute, so both evaluate z with identical float32 operations.
__device__ __forceinline__ void bn_coeffs(float mean, float rstd, float w, float b, float *a, float *s) {
    *a = w * rstd;
    *s = fmaf(-mean, *a, b);
}

// Pre-activation z = (x - mean) * a + b with a = w * rstd.  Float32 I/O forms
// it centred, so a channel whose mean lies far from zero relative to its
// spread keeps full precision (the folded form cancels two products of size
// |mean| * a); 16-bit I/O, whose inputs cannot resolve such a channel anyway,
// uses z = x * a + s with s = b - mean * a (one operation fewer).
template <typename T>
__device__ __forceinline__ float bn_pre(float x, float a, float s, float mean, float bias) {
    if constexpr (sizeof(T) == 4)
        return fmaf(x - mean, a, bias);
    else
        return fmaf(x, a, s);
}

// ------------------------------------------------------ pairwise statistics
struct WelfF {
    float n, mean, m2;
};
struct WelfD {
    double n, mean, m2;
};

// Fold a chunk of `cnt` values with mean `cm` and sum of squared deviations
// `cm2` into the running state (Chan et al. pairwise update).
__device__ __forceinline__ void welf_fold(WelfF &s, float cnt, float cm, float cm2) {
    const float n = s.n + cnt;
    const float f = cnt * __builtin_amdgcn_rcpf(n);
    const float d = cm - s.mean;
    s.mean = fmaf(d, f, s.mean);
    s.m2 += cm2 + d * d * (s.n * f);
    s.n = n;
}

// Symmetric merge (identical result for merge(a,b) and merge(b,a), so every
// lane of a butterfly holds the same value).
__device__ __forceinline__ WelfF welf_merge(const WelfF &a, const WelfF &b) {
    const float n = a.n + b.n;
    if (n == 0.0f) return WelfF{0.0f, 0.0f, 0.0f};
    const float r = __builtin_amdgcn_rcpf(n);
    const float d = b.mean - a.mean;
    return WelfF{n, (a.n * a.mean + b.n * b.mean) * r, (a.m2 + b.m2) + d * d * (a.n * b.n) * r};
}
__device__ __forceinline__ WelfD welf_merge(const WelfD &a, const WelfD &b) {
    const double n = a.n + b.n;
    if (n == 0.0) return WelfD{0.0, 0.0, 0.0};
    const double d = b.mean - a.mean;
    return WelfD{n, (a.n * a.mean + b.n * b.mean) / n, (a.m2 + b.m2) + d * d * (a.n * b.n) / n};
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ WelfF wave_merge(WelfF s) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        WelfF o{shfl_xor_f(s.n, m), shfl_xor_f(s.mean, m), shfl_xor_f(s.m2, m)};
        s = welf_merge(s, o);
    }
    return s;
}

__device__ __forceinline__ WelfD wave_merge(WelfD s) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        WelfD o{shfl_xor_d(s.n, m), shfl_xor_d(s.mean, m), shfl_xor_d(s.m2, m)};
        s = welf_merge(s, o);
    }
    return s;
}


// ------------------------------------------------- backward coefficients
// With m the saved (float32) mean, the channel sums are S_dz = sum dz,
// S_dzx = sum dz (x - m) and S_xc = sum (x - m); the exact batch mean is
// m + S_xc / n, so ([NormPage] "BatchNorm", the BN gradient)
//   db = S_dz,   dw = rstd * (S_dzx - S_xc * S_dz / n)   (= sum dz * xhat)
// and dx = (w rstd / n)(n dz - db - xhat dw) = k1 dz + k2 (x - m) + k3 with
//   k1 = w rstd,  k2 = -w rstd^2 dw / n,  k3 = -w rstd db / n - k2 S_xc / n;
// k3m = k3 - k2 m folds the mean in, for dx = k1 dz + k2 x + k3m.
struct BnDxCoef {
    double dbeta, dgamma;
    float k1, k2, k3, k3m;
};

__device__ __forceinline__ BnDxCoef bn_dx_coeffs(const double sums[3], float mean, float rstd_f,
                                                 float wc_f, double n_total) {
    const double r = (double)rstd_f, wc = (double)wc_f;
    const double mean_shift = sums[2] / n_total;  // exact mean minus saved mean
    BnDxCoef k;
    k.dbeta = sums[0];
    k.dgamma = r * (sums[1] - mean_shift * sums[0]);
    const double k2d = -wc * r * r * k.dgamma / n_total;
    const double k3d = -wc * r * k.dbeta / n_total - k2d * mean_shift;
    k.k1 = (float)(wc * r);
    k.k2 = (float)k2d;
    k.k3 = (float)k3d;
    k.k3m = (float)(k3d - k2d * (double)mean);
    return k;
}

// Training statistics -> the saved float32 mean / rstd and the momentum
// update of the running statistics ([MathPage] "Practice 2": new =
// (1 - momentum) * old + momentum * batch, the running variance taking the
// unbiased batch variance).  One thread per channel.
__device__ __forceinline__ void bn_save_stats(const WelfD &st, int64_t c, float eps, float momentum,
                                              float *running_mean, float *running_var,
                                              float *save_mean, float *save_rstd) {
    save_mean[c] = (float)st.mean;
    save_rstd[c] = (float)(1.0 / sqrt(st.m2 / st.n + (double)eps));
    const double m = (double)momentum;
    if (running_mean) running_mean[c] = (float)((1.0 - m) * running_mean[c] + m * st.mean);
    if (running_var) running_var[c] = (float)((1.0 - m) * running_var[c] + m * (st.m2 / (st.n - 1.0)));
}

// -------------------------------------------------------------- geometry
// Plane path: x is [Nb][C][HW]; channel c's values are the Nb contiguous
// planes (n, c).  Each channel is split into `tiles` workgroups of `ppb`
// planes; the grid is C * tiles, blockIdx = tile * C + c.
struct BnGeom {
    int64_t Nb, HW;
    int C, ppb, tiles;
};

// Column path: x is seen as Nb rows of K = C * HW contiguous values (one
// row per sample); column j belongs to channel j / HW.  A workgroup covers
// a chunk of CV vectors (CV * V columns) of RT consecutive rows: its
// threads are RPP row slices of CV lanes, lane cv of slice rs owning the
// V columns of vector chunk * CV + cv in rows tile * RT + rs, + RPP, ...
// The grid is NCH * T, blockIdx = tile * NCH + chunk.
struct BnColGeom {
    int64_t Nb, K, KV, HW;  // rows, columns per row, vectors per row, plane size
    int C;
    int RT, T;              // rows per tile, row tiles
    int CV, RPP, NCH;       // vectors per chunk row, row slices, chunks
};

// Column-path workspace: three float64 sums per (row tile, column) -- two in
// the forward -- followed by float32 [C][4] dx coefficients.
inline size_t col_part_bytes_host(const BnColGeom &g) {
    return (size_t)g.T * (size_t)g.K * 3 * sizeof(double);
}

// Everything an entry point passes to a launcher.
struct BnArgs {
    hipStream_t st;
    norm_act act;
    float act_p, eps, momentum;
    const void *x, *res, *w, *b, *dy;
    float *rm, *rv, *sm, *sr;  // running (written by training, read by eval), saved
    void *y, *dx, *dres, *dw, *db, *ws;
};

// Launchers (defined in bn_plane.hpp / bn_cols.hpp, instantiated per dtype
// in bn_inst.hip).  Each enqueues the kernels of one operation.
template <typename T, int V> norm_status bn_plane_fwd_train(const BnGeom &g, const BnArgs &a);
template <typename T, int V> norm_status bn_plane_fwd_eval(const BnGeom &g, const BnArgs &a);
template <typename T, int V> norm_status bn_plane_bwd(const BnGeom &g, const BnArgs &a);
// Column path: g the reduction geometry, gs the streaming one (apply, dx).
template <typename T, int V> norm_status bn_col_fwd_train(const BnColGeom &g, const BnColGeom &gs, const BnArgs &a);
template <typename T, int V> norm_status bn_col_fwd_eval(const BnColGeom &gs, const BnArgs &a);
template <typename T, int V> norm_status bn_col_bwd(const BnColGeom &g, const BnColGeom &gs, const BnArgs &a);

}  // namespace mi355norm
