// batchnorm.hip -- BatchNorm training/eval forward and backward for gfx950,
// with an optional fused residual add and ReLU / exact-GELU activation.
//
// Pages (by title):
//   [NormPage] "How attorch implements LayerNorm, BatchNorm and RMSNorm:
//               the three normalization Triton kernels explained"
//   [MathPage] "Building custom GPU operators quickly with attorch.math:
//               an operator-fusion guide for advanced developers"
//   [ActPage]  "Operator fusion in practice: attorch's activation and
//               dropout fusion kernels"
//
// Layout.  x is NCHW, seen as [Nb][C][HW]: the (n, c) "plane" of HW values
// is contiguous, consecutive planes belong to consecutive channels.  A
// channel's n = Nb*HW values are the Nb planes (0, c), (1, c), ...
//
// Work split.  [NormPage] "BatchNorm" section gives one program per channel
// looping over blocks of batch x spatial values.  MI355X has 256 CUs and the
// workloads have 64-256 channels, so here each channel is split into
// `tiles` workgroups of `ppb` planes; every kernel's grid is C * tiles
// workgroups, blockIdx = tile * C + c.
//
//   forward (training)
//     bn_stats_kernel   one-pass statistics of each tile: every thread folds
//                       its 128-bit chunks into a running (count, mean, M2)
//                       with the pairwise update, merges across the wave in
//                       float32 and across waves in float64, and writes one
//                       float64 triple per tile ([NormPage] "BatchNorm":
//                       online correction by the difference from the previous
//                       mean, no second pass; [MathPage] "Practice 2").
//     bn_apply_kernel   each workgroup first combines its channel's tile
//                       triples (float64, exact parallel-axis identity, fixed
//                       order: every workgroup of a channel gets the same
//                       bits), the channel's first
//                       workgroup saves mean / rstd and applies the momentum
//                       update, then z = x * a_c + s_c (+ res), y = act(z)
//                       with a_c = w_c * rstd_c, s_c = b_c - mean_c * a_c.
//   forward (eval)      bn_apply_kernel with mean / rstd from running stats.
//   backward
//     bn_bwd_reduce_kernel  recomputes z exactly as the forward did,
//                       dz = dy * act'(z), stores dres = dz when a residual
//                       was added, and sums dz, dz * (x - mean) and x - mean
//                       per tile (float64 per element for float32 I/O,
//                       float32 per thread for bf16; float64 beyond).
//     bn_bwd_dx_kernel  each workgroup adds its channel's tile sums, forms
//                       db, dw and dx = k1*dz + k2*(x - mean) + k3 (the first
//                       workgroup writes db, dw), then streams dz (re-read
//                       from dres, or recomputed from dy, x, res) into dx.
// Folding the per-channel merges into the following kernel saves a launch
// and the gap between dependent kernels (several microseconds each).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdlib.h>

#include <initializer_list>
#include <type_traits>

#include "norm_device.hpp"
#include "norm_host.hpp"

namespace mi355norm {

constexpr int kBnBlock = 256;
constexpr int kBnWaves = kBnBlock / kWave;
constexpr int kBnUnroll = 4;             // vectors in flight per thread per step
constexpr int64_t kBnTileBytes = 16384;  // target input bytes per workgroup

// Per-channel scale and shift shared by the forward apply and the backward
// recompute, so both evaluate z with identical float32 operations.
__device__ __forceinline__ void bn_coeffs(float mean, float rstd, float w, float b, float *a, float *s) {
    *a = w * rstd;
    *s = fmaf(-mean, *a, b);
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

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_d(v, m);
    return v;
}

// ------------------------------------------------------------------- tiles
struct BnGeom {
    int64_t Nb, HW;
    int C, ppb, tiles;
};

__device__ __forceinline__ void tile_of_block(const BnGeom &g, int *c, int64_t *n0, int64_t *n1) {
    *c = (int)(blockIdx.x % (unsigned)g.C);
    const int t = (int)(blockIdx.x / (unsigned)g.C);
    *n0 = (int64_t)t * g.ppb;
    const int64_t e = *n0 + g.ppb;
    *n1 = e < g.Nb ? e : g.Nb;
}

__device__ __forceinline__ int64_t plane_offset(const BnGeom &g, int64_t n, int c) {
    return (n * g.C + c) * g.HW;
}

// -------------------------------------------------------- forward: stats
template <typename T, int V>
__global__ void __launch_bounds__(kBnBlock)
bn_stats_kernel(const T *__restrict__ x, BnGeom g, double *__restrict__ part) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    int c; int64_t n0, n1;
    tile_of_block(g, &c, &n0, &n1);
    const int64_t nvp = g.HW / V;  // vectors per plane

    WelfF st{0.0f, 0.0f, 0.0f};
    for (int64_t n = n0; n < n1; ++n) {
        const T *p = x + plane_offset(g, n, c);
        for (int64_t v0 = threadIdx.x; v0 < nvp; v0 += (int64_t)kBnBlock * kBnUnroll) {
            raw_t r[kBnUnroll];
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < nvp) r[u] = vload_stream<T, V>(p + v * V);
            }
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < nvp) {
                    float f[V];
                    VT::unpack(r[u], f);
                    float s = 0.0f;
#pragma unroll
                    for (int e = 0; e < V; ++e) s += f[e];
                    const float cm = s * (1.0f / V);
                    float cm2 = 0.0f;
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const float d = f[e] - cm;
                        cm2 = fmaf(d, d, cm2);
                    }
                    welf_fold(st, (float)V, cm, cm2);
                }
            }
        }
    }
    st = wave_merge(st);

    __shared__ WelfD wave_part[kBnWaves];
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) wave_part[wave] = WelfD{st.n, st.mean, st.m2};
    __syncthreads();
    if (threadIdx.x == 0) {
        WelfD acc = wave_part[0];
        for (int i = 1; i < kBnWaves; ++i) acc = welf_merge(acc, wave_part[i]);
        double *dst = part + ((int64_t)c * g.tiles + blockIdx.x / (unsigned)g.C) * 3;
        dst[0] = acc.n;
        dst[1] = acc.mean;
        dst[2] = acc.m2;
    }
}

// ------------------------------------------- forward: channel statistics
// Combines channel c's tile triples (n_t, mean_t, M2_t) in float64 on the
// block's first wave with the exact parallel-axis identity
//   mean = sum n_t mean_t / n,   M2 = sum [M2_t + n_t (mean_t - mean)^2],
// two butterfly sums and one division (a chain of pairwise merges would
// need a division per step, and every workgroup of the channel repeats
// this).  The order is fixed, so every workgroup of channel c obtains the
// same bits; the result is shared through LDS.
__device__ __forceinline__ WelfD merge_channel_tiles(const double *__restrict__ part, int c, int tiles) {
    __shared__ WelfD sh;
    if (threadIdx.x < kWave) {
        const double *q = part + (int64_t)c * tiles * 3;
        double sn = 0.0, snm = 0.0;
        for (int t = threadIdx.x; t < tiles; t += kWave) {
            sn += q[t * 3 + 0];
            snm = fma(q[t * 3 + 0], q[t * 3 + 1], snm);
        }
        sn = wave_sum_d(sn);
        snm = wave_sum_d(snm);
        const double mean = snm / sn;
        double m2 = 0.0;
        for (int t = threadIdx.x; t < tiles; t += kWave) {
            const double d = q[t * 3 + 1] - mean;
            m2 += fma(q[t * 3 + 0] * d, d, q[t * 3 + 2]);
        }
        m2 = wave_sum_d(m2);
        if (threadIdx.x == 0) sh = WelfD{sn, mean, m2};
    }
    __syncthreads();
    return sh;
}

// ---------------------------------------------------- forward: apply
// MODE 0 (training): mean and rstd come from the merged tile statistics
// (biased variance); the channel's first workgroup also writes them to
// save_mean / save_rstd and applies the momentum update ([MathPage]
// "Practice 2": new = (1 - momentum) * old + momentum * batch, the running
// variance taking the unbiased batch variance).
// MODE 1 (eval): mean = running_mean, rstd = 1 / sqrt(running_var + eps).
// Then z = x * a_c + s_c (+ res), y = act(z).
template <typename T, int V, int ACT, bool RES, int MODE>
__global__ void __launch_bounds__(kBnBlock)
bn_apply_kernel(const T *__restrict__ x, const T *__restrict__ res, const T *__restrict__ w,
                const T *__restrict__ b, const double *__restrict__ part, float eps, float momentum,
                float *__restrict__ running_mean, float *__restrict__ running_var,
                float *__restrict__ save_mean, float *__restrict__ save_rstd, T *__restrict__ y,
                BnGeom g, int act_rt, float act_p) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    constexpr bool kFast = std::is_same<T, bf16_t>::value;  // fp16 keeps the exact forms
    int c; int64_t n0, n1;
    tile_of_block(g, &c, &n0, &n1);
    float mean, rstd;
    if (MODE == 0) {
        const WelfD st = merge_channel_tiles(part, c, g.tiles);
        mean = (float)st.mean;
        rstd = (float)(1.0 / sqrt(st.m2 / st.n + (double)eps));
        if (n0 == 0 && threadIdx.x == 0) {
            save_mean[c] = mean;
            save_rstd[c] = rstd;
            const double m = (double)momentum;
            if (running_mean) running_mean[c] = (float)((1.0 - m) * running_mean[c] + m * st.mean);
            if (running_var)
                running_var[c] = (float)((1.0 - m) * running_var[c] + m * (st.m2 / (st.n - 1.0)));
        }
    } else {
        mean = running_mean[c];
        rstd = 1.0f / sqrtf(running_var[c] + eps);
    }
    float a, s;
    bn_coeffs(mean, rstd, w ? ld1(w + c) : 1.0f, b ? ld1(b + c) : 0.0f, &a, &s);
    const int64_t nvp = g.HW / V;

    for (int64_t n = n0; n < n1; ++n) {
        const int64_t off = plane_offset(g, n, c);
        for (int64_t v0 = threadIdx.x; v0 < nvp; v0 += (int64_t)kBnBlock * kBnUnroll) {
            raw_t rx[kBnUnroll], rr[kBnUnroll];
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < nvp) {
                    rx[u] = vload_stream<T, V>(x + off + v * V);
                    if (RES) rr[u] = vload_stream<T, V>(res + off + v * V);
                }
            }
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < nvp) {
                    float f[V], rf[V], o[V];
                    VT::unpack(rx[u], f);
                    if (RES) VT::unpack(rr[u], rf);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        float z = fmaf(f[e], a, s);
                        if (RES) z += rf[e];
                        o[e] = act_fwd_any<ACT, kFast>(z, act_rt, act_p);
                    }
                    vstore_stream<T, V>(y + off + v * V, VT::pack(o));
                }
            }
        }
    }
}

// --------------------------------------------------- backward: pass 1
template <typename T, int V, int ACT, bool RES>
__global__ void __launch_bounds__(kBnBlock)
bn_bwd_reduce_kernel(const T *__restrict__ dy, const T *__restrict__ x, const T *__restrict__ res,
                     const T *__restrict__ w, const T *__restrict__ b,
                     const float *__restrict__ save_mean, const float *__restrict__ save_rstd,
                     T *__restrict__ dres, BnGeom g, double *__restrict__ part, int act_rt,
                     float act_p) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    int c; int64_t n0, n1;
    tile_of_block(g, &c, &n0, &n1);
    const float mean = save_mean[c];
    float a, s;
    bn_coeffs(mean, save_rstd[c], w ? ld1(w + c) : 1.0f, b ? ld1(b + c) : 0.0f, &a, &s);
    const int64_t nvp = g.HW / V;

    // Accumulation.  Float32 I/O: float64 per element, so x - mean and
    // dz * (x - mean) are exact -- the 1e-5 tolerance on the channel sums
    // needs it when a channel's dw lands near zero -- plus the sum of
    // x - mean, which corrects for the saved mean being rounded to float32.
    // bf16 I/O: float32 per thread of dz and dz * x (the mean is taken out
    // once per tile in float64); ample for bf16 outputs and two VALU
    // operations per element cheaper where the GELU backward is VALU-bound.
    // Threads and tiles are always combined in float64.
    constexpr bool kExact = sizeof(T) == 4;
    using Acc = typename std::conditional<kExact, double, float>::type;
    Acc s_dz = 0, s_dzx = 0, s_xc = 0;
    const Acc mean_a = kExact ? (Acc)mean : (Acc)0;
    for (int64_t n = n0; n < n1; ++n) {
        const int64_t off = plane_offset(g, n, c);
        for (int64_t v0 = threadIdx.x; v0 < nvp; v0 += (int64_t)kBnBlock * kBnUnroll) {
            raw_t rd[kBnUnroll], rx[kBnUnroll], rr[kBnUnroll];
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < nvp) {
                    rd[u] = vload_stream<T, V>(dy + off + v * V);
                    rx[u] = vload_stream<T, V>(x + off + v * V);
                    if (RES && ACT != kActNone) rr[u] = vload_stream<T, V>(res + off + v * V);
                }
            }
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < nvp) {
                    float df[V], xf[V], rf[V], dz[V];
                    VT::unpack(rd[u], df);
                    VT::unpack(rx[u], xf);
                    if (RES && ACT != kActNone) VT::unpack(rr[u], rf);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        if (ACT != kActNone) {
                            float z = fmaf(xf[e], a, s);
                            if (RES) z += rf[e];
                            dz[e] = df[e] * act_grad_any<ACT, std::is_same<T, bf16_t>::value>(z, act_rt, act_p);
                        } else {
                            dz[e] = df[e];
                        }
                        const Acc xc = kExact ? (Acc)xf[e] - mean_a : (Acc)xf[e];
                        const Acc d = (Acc)dz[e];
                        s_dz += d;
                        s_dzx = fma(d, xc, s_dzx);
                        if (kExact) s_xc += xc;
                    }
                    if (RES) vstore_stream<T, V>(dres + off + v * V, VT::pack(dz));
                }
            }
        }
    }
    const double t_dz = wave_sum_d((double)s_dz);
    const double t_dzx = wave_sum_d((double)s_dzx);
    const double t_xc = wave_sum_d((double)s_xc);
    __shared__ double wave_part[kBnWaves][3];
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        wave_part[wave][0] = t_dz;
        wave_part[wave][1] = t_dzx;
        wave_part[wave][2] = t_xc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double p0 = 0.0, p1 = 0.0, p2 = 0.0;
        for (int i = 0; i < kBnWaves; ++i) {
            p0 += wave_part[i][0];
            p1 += wave_part[i][1];
            p2 += wave_part[i][2];
        }
        if (!kExact) p1 -= (double)mean * p0;  // sum dz * x  ->  sum dz * (x - mean)
        double *dst = part + ((int64_t)c * g.tiles + blockIdx.x / (unsigned)g.C) * 3;
        dst[0] = p0;
        dst[1] = p1;
        dst[2] = p2;
    }
}

// ------------------------------------------- backward: channel sums
// Adds channel c's three tile sums in float64 on the block's first wave
// (fixed order, identical in every workgroup of the channel).
__device__ __forceinline__ void sum_channel_tiles(const double *__restrict__ part, int c, int tiles,
                                                  double out[3]) {
    __shared__ double sh[3];
    if (threadIdx.x < kWave) {
        double s0 = 0.0, s1 = 0.0, s2 = 0.0;
        for (int t = threadIdx.x; t < tiles; t += kWave) {
            const double *q = part + ((int64_t)c * tiles + t) * 3;
            s0 += q[0];
            s1 += q[1];
            s2 += q[2];
        }
        s0 = wave_sum_d(s0);
        s1 = wave_sum_d(s1);
        s2 = wave_sum_d(s2);
        if (threadIdx.x == 0) {
            sh[0] = s0;
            sh[1] = s1;
            sh[2] = s2;
        }
    }
    __syncthreads();
    out[0] = sh[0];
    out[1] = sh[1];
    out[2] = sh[2];
}

// ----------------------------------------------------- backward: pass 2
// With m the saved (float32) mean, the channel sums are S_dz = sum dz,
// S_dzx = sum dz (x - m) and S_xc = sum (x - m); the exact batch mean is
// m + S_xc / n, so
//   db = S_dz,   dw = rstd * (S_dzx - S_xc * S_dz / n)   (= sum dz * xhat)
// and dx = (w rstd / n)(n dz - db - xhat dw) = k1 dz + k2 (x - m) + k3 with
//   k1 = w rstd,  k2 = -w rstd^2 dw / n,  k3 = -w rstd db / n - k2 S_xc / n.
// The channel's first workgroup writes dw and db.
// DZ_SRC 0: dz = dy (no activation, no residual recompute needed);
//        1: dz re-read from dres (written by pass 1, exact in float32);
//        2: dz recomputed from dy, x (and res) as in pass 1.
template <typename T, int V, int ACT, bool RES, int DZ_SRC>
__global__ void __launch_bounds__(kBnBlock)
bn_bwd_dx_kernel(const T *__restrict__ dy, const T *__restrict__ x, const T *__restrict__ res,
                 const T *__restrict__ dres, const T *__restrict__ w, const T *__restrict__ b,
                 const float *__restrict__ save_mean, const float *__restrict__ save_rstd,
                 const double *__restrict__ part, double n_total, T *__restrict__ dw, T *__restrict__ db,
                 T *__restrict__ dx, BnGeom g, int act_rt, float act_p) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    constexpr bool kFast = std::is_same<T, bf16_t>::value;  // fp16 keeps the exact forms
    int c; int64_t n0, n1;
    tile_of_block(g, &c, &n0, &n1);
    double sums[3];
    sum_channel_tiles(part, c, g.tiles, sums);
    const float mean = save_mean[c];
    const float rstd_f = save_rstd[c];
    const float wc_f = w ? ld1(w + c) : 1.0f;
    const double r = (double)rstd_f, wc = (double)wc_f;
    const double mean_shift = sums[2] / n_total;  // exact mean minus saved mean
    const double dbeta = sums[0];
    const double dgamma = r * (sums[1] - mean_shift * sums[0]);
    if (n0 == 0 && threadIdx.x == 0) {
        if (db) st1(db + c, (float)dbeta);
        if (dw) st1(dw + c, (float)dgamma);
    }
    const double k2d = -wc * r * r * dgamma / n_total;
    const float k1 = (float)(wc * r), k2 = (float)k2d;
    const float k3 = (float)(-wc * r * dbeta / n_total - k2d * mean_shift);
    // bf16 I/O: fold the mean into the constant, dx = k1 dz + k2 x + k3m.
    constexpr bool kExact = sizeof(T) == 4;
    const float k3m = (float)(-wc * r * dbeta / n_total - k2d * mean_shift - k2d * (double)mean);
    float a = 0.0f, s = 0.0f;
    if (DZ_SRC == 2) bn_coeffs(mean, rstd_f, wc_f, b ? ld1(b + c) : 0.0f, &a, &s);
    const int64_t nvp = g.HW / V;
    const T *dzsrc = DZ_SRC == 1 ? dres : dy;

    for (int64_t n = n0; n < n1; ++n) {
        const int64_t off = plane_offset(g, n, c);
        for (int64_t v0 = threadIdx.x; v0 < nvp; v0 += (int64_t)kBnBlock * kBnUnroll) {
            raw_t rd[kBnUnroll], rx[kBnUnroll], rr[kBnUnroll];
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < nvp) {
                    rd[u] = vload_stream<T, V>(dzsrc + off + v * V);
                    rx[u] = vload_stream<T, V>(x + off + v * V);
                    if (DZ_SRC == 2 && RES) rr[u] = vload_stream<T, V>(res + off + v * V);
                }
            }
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < nvp) {
                    float df[V], xf[V], rf[V], o[V];
                    VT::unpack(rd[u], df);
                    VT::unpack(rx[u], xf);
                    if (DZ_SRC == 2 && RES) VT::unpack(rr[u], rf);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        float dz = df[e];
                        if (DZ_SRC == 2 && ACT != kActNone) {
                            float z = fmaf(xf[e], a, s);
                            if (RES) z += rf[e];
                            dz = df[e] * act_grad_any<ACT, kFast>(z, act_rt, act_p);
                        }
                        o[e] = kExact ? fmaf(k1, dz, fmaf(k2, xf[e] - mean, k3)) : fmaf(k1, dz, fmaf(k2, xf[e], k3m));
                    }
                    vstore_stream<T, V>(dx + off + v * V, VT::pack(o));
                }
            }
        }
    }
}

// ------------------------------------------------------------- host side
// Values per workgroup: 16 KiB of input (4096 float32 or 8192 bf16 values,
// rounded up to whole planes), the best of a sweep over the two BatchNorm
// workloads.  MI355NORM_BN_TILE (values) overrides it for tuning sweeps; it
// is read per call, so the workspace query and the call must see the same.
static int64_t tile_elems(norm_dtype dt) {
    const char *e = getenv("MI355NORM_BN_TILE");
    if (e && *e) {
        const long long v = atoll(e);
        if (v >= 256 && v <= (1LL << 26)) return v;
    }
    return kBnTileBytes / (int64_t)dtype_size(dt);
}

static BnGeom make_geom(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW) {
    BnGeom g;
    g.Nb = Nb;
    g.HW = HW;
    g.C = (int)C;
    int64_t ppb = HW > 0 ? ceil_div(tile_elems(dt), HW) : 1;
    if (ppb > Nb) ppb = Nb > 0 ? Nb : 1;
    if (ppb < 1) ppb = 1;
    g.ppb = (int)ppb;
    g.tiles = (int)(Nb > 0 ? ceil_div(Nb, ppb) : 1);
    return g;
}

static norm_status check_bn(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW) {
    if (!dtype_ok(dt)) return NORM_ERR_DTYPE;
    if (Nb < 0 || C < 0 || HW < 0) return NORM_ERR_SHAPE;
    if (C > (int64_t)1 << 24 || Nb > (int64_t)1 << 31 || HW > (int64_t)1 << 40) return NORM_ERR_SHAPE;
    if (C > 0 && Nb > 0 && HW > 0 && Nb * C > ((int64_t)1 << 31) - 1) return NORM_ERR_SHAPE;
    return NORM_OK;
}

static bool bn_vec_ok(norm_dtype dt, int64_t HW, std::initializer_list<const void *> ptrs) {
    if ((HW * (int64_t)dtype_size(dt)) % 16 != 0) return false;
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return false;
    return true;
}

// Workspace: one float64 triple per (channel, tile) -- the forward's
// (count, mean, M2) or the backward's three sums.
static size_t ws_layout(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW) {
    const BnGeom g = make_geom(dt, Nb, C, HW);
    return (size_t)C * g.tiles * 3 * sizeof(double);
}

template <typename T, int V>
static norm_status launch_fwd_train(const BnGeom &g, hipStream_t st, norm_act act, float act_p, float eps,
                                    float momentum, const void *x, const void *res, const void *w,
                                    const void *b, float *rm, float *rv, float *sm, float *sr, void *y,
                                    void *ws) {
    const dim3 grid((unsigned)(g.C * (int64_t)g.tiles));
    double *part = static_cast<double *>(ws);
    launch("bn_stats_kernel", false, bn_stats_kernel<T, V>, grid, dim3(kBnBlock), 0, st, (const T *)x, g, part);
    using fn_t = void (*)(const T *, const T *, const T *, const T *, const double *, float, float, float *,
                          float *, float *, float *, T *, BnGeom, int, float);
    fn_t fn = nullptr;
    const bool r = res != nullptr;
    switch (act) {
    case NORM_ACT_NONE: fn = r ? bn_apply_kernel<T, V, kActNone, true, 0> : bn_apply_kernel<T, V, kActNone, false, 0>; break;
    case NORM_ACT_RELU: fn = r ? bn_apply_kernel<T, V, kActRelu, true, 0> : bn_apply_kernel<T, V, kActRelu, false, 0>; break;
    case NORM_ACT_GELU: fn = r ? bn_apply_kernel<T, V, kActGelu, true, 0> : bn_apply_kernel<T, V, kActGelu, false, 0>; break;
    default: fn = r ? bn_apply_kernel<T, V, kActGeneric, true, 0> : bn_apply_kernel<T, V, kActGeneric, false, 0>; break;
    }
    launch("bn_apply_kernel<train>", true, fn, grid, dim3(kBnBlock), 0, st, (const T *)x, (const T *)res,
           (const T *)w, (const T *)b, (const double *)part, eps, momentum, rm, rv, sm, sr, (T *)y, g, (int)act,
           act_p);
    return launch_status();
}

template <typename T, int V>
static norm_status launch_fwd_eval(const BnGeom &g, hipStream_t st, norm_act act, float act_p, float eps,
                                   const void *x, const void *res, const void *w, const void *b,
                                   const float *rm, const float *rv, void *y) {
    const dim3 grid((unsigned)(g.C * (int64_t)g.tiles));
    using fn_t = void (*)(const T *, const T *, const T *, const T *, const double *, float, float, float *,
                          float *, float *, float *, T *, BnGeom, int, float);
    fn_t fn = nullptr;
    const bool r = res != nullptr;
    switch (act) {
    case NORM_ACT_NONE: fn = r ? bn_apply_kernel<T, V, kActNone, true, 1> : bn_apply_kernel<T, V, kActNone, false, 1>; break;
    case NORM_ACT_RELU: fn = r ? bn_apply_kernel<T, V, kActRelu, true, 1> : bn_apply_kernel<T, V, kActRelu, false, 1>; break;
    case NORM_ACT_GELU: fn = r ? bn_apply_kernel<T, V, kActGelu, true, 1> : bn_apply_kernel<T, V, kActGelu, false, 1>; break;
    default: fn = r ? bn_apply_kernel<T, V, kActGeneric, true, 1> : bn_apply_kernel<T, V, kActGeneric, false, 1>; break;
    }
    // Eval reads the running statistics; they are not written.
    launch("bn_apply_kernel<eval>", true, fn, grid, dim3(kBnBlock), 0, st, (const T *)x, (const T *)res,
           (const T *)w, (const T *)b, (const double *)nullptr, eps, 0.0f, const_cast<float *>(rm),
           const_cast<float *>(rv), (float *)nullptr, (float *)nullptr, (T *)y, g, (int)act, act_p);
    return launch_status();
}

template <typename T, int V, int ACT>
static void launch_bwd_act(const BnGeom &g, hipStream_t st, bool has_res, int act_rt, float act_p,
                           const void *dy, const void *x, const void *res, const void *w, const void *b,
                           const float *sm, const float *sr, void *dx, void *dres, void *dw, void *db,
                           void *ws) {
    const dim3 grid((unsigned)(g.C * (int64_t)g.tiles));
    const dim3 blk(kBnBlock);
    double *part = static_cast<double *>(ws);
    const double n_total = (double)g.Nb * (double)g.HW;
    // The main (largest) kernel: pass 1 with a residual (it reads dy, x, res
    // and writes dres), pass 2 otherwise.
    if (has_res)
        launch("bn_bwd_reduce_kernel", true, bn_bwd_reduce_kernel<T, V, ACT, true>, grid, blk, 0, st,
               (const T *)dy, (const T *)x, (const T *)res, (const T *)w, (const T *)b, sm, sr, (T *)dres, g, part,
               act_rt, act_p);
    else
        launch("bn_bwd_reduce_kernel", false, bn_bwd_reduce_kernel<T, V, ACT, false>, grid, blk, 0, st,
               (const T *)dy, (const T *)x, (const T *)res, (const T *)w, (const T *)b, sm, sr, (T *)dres, g, part,
               act_rt, act_p);
    // dz for pass 2: float32 dres holds dz exactly; 16-bit dres is rounded, so
    // there dz is recomputed from dy and x (and res).
    const bool fp32 = sizeof(T) == 4;
    const bool main = !has_res;
    const double *cp = part;
    if (ACT == kActNone && !has_res) {
        launch("bn_bwd_dx_kernel", main, bn_bwd_dx_kernel<T, V, ACT, false, 0>, grid, blk, 0, st, (const T *)dy,
               (const T *)x, (const T *)res, (const T *)dres, (const T *)w, (const T *)b, sm, sr, cp, n_total,
               (T *)dw, (T *)db, (T *)dx, g, act_rt, act_p);
    } else if (has_res && (fp32 || ACT == kActNone)) {
        launch("bn_bwd_dx_kernel", main, bn_bwd_dx_kernel<T, V, ACT, true, 1>, grid, blk, 0, st, (const T *)dy,
               (const T *)x, (const T *)res, (const T *)dres, (const T *)w, (const T *)b, sm, sr, cp, n_total,
               (T *)dw, (T *)db, (T *)dx, g, act_rt, act_p);
    } else if (has_res) {
        launch("bn_bwd_dx_kernel", main, bn_bwd_dx_kernel<T, V, ACT, true, 2>, grid, blk, 0, st, (const T *)dy,
               (const T *)x, (const T *)res, (const T *)dres, (const T *)w, (const T *)b, sm, sr, cp, n_total,
               (T *)dw, (T *)db, (T *)dx, g, act_rt, act_p);
    } else {
        launch("bn_bwd_dx_kernel", main, bn_bwd_dx_kernel<T, V, ACT, false, 2>, grid, blk, 0, st, (const T *)dy,
               (const T *)x, (const T *)res, (const T *)dres, (const T *)w, (const T *)b, sm, sr, cp, n_total,
               (T *)dw, (T *)db, (T *)dx, g, act_rt, act_p);
    }
}

template <typename T, int V>
static norm_status launch_bwd(const BnGeom &g, hipStream_t st, norm_act act, float act_p, const void *dy,
                              const void *x, const void *res, const void *w, const void *b, const float *sm,
                              const float *sr, void *dx, void *dres, void *dw, void *db, void *ws) {
    const bool r = res != nullptr;
    const int a = (int)act;
    switch (act) {
    case NORM_ACT_NONE: launch_bwd_act<T, V, kActNone>(g, st, r, a, act_p, dy, x, res, w, b, sm, sr, dx, dres, dw, db, ws); break;
    case NORM_ACT_RELU: launch_bwd_act<T, V, kActRelu>(g, st, r, a, act_p, dy, x, res, w, b, sm, sr, dx, dres, dw, db, ws); break;
    case NORM_ACT_GELU: launch_bwd_act<T, V, kActGelu>(g, st, r, a, act_p, dy, x, res, w, b, sm, sr, dx, dres, dw, db, ws); break;
    default: launch_bwd_act<T, V, kActGeneric>(g, st, r, a, act_p, dy, x, res, w, b, sm, sr, dx, dres, dw, db, ws); break;
    }
    return launch_status();
}

static bool act_ok(norm_act a) { return (int)a >= 0 && (int)a < kActCount; }

// The activation parameter must be finite; CELU divides by it.
static bool act_param_ok(norm_act a, float p) {
    if (!(p == p) || p == __builtin_inff() || p == -__builtin_inff()) return false;
    return !(a == NORM_ACT_CELU && p == 0.0f);
}

}  // namespace mi355norm

using namespace mi355norm;

extern "C" size_t bn_workspace_bytes(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW) {
    if (check_bn(dt, Nb, C, HW) != NORM_OK) return 0;
    return ws_layout(dt, Nb, C, HW);
}

extern "C" norm_status bn_fwd_train(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW, float eps, float momentum,
                                    norm_act act, float act_param, const void *x, const void *res, const void *w, const void *b,
                                    float *running_mean, float *running_var, float *save_mean, float *save_rstd,
                                    void *y, void *ws, size_t ws_bytes, void *stream) {
    CallScope scope;
    norm_status s = check_bn(dt, Nb, C, HW);
    if (s != NORM_OK) return s;
    if (!act_ok(act)) return NORM_ERR_ACT;
    if (!(eps >= 0.0f) || !(momentum >= 0.0f && momentum <= 1.0f)) return NORM_ERR_ARG;
    if (!act_param_ok(act, act_param)) return NORM_ERR_ARG;
    if (C == 0) return NORM_OK;
    if (Nb * HW < 2) return NORM_ERR_ARG;  // the unbiased running variance needs n >= 2
    if (!x || !y || !save_mean || !save_rstd) return NORM_ERR_NULL;
    if (!ws || ws_bytes < ws_layout(dt, Nb, C, HW)) return NORM_ERR_WORKSPACE;
    const BnGeom g = make_geom(dt, Nb, C, HW);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool vec = bn_vec_ok(dt, HW, {x, res, y});
    return with_io_type(dt, [&](auto tag) {
        using T = typename decltype(tag)::type;
        constexpr int VW = 16 / (int)sizeof(T);
        return vec ? launch_fwd_train<T, VW>(g, st, act, act_param, eps, momentum, x, res, w, b, running_mean, running_var, save_mean, save_rstd, y, ws)
                   : launch_fwd_train<T, 1>(g, st, act, act_param, eps, momentum, x, res, w, b, running_mean, running_var, save_mean, save_rstd, y, ws);
    });
}

extern "C" norm_status bn_fwd_eval(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW, float eps, norm_act act,
                                   float act_param, const void *x, const void *res, const void *w, const void *b,
                                   const float *running_mean, const float *running_var, void *y, void *stream) {
    CallScope scope;
    norm_status s = check_bn(dt, Nb, C, HW);
    if (s != NORM_OK) return s;
    if (!act_ok(act)) return NORM_ERR_ACT;
    if (!(eps >= 0.0f) || !act_param_ok(act, act_param)) return NORM_ERR_ARG;
    if (C == 0 || Nb * HW == 0) return NORM_OK;
    if (!x || !y || !running_mean || !running_var) return NORM_ERR_NULL;
    const BnGeom g = make_geom(dt, Nb, C, HW);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool vec = bn_vec_ok(dt, HW, {x, res, y});
    return with_io_type(dt, [&](auto tag) {
        using T = typename decltype(tag)::type;
        constexpr int VW = 16 / (int)sizeof(T);
        return vec ? launch_fwd_eval<T, VW>(g, st, act, act_param, eps, x, res, w, b, running_mean, running_var, y)
                   : launch_fwd_eval<T, 1>(g, st, act, act_param, eps, x, res, w, b, running_mean, running_var, y);
    });
}

extern "C" norm_status bn_bwd(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW, norm_act act, float act_param,
                              const void *dy,
                              const void *x, const void *res, const void *w, const void *b, const float *save_mean,
                              const float *save_rstd, void *dx, void *dres, void *dw, void *db, void *ws,
                              size_t ws_bytes, void *stream) {
    CallScope scope;
    norm_status s = check_bn(dt, Nb, C, HW);
    if (s != NORM_OK) return s;
    if (!act_ok(act)) return NORM_ERR_ACT;
    if (!act_param_ok(act, act_param)) return NORM_ERR_ARG;
    if (C == 0) return NORM_OK;
    if (Nb * HW < 2) return NORM_ERR_ARG;
    if (!dy || !x || !dx || !save_mean || !save_rstd) return NORM_ERR_NULL;
    if (res && !dres) return NORM_ERR_NULL;
    if (!ws || ws_bytes < ws_layout(dt, Nb, C, HW)) return NORM_ERR_WORKSPACE;
    const BnGeom g = make_geom(dt, Nb, C, HW);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool vec = bn_vec_ok(dt, HW, {dy, x, res, dx, dres});
    return with_io_type(dt, [&](auto tag) {
        using T = typename decltype(tag)::type;
        constexpr int VW = 16 / (int)sizeof(T);
        return vec ? launch_bwd<T, VW>(g, st, act, act_param, dy, x, res, w, b, save_mean, save_rstd, dx, dres, dw, db, ws)
                   : launch_bwd<T, 1>(g, st, act, act_param, dy, x, res, w, b, save_mean, save_rstd, dx, dres, dw, db, ws);
    });
}
