// bn_plane.hpp -- BatchNorm plane path: kernels and launchers for inputs
// whose (n, c) planes of HW values are long enough to stream on their own.
//
// Pages (by title):
//   [NormPage] "How attorch implements LayerNorm, BatchNorm and RMSNorm:
//               the three normalization Triton kernels explained"
//   [MathPage] "Building custom GPU operators quickly with attorch.math:
//               an operator-fusion guide for advanced developers"
//   [ActPage]  "Operator fusion in practice: attorch's activation and
//               dropout fusion kernels"
//
// Work split.  [NormPage] "BatchNorm" section gives one program per channel
// looping over blocks of batch x spatial values.  MI355X has 256 CUs and
// networks have 64-256 channels per layer, so here each channel is split
// into `tiles` workgroups of `ppb` planes (BnGeom).
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
//                       bits), the channel's first workgroup saves mean /
//                       rstd and applies the momentum update, then
//                       z = x * a_c + s_c (+ res), y = act(z) with
//                       a_c = w_c * rstd_c, s_c = b_c - mean_c * a_c.
//   forward (eval)      bn_apply_kernel with mean / rstd from running stats.
//   backward
//     bn_bwd_reduce_kernel  recomputes z exactly as the forward did,
//                       dz = dy * act'(z), stores dres = dz when a residual
//                       was added, and sums dz, dz * (x - mean) and x - mean
//                       per tile (float64 per element for float32 I/O,
//                       float32 per thread for 16-bit I/O; float64 beyond).
//     bn_bwd_dx_kernel  each workgroup adds its channel's tile sums, forms
//                       db, dw and dx = k1*dz + k2*(x - mean) + k3 (the first
//                       workgroup writes db, dw), then streams dz (re-read
//                       from dres, or recomputed from dy, x, res) into dx.
// Folding the per-channel merges into the following kernel saves a launch
// and the gap between dependent kernels (several microseconds each).
#pragma once

#include "bn_common.hpp"

namespace mi355norm {

// ------------------------------------------------------------------- tiles

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

// Output store of vector v of the plane that starts at element `off`.  A
// plane under 4 GiB is addressed from its first element (the same in every
// lane) and written with the device-scope buffer store; a larger one with a
// non-temporal global store.
template <typename T, int V>
__device__ __forceinline__ void plane_store(T *out, int64_t off, int64_t v, const typename Vec<T, V>::raw_t &r,
                                            bool sc1_ok) {
    if (sc1_ok)
        vstore_out<T, V>(out + off, (uint32_t)(v * V), r);
    else
        vstore_stream<T, V>(out + off + v * V, r);
}
template <typename T>
__device__ __forceinline__ bool plane_sc1_ok(const BnGeom &g) {
    return g.HW * (int64_t)sizeof(T) <= (int64_t)0xffffffff;
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

    // Each thread folds its chunks into a float32 running state.  A plane
    // longer than kBnStatsChunk vectors (then the whole tile) is walked in
    // pieces of that many vectors, after each of which the state moves into
    // a float64 one: a float32 state never spans more than 1024 float32 or
    // 2048 16-bit values per thread (a single 4 GiB plane is one tile).
    // Shorter planes keep the float32 state and wave merge throughout.
    const bool long_plane = nvp > kBnStatsChunk;  // the same in every lane
    // Float32 I/O: when the tile's first vector shows a mean more than four
    // of its own spreads from zero, values are folded relative to that mean,
    // so the float32 state's rounding scales with the channel's spread
    // rather than its mean.  Otherwise (and for 16-bit I/O) no shift: moving
    // the origin by a value a few spreads from a near-zero mean would make
    // the rounding larger, not smaller.  Every lane computes the same shift.
    float shift = 0.0f;
    if constexpr (sizeof(T) == 4 && V > 1) {  // one value has no spread to compare
        if (nvp > 0) {
            float f0[V];
            VT::unpack(vload<T, V>(x + plane_offset(g, n0, c)), f0);
            float s0 = 0.0f;
#pragma unroll
            for (int e = 0; e < V; ++e) s0 += f0[e];
            const float m0 = s0 * (1.0f / V);
            float q0 = 0.0f;
#pragma unroll
            for (int e = 0; e < V; ++e) q0 = fmaf(f0[e] - m0, f0[e] - m0, q0);
            if (m0 * m0 > 16.0f * (q0 * (1.0f / V))) shift = m0;
        }
    }
    WelfF st{0.0f, 0.0f, 0.0f};
    WelfD acc{0.0, 0.0, 0.0};
    for (int64_t n = n0; n < n1; ++n) {
        const T *p = x + plane_offset(g, n, c);
        for (int64_t vc = 0; vc < nvp; vc += kBnStatsChunk) {
            const int64_t ve = nvp - vc > kBnStatsChunk ? vc + kBnStatsChunk : nvp;
            for (int64_t v0 = vc + threadIdx.x; v0 < ve; v0 += (int64_t)kBnBlock * kBnUnroll) {
                raw_t r[kBnUnroll];
#pragma unroll
                for (int u = 0; u < kBnUnroll; ++u) {
                    const int64_t v = v0 + (int64_t)u * kBnBlock;
                    if (v < ve) r[u] = vload_stream<T, V>(p + v * V);
                }
#pragma unroll
                for (int u = 0; u < kBnUnroll; ++u) {
                    const int64_t v = v0 + (int64_t)u * kBnBlock;
                    if (v < ve) {
                        float f[V];
                        VT::unpack(r[u], f);
#pragma unroll
                        for (int e = 0; e < V; ++e) f[e] -= shift;
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
            if (long_plane) {
                acc = welf_merge(acc, WelfD{st.n, (double)st.mean + shift, st.m2});
                st = WelfF{0.0f, 0.0f, 0.0f};
            }
        }
    }
    if (long_plane) {
        acc = wave_merge(acc);
    } else {
        st = wave_merge(st);
        acc = WelfD{st.n, (double)st.mean + shift, st.m2};
    }

    __shared__ WelfD wave_part[kBnWaves];
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) wave_part[wave] = acc;
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
        const int lane = threadIdx.x;
        double sn = 0.0, snm = 0.0, m2 = 0.0, mean;
        constexpr int R = 4;  // tiles held per lane on the one-round path
        if (tiles <= R * kWave) {  // the same in every lane: one round of loads
            double tn[R], tm[R], tq[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int t = lane + r * kWave;
                tn[r] = tm[r] = tq[r] = 0.0;
                if (t < tiles) {
                    tn[r] = q[t * 3 + 0];
                    tm[r] = q[t * 3 + 1];
                    tq[r] = q[t * 3 + 2];
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                sn += tn[r];
                snm = fma(tn[r], tm[r], snm);
            }
            sn = wave_sum_dpp_d(sn);
            snm = wave_sum_dpp_d(snm);
            mean = snm / sn;
#pragma unroll
            for (int r = 0; r < R; ++r) {  // absent tiles have n = M2 = 0
                const double d = tm[r] - mean;
                m2 += fma(tn[r] * d, d, tq[r]);
            }
        } else {
            for (int t = lane; t < tiles; t += kWave) {
                sn += q[t * 3 + 0];
                snm = fma(q[t * 3 + 0], q[t * 3 + 1], snm);
            }
            sn = wave_sum_dpp_d(sn);
            snm = wave_sum_dpp_d(snm);
            mean = snm / sn;
            for (int t = lane; t < tiles; t += kWave) {
                const double d = q[t * 3 + 1] - mean;
                m2 += fma(q[t * 3 + 0] * d, d, q[t * 3 + 2]);
            }
        }
        m2 = wave_sum_dpp_d(m2);
        if (lane == 0) sh = WelfD{sn, mean, m2};
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
    int c; int64_t n0, n1;
    tile_of_block(g, &c, &n0, &n1);
    const int64_t nvp = g.HW / V;
    // Vectors in flight per thread: 8, or 4 for the 16-bit training apply
    // (bf16 GELU BatchNorm2d 256x64x112x112: 125.7 -> 123.0 us; the float32
    // apply measured flat at 4, the eval apply keeps 8).
    constexpr int U = (sizeof(T) == 2 && MODE == 0) ? 4 : kBnUnrollStream;
    raw_t rx[U], rr[U];
    auto load = [&](int64_t off, int64_t v0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + (int64_t)u * kBnBlock;
            if (v < nvp) {
                rx[u] = vload_stream<T, V>(x + off + v * V);
                if (RES) rr[u] = vload_stream<T, V>(res + off + v * V);
            }
        }
    };
    // Float32 I/O: the block's first vectors are requested before the
    // channel's statistics are formed, so that read overlaps them (apply
    // 89.4 -> 87.9 us on the float32 BatchNorm2d workload; the 16-bit
    // kernels measured slower with it: eval apply 120.7 -> 127.2 us).
    bool loaded = sizeof(T) == 4 && n0 < n1;
    if (loaded) load(plane_offset(g, n0, c), threadIdx.x);
    float mean, rstd;
    if (MODE == 0) {
        const WelfD st = merge_channel_tiles(part, c, g.tiles);
        mean = (float)st.mean;
        rstd = (float)(1.0 / sqrt(st.m2 / st.n + (double)eps));
        if (n0 == 0 && threadIdx.x == 0)
            bn_save_stats(st, c, eps, momentum, running_mean, running_var, save_mean, save_rstd);
    } else {
        mean = running_mean[c];
        rstd = 1.0f / sqrtf(running_var[c] + eps);
    }
    float a, s;
    const float bias = b ? ld1(b + c) : 0.0f;
    bn_coeffs(mean, rstd, w ? ld1(w + c) : 1.0f, bias, &a, &s);
    const bool sc1_ok = plane_sc1_ok<T>(g);

    for (int64_t n = n0; n < n1; ++n) {
        const int64_t off = plane_offset(g, n, c);
        for (int64_t v0 = threadIdx.x; v0 < nvp; v0 += (int64_t)kBnBlock * U) {
            if (!loaded) load(off, v0);  // else: the first plane's first vectors, loaded above
            loaded = false;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < nvp) {
                    float f[V], rf[V], o[V];
                    VT::unpack(rx[u], f);
                    if (RES) VT::unpack(rr[u], rf);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        float z = bn_pre<T>(f[e], a, s, mean, bias);
                        if (RES) z += rf[e];
                        o[e] = act_fwd_io<T, ACT>(z, act_rt, act_p);
                    }
                    plane_store<T, V>(y, off, v, VT::pack(o), sc1_ok);
                }
            }
        }
        loaded = false;  // a thread past the first plane's last vector did not use it
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
    const float bias = b ? ld1(b + c) : 0.0f;
    bn_coeffs(mean, save_rstd[c], w ? ld1(w + c) : 1.0f, bias, &a, &s);
    constexpr bool kPre = kGeluPrescale<T, ACT, RES>;
    if (kPre) {
        a *= kGeluWScale;
        s *= kGeluWScale;
    }
    const int64_t nvp = g.HW / V;
    const bool sc1_ok = plane_sc1_ok<T>(g);

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
    // 16-bit I/O: a plane longer than kBnStatsChunk vectors is walked in
    // pieces of that many, after each of which the float32 sums move into
    // float64 ones, so none spans more than 2048 values per thread.
    const bool long_plane = nvp > kBnStatsChunk;  // the same in every lane
    double f_dz = 0.0, f_dzx = 0.0;
    const Acc mean_a = kExact ? (Acc)mean : (Acc)0;
    for (int64_t n = n0; n < n1; ++n) {
        const int64_t off = plane_offset(g, n, c);
        for (int64_t vc = 0; vc < nvp; vc += kBnStatsChunk) {
          const int64_t ve = nvp - vc > kBnStatsChunk ? vc + kBnStatsChunk : nvp;
          for (int64_t v0 = vc + threadIdx.x; v0 < ve; v0 += (int64_t)kBnBlock * kBnUnroll) {
            raw_t rd[kBnUnroll], rx[kBnUnroll], rr[kBnUnroll];
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < ve) {
                    rd[u] = vload_stream<T, V>(dy + off + v * V);
                    rx[u] = vload_stream<T, V>(x + off + v * V);
                    if (RES && ACT != kActNone) rr[u] = vload_stream<T, V>(res + off + v * V);
                }
            }
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t v = v0 + (int64_t)u * kBnBlock;
                if (v < ve) {
                    float df[V], xf[V], rf[V], dz[V];
                    VT::unpack(rd[u], df);
                    VT::unpack(rx[u], xf);
                    if (RES && ACT != kActNone) VT::unpack(rr[u], rf);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        if (ACT != kActNone) {
                            float z = bn_pre<T>(xf[e], a, s, mean, bias);
                            if (RES) z += rf[e];
                            dz[e] = df[e] * (kPre ? gelu_grad_fast_w(z)
                                                  : act_grad_any<ACT, kFastGrad<T>>(z, act_rt, act_p));
                        } else {
                            dz[e] = df[e];
                        }
                        const Acc xc = kExact ? (Acc)xf[e] - mean_a : (Acc)xf[e];
                        const Acc d = (Acc)dz[e];
                        s_dz += d;
                        s_dzx = fma(d, xc, s_dzx);
                        if (kExact) s_xc += xc;
                    }
                    if (RES) plane_store<T, V>(dres, off, v, VT::pack(dz), sc1_ok);
                }
            }
          }
          if (!kExact && long_plane) {
              f_dz += (double)s_dz;
              f_dzx += (double)s_dzx;
              s_dz = s_dzx = 0;
          }
        }
    }
    const double t_dz = wave_sum_d((double)s_dz + f_dz);
    const double t_dzx = wave_sum_d((double)s_dzx + f_dzx);
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
// Every workgroup adds its channel's tile sums and forms db, dw and the dx
// coefficients (bn_dx_coeffs); the channel's first workgroup writes dw, db.
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
    constexpr bool kFast = kFastGrad<T>;
    int c; int64_t n0, n1;
    tile_of_block(g, &c, &n0, &n1);
    const int64_t nvp = g.HW / V;
    const T *dzsrc = DZ_SRC == 1 ? dres : dy;
    raw_t rd[kBnUnrollStream], rx[kBnUnrollStream], rr[kBnUnrollStream];
    auto load = [&](int64_t off, int64_t v0) {
#pragma unroll
        for (int u = 0; u < kBnUnrollStream; ++u) {
            const int64_t v = v0 + (int64_t)u * kBnBlock;
            if (v < nvp) {
                rd[u] = vload_stream<T, V>(dzsrc + off + v * V);
                rx[u] = vload_stream<T, V>(x + off + v * V);
                if (DZ_SRC == 2 && RES) rr[u] = vload_stream<T, V>(res + off + v * V);
            }
        }
    };
    // Float32 I/O: the block's first vectors are requested before the
    // channel's sums are added, so that read overlaps them (dx 88.4 -> 86.3
    // us on the float32 BatchNorm2d workload; the 16-bit dx kernel measured
    // far slower with it, 181 -> 242 us).
    bool loaded = sizeof(T) == 4 && n0 < n1;
    if (loaded) load(plane_offset(g, n0, c), threadIdx.x);
    double sums[3];
    sum_channel_tiles(part, c, g.tiles, sums);
    const float mean = save_mean[c];
    const float rstd_f = save_rstd[c];
    const float wc_f = w ? ld1(w + c) : 1.0f;
    const BnDxCoef kc = bn_dx_coeffs(sums, mean, rstd_f, wc_f, n_total);
    if (n0 == 0 && threadIdx.x == 0) {
        if (db) st1(db + c, (float)kc.dbeta);
        if (dw) st1(dw + c, (float)kc.dgamma);
    }
    const float k1 = kc.k1, k2 = kc.k2, k3 = kc.k3;
    // 16-bit I/O: the mean folded into the constant, dx = k1 dz + k2 x + k3m.
    constexpr bool kExact = sizeof(T) == 4;
    const float k3m = kc.k3m;
    float a = 0.0f, s = 0.0f;
    const float bias = b ? ld1(b + c) : 0.0f;
    if (DZ_SRC == 2) bn_coeffs(mean, rstd_f, wc_f, bias, &a, &s);
    constexpr bool kPre = kGeluPrescale<T, ACT, RES>;
    if (kPre) {
        a *= kGeluWScale;
        s *= kGeluWScale;
    }
    const bool sc1_ok = plane_sc1_ok<T>(g);

    for (int64_t n = n0; n < n1; ++n) {
        const int64_t off = plane_offset(g, n, c);
        for (int64_t v0 = threadIdx.x; v0 < nvp; v0 += (int64_t)kBnBlock * kBnUnrollStream) {
            if (!loaded) load(off, v0);  // else: the first plane's first vectors, loaded above
            loaded = false;
#pragma unroll
            for (int u = 0; u < kBnUnrollStream; ++u) {
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
                            float z = bn_pre<T>(xf[e], a, s, mean, bias);
                            if (RES) z += rf[e];
                            dz = df[e] * (kPre ? gelu_grad_fast_w(z) : act_grad_any<ACT, kFast>(z, act_rt, act_p));
                        }
                        o[e] = kExact ? fmaf(k1, dz, fmaf(k2, xf[e] - mean, k3)) : fmaf(k1, dz, fmaf(k2, xf[e], k3m));
                    }
                    plane_store<T, V>(dx, off, v, VT::pack(o), sc1_ok);
                }
            }
        }
        loaded = false;  // a thread past the first plane's last vector did not use it
    }
}

// ------------------------------------------------------------- launchers
template <typename T, int V, int MODE>
static auto plane_apply_kernel(norm_act act, bool r) {
    switch (act) {
    case NORM_ACT_NONE: return r ? bn_apply_kernel<T, V, kActNone, true, MODE> : bn_apply_kernel<T, V, kActNone, false, MODE>;
    case NORM_ACT_RELU: return r ? bn_apply_kernel<T, V, kActRelu, true, MODE> : bn_apply_kernel<T, V, kActRelu, false, MODE>;
    case NORM_ACT_GELU: return r ? bn_apply_kernel<T, V, kActGelu, true, MODE> : bn_apply_kernel<T, V, kActGelu, false, MODE>;
    default: return r ? bn_apply_kernel<T, V, kActGeneric, true, MODE> : bn_apply_kernel<T, V, kActGeneric, false, MODE>;
    }
}

template <typename T, int V>
norm_status bn_plane_fwd_train(const BnGeom &g, const BnArgs &a) {
    const dim3 grid((unsigned)(g.C * (int64_t)g.tiles));
    double *part = static_cast<double *>(a.ws);
    launch("bn_stats_kernel", false, bn_stats_kernel<T, V>, grid, dim3(kBnBlock), 0, a.st, (const T *)a.x, g,
           part);
    launch("bn_apply_kernel<train>", true, plane_apply_kernel<T, V, 0>(a.act, a.res != nullptr), grid,
           dim3(kBnBlock), 0, a.st, (const T *)a.x, (const T *)a.res, (const T *)a.w, (const T *)a.b,
           (const double *)part, a.eps, a.momentum, a.rm, a.rv, a.sm, a.sr, (T *)a.y, g, (int)a.act, a.act_p);
    return launch_status();
}

template <typename T, int V>
norm_status bn_plane_fwd_eval(const BnGeom &g, const BnArgs &a) {
    const dim3 grid((unsigned)(g.C * (int64_t)g.tiles));
    // Eval reads the running statistics; they are not written.
    launch("bn_apply_kernel<eval>", true, plane_apply_kernel<T, V, 1>(a.act, a.res != nullptr), grid,
           dim3(kBnBlock), 0, a.st, (const T *)a.x, (const T *)a.res, (const T *)a.w, (const T *)a.b,
           (const double *)nullptr, a.eps, 0.0f, a.rm, a.rv, (float *)nullptr, (float *)nullptr, (T *)a.y, g,
           (int)a.act, a.act_p);
    return launch_status();
}

template <typename T, int V, int ACT>
static void plane_bwd_act(const BnGeom &g, const BnArgs &a) {
    const dim3 grid((unsigned)(g.C * (int64_t)g.tiles));
    const dim3 blk(kBnBlock);
    double *part = static_cast<double *>(a.ws);
    const double n_total = (double)g.Nb * (double)g.HW;
    const bool has_res = a.res != nullptr;
    const int act_rt = (int)a.act;
    // The main (largest) kernel: pass 1 with a residual (it reads dy, x, res
    // and writes dres), pass 2 otherwise.
    launch("bn_bwd_reduce_kernel", has_res,
           has_res ? bn_bwd_reduce_kernel<T, V, ACT, true> : bn_bwd_reduce_kernel<T, V, ACT, false>, grid, blk, 0,
           a.st, (const T *)a.dy, (const T *)a.x, (const T *)a.res, (const T *)a.w, (const T *)a.b,
           (const float *)a.sm, (const float *)a.sr, (T *)a.dres, g, part, act_rt, a.act_p);
    // dz for pass 2: float32 dres holds dz exactly; 16-bit dres is rounded, so
    // there dz is recomputed from dy and x (and res).
    const bool fp32 = sizeof(T) == 4;
    auto fn = bn_bwd_dx_kernel<T, V, ACT, false, 2>;
    if (ACT == kActNone && !has_res) fn = bn_bwd_dx_kernel<T, V, ACT, false, 0>;
    else if (has_res && (fp32 || ACT == kActNone)) fn = bn_bwd_dx_kernel<T, V, ACT, true, 1>;
    else if (has_res) fn = bn_bwd_dx_kernel<T, V, ACT, true, 2>;
    launch("bn_bwd_dx_kernel", !has_res, fn, grid, blk, 0, a.st, (const T *)a.dy, (const T *)a.x,
           (const T *)a.res, (const T *)a.dres, (const T *)a.w, (const T *)a.b, (const float *)a.sm,
           (const float *)a.sr, (const double *)part, n_total, (T *)a.dw, (T *)a.db, (T *)a.dx, g, act_rt,
           a.act_p);
}

template <typename T, int V>
norm_status bn_plane_bwd(const BnGeom &g, const BnArgs &a) {
    switch (a.act) {
    case NORM_ACT_NONE: plane_bwd_act<T, V, kActNone>(g, a); break;
    case NORM_ACT_RELU: plane_bwd_act<T, V, kActRelu>(g, a); break;
    case NORM_ACT_GELU: plane_bwd_act<T, V, kActGelu>(g, a); break;
    default: plane_bwd_act<T, V, kActGeneric>(g, a); break;
    }
    return launch_status();
}

}  // namespace mi355norm
