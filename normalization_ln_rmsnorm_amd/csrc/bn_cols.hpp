// bn_cols.hpp -- BatchNorm column path: kernels and launchers for inputs
// whose (n, c) planes are too short to stream on their own -- BatchNorm1d's
// (N, C) inputs (HW = 1) and (N, C, L) inputs with small L, and small
// feature maps.
//
// Pages (by title):
//   [NormPage] "How attorch implements LayerNorm, BatchNorm and RMSNorm:
//               the three normalization Triton kernels explained"
//   [MathPage] "Building custom GPU operators quickly with attorch.math:
//               an operator-fusion guide for advanced developers"
//
// Layout.  Each sample n is one contiguous row of K = C * HW values; column
// j holds channel j / HW.  The channel's statistics run down the columns,
// so a wave reads whole 128-bit vectors along a row and walks down the rows
// (BnColGeom): every load is a full contiguous segment, whatever HW is.
//
//   forward (training)
//     bn_col_stats_kernel     Welford update per column over the thread's
//                             rows (float32), merged across the workgroup's
//                             row slices in float64 (Chan's pairwise merge,
//                             a fixed tree); one (mean, M2) per column and
//                             row tile
//     bn_col_finalize_kernel  one wave per channel combines its HW columns x
//                             T tiles with the exact parallel-axis identity
//                             (float64), saves mean / rstd and applies the
//                             momentum update
//     bn_col_apply_kernel     z = x * a_c + s_c (+ res), y = act(z)
//   forward (eval)            bn_col_apply_kernel from the running stats
//   backward
//     bn_col_bwd_reduce_kernel   dz = dy * act'(z) at the recomputed z,
//                             dres = dz, and per column and tile the sums
//                             of dz, dz (x - mean) and x - mean
//     bn_col_bwd_finalize_kernel one wave per channel adds them, writes dw,
//                             db and the dx coefficients (bn_dx_coeffs)
//     bn_col_bwd_dx_kernel    dx = k1 dz + k2 (x - mean) + k3
// The per-element arithmetic is the plane path's (same coefficient and
// activation functions), so both paths compute the same z.
#pragma once

#include "bn_common.hpp"

namespace mi355norm {

// Position of this thread in the column geometry.
struct ColPos {
    int64_t col0;    // first of the thread's V columns
    int64_t cb;      // first column of the block's chunk (the same in every lane)
    int64_t r0, r1;  // the tile's rows [r0, r1)
    int rs;          // row slice: rows r0 + rs, r0 + rs + RPP, ...
    int tile;
    bool active;     // lane maps to a real vector of a real slice
};

// The column chunks of one row tile take consecutive slots on one XCD
// (xcd_swizzle), so the rows they share are read through one L2 in a short
// window rather than as 1 KiB slices by every XCD.
__device__ __forceinline__ ColPos col_pos(const BnColGeom &g, int V) {
    ColPos p;
    const unsigned id = xcd_swizzle(blockIdx.x, gridDim.x);
    const int chunk = (int)(id % (unsigned)g.NCH);
    p.tile = (int)(id / (unsigned)g.NCH);
    const int cv = (int)(threadIdx.x % (unsigned)g.CV);
    p.rs = (int)(threadIdx.x / (unsigned)g.CV);
    const int64_t vi = (int64_t)chunk * g.CV + cv;
    p.active = p.rs < g.RPP && vi < g.KV;
    p.col0 = vi * V;
    p.cb = (int64_t)chunk * g.CV * V;
    p.r0 = (int64_t)p.tile * g.RT;
    const int64_t e = p.r0 + g.RT;
    p.r1 = e < g.Nb ? e : g.Nb;
    return p;
}

// Output store of the thread's vector in row `row`.  When the block's tile
// spans under 4 GiB it is addressed from the tile's first row and the
// chunk's first column (the same in every lane) and written with the
// device-scope buffer store; otherwise with a non-temporal global store.
template <typename T>
__device__ __forceinline__ bool col_sc1_ok(const BnColGeom &g) {
    return (int64_t)g.RT * g.K * (int64_t)sizeof(T) <= (int64_t)0xffffffff;
}
template <typename T, int V>
__device__ __forceinline__ void col_store(T *out, const BnColGeom &g, const ColPos &p, int64_t row,
                                          const typename Vec<T, V>::raw_t &r, bool sc1_ok) {
    if (sc1_ok)
        vstore_out<T, V>(out + p.r0 * g.K + p.cb, (uint32_t)((row - p.r0) * g.K + (p.col0 - p.cb)), r);
    else
        vstore_stream<T, V>(out + row * g.K + p.col0, r);
}

__device__ __forceinline__ int tree_start(int rpp) {
    int h = 1;
    while (h < rpp) h <<= 1;
    return h >> 1;
}

// -------------------------------------------------------- forward: stats
template <typename T, int V>
__global__ void __launch_bounds__(kBnBlock)
bn_col_stats_kernel(const T *__restrict__ x, BnColGeom g, double *__restrict__ part) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    const ColPos p = col_pos(g, V);
    // Float32 I/O: a column whose first two rows in the tile lie more than
    // four times their difference from zero is folded relative to the first
    // row's value, so the float32 state's rounding scales with the spread
    // rather than the mean; otherwise (and for 16-bit I/O) no shift, since a
    // shift a few spreads from a near-zero mean would enlarge the rounding.
    // The shift depends only on the tile and column, so the row slices of a
    // column agree.
    float n = 0.0f, mean[V], m2[V], shift[V];
#pragma unroll
    for (int e = 0; e < V; ++e) mean[e] = m2[e] = shift[e] = 0.0f;
    if (p.active) {
        const T *base = x + p.col0;
        if constexpr (sizeof(T) == 4) {
            if (p.r0 + 1 < p.r1) {
                float f0[V], f1[V];
                VT::unpack(vload<T, V>(base + p.r0 * g.K), f0);
                VT::unpack(vload<T, V>(base + (p.r0 + 1) * g.K), f1);
#pragma unroll
                for (int e = 0; e < V; ++e)
                    shift[e] = fabsf(f0[e]) > 4.0f * fabsf(f0[e] - f1[e]) ? f0[e] : 0.0f;
            }
        }
        const int64_t step = (int64_t)g.RPP;
        for (int64_t r = p.r0 + p.rs; r < p.r1; r += step * kBnUnroll) {
            raw_t buf[kBnUnroll];
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t rr = r + u * step;
                if (rr < p.r1) buf[u] = vload_stream<T, V>(base + rr * g.K);
            }
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t rr = r + u * step;
                if (rr < p.r1) {
                    float f[V];
                    VT::unpack(buf[u], f);
                    n += 1.0f;
                    const float inv = 1.0f / n;
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const float fs = f[e] - shift[e];
                        const float d = fs - mean[e];
                        mean[e] = fmaf(d, inv, mean[e]);
                        m2[e] = fmaf(d, fs - mean[e], m2[e]);
                    }
                }
            }
        }
    }
    // Merge the row slices of each column: a fixed float64 tree over rs.
    __shared__ double sh_n[kBnBlock];
    __shared__ double sh_mean[kBnBlock * V];
    __shared__ double sh_m2[kBnBlock * V];
    const int t = threadIdx.x;
    sh_n[t] = n;
#pragma unroll
    for (int e = 0; e < V; ++e) {
        sh_mean[t * V + e] = (double)mean[e] + shift[e];
        sh_m2[t * V + e] = m2[e];
    }
    for (int h = tree_start(g.RPP); h >= 1; h >>= 1) {
        __syncthreads();
        if (p.active && p.rs < h && p.rs + h < g.RPP) {
            const int o = t + h * g.CV;
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const WelfD m = welf_merge(WelfD{sh_n[t], sh_mean[t * V + e], sh_m2[t * V + e]},
                                           WelfD{sh_n[o], sh_mean[o * V + e], sh_m2[o * V + e]});
                sh_mean[t * V + e] = m.mean;
                sh_m2[t * V + e] = m.m2;
            }
            sh_n[t] += sh_n[o];
        }
    }
    __syncthreads();
    if (p.active && p.rs == 0) {
        double *dst = part + ((int64_t)p.tile * g.K + p.col0) * 2;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            dst[2 * e] = sh_mean[t * V + e];
            dst[2 * e + 1] = sh_m2[t * V + e];
        }
    }
}

// ------------------------------------------- forward: channel statistics
// One wave per channel.  Entry (tile, column) holds the n_t rows of the
// tile as (mean, M2).  The lanes sum n_t and n_t mean_t over their entries
// (up to eight each held in registers, else two passes over the entries),
// one division gives the channel mean, and a second sum adds M2_t + n_t
// (mean_t - mean)^2, all in float64 and in a fixed order.  (T is only the
// dtype of the operation, so each dtype's translation unit has its own
// instance.)
template <typename T>
__global__ void __launch_bounds__(kBnBlock)
bn_col_finalize_kernel(const double *__restrict__ part, BnColGeom g, float eps, float momentum,
                       float *__restrict__ running_mean, float *__restrict__ running_var,
                       float *__restrict__ save_mean, float *__restrict__ save_rstd) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t c = (int64_t)blockIdx.x * kBnWaves + threadIdx.x / kWave;
    if (c >= g.C) return;  // the whole wave leaves; no barrier follows
    const int64_t ne = (int64_t)g.T * g.HW;
    // Entry e: tile e / HW (its row count), column c HW + e mod HW.
    auto entry = [&](int64_t e, double &nt, double &m, double &q) {
        const int64_t t = e / g.HW, j = c * g.HW + e % g.HW;
        const int64_t left = g.Nb - t * g.RT;
        nt = (double)(left < g.RT ? left : g.RT);
        m = part[(t * g.K + j) * 2];
        q = part[(t * g.K + j) * 2 + 1];
    };
    // The exact parallel-axis identity, mean = sum n_t m_t / n and M2 =
    // sum [M2_t + n_t (m_t - mean)^2], in a fixed order: one division per
    // channel instead of one per pairwise merge (a chain of dependent
    // float64 divisions per lane).
    double sn = 0.0, snm = 0.0, m2 = 0.0;
    constexpr int R = 8;  // entries held per lane on the one-round path
    if (ne <= (int64_t)R * kWave) {  // the same in every lane
        double nt[R], m[R], q[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t e = lane + (int64_t)r * kWave;
            nt[r] = m[r] = q[r] = 0.0;
            if (e < ne) entry(e, nt[r], m[r], q[r]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            sn += nt[r];
            snm = fma(nt[r], m[r], snm);
        }
        sn = wave_sum_dpp_d(sn);
        snm = wave_sum_dpp_d(snm);
        const double mean = sn > 0.0 ? snm / sn : 0.0;
#pragma unroll
        for (int r = 0; r < R; ++r) {  // absent entries have n = M2 = 0
            const double d = m[r] - mean;
            m2 += fma(nt[r] * d, d, q[r]);
        }
        m2 = wave_sum_dpp_d(m2);
        if (lane == 0) bn_save_stats(WelfD{sn, mean, m2}, c, eps, momentum, running_mean, running_var, save_mean, save_rstd);
        return;
    }
    for (int64_t e = lane; e < ne; e += kWave) {
        double nt, m, q;
        entry(e, nt, m, q);
        sn += nt;
        snm = fma(nt, m, snm);
    }
    sn = wave_sum_dpp_d(sn);
    snm = wave_sum_dpp_d(snm);
    const double mean = sn > 0.0 ? snm / sn : 0.0;
    for (int64_t e = lane; e < ne; e += kWave) {
        double nt, m, q;
        entry(e, nt, m, q);
        const double d = m - mean;
        m2 += fma(nt * d, d, q);
    }
    m2 = wave_sum_dpp_d(m2);
    const WelfD acc{sn, mean, m2};
    if (lane == 0) bn_save_stats(acc, c, eps, momentum, running_mean, running_var, save_mean, save_rstd);
}

// ---------------------------------------------------- forward: apply
// MODE 0 (training): mean / rstd from save_mean / save_rstd (just written
// by the finalize kernel).  MODE 1 (eval): from the running statistics.
template <typename T, int V, int ACT, bool RES, int MODE>
__global__ void __launch_bounds__(kBnBlock)
bn_col_apply_kernel(const T *__restrict__ x, const T *__restrict__ res, const T *__restrict__ w,
                    const T *__restrict__ b, const float *__restrict__ mean_src,
                    const float *__restrict__ scale_src, float eps, T *__restrict__ y, BnColGeom g,
                    int act_rt, float act_p) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    const ColPos p = col_pos(g, V);
    const bool sc1_ok = col_sc1_ok<T>(g);
    if (!p.active) return;  // no barriers in this kernel
    float a[V], s[V], mn[V], bs[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const int64_t c = (p.col0 + e) / g.HW;
        mn[e] = mean_src[c];
        bs[e] = b ? ld1(b + c) : 0.0f;
        const float rstd = MODE == 0 ? scale_src[c] : 1.0f / sqrtf(scale_src[c] + eps);
        bn_coeffs(mn[e], rstd, w ? ld1(w + c) : 1.0f, bs[e], &a[e], &s[e]);
    }
    const int64_t step = (int64_t)g.RPP;
    for (int64_t r = p.r0 + p.rs; r < p.r1; r += step * kBnUnroll) {
        raw_t rx[kBnUnroll], rr_[kBnUnroll];
#pragma unroll
        for (int u = 0; u < kBnUnroll; ++u) {
            const int64_t row = r + u * step;
            if (row < p.r1) {
                rx[u] = vload_stream<T, V>(x + row * g.K + p.col0);
                if (RES) rr_[u] = vload_stream<T, V>(res + row * g.K + p.col0);
            }
        }
#pragma unroll
        for (int u = 0; u < kBnUnroll; ++u) {
            const int64_t row = r + u * step;
            if (row < p.r1) {
                float f[V], rf[V], o[V];
                VT::unpack(rx[u], f);
                if (RES) VT::unpack(rr_[u], rf);
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    float z = bn_pre<T>(f[e], a[e], s[e], mn[e], bs[e]);
                    if (RES) z += rf[e];
                    o[e] = act_fwd_io<T, ACT>(z, act_rt, act_p);
                }
                col_store<T, V>(y, g, p, row, VT::pack(o), sc1_ok);
            }
        }
    }
}

// --------------------------------------------------- backward: pass 1
// Accumulation as on the plane path: float64 per element for float32 I/O
// (with the sum of x - mean), float32 dz and dz * x per thread for 16-bit
// I/O (the mean taken out per tile in float64); the row slices are added
// in float64 by a fixed tree.
template <typename T, int V, int ACT, bool RES>
__global__ void __launch_bounds__(kBnBlock)
bn_col_bwd_reduce_kernel(const T *__restrict__ dy, const T *__restrict__ x, const T *__restrict__ res,
                         const T *__restrict__ w, const T *__restrict__ b,
                         const float *__restrict__ save_mean, const float *__restrict__ save_rstd,
                         T *__restrict__ dres, BnColGeom g, double *__restrict__ part, int act_rt,
                         float act_p) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    constexpr bool kExact = sizeof(T) == 4;
    constexpr bool kFast = kFastGrad<T>;
    constexpr bool kPre = kGeluPrescale<T, ACT, RES>;
    constexpr int NS = kExact ? 3 : 2;
    using Acc = typename std::conditional<kExact, double, float>::type;
    const ColPos p = col_pos(g, V);
    const bool sc1_ok = col_sc1_ok<T>(g);
    Acc s_dz[V], s_dzx[V], s_xc[V];
    float a[V], s[V], mean[V], bs[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        s_dz[e] = s_dzx[e] = s_xc[e] = 0;
        a[e] = s[e] = mean[e] = bs[e] = 0.0f;
    }
    if (p.active) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const int64_t c = (p.col0 + e) / g.HW;
            mean[e] = save_mean[c];
            bs[e] = b ? ld1(b + c) : 0.0f;
            bn_coeffs(mean[e], save_rstd[c], w ? ld1(w + c) : 1.0f, bs[e], &a[e], &s[e]);
            if (kPre) {
                a[e] *= kGeluWScale;
                s[e] *= kGeluWScale;
            }
        }
        const int64_t step = (int64_t)g.RPP;
        for (int64_t r = p.r0 + p.rs; r < p.r1; r += step * kBnUnroll) {
            raw_t rd[kBnUnroll], rx[kBnUnroll], rr_[kBnUnroll];
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t row = r + u * step;
                if (row < p.r1) {
                    const int64_t off = row * g.K + p.col0;
                    rd[u] = vload_stream<T, V>(dy + off);
                    rx[u] = vload_stream<T, V>(x + off);
                    if (RES && ACT != kActNone) rr_[u] = vload_stream<T, V>(res + off);
                }
            }
#pragma unroll
            for (int u = 0; u < kBnUnroll; ++u) {
                const int64_t row = r + u * step;
                if (row < p.r1) {
                    float df[V], xf[V], rf[V], dz[V];
                    VT::unpack(rd[u], df);
                    VT::unpack(rx[u], xf);
                    if (RES && ACT != kActNone) VT::unpack(rr_[u], rf);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        if (ACT != kActNone) {
                            float z = bn_pre<T>(xf[e], a[e], s[e], mean[e], bs[e]);
                            if (RES) z += rf[e];
                            dz[e] = df[e] * (kPre ? gelu_grad_fast_w(z) : act_grad_any<ACT, kFast>(z, act_rt, act_p));
                        } else {
                            dz[e] = df[e];
                        }
                        const Acc xc = kExact ? (Acc)xf[e] - (Acc)mean[e] : (Acc)xf[e];
                        const Acc d = (Acc)dz[e];
                        s_dz[e] += d;
                        s_dzx[e] = fma(d, xc, s_dzx[e]);
                        if (kExact) s_xc[e] += xc;
                    }
                    if (RES) col_store<T, V>(dres, g, p, row, VT::pack(dz), sc1_ok);
                }
            }
        }
    }
    __shared__ double sh[NS][kBnBlock * V];
    const int t = threadIdx.x;
#pragma unroll
    for (int e = 0; e < V; ++e) {
        sh[0][t * V + e] = (double)s_dz[e];
        sh[1][t * V + e] = (double)s_dzx[e];
        if (kExact) sh[NS - 1][t * V + e] = (double)s_xc[e];
    }
    for (int h = tree_start(g.RPP); h >= 1; h >>= 1) {
        __syncthreads();
        if (p.active && p.rs < h && p.rs + h < g.RPP) {
            const int o = t + h * g.CV;
#pragma unroll
            for (int k = 0; k < NS; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) sh[k][t * V + e] += sh[k][o * V + e];
        }
    }
    __syncthreads();
    if (p.active && p.rs == 0) {
        double *dst = part + ((int64_t)p.tile * g.K + p.col0) * 3;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const double p0 = sh[0][t * V + e];
            double p1 = sh[1][t * V + e];
            if (!kExact) p1 -= (double)mean[e] * p0;  // sum dz * x  ->  sum dz * (x - mean)
            dst[3 * e] = p0;
            dst[3 * e + 1] = p1;
            dst[3 * e + 2] = kExact ? sh[NS - 1][t * V + e] : 0.0;
        }
    }
}

// ------------------------------------------- backward: channel sums
// One wave per channel: adds the (tile, column) sums in a fixed order,
// writes db and dw, and stores k1, k2, k3, k3m for the dx kernel.
template <typename T>
__global__ void __launch_bounds__(kBnBlock)
bn_col_bwd_finalize_kernel(const double *__restrict__ part, BnColGeom g, const T *__restrict__ w,
                           const float *__restrict__ save_mean, const float *__restrict__ save_rstd,
                           T *__restrict__ dw, T *__restrict__ db, float *__restrict__ coef) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t c = (int64_t)blockIdx.x * kBnWaves + threadIdx.x / kWave;
    if (c >= g.C) return;  // the whole wave leaves; no barrier follows
    constexpr int U = 4;  // entries in flight per lane
    const int64_t ne = (int64_t)g.T * g.HW;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
    for (int64_t e0 = lane; e0 < ne; e0 += (int64_t)kWave * U) {
        double v[U][3];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = e0 + (int64_t)u * kWave;
            v[u][0] = v[u][1] = v[u][2] = 0.0;
            if (e < ne) {
                const int64_t t = e / g.HW, j = c * g.HW + e % g.HW;
                const double *q = part + (t * g.K + j) * 3;
                v[u][0] = q[0];
                v[u][1] = q[1];
                v[u][2] = q[2];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            s0 += v[u][0];
            s1 += v[u][1];
            s2 += v[u][2];
        }
    }
    double sums[3] = {wave_sum_d(s0), wave_sum_d(s1), wave_sum_d(s2)};
    if (lane == 0) {
        const double n_total = (double)g.Nb * (double)g.HW;
        const BnDxCoef k = bn_dx_coeffs(sums, save_mean[c], save_rstd[c], w ? ld1(w + c) : 1.0f, n_total);
        if (db) st1(db + c, (float)k.dbeta);
        if (dw) st1(dw + c, (float)k.dgamma);
        coef[c * 4 + 0] = k.k1;
        coef[c * 4 + 1] = k.k2;
        coef[c * 4 + 2] = k.k3;
        coef[c * 4 + 3] = k.k3m;
    }
}

// ----------------------------------------------------- backward: pass 2
// DZ_SRC as on the plane path: 0 dz = dy; 1 dz re-read from dres; 2 dz
// recomputed from dy, x (and res).
template <typename T, int V, int ACT, bool RES, int DZ_SRC>
__global__ void __launch_bounds__(kBnBlock)
bn_col_bwd_dx_kernel(const T *__restrict__ dy, const T *__restrict__ x, const T *__restrict__ res,
                     const T *__restrict__ dres, const T *__restrict__ w, const T *__restrict__ b,
                     const float *__restrict__ save_mean, const float *__restrict__ save_rstd,
                     const float *__restrict__ coef, T *__restrict__ dx, BnColGeom g, int act_rt,
                     float act_p) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    constexpr bool kExact = sizeof(T) == 4;
    constexpr bool kFast = kFastGrad<T>;
    constexpr bool kPre = kGeluPrescale<T, ACT, RES>;
    const ColPos p = col_pos(g, V);
    const bool sc1_ok = col_sc1_ok<T>(g);
    if (!p.active) return;  // no barriers in this kernel
    float k1[V], k2[V], k3[V], mean[V], a[V], s[V], bs[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const int64_t c = (p.col0 + e) / g.HW;
        k1[e] = coef[c * 4 + 0];
        k2[e] = coef[c * 4 + 1];
        k3[e] = kExact ? coef[c * 4 + 2] : coef[c * 4 + 3];
        mean[e] = save_mean[c];
        a[e] = s[e] = 0.0f;
        bs[e] = b ? ld1(b + c) : 0.0f;
        if (DZ_SRC == 2) bn_coeffs(mean[e], save_rstd[c], w ? ld1(w + c) : 1.0f, bs[e], &a[e], &s[e]);
        if (kPre) {
            a[e] *= kGeluWScale;
            s[e] *= kGeluWScale;
        }
    }
    const T *dzsrc = DZ_SRC == 1 ? dres : dy;
    const int64_t step = (int64_t)g.RPP;
    for (int64_t r = p.r0 + p.rs; r < p.r1; r += step * kBnUnroll) {
        raw_t rd[kBnUnroll], rx[kBnUnroll], rr_[kBnUnroll];
#pragma unroll
        for (int u = 0; u < kBnUnroll; ++u) {
            const int64_t row = r + u * step;
            if (row < p.r1) {
                const int64_t off = row * g.K + p.col0;
                rd[u] = vload_stream<T, V>(dzsrc + off);
                rx[u] = vload_stream<T, V>(x + off);
                if (DZ_SRC == 2 && RES) rr_[u] = vload_stream<T, V>(res + off);
            }
        }
#pragma unroll
        for (int u = 0; u < kBnUnroll; ++u) {
            const int64_t row = r + u * step;
            if (row < p.r1) {
                float df[V], xf[V], rf[V], o[V];
                VT::unpack(rd[u], df);
                VT::unpack(rx[u], xf);
                if (DZ_SRC == 2 && RES) VT::unpack(rr_[u], rf);
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    float dz = df[e];
                    if (DZ_SRC == 2 && ACT != kActNone) {
                        float z = bn_pre<T>(xf[e], a[e], s[e], mean[e], bs[e]);
                        if (RES) z += rf[e];
                        dz = df[e] * (kPre ? gelu_grad_fast_w(z) : act_grad_any<ACT, kFast>(z, act_rt, act_p));
                    }
                    o[e] = kExact ? fmaf(k1[e], dz, fmaf(k2[e], xf[e] - mean[e], k3[e]))
                                  : fmaf(k1[e], dz, fmaf(k2[e], xf[e], k3[e]));
                }
                col_store<T, V>(dx, g, p, row, VT::pack(o), sc1_ok);
            }
        }
    }
}

// ------------------------------------------------------------- launchers

template <typename T, int V, int MODE>
static auto col_apply_kernel(norm_act act, bool r) {
    switch (act) {
    case NORM_ACT_NONE: return r ? bn_col_apply_kernel<T, V, kActNone, true, MODE> : bn_col_apply_kernel<T, V, kActNone, false, MODE>;
    case NORM_ACT_RELU: return r ? bn_col_apply_kernel<T, V, kActRelu, true, MODE> : bn_col_apply_kernel<T, V, kActRelu, false, MODE>;
    case NORM_ACT_GELU: return r ? bn_col_apply_kernel<T, V, kActGelu, true, MODE> : bn_col_apply_kernel<T, V, kActGelu, false, MODE>;
    default: return r ? bn_col_apply_kernel<T, V, kActGeneric, true, MODE> : bn_col_apply_kernel<T, V, kActGeneric, false, MODE>;
    }
}

// g: the reduction geometry (statistics, finalize, workspace layout); gs:
// the streaming geometry of the apply and dx passes.
template <typename T, int V>
norm_status bn_col_fwd_train(const BnColGeom &g, const BnColGeom &gs, const BnArgs &a) {
    const dim3 grid((unsigned)((int64_t)g.NCH * g.T));
    const dim3 sgrid((unsigned)((int64_t)gs.NCH * gs.T));
    const dim3 fgrid((unsigned)ceil_div(g.C, kBnWaves));
    double *part = static_cast<double *>(a.ws);
    launch("bn_col_stats_kernel", false, bn_col_stats_kernel<T, V>, grid, dim3(kBnBlock), 0, a.st,
           (const T *)a.x, g, part);
    launch("bn_col_finalize_kernel", false, bn_col_finalize_kernel<T>, fgrid, dim3(kBnBlock), 0, a.st,
           (const double *)part, g, a.eps, a.momentum, a.rm, a.rv, a.sm, a.sr);
    launch("bn_col_apply_kernel<train>", true, col_apply_kernel<T, V, 0>(a.act, a.res != nullptr), sgrid,
           dim3(kBnBlock), 0, a.st, (const T *)a.x, (const T *)a.res, (const T *)a.w, (const T *)a.b,
           (const float *)a.sm, (const float *)a.sr, a.eps, (T *)a.y, gs, (int)a.act, a.act_p);
    return launch_status();
}

template <typename T, int V>
norm_status bn_col_fwd_eval(const BnColGeom &g, const BnArgs &a) {
    const dim3 grid((unsigned)((int64_t)g.NCH * g.T));
    launch("bn_col_apply_kernel<eval>", true, col_apply_kernel<T, V, 1>(a.act, a.res != nullptr), grid,
           dim3(kBnBlock), 0, a.st, (const T *)a.x, (const T *)a.res, (const T *)a.w, (const T *)a.b,
           (const float *)a.rm, (const float *)a.rv, a.eps, (T *)a.y, g, (int)a.act, a.act_p);
    return launch_status();
}

template <typename T, int V, int ACT>
static void col_bwd_act(const BnColGeom &g, const BnColGeom &gs, const BnArgs &a) {
    const dim3 grid((unsigned)((int64_t)g.NCH * g.T));
    const dim3 sgrid((unsigned)((int64_t)gs.NCH * gs.T));
    const dim3 fgrid((unsigned)ceil_div(g.C, kBnWaves));
    const dim3 blk(kBnBlock);
    double *part = static_cast<double *>(a.ws);
    float *coef = reinterpret_cast<float *>(static_cast<char *>(a.ws) + col_part_bytes_host(g));
    const bool has_res = a.res != nullptr;
    const int act_rt = (int)a.act;
    launch("bn_col_bwd_reduce_kernel", has_res,
           has_res ? bn_col_bwd_reduce_kernel<T, V, ACT, true> : bn_col_bwd_reduce_kernel<T, V, ACT, false>, grid,
           blk, 0, a.st, (const T *)a.dy, (const T *)a.x, (const T *)a.res, (const T *)a.w, (const T *)a.b,
           (const float *)a.sm, (const float *)a.sr, (T *)a.dres, g, part, act_rt, a.act_p);
    launch("bn_col_bwd_finalize_kernel", false, bn_col_bwd_finalize_kernel<T>, fgrid, blk, 0, a.st,
           (const double *)part, g, (const T *)a.w, (const float *)a.sm, (const float *)a.sr, (T *)a.dw,
           (T *)a.db, coef);
    const bool fp32 = sizeof(T) == 4;
    auto fn = bn_col_bwd_dx_kernel<T, V, ACT, false, 2>;
    if (ACT == kActNone && !has_res) fn = bn_col_bwd_dx_kernel<T, V, ACT, false, 0>;
    else if (has_res && (fp32 || ACT == kActNone)) fn = bn_col_bwd_dx_kernel<T, V, ACT, true, 1>;
    else if (has_res) fn = bn_col_bwd_dx_kernel<T, V, ACT, true, 2>;
    launch("bn_col_bwd_dx_kernel", !has_res, fn, sgrid, blk, 0, a.st, (const T *)a.dy, (const T *)a.x,
           (const T *)a.res, (const T *)a.dres, (const T *)a.w, (const T *)a.b, (const float *)a.sm,
           (const float *)a.sr, (const float *)coef, (T *)a.dx, gs, act_rt, a.act_p);
}

template <typename T, int V>
norm_status bn_col_bwd(const BnColGeom &g, const BnColGeom &gs, const BnArgs &a) {
    switch (a.act) {
    case NORM_ACT_NONE: col_bwd_act<T, V, kActNone>(g, gs, a); break;
    case NORM_ACT_RELU: col_bwd_act<T, V, kActRelu>(g, gs, a); break;
    case NORM_ACT_GELU: col_bwd_act<T, V, kActGelu>(g, gs, a); break;
    default: col_bwd_act<T, V, kActGeneric>(g, gs, a); break;
    }
    return launch_status();
}

}  // namespace mi355norm
