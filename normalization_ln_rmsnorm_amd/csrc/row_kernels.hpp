// row_kernels.hpp -- LayerNorm and RMSNorm kernels for gfx950 and their
// launchers (the entry points and the launch planner are in rownorm.hip).
//
// Pages (by title):
//   [NormPage] "How attorch implements LayerNorm, BatchNorm and RMSNorm:
//               the three normalization Triton kernels explained"
//
// Design.  Every row is normalized by a group of `tpr` threads (a power of
// two from 1 to 1024) that holds the whole row in registers: thread `l` of
// the group owns the 128-bit vectors l, l + tpr, l + 2*tpr, ... (IT of them),
// so each load instruction of a wave reads consecutive 16-byte chunks.  The
// row sums are reduced inside the wave with DPP / ds_swizzle / readlane and,
// when a row spans several waves, combined through LDS in a fixed order.
// Blocks are persistent: each walks rows blockIdx*rpb, +grid*rpb, ... so the
// weight (and bias) vectors are loaded once per block and kept in registers.
// Nothing here is a dense contraction; the kernels are bound by HBM traffic
// (read x, write y forward; read x and dy, write dx backward).
//
// Backward.  dx needs two row sums ([NormPage] "LayerNorm" section:
// mean_j(g) and mean_j(g * xhat)); RMSNorm needs only the second
// ([NormPage] "RMSNorm" section).  The weight/bias gradients are column sums
// over rows: each thread accumulates its own columns over the rows its block
// visits, the row slots of a block are combined in LDS, and each block
// writes one partial row to the workspace ([NormPage] "Engineering tricks":
// per-row-block partials followed by a sum).  A second kernel adds the
// partial rows in a fixed order (float64), so dw/db are reproducible.
#pragma once

#include "row_common.hpp"

namespace mi355norm {

constexpr int kMaxWavesPerBlock = 16;


template <typename VT> __device__ __forceinline__ typename VT::raw_t ones_raw() {
    float f[VT::n];
#pragma unroll
    for (int e = 0; e < VT::n; ++e) f[e] = 1.0f;
    return VT::pack(f);
}
template <typename VT> __device__ __forceinline__ typename VT::raw_t zeros_raw() {
    float f[VT::n];
#pragma unroll
    for (int e = 0; e < VT::n; ++e) f[e] = 0.0f;
    return VT::pack(f);
}

// Sum of `v` over the threads of one row group.  `slot` alternates between
// two LDS areas so that back-to-back reductions need one barrier each.
__device__ __forceinline__ float row_sum(float v, int tpr, float (*lds)[kMaxWavesPerBlock], int slot) {
    v = seg_sum(v, tpr < kWave ? tpr : kWave);
    if (tpr > kWave) {  // block-uniform: the row spans tpr/64 waves
        const int wave = threadIdx.x / kWave;
        if ((threadIdx.x & (kWave - 1)) == 0) lds[slot][wave] = v;
        __syncthreads();
        const int wpr = tpr / kWave;
        const int first = (wave / wpr) * wpr;
        float s = 0.0f;
        for (int i = 0; i < wpr; ++i) s += lds[slot][first + i];
        v = s;
    }
    return v;
}

__device__ __forceinline__ void row_sum2(float &a, float &b, int tpr, float (*lds)[kMaxWavesPerBlock][2], int slot) {
    seg_sum2(a, b, tpr < kWave ? tpr : kWave);
    if (tpr > kWave) {
        const int wave = threadIdx.x / kWave;
        if ((threadIdx.x & (kWave - 1)) == 0) {
            lds[slot][wave][0] = a;
            lds[slot][wave][1] = b;
        }
        __syncthreads();
        const int wpr = tpr / kWave;
        const int first = (wave / wpr) * wpr;
        float sa = 0.0f, sb = 0.0f;
        for (int i = 0; i < wpr; ++i) {
            sa += lds[slot][first + i][0];
            sb += lds[slot][first + i][1];
        }
        a = sa;
        b = sb;
    }
}

// The row is kept in registers in its packed I/O form and unpacked again
// for each pass over it; `opaque` stops the compiler from keeping the first
// unpacked copy alive instead (float32 copies of a bf16 row double the
// register footprint and halve the number of waves a CU can hold).
template <typename R> __device__ __forceinline__ void opaque(R &r) { asm volatile("" : "+v"(r)); }

// ------------------------------------------------------------------ forward
// LayerNorm ([NormPage] "LayerNorm" section): mean, then the sum of squared
// deviations (exact two-pass over the register-resident row), rstd by rsqrt,
// y = (x - mean) * rstd * w + b.  RMSNorm ([NormPage] "RMSNorm" section):
// no mean; rstd from the mean of squares; y = x * rstd * w.
// ONE: the grid gives every block exactly one row group (the default
// plan); the kernel then neither loops nor holds a prefetched next row,
// which frees IT vectors of registers per thread for more waves per CU.
template <typename T, int V, int IT, bool RMS, int MAXB, bool ONE>
__global__ void __launch_bounds__(MAXB)
row_fwd_kernel(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ b,
               T *__restrict__ y, float *__restrict__ mean_out, float *__restrict__ rstd_out,
               int64_t M, int N, float inv_n, float eps, int tpr) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    __shared__ float lds[2][kMaxWavesPerBlock];

    const int nv = N / V;
    const int lane = threadIdx.x & (tpr - 1);
    const int rpb = blockDim.x / tpr;
    const int slot_in_block = threadIdx.x / tpr;

    // Row loop (one pass per block on the default, non-persistent grid; more
    // on a persistent grid).  The next row's loads are issued before this
    // row is reduced and stored.
    const int64_t step = (int64_t)gridDim.x * rpb;
    int64_t base = (int64_t)blockIdx.x * rpb;

    // x of the row group starting at row `gbase`, this thread's slots.  On
    // the 16-byte path a buffer resource spans the group's rows, so lanes
    // past the last row or past the row's end read zeros without a branch:
    // branches around the loads made the compiler wait for each load before
    // issuing the next.  The group spans at most 1024 x 8 x 8 elements, so
    // its byte offsets fit 32 bits.
    auto load_group = [&](raw_t *dst, int64_t gbase) {
        if constexpr (sizeof(raw_t) == 16) {
            const int64_t rows = gbase < M ? (M - gbase < rpb ? M - gbase : (int64_t)rpb) : 0;
            const auto rs = load_rsrc(rows ? x + gbase * N : x, (uint32_t)(rows * N * (int64_t)sizeof(T)));
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                const int v = lane + k * tpr;
                const uint32_t off =
                    v < nv ? (uint32_t)(((int64_t)slot_in_block * N + (int64_t)v * V) * (int64_t)sizeof(T)) : kOffNone;
                dst[k] = vload16_rsrc<2>(rs, off);
            }
        } else {
            const int64_t row = gbase + slot_in_block;
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                const int v = lane + k * tpr;
                dst[k] = zeros_raw<VT>();
                if (row < M && v < nv) dst[k] = vload_stream<T, V>(x + row * N + (int64_t)v * V);
            }
        }
    };
    raw_t xr[IT];
    load_group(xr, base);

    raw_t wr[IT], br[IT];
    if constexpr (sizeof(raw_t) == 16) {
        // A null w or b gets an empty range (its loads read zeros); a null w
        // then becomes all ones through the fill pattern, with no branch.
        const uint32_t pbytes = (uint32_t)(N * (int64_t)sizeof(T));
        const auto rw = load_rsrc(w, w ? pbytes : 0u);
        const auto rb = load_rsrc(b, b ? pbytes : 0u);
        const raw_t wfill = w ? zeros_raw<VT>() : ones_raw<VT>();
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int v = lane + k * tpr;
            const uint32_t off = v < nv ? (uint32_t)v * 16u : kOffNone;
            wr[k] = vload16_rsrc<0>(rw, off) | wfill;
            br[k] = zeros_raw<VT>();
            if constexpr (!RMS) br[k] = vload16_rsrc<0>(rb, off);
        }
    } else {
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int v = lane + k * tpr;
            wr[k] = ones_raw<VT>();
            br[k] = zeros_raw<VT>();
            if (v < nv) {
                if (w) wr[k] = vload<T, V>(w + (int64_t)v * V);
                if (!RMS && b) br[k] = vload<T, V>(b + (int64_t)v * V);
            }
        }
    }

    // LDS slot of the sum of squares.  A row spanning several waves reads
    // every wave's partial after one barrier; a fast wave may reach the next
    // row's write before a slow one has read this row's partials, so two
    // consecutive reductions never use the same slot: LayerNorm takes slot 0
    // (mean) then 1 (squares) in every row, RMSNorm alternates its single
    // reduction between the slots from row to row.
    int qslot = 1;
    for (; base < M; base += step) {
        const int64_t row = base + slot_in_block;
        const bool active = row < M;
        raw_t nx[IT];
        if constexpr (!ONE) load_group(nx, base + step);
#pragma unroll
        for (int k = 0; k < IT; ++k) {  // keep w, b packed (no hoisted float copies)
            opaque(wr[k]);
            if (!RMS) opaque(br[k]);
        }

        float mean = 0.0f;
        if (!RMS) {
            // Float32 I/O sums the row relative to its first element, so a
            // row far from zero relative to its spread keeps its mean's
            // precision (16-bit inputs cannot resolve such a row).
            float x0 = 0.0f;
            if constexpr (sizeof(T) == 4) {
                if (active) x0 = ld1(x + row * N);
            }
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                float f[V];
                VT::unpack(xr[k], f);
                if constexpr (sizeof(T) == 4) {
                    const bool valid = lane + k * tpr < nv;  // out-of-range slots hold 0, not x0
#pragma unroll
                    for (int e = 0; e < V; ++e) s += valid ? f[e] - x0 : 0.0f;
                } else {
#pragma unroll
                    for (int e = 0; e < V; ++e) s += f[e];
                }
            }
            if constexpr (sizeof(T) == 4)
                mean = x0 + row_sum(s, tpr, lds, 0) * inv_n;
            else
                mean = row_sum(s, tpr, lds, 0) * inv_n;
#pragma unroll
            for (int k = 0; k < IT; ++k) opaque(xr[k]);
        }
        // Slots past the row's end hold zeros: they add nothing for RMSNorm
        // but mean^2 for LayerNorm, so LayerNorm masks them, only in a slice
        // k that reaches past the row's end (a uniform test: full slices
        // skip the per-element select).
        float q = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            float f[V];
            VT::unpack(xr[k], f);
            if (RMS || (k + 1) * tpr <= nv) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = f[e] - mean;
                    q += d * d;
                }
            } else {
                const bool valid = lane + k * tpr < nv;
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = f[e] - mean;
                    q += valid ? d * d : 0.0f;
                }
            }
        }
        const float rstd = rsqrtf(row_sum(q, tpr, lds, qslot) * inv_n + eps);
        if (RMS) qslot ^= 1;
#pragma unroll
        for (int k = 0; k < IT; ++k) opaque(xr[k]);

        if (active) {
            T *ygrp = y + base * N;  // the block's row group: the same in every lane
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                const int v = lane + k * tpr;
                if (v < nv) {
                    float f[V], wf[V], bf[V], o[V];
                    VT::unpack(xr[k], f);
                    VT::unpack(wr[k], wf);
                    VT::unpack(br[k], bf);
#pragma unroll
                    for (int e = 0; e < V; ++e) o[e] = (f[e] - mean) * rstd * wf[e] + bf[e];
                    vstore_out<T, V>(ygrp, (uint32_t)(slot_in_block * N + v * V), VT::pack(o));
                }
            }
            if (lane == 0) {
                if (!RMS && mean_out) mean_out[row] = mean;
                if (rstd_out) rstd_out[row] = rstd;
            }
        }
        if constexpr (ONE) break;
#pragma unroll
        for (int k = 0; k < IT; ++k) xr[k] = nx[k];
    }
}

// ----------------------------------------------------------------- backward
// With g = dy * w and xhat = (x - mean) * rstd (RMSNorm: xhat = x * rstd):
//   LayerNorm  dx = rstd * (g - mean_j(g) - xhat * mean_j(g * xhat))
//   RMSNorm    dx = rstd * (g - xhat * mean_j(g * xhat))
// (for RMSNorm, x * rstd^2 * mean_j(g * x) = xhat * mean_j(g * xhat)).
// Column partials: dw += dy * xhat, db += dy, per thread, then per block:
// one float32 partial row per block into part_w / part_b, or, when the grid
// is a single block, the final dw / db straight into dw_out / db_out (the
// block's partial row is then the whole sum; no second kernel).
template <typename T, int V, int IT, bool RMS, int MAXB>
__global__ void __launch_bounds__(MAXB)
row_bwd_kernel(const T *__restrict__ dy, const T *__restrict__ x, const T *__restrict__ w,
               const float *__restrict__ mean_in, const float *__restrict__ rstd_in,
               T *__restrict__ dx, float *__restrict__ part_w, float *__restrict__ part_b,
               T *__restrict__ dw_out, T *__restrict__ db_out, int64_t M, int N, float inv_n, int tpr) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    __shared__ float lds[2][kMaxWavesPerBlock][2];
    __shared__ float lds_c[2][kMaxWavesPerBlock];  // float32 LayerNorm: the mean correction

    const int nv = N / V;
    const int lane = threadIdx.x & (tpr - 1);
    const int rpb = blockDim.x / tpr;
    const int slot_in_block = threadIdx.x / tpr;
    const bool full_rows = nv == tpr * IT;  // every thread's IT vectors lie inside the row

    raw_t wr[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int v = lane + k * tpr;
        wr[k] = ones_raw<VT>();
        if (w && v < nv) wr[k] = vload<T, V>(w + (int64_t)v * V);
    }

    float acc_w[IT][V], acc_b[IT][V];
#pragma unroll
    for (int k = 0; k < IT; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) acc_w[k][e] = acc_b[k][e] = 0.0f;

    // The next row's x, dy and statistics are issued before this row is
    // reduced and written.  The loads sit under bounds branches, so the
    // compiler waits for all outstanding loads before the first pass: in
    // effect one row's reads are in flight per wave at a time.  Unconditional
    // (clamped) loads that keep the next row in flight through the passes
    // measured slower on the RMSNorm 16384 x 4096 backward: more reads in
    // flight per CU lower this two-read, one-write pass's bandwidth.
    int slot = 0, slot_c = 0;
    const int64_t step = (int64_t)gridDim.x * rpb;
    int64_t base = (int64_t)blockIdx.x * rpb;
    raw_t rx[IT], rd[IT];
    float mean = 0.0f, rstd = 0.0f;
    {
        const int64_t row = base + slot_in_block;
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int v = lane + k * tpr;
            rx[k] = zeros_raw<VT>();
            rd[k] = zeros_raw<VT>();
            if (row < M && v < nv) {
                rx[k] = vload_stream<T, V>(x + row * N + (int64_t)v * V);
                rd[k] = vload_stream<T, V>(dy + row * N + (int64_t)v * V);
            }
        }
        if (row < M) {
            if (!RMS) mean = mean_in[row];
            rstd = rstd_in[row];
        }
    }
    for (; base < M; base += step) {
        const int64_t row = base + slot_in_block;
        const bool active = row < M;
        const int64_t nrow = row + step;
        raw_t nx[IT], nd[IT];
        float nmean = 0.0f, nrstd = 0.0f;
        if (full_rows && base + step + rpb <= M) {  // block-uniform: every slot's next row is in range
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                const int v = lane + k * tpr;
                nx[k] = vload_stream<T, V>(x + nrow * N + (int64_t)v * V);
                nd[k] = vload_stream<T, V>(dy + nrow * N + (int64_t)v * V);
            }
        } else {
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                const int v = lane + k * tpr;
                nx[k] = zeros_raw<VT>();
                nd[k] = zeros_raw<VT>();
                if (nrow < M && v < nv) {
                    nx[k] = vload_stream<T, V>(x + nrow * N + (int64_t)v * V);
                    nd[k] = vload_stream<T, V>(dy + nrow * N + (int64_t)v * V);
                }
            }
        }
        if (nrow < M) {
            if (!RMS) nmean = mean_in[nrow];
            nrstd = rstd_in[nrow];
        }
#pragma unroll
        for (int k = 0; k < IT; ++k) opaque(wr[k]);  // keep w packed (no hoisted float copy)

        // Float32 LayerNorm: the saved mean is the float32 rounding of the
        // row mean, an error shared by every element of the row that would
        // add coherently into dw.  One more row sum, of x - mean, gives the
        // exact mean as mean + corr (kept in two parts: x - mean is exact for
        // x near the mean, corr is small), as the BatchNorm backward does
        // with its channel sums.  16-bit I/O: corr = 0.
        float corr = 0.0f;
        if constexpr (sizeof(T) == 4 && !RMS) {
            float sc = 0.0f;
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                const bool valid = lane + k * tpr < nv;
                float xf[V];
                VT::unpack(rx[k], xf);
#pragma unroll
                for (int e = 0; e < V; ++e) sc += valid ? xf[e] - mean : 0.0f;
            }
            corr = row_sum(sc, tpr, lds_c, slot_c) * inv_n;
            slot_c ^= 1;
#pragma unroll
            for (int k = 0; k < IT; ++k) opaque(rx[k]);
        }

        // Pass 1: the row sums and the column partials.  Out-of-range
        // elements hold x = dy = 0 and add nothing (their g is 0).  g is
        // kept in float32 for pass 2, which then needs neither dy nor w.
        float s_gx = 0.0f, s_g = 0.0f;
        float gr[IT][V];
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            float xf[V], df[V], wf[V];
            VT::unpack(rx[k], xf);
            VT::unpack(rd[k], df);
            VT::unpack(wr[k], wf);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float xc = RMS ? xf[e] : xf[e] - mean;
                if constexpr (sizeof(T) == 4 && !RMS) xc -= corr;
                const float xh = xc * rstd;
                acc_w[k][e] = fmaf(df[e], xh, acc_w[k][e]);
                if (!RMS) acc_b[k][e] += df[e];
                const float g = df[e] * wf[e];
                gr[k][e] = g;
                s_gx = fmaf(g, xh, s_gx);
                if (!RMS) s_g += g;
            }
        }
        row_sum2(s_gx, s_g, tpr, lds, slot);
        slot ^= 1;
        // dx = rstd * (g - c_g - xhat * c_gx) with xhat = (x - mean) * rstd,
        // evaluated as rstd * g + ((x - mean) * k1 + k0): two FMAs per
        // element after the centring subtraction (none for RMSNorm).
        const float c_gx = s_gx * inv_n, c_g = s_g * inv_n;
        const float k1 = -(rstd * rstd) * c_gx;
        float k0 = -rstd * c_g;
        if constexpr (sizeof(T) == 4 && !RMS) k0 = fmaf(-k1, corr, k0);  // (x - mean - corr) k1 + k0
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            opaque(rx[k]);
            opaque(wr[k]);
        }

        // Pass 2: dx from the packed x and the float32 g.
        if (active) {
            T *dxgrp = dx + base * N;  // the block's row group: the same in every lane
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                const int v = lane + k * tpr;
                if (v < nv) {
                    float xf[V], o[V];
                    VT::unpack(rx[k], xf);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const float lin = RMS ? xf[e] * k1 : fmaf(xf[e] - mean, k1, k0);
                        o[e] = fmaf(gr[k][e], rstd, lin);
                    }
                    vstore_out<T, V>(dxgrp, (uint32_t)(slot_in_block * N + v * V), VT::pack(o));
                }
            }
        }
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            rx[k] = nx[k];
            rd[k] = nd[k];
        }
        mean = nmean;
        rstd = nrstd;
    }

    // Combine the row slots of this block column by column and write one
    // partial row per block (dW, and dB when wanted); slots are added in
    // increasing order.  Partial rows go out through 16-byte device-scope
    // stores where the width allows.
    if (!part_w && !part_b && !dw_out && !db_out) return;
    if (rpb == 1) {  // one row slot: every thread owns distinct columns
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int v = lane + k * tpr;
            if (v >= nv) continue;
            const int64_t off = (int64_t)blockIdx.x * N + (int64_t)v * V;
            if constexpr (V % 4 == 0) {  // N is a multiple of V here: 16-byte stores
#pragma unroll
                for (int e = 0; e < V; e += 4) {
                    const uint32_t c = (uint32_t)(v * V + e);
                    if (part_w) vstore_out<float, 4>(part_w + (int64_t)blockIdx.x * N, c, Vec<float, 4>::pack(&acc_w[k][e]));
                    if (part_b) vstore_out<float, 4>(part_b + (int64_t)blockIdx.x * N, c, Vec<float, 4>::pack(&acc_b[k][e]));
                }
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const uint32_t c = (uint32_t)(v * V + e);
                    if (part_w) vstore_out<float, 1>(part_w + (int64_t)blockIdx.x * N, c, __float_as_uint(acc_w[k][e]));
                    if (part_b) vstore_out<float, 1>(part_b + (int64_t)blockIdx.x * N, c, __float_as_uint(acc_b[k][e]));
                }
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if (dw_out) st1(dw_out + (off + e), acc_w[k][e]);
                if (db_out) st1(db_out + (off + e), acc_b[k][e]);
            }
        }
        return;
    }
    // Several row slots: stage every slot's column partials in LDS as
    // [which][slot][column] (dW, then dB when wanted: one staging between
    // two barriers), then let all threads add over the slots (in slot order)
    // for their own columns and write the block's partial rows.
    extern __shared__ __align__(16) float colbuf[];  // (1 or 2) * rpb * N floats; 16-byte access below
    const bool want_b = part_b != nullptr || db_out != nullptr;
    __syncthreads();
    for (int which = 0; which < (want_b ? 2 : 1); ++which) {
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int v = lane + k * tpr;
            if (v < nv) {
                float *dst = colbuf + (which * rpb + slot_in_block) * N + v * V;
                if constexpr (V % 4 == 0) {  // N is a multiple of V here: 16-byte writes
#pragma unroll
                    for (int e = 0; e < V; e += 4) {
                        const float *a = which == 0 ? &acc_w[k][e] : &acc_b[k][e];
                        *reinterpret_cast<float4 *>(dst + e) = make_float4(a[0], a[1], a[2], a[3]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < V; ++e) dst[e] = which == 0 ? acc_w[k][e] : acc_b[k][e];
                }
            }
        }
    }
    __syncthreads();
    for (int which = 0; which < 2; ++which) {
        float *part = which == 0 ? part_w : part_b;
        T *out = which == 0 ? dw_out : db_out;
        if (part == nullptr && out == nullptr) continue;
        const float *src = colbuf + which * rpb * N;
        if (out == nullptr && (N & 3) == 0) {
            // Four columns per thread: 16-byte LDS reads and one 16-byte
            // device-scope store (as for dx) per four columns, so the partial
            // rows leave no dirty L2 lines for the write-back at the end of
            // the kernel.  Each column's slots are added in the same order.
            float *prow = part + (int64_t)blockIdx.x * N;
            for (int col = threadIdx.x * 4; col < N; col += blockDim.x * 4) {
                float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                for (int r = 0; r < rpb; ++r) {
                    const float4 q = *reinterpret_cast<const float4 *>(src + r * N + col);
                    sum[0] += q.x;
                    sum[1] += q.y;
                    sum[2] += q.z;
                    sum[3] += q.w;
                }
                vstore_out<float, 4>(prow, (uint32_t)col, Vec<float, 4>::pack(sum));
            }
            continue;
        }
        for (int col = threadIdx.x; col < N; col += blockDim.x) {
            float sum = 0.0f;
            for (int r = 0; r < rpb; ++r) sum += src[r * N + col];
            if (out)
                st1(out + col, sum);
            else
                vstore_out<float, 1>(part + (int64_t)blockIdx.x * N, (uint32_t)col, __float_as_uint(sum));
        }
    }
}

// Column sums of G partial rows (float64, fixed order) -> dw / db in T.
// blockDim = (16 columns, 16 row slices); grid = (ceil(N/16), 1 or 2).
// Each thread adds rows slice, slice+16, ... with eight loads in flight,
// then the 16 slices are added in order through LDS.
constexpr int kColsumCols = 16;
constexpr int kColsumSlices = 16;
template <typename T>
__global__ void __launch_bounds__(kColsumCols * kColsumSlices)
colsum_kernel(const float *__restrict__ part_w, const float *__restrict__ part_b, int G, int N,
              T *__restrict__ dw, T *__restrict__ db) {
    __shared__ double red[kColsumSlices][kColsumCols];
    const float *part = blockIdx.y == 0 ? part_w : part_b;
    T *out = blockIdx.y == 0 ? dw : db;
    if (part == nullptr || out == nullptr) return;  // uniform per block
    const int col = blockIdx.x * kColsumCols + threadIdx.x;
    double s = 0.0;
    if (col < N) {
        int g = threadIdx.y;
        for (; g + 7 * kColsumSlices < G; g += 8 * kColsumSlices) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(g + u * kColsumSlices) * N + col];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += (double)v[u];
        }
        for (; g < G; g += kColsumSlices) s += (double)part[(int64_t)g * N + col];
    }
    red[threadIdx.y][threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.y == 0 && col < N) {
        double t = 0.0;
        for (int i = 0; i < kColsumSlices; ++i) t += red[i][threadIdx.x];
        st1(out + col, (float)t);
    }
}

// Zero fill (used for parameter gradients of an empty batch; a kernel rather
// than a memset so the call stays safe under stream capture).
template <typename T>
__global__ void zero_fill_kernel(T *__restrict__ out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) st1(out + i, 0.0f);
}

// ------------------------------------------------------------- launchers
template <typename T, bool RMS, int V>
norm_status row_launch_fwd(const RowPlan &p, hipStream_t s, const void *x, const void *w, const void *b,
                           void *y, float *mean, float *rstd, int64_t M, int N, float eps) {
    using fn_t = void (*)(const T *, const T *, const T *, T *, float *, float *, int64_t, int,
                          float, float, int);
    fn_t fn = nullptr;
    const int64_t rpb = p.block / p.tpr;
    const bool one = (int64_t)p.grid * rpb >= M;  // every block one row group
#define MI355NORM_FWD(IT)                                                                              \
    (p.block > 256 ? (one ? row_fwd_kernel<T, V, IT, RMS, 1024, true> : row_fwd_kernel<T, V, IT, RMS, 1024, false>) \
                   : (one ? row_fwd_kernel<T, V, IT, RMS, 256, true> : row_fwd_kernel<T, V, IT, RMS, 256, false>))
    switch (p.it) {
    case 1: fn = MI355NORM_FWD(1); break;
    case 2: fn = MI355NORM_FWD(2); break;
    case 3: if constexpr (V > 1) fn = MI355NORM_FWD(3); break;
    case 4: fn = MI355NORM_FWD(4); break;
    case 6: if constexpr (V > 1) fn = MI355NORM_FWD(6); break;
    case 8: fn = MI355NORM_FWD(8); break;
    case 16: if constexpr (V == 1) fn = MI355NORM_FWD(16); break;
    case 32: if constexpr (V == 1) fn = MI355NORM_FWD(32); break;
    case 64: if constexpr (V == 1) fn = MI355NORM_FWD(64); break;
    }
#undef MI355NORM_FWD
    if (!fn) return NORM_ERR_SHAPE;
    launch(RMS ? "row_fwd_kernel<rms>" : "row_fwd_kernel<ln>", true, fn, dim3(p.grid), dim3(p.block), 0, s,
           (const T *)x, (const T *)w, (const T *)b, (T *)y, mean, rstd, M, N, 1.0f / (float)N, eps, p.tpr);
    return launch_status();
}

template <typename T, bool RMS, int V>
norm_status row_launch_bwd(const RowPlan &p, hipStream_t s, const void *dy, const void *x, const void *w,
                           const float *mean, const float *rstd, void *dx, float *part_w, float *part_b,
                           void *dw_out, void *db_out, int64_t M, int N) {
    using fn_t = void (*)(const T *, const T *, const T *, const float *, const float *, T *,
                          float *, float *, T *, T *, int64_t, int, float, int);
    fn_t fn = nullptr;
    switch (p.it) {
    case 1: fn = p.block > 256 ? row_bwd_kernel<T, V, 1, RMS, 1024> : row_bwd_kernel<T, V, 1, RMS, 256>; break;
    case 2: fn = p.block > 256 ? row_bwd_kernel<T, V, 2, RMS, 1024> : row_bwd_kernel<T, V, 2, RMS, 256>; break;
    case 3: if constexpr (V > 1) fn = p.block > 256 ? row_bwd_kernel<T, V, 3, RMS, 1024> : row_bwd_kernel<T, V, 3, RMS, 256>; break;
    case 4: fn = p.block > 256 ? row_bwd_kernel<T, V, 4, RMS, 1024> : row_bwd_kernel<T, V, 4, RMS, 256>; break;
    case 6: if constexpr (V > 1) fn = p.block > 256 ? row_bwd_kernel<T, V, 6, RMS, 1024> : row_bwd_kernel<T, V, 6, RMS, 256>; break;
    case 8: fn = p.block > 256 ? row_bwd_kernel<T, V, 8, RMS, 1024> : row_bwd_kernel<T, V, 8, RMS, 256>; break;
    case 16: if constexpr (V == 1) fn = p.block > 256 ? row_bwd_kernel<T, V, 16, RMS, 1024> : row_bwd_kernel<T, V, 16, RMS, 256>; break;
    case 32: if constexpr (V == 1) fn = p.block > 256 ? row_bwd_kernel<T, V, 32, RMS, 1024> : row_bwd_kernel<T, V, 32, RMS, 256>; break;
    case 64: if constexpr (V == 1) fn = p.block > 256 ? row_bwd_kernel<T, V, 64, RMS, 1024> : row_bwd_kernel<T, V, 64, RMS, 256>; break;
    }
    if (!fn) return NORM_ERR_SHAPE;
    const int rpb = p.block / p.tpr;
    const bool sums = part_w || part_b || dw_out || db_out;
    const size_t nstage = (part_b || db_out) ? 2 : 1;  // dW, and dB when wanted
    const size_t shmem = (sums && rpb > 1) ? nstage * rpb * N * sizeof(float) : 0;
    if (shmem > 65536) return NORM_ERR_SHAPE;  // only reachable through the tuning override
    launch(RMS ? "row_bwd_kernel<rms>" : "row_bwd_kernel<ln>", true, fn, dim3(p.grid), dim3(p.block), shmem, s,
           (const T *)dy, (const T *)x, (const T *)w, mean, rstd, (T *)dx, part_w, part_b, (T *)dw_out,
           (T *)db_out, M, N, 1.0f / (float)N, p.tpr);
    return launch_status();
}

template <typename T>
void row_launch_colsum(hipStream_t s, const float *part_w, const float *part_b, int parts, int N, void *dw,
                       void *db) {
    dim3 grid((unsigned)ceil_div(N, kColsumCols), part_b ? 2 : 1);
    dim3 block(kColsumCols, kColsumSlices);
    launch("colsum_kernel", false, colsum_kernel<T>, grid, block, 0, s, part_w, part_b, parts, N, (T *)dw,
           (T *)db);
}

template <typename T>
void row_launch_zero(hipStream_t s, void *out, int n) {
    const dim3 grid((unsigned)ceil_div(n, 256));
    launch("zero_fill_kernel", false, zero_fill_kernel<T>, grid, dim3(256), 0, s, (T *)out, n);
}

}  // namespace mi355norm
