// ad_kernels.hpp -- fused activation + dropout, element-wise, for gfx950.
//
// Page (by title):
//   [ActPage] "Operator fusion in practice: attorch's activation and
//             dropout fusion kernels" -- sections 3-5 (one load and one
//             store per element, the activation and inverted dropout applied
//             in registers; the mask a function of (seed, element offset)
//             recomputed in the backward instead of stored) and 6 (one
//             kernel per activation, the rest pruned at compile time).
//
// Mask.  Element e (the caller's offset, a multiple of 8, plus the flat
// index) takes 16 bits of Philox4x32-10 (Salmon et al., SC 2011) under key
// (seed low, seed high) and counter (e / 8 low, e / 8 high, 0, 0): word
// (e mod 8) / 2, its low half for even e, its high half for odd e.  One
// generator call serves eight consecutive elements, one 16-bit vector (a
// float32 vector uses half a call).  The element is dropped when its 16
// bits are below thresh (thresh / 2^16 is the drop probability); survivors
// are scaled by 1 / (1 - p).
//
// Both directions are bound by HBM traffic (2 tensors forward, 3 backward);
// the ten Philox rounds are 20 64-bit multiplies and 20 three-input XORs
// per call, so taking 16 bits per element (one call per 16-bit vector, not
// two) is what keeps the 16-bit GELU forward near the HBM rate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "norm_device.hpp"
#include "norm_host.hpp"

namespace mi355norm {

constexpr int kAdBlock = 256;
// Vectors per thread and pass, as measured on the bf16 GELU 16384 x 4096
// workload: the forward (VALU-heavy with the generator) runs best with one
// (48.5 -> 46.9 us against four), the backward with two (63.7 -> 58.5 us):
// more threads in flight, each with fewer loads, hide the per-element
// arithmetic better than more loads per thread.
constexpr int kAdUnrollFwd = 1;
constexpr int kAdUnrollBwd = 2;

struct AdArgs {
    int64_t n;           // elements
    uint32_t k0, k1;     // Philox key (seed)
    uint64_t blk0;       // offset / 8: the counter of element 0's group
    uint32_t thresh;     // drop when the element's 16 bits are below thresh
    float scale;         // 1 / (1 - p)
    int act_rt;          // activation for the run-time dispatched instance
    float act_p;         // its parameter
};

// a ^ b ^ c as one v_bitop3_b32: 0x96 is the truth table of the three
// inputs' parity (the compiler leaves a chain of two-input XORs unfused).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32-10 on counter (c0, c1, 0, 0): ten rounds of the published
// round function, the key bumped by the Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1,
                                              uint32_t w[4]) {
    uint32_t c2 = 0u, c3 = 0u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // One 32 x 32 -> 64-bit product per multiplier (v_mad_u64_u32)
        // instead of separate high and low multiplies.
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = xor3(hi1, c1, k0);
        const uint32_t n2 = xor3(hi0, c3, k1);
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    w[0] = c0;
    w[1] = c1;
    w[2] = c2;
    w[3] = c3;
}

// The 16 bits of word w that element parity `odd` takes.
__device__ __forceinline__ uint32_t half16(uint32_t w, bool odd) { return odd ? (w >> 16) : (w & 0xffffu); }

// Keep flags of the V elements of vector vi (V = 8 or 4), or of element vi
// for V = 1.
template <int V>
__device__ __forceinline__ void keep_flags(const AdArgs &a, int64_t vi, bool keep[V]) {
    uint32_t w[4];
    if constexpr (V == 8) {  // elements 8 vi .. 8 vi + 7: one whole call
        const uint64_t blk = a.blk0 + (uint64_t)vi;
        philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), a.k0, a.k1, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) keep[e] = half16(w[e >> 1], e & 1) >= a.thresh;
    } else if constexpr (V == 4) {  // elements 4 vi .. 4 vi + 3: words 0-1 or 2-3
        const uint64_t blk = a.blk0 + (uint64_t)(vi >> 1);
        philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), a.k0, a.k1, w);
        const bool upper = vi & 1;
        const uint32_t wa = upper ? w[2] : w[0], wb = upper ? w[3] : w[1];
        keep[0] = half16(wa, false) >= a.thresh;
        keep[1] = half16(wa, true) >= a.thresh;
        keep[2] = half16(wb, false) >= a.thresh;
        keep[3] = half16(wb, true) >= a.thresh;
    } else {  // element vi
        const uint64_t blk = a.blk0 + (uint64_t)(vi >> 3);
        philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), a.k0, a.k1, w);
        const int q = (int)(vi & 7) >> 1;
        const uint32_t word = q == 0 ? w[0] : q == 1 ? w[1] : q == 2 ? w[2] : w[3];
        keep[0] = half16(word, vi & 1) >= a.thresh;
    }
}

// Forward over vectors v0, v0 + stride, ... below nvec, kAdUnrollFwd loads in
// flight (vector v holds elements v * V .. v * V + V - 1).  DROP = false is
// the plain activation (p = 0: no generator calls).  `ub` is a vector index
// at or below v0 that is the same in every lane (the range's first vector);
// outputs are stored relative to it.
template <typename T, int V, int ACT, bool DROP>
__device__ __forceinline__ void ad_fwd_range(const T *__restrict__ x, T *__restrict__ y, int64_t nvec,
                                             int64_t v0, int64_t stride, int64_t ub, const AdArgs &a) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    for (int64_t vb = v0; vb < nvec; vb += stride * kAdUnrollFwd) {
        raw_t r[kAdUnrollFwd];
#pragma unroll
        for (int u = 0; u < kAdUnrollFwd; ++u) {
            const int64_t v = vb + u * stride;
            if (v < nvec) r[u] = vload_stream<T, V>(x + v * V);
        }
#pragma unroll
        for (int u = 0; u < kAdUnrollFwd; ++u) {
            const int64_t v = vb + u * stride;
            if (v < nvec) {
                float f[V], o[V];
                VT::unpack(r[u], f);
                bool keep[V];
                if (DROP) keep_flags<V>(a, v, keep);
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float t = act_fwd_io<T, ACT>(f[e], a.act_rt, a.act_p);
                    o[e] = DROP ? (keep[e] ? t * a.scale : 0.0f) : t;
                }
                vstore_out<T, V>(y + ub * V, (uint32_t)((v - ub) * V), VT::pack(o));
            }
        }
    }
}

template <typename T, int V, int ACT, bool DROP>
__device__ __forceinline__ void ad_bwd_range(const T *__restrict__ dy, const T *__restrict__ x,
                                             T *__restrict__ dx, int64_t nvec, int64_t v0, int64_t stride,
                                             int64_t ub, const AdArgs &a) {
    using VT = Vec<T, V>;
    using raw_t = typename VT::raw_t;
    constexpr bool kFast = sizeof(T) == 2;
    for (int64_t vb = v0; vb < nvec; vb += stride * kAdUnrollBwd) {
        raw_t rd[kAdUnrollBwd], rx[kAdUnrollBwd];
#pragma unroll
        for (int u = 0; u < kAdUnrollBwd; ++u) {
            const int64_t v = vb + u * stride;
            if (v < nvec) {
                rd[u] = vload_stream<T, V>(dy + v * V);
                rx[u] = vload_stream<T, V>(x + v * V);
            }
        }
#pragma unroll
        for (int u = 0; u < kAdUnrollBwd; ++u) {
            const int64_t v = vb + u * stride;
            if (v < nvec) {
                float df[V], xf[V], o[V];
                VT::unpack(rd[u], df);
                VT::unpack(rx[u], xf);
                bool keep[V];
                if (DROP) keep_flags<V>(a, v, keep);
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float g = df[e] * act_grad_any<ACT, kFast>(xf[e], a.act_rt, a.act_p);
                    o[e] = DROP ? (keep[e] ? g * a.scale : 0.0f) : g;
                }
                vstore_out<T, V>(dx + ub * V, (uint32_t)((v - ub) * V), VT::pack(o));
            }
        }
    }
}

// One launch covers the n / V full vectors (V-wide path) and the n mod V
// tail elements (scalar, by the first threads of the grid).
template <typename T, int V, int ACT, bool DROP>
__global__ void __launch_bounds__(kAdBlock)
act_dropout_fwd_kernel(const T *__restrict__ x, T *__restrict__ y, AdArgs a) {
    const int64_t nvec = a.n / V;
    const int64_t t0 = (int64_t)blockIdx.x * kAdBlock * kAdUnrollFwd + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kAdBlock * kAdUnrollFwd;
    // Each block covers kAdUnrollFwd * kAdBlock consecutive vectors per pass.
    for (int64_t base = (int64_t)blockIdx.x * kAdBlock * kAdUnrollFwd; base < nvec; base += stride)
        ad_fwd_range<T, V, ACT, DROP>(x, y, base + kAdBlock * kAdUnrollFwd < nvec ? base + kAdBlock * kAdUnrollFwd : nvec,
                                      base + threadIdx.x, kAdBlock, base, a);
    if (V > 1) {
        const int64_t tail = a.n - nvec * V;
        if (t0 < tail) {
            const int64_t i = nvec * V + t0;
            ad_fwd_range<T, 1, ACT, DROP>(x, y, i + 1, i, 1, nvec * V, a);
        }
    }
}

template <typename T, int V, int ACT, bool DROP>
__global__ void __launch_bounds__(kAdBlock)
act_dropout_bwd_kernel(const T *__restrict__ dy, const T *__restrict__ x, T *__restrict__ dx, AdArgs a) {
    const int64_t nvec = a.n / V;
    const int64_t t0 = (int64_t)blockIdx.x * kAdBlock * kAdUnrollBwd + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kAdBlock * kAdUnrollBwd;
    for (int64_t base = (int64_t)blockIdx.x * kAdBlock * kAdUnrollBwd; base < nvec; base += stride)
        ad_bwd_range<T, V, ACT, DROP>(dy, x, dx, base + kAdBlock * kAdUnrollBwd < nvec ? base + kAdBlock * kAdUnrollBwd : nvec,
                                      base + threadIdx.x, kAdBlock, base, a);
    if (V > 1) {
        const int64_t tail = a.n - nvec * V;
        if (t0 < tail) {
            const int64_t i = nvec * V + t0;
            ad_bwd_range<T, 1, ACT, DROP>(dy, x, dx, i + 1, i, 1, nvec * V, a);
        }
    }
}

// Launchers (instantiated per dtype in ad_inst.hip).
template <typename T, int V> norm_status ad_launch_fwd(const AdArgs &a, const void *x, void *y, hipStream_t s);
template <typename T, int V>
norm_status ad_launch_bwd(const AdArgs &a, const void *dy, const void *x, void *dx, hipStream_t s);

}  // namespace mi355norm
