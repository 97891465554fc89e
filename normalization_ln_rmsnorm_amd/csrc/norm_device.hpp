// norm_device.hpp -- device-side building blocks for the gfx950 kernels:
// element I/O (float32 / bf16 / fp16, 128-bit vectors), wave64 reductions (DPP,
// ds_swizzle, readlane), and the activation functions.
//
// [ActPage] = "Operator fusion in practice: attorch's activation and dropout
// fusion kernels".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mi355norm {

constexpr int kWave = 64;

// ----------------------------------------------------------------- dtypes
// bf16 is carried as its 16-bit pattern.  Widening is exact (the pattern is
// the top half of a float32); narrowing uses gfx950's v_cvt_pk_bf16_f32,
// which rounds to nearest-even.
struct bf16_t {
    uint16_t bits;
};

// fp16 (IEEE binary16) likewise travels as its bit pattern; widening is exact
// and narrowing rounds to nearest-even (the hardware conversion in the
// default rounding mode).
struct f16_t {
    uint16_t bits;
};

typedef __bf16 hw_bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 hw_f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float hw_f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    hw_f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hw_bf16x2));
}

__device__ __forceinline__ void unpack_f16x2(uint32_t u, float *f) {
    const hw_f32x2 v = __builtin_convertvector(__builtin_bit_cast(hw_f16x2, u), hw_f32x2);
    f[0] = v.x;
    f[1] = v.y;
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    hw_f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hw_f16x2));
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Vec<T, V>: V consecutive elements of type T moved by one load/store
// instruction, unpacked into V floats.  V * sizeof(T) is 16 bytes on the
// vector path and sizeof(T) on the scalar path.
template <typename T, int V> struct Vec;

template <> struct Vec<float, 4> {
    static constexpr int n = 4;
    using raw_t = u32x4;
    __device__ __forceinline__ static void unpack(const raw_t &r, float *f) {
        f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
    __device__ __forceinline__ static raw_t pack(const float *f) {
        return raw_t{__float_as_uint(f[0]), __float_as_uint(f[1]),
                     __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
};

template <> struct Vec<float, 1> {
    static constexpr int n = 1;
    using raw_t = uint32_t;
    __device__ __forceinline__ static void unpack(const raw_t &r, float *f) { f[0] = __uint_as_float(r); }
    __device__ __forceinline__ static raw_t pack(const float *f) { return __float_as_uint(f[0]); }
};

template <> struct Vec<bf16_t, 8> {
    static constexpr int n = 8;
    using raw_t = u32x4;
    __device__ __forceinline__ static void unpack(const raw_t &r, float *f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
    __device__ __forceinline__ static raw_t pack(const float *f) {
        return raw_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                     pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
    }
};

template <> struct Vec<bf16_t, 1> {
    static constexpr int n = 1;
    using raw_t = uint16_t;
    __device__ __forceinline__ static void unpack(const raw_t &r, float *f) {
        f[0] = __uint_as_float(uint32_t(r) << 16);
    }
    __device__ __forceinline__ static raw_t pack(const float *f) {
        return raw_t(pack_bf16x2(f[0], 0.0f) & 0xffffu);
    }
};

template <> struct Vec<f16_t, 8> {
    static constexpr int n = 8;
    using raw_t = u32x4;
    __device__ __forceinline__ static void unpack(const raw_t &r, float *f) {
        unpack_f16x2(r.x, f); unpack_f16x2(r.y, f + 2);
        unpack_f16x2(r.z, f + 4); unpack_f16x2(r.w, f + 6);
    }
    __device__ __forceinline__ static raw_t pack(const float *f) {
        return raw_t{pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]),
                     pack_f16x2(f[4], f[5]), pack_f16x2(f[6], f[7])};
    }
};

template <> struct Vec<f16_t, 1> {
    static constexpr int n = 1;
    using raw_t = uint16_t;
    __device__ __forceinline__ static void unpack(const raw_t &r, float *f) { f[0] = f16_to_f32(r); }
    __device__ __forceinline__ static raw_t pack(const float *f) {
        return raw_t(pack_f16x2(f[0], 0.0f) & 0xffffu);
    }
};

// Vector loads and stores.  `p` points at element 0 of the vector.
template <typename T, int V>
__device__ __forceinline__ typename Vec<T, V>::raw_t vload(const T *p) {
    return *reinterpret_cast<const typename Vec<T, V>::raw_t *>(p);
}
template <typename T, int V>
__device__ __forceinline__ void vstore(T *p, const typename Vec<T, V>::raw_t &r) {
    *reinterpret_cast<typename Vec<T, V>::raw_t *>(p) = r;
}
// Streaming loads: the data is read once, so mark it non-temporal.
template <typename T, int V>
__device__ __forceinline__ typename Vec<T, V>::raw_t vload_stream(const T *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const typename Vec<T, V>::raw_t *>(p));
}
// Non-temporal streaming store: the fallback where an output region is
// 4 GiB or more (vstore_out below needs 32-bit offsets from its base).
template <typename T, int V>
__device__ __forceinline__ void vstore_stream(T *p, const typename Vec<T, V>::raw_t &r) {
    __builtin_nontemporal_store(r, reinterpret_cast<typename Vec<T, V>::raw_t *>(p));
}
// Streaming stores.  On gfx950, stores tagged with device scope (sc1) and no
// non-temporal hint stream faster than non-temporal ones (RMSNorm 16384 x
// 4096 bf16 backward: 64.0 vs 70.6 us for the same kernel, loads unchanged).
// A global store cannot carry that tag from C++, so the store goes through a
// raw buffer resource over `base`.  `base` must be the same in every lane of
// the wave (it is then held in scalar registers; otherwise the compiler
// serialises the store over the distinct values), and `idx` is the lane's
// element offset from it, below 2^32 bytes.
constexpr int kStoreCachePolicy = 0x10;  // sc1 = 1, sc0 = 0, nt = 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)0xffffffffu, 0x00020000);
}
template <typename T, int V>
__device__ __forceinline__ void vstore_out(T *base, uint32_t idx, const typename Vec<T, V>::raw_t &r) {
    const int off = (int)(idx * (uint32_t)sizeof(T));
    using raw_t = typename Vec<T, V>::raw_t;
    if constexpr (sizeof(raw_t) == 16)
        __builtin_amdgcn_raw_buffer_store_b128(r, store_rsrc(base), off, 0, kStoreCachePolicy);
    else if constexpr (sizeof(raw_t) == 4)
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)r, store_rsrc(base), off, 0, kStoreCachePolicy);
    else
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)r, store_rsrc(base), off, 0, kStoreCachePolicy);
}

// Range-checked 16-byte loads through a raw buffer resource of `bytes`
// bytes over `base` (the same in every lane): a lane whose byte offset lies
// outside the range reads zeros, so bounds need no branch per load.  Lanes
// that must read zeros pass kOffNone, far past any range used here.
constexpr uint32_t kOffNone = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t load_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
// POLICY: 0 for data read again (w, b), 2 (non-temporal) for streams.
template <int POLICY>
__device__ __forceinline__ u32x4 vload16_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY);
}

// Scalar parameter load (w, b, statistics) widened to float.
__device__ __forceinline__ float ld1(const float *p) { return *p; }
__device__ __forceinline__ float ld1(const bf16_t *p) { return __uint_as_float(uint32_t(p->bits) << 16); }
__device__ __forceinline__ void st1(float *p, float v) { *p = v; }
__device__ __forceinline__ void st1(bf16_t *p, float v) { p->bits = uint16_t(pack_bf16x2(v, 0.0f) & 0xffffu); }
__device__ __forceinline__ float ld1(const f16_t *p) { return f16_to_f32(p->bits); }
__device__ __forceinline__ void st1(f16_t *p, float v) { p->bits = uint16_t(pack_f16x2(v, 0.0f) & 0xffffu); }

// ------------------------------------------------------- wave reductions
// DPP control codes (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;       // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float swz_xor16(float v) {
    // ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask 0x10.
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float lane_read(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of `seg` lanes (seg a power of two, 1..64); every
// lane of a group receives the group's sum.  All 64 lanes must be active.
// The combining order depends only on lane positions, so results are
// reproducible.  `seg` is wave-uniform, so its tests are scalar branches.
__device__ __forceinline__ float seg_sum(float v, int seg) {
    if (seg > 1) v += dpp<kDppXor1>(v);
    if (seg > 2) v += dpp<kDppXor2>(v);
    if (seg > 4) v += dpp<kDppHalfMirror>(v);
    if (seg > 8) v += dpp<kDppMirror>(v);
    if (seg > 16) v += swz_xor16(v);
    if (seg > 32) v = lane_read(v, 0) + lane_read(v, 32);
    return v;
}

// Full-wave float64 sum with the same lane pattern (each 64-bit value moves
// as its two 32-bit halves); every lane receives the sum.  All 64 lanes must
// be active.
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double swz_xor16_d(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)u, 0x401F);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)(u >> 32), 0x401F);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double lane_read_d(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_dpp_d(double v) {
    v += dpp_d<kDppXor1>(v);
    v += dpp_d<kDppXor2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    v += dpp_d<kDppMirror>(v);
    v += swz_xor16_d(v);
    return lane_read_d(v, 0) + lane_read_d(v, 32);
}

// Two sums at once (keeps the dependency chains interleaved).
__device__ __forceinline__ void seg_sum2(float &a, float &b, int seg) {
    if (seg > 1) { a += dpp<kDppXor1>(a); b += dpp<kDppXor1>(b); }
    if (seg > 2) { a += dpp<kDppXor2>(a); b += dpp<kDppXor2>(b); }
    if (seg > 4) { a += dpp<kDppHalfMirror>(a); b += dpp<kDppHalfMirror>(b); }
    if (seg > 8) { a += dpp<kDppMirror>(a); b += dpp<kDppMirror>(b); }
    if (seg > 16) { a += swz_xor16(a); b += swz_xor16(b); }
    if (seg > 32) {
        a = lane_read(a, 0) + lane_read(a, 32);
        b = lane_read(b, 0) + lane_read(b, 32);
    }
}

// Lane exchange of doubles through ds_bpermute, for the float64 Welford
// wave merges (each step merges with the lane `mask` away).
__device__ __forceinline__ double shfl_xor_d(double v, int mask) {
    return __shfl_xor(v, mask, kWave);
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_d(v, m);
    return v;
}

// Workgroups are dispatched to the chip's 8 XCDs round-robin by linear
// index, and each XCD has its own L2.  xcd_swizzle maps dispatch index b to
// a logical index such that consecutive logical indices run on the same XCD:
// XCD x takes a contiguous range of them.  A bijection on [0, G) for any G
// (the first G mod 8 XCDs take one more).
constexpr unsigned kXcds = 8;
__device__ __forceinline__ unsigned xcd_swizzle(unsigned b, unsigned G) {
    const unsigned q = G / kXcds, r = G % kXcds;
    const unsigned x = b % kXcds, j = b / kXcds;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

// ------------------------------------------------------------ activations
// ReLU and the exact error-function GELU ([ActPage] sections 5-6), computed
// in float32.  GELU(z) = z * Phi(z), Phi(z) = (1 + erf(z / sqrt 2)) / 2;
// GELU'(z) = Phi(z) + z * phi(z), phi(z) = exp(-z^2 / 2) / sqrt(2 pi).
//
// Two evaluations of Phi:
//  * accurate (FAST = false): the device erff and expf, for float32 I/O,
//    whose 1e-5 tolerance on channel sums over millions of values leaves no
//    room for a systematic per-element error;
//  * fast (FAST = true), for bf16 I/O, where the BatchNorm GELU backward is
//    otherwise bound by VALU time: Abramowitz & Stegun, Handbook of
//    Mathematical Functions, eq. 7.1.26 (Hastings' approximation),
//    erfc(u) ~= t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-u^2),
//    t = 1 / (1 + p u), u >= 0, with |error in erf| <= 1.5e-7.  With
//    u = |z| / sqrt 2 the exp(-u^2) is exp(-z^2 / 2), the same factor phi
//    needs, so Phi and phi share one exp; in float32 the result is within
//    3e-7 of Phi (and of GELU') everywhere -- far inside 2 bf16 ulp.
//    Divided by the sqrt(2 pi) / 2 that relates exp(-u^2) / 2 to phi, the
//    coefficients are A&S eq. 26.2.17's b1..b5 (Phi(-|z|) = phi(z) t B(t),
//    |error| < 7.5e-8).  This form serves the derivative, which needs both
//    Phi and phi; the forward uses the cheaper gelu_fast below.
enum Act : int {
    kActNone = 0, kActRelu = 1, kActGelu = 2, kActSigmoid = 3, kActTanh = 4, kActSilu = 5,
    kActMish = 6, kActLeakyRelu = 7, kActElu = 8, kActSelu = 9, kActCelu = 10,
    kActSoftplus = 11, kActRelu6 = 12, kActHardsigmoid = 13, kActHardswish = 14,
    kActCount = 15,
    kActGeneric = 255  // template tag: the activation is chosen at run time
};

constexpr float kInvSqrt2 = 0.70710678118654752440f;
constexpr float kInvSqrt2Pi = 0.39894228040143267794f;
constexpr float kNegHalfLog2e = -0.72134752044448170368f;  // -log2(e) / 2

// Accurate GELU'(z) = Phi(z) + z phi(z) from the device erff and expf.
__device__ __forceinline__ float gelu_grad_exact(float z) {
    return fmaf(z * kInvSqrt2Pi, expf(-0.5f * z * z), 0.5f * (1.0f + erff(z * kInvSqrt2)));
}

// Fast GELU'(z) (FAST = true).  With phi(z) = exp(-z^2 / 2) / sqrt(2 pi)
// and Phi(-|z|) = phi(z) t B(t) (B the 7.1.26 polynomial divided by
// sqrt(2 pi) / 2, i.e. the b1..b5 of A&S eq. 26.2.17; t = 1 / (1 + p |z|),
// p = 0.2316419): Phi(z) = H(z) - s phi(z) t B(t) with s = sign(z) and
// H = (1 + s) / 2 (1 for z >= 0, 0 below), so GELU'(z) = H + phi(z) (z -
// B(t) s t).  phi(z) is one exp2 whose argument carries log2(1 / sqrt(2 pi))
// (so z needs no scaling multiply).  The sign rides in the reciprocal:
// s t = 1 / (s + p z) (both terms carry the sign of z), and B takes
// |s t| = t through the operand's absolute-value modifier; s itself is one
// bit-select (copysign), H one FMA.  That replaces the compare and the two
// selects of the plain form.
constexpr float kLog2InvSqrt2Pi = -1.32574806f;  // log2(1 / sqrt(2 pi))
__device__ __forceinline__ float sign_of(float v) { return __builtin_copysignf(1.0f, v); }
__device__ __forceinline__ float gelu_grad_fast(float z) {
    const float e = __builtin_amdgcn_exp2f(fmaf(z * z, kNegHalfLog2e, kLog2InvSqrt2Pi));  // phi(z)
    const float sg = sign_of(z);
    const float st = __builtin_amdgcn_rcpf(fmaf(0.2316419f, z, sg));  // s t
    const float t = fabsf(st);
    float b = fmaf(t, 1.330274429f, -1.821255978f);
    b = fmaf(t, b, 1.781477937f);
    b = fmaf(t, b, -0.356563782f);
    b = fmaf(t, b, 0.319381530f);
    return fmaf(e, fmaf(-b, st, z), fmaf(0.5f, sg, 0.5f));
}

// gelu_grad_fast of z = w / kGeluWScale.  A caller that forms z as x a + s
// can scale a and s by kGeluWScale = sqrt(log2(e) / 2) once and pass w: the
// exp2 argument -z^2 log2(e) / 2 is then -w^2 (one multiply per element
// fewer), phi(z) = exp2(log2(1 / sqrt(2 pi)) - w^2), and GELU'(z) = H +
// (phi / kGeluWScale) (w - kGeluWScale B(t) s t): the factor 1 /
// kGeluWScale joins the exponent (log2 of 1 / (sqrt(2 pi) kGeluWScale)),
// kGeluWScale joins B's coefficients and p.  Same error bound.
constexpr float kGeluWScale = 0.84932180f;
__device__ __forceinline__ float gelu_grad_fast_w(float w) {
    const float e = __builtin_amdgcn_exp2f(fmaf(-w, w, -1.09013125f));  // phi / kGeluWScale
    const float sg = sign_of(w);
    const float st = __builtin_amdgcn_rcpf(fmaf(0.27273747f, w, sg));  // p / kGeluWScale
    const float t = fabsf(st);
    float b = fmaf(t, 1.129831073f, -1.546832407f);  // kGeluWScale b5, b4
    b = fmaf(t, b, 1.513048048f);
    b = fmaf(t, b, -0.3028373926f);
    b = fmaf(t, b, 0.2712576963f);
    return fmaf(e, fmaf(-b, st, w), fmaf(0.5f, sg, 0.5f));
}

// Fast forward GELU (FAST = true).  The forward needs Phi but not phi, so it
// uses Abramowitz & Stegun eq. 7.1.28, erf(u) ~= 1 - 1 / (1 + a1 u + ... +
// a6 u^6)^16 for u >= 0, |error| <= 3e-7, which costs one reciprocal and no
// exp.  With r16 = (1 + a1 u + ... + a6 u^6)^-16 and u = |z| / sqrt 2,
// z * Phi(z) = max(z, 0) - |z| * r16 / 2 for either sign of z.  The
// polynomial is evaluated in |z| with every coefficient (the constant 1
// included) scaled by 2^(1/16): a_i 2^(-i/2) 2^(1/16) for u^i, so its
// reciprocal's 16th power is r16 / 2 and the result one FMA.  In float32
// the result is within 7.1e-7 of GELU(z) (below 0.04 bf16 ulp wherever
// |GELU(z)| > 2^-10).
// max(z, 0) as one integer max on the bits: a float with the sign bit set is
// a negative int32 and gives +0, any other float passes unchanged.  fmaxf
// costs a second v_max_f32 that quiets signalling NaNs of a value that came
// straight from memory.  Used where it is added to a term that carries z's
// NaN or infinity anyway, and where the sign of a zero result is immaterial.
__device__ __forceinline__ float max0_bits(float z) {
    return __int_as_float(max(__float_as_int(z), 0));
}

__device__ __forceinline__ float gelu_fast(float z) {
    const float az = fabsf(z);
    float p = fmaf(5.6212998e-06f, az, 5.1055209e-05f);
    p = fmaf(p, az, 3.9686136e-05f);
    p = fmaf(p, az, 3.4227392e-03f);
    p = fmaf(p, az, 2.2076998e-02f);
    p = fmaf(p, az, 5.2075163e-02f);
    p = fmaf(p, az, 1.0442737f);  // 2^(1/16)
    float r = __builtin_amdgcn_rcpf(p);
    r *= r;
    r *= r;
    r *= r;
    r *= r;  // r = p^-16 = r16 / 2
    return fmaf(-az, r, max0_bits(z));
}

// GELU with a small relative error everywhere, the forward for fp16 I/O:
// fp16 results reach 2^-24 in the negative tail, where the absolute error of
// eq. 7.1.28 above is several fp16 ulps.  The form is the one of Press et
// al., Numerical Recipes (2nd ed., section 6.2): erfc(u) ~= t exp(-u^2 +
// P(t)), t = 1 / (1 + u / 2), u >= 0, which keeps the error relative all
// along the tail.  Their P has degree 9 (fractional error 1.2e-7, far below
// what an fp16 result resolves); P here is a degree-5 fit of our own
// (weighted least squares towards minimax on u in [0, 8], gelu_erfc_fit.py
// beside this file): erfc's relative error stays below 7.7e-6 there.  With
// u = |z| / sqrt 2, z Phi(z) = max(z, 0) - |z| erfc(u) / 2; P is kept in
// log2 units with the 1/2 folded into its constant, so the exponential is
// one exp2.  Evaluated in float32 the result is within 9.2e-6 of GELU(z),
// relatively, wherever |GELU(z)| > 2^-24 (|z| <= 12; 0.01 fp16 ulp).
__device__ __forceinline__ float gelu_fast_rel(float z) {
    const float az = fabsf(z);
    const float t = __builtin_amdgcn_rcpf(fmaf(az, 3.535533845e-01f, 1.0f));  // 1 / (1 + u / 2)
    float p = fmaf(t, 3.300003556e-01f, -1.022894649e+00f);
    p = fmaf(t, p, 6.842195693e-01f);
    p = fmaf(t, p, 3.672914762e-01f);
    p = fmaf(t, p, 1.468620589e+00f);
    const float arg = fmaf(t, p, fmaf(z, z * -7.213475108e-01f, -2.827226368e+00f));
    const float h = t * __builtin_amdgcn_exp2f(arg);  // erfc(u) / 2
    return fmaf(-az, h, max0_bits(z));
}

template <int ACT, bool FAST = false> __device__ __forceinline__ float act_fwd(float z) {
    if constexpr (ACT == kActRelu) return z > 0.0f ? z : 0.0f;
    else if constexpr (ACT == kActGelu) {
        if constexpr (FAST) return gelu_fast(z);
        else return 0.5f * z * (1.0f + erff(z * kInvSqrt2));
    } else return z;
}

template <int ACT, bool FAST = false> __device__ __forceinline__ float act_grad(float z) {
    if constexpr (ACT == kActRelu) return z > 0.0f ? 1.0f : 0.0f;
    else if constexpr (ACT == kActGelu) {
        if constexpr (FAST) return gelu_grad_fast(z);
        else return gelu_grad_exact(z);
    } else return 1.0f;
}

// The rest of the family ([ActPage] section 6), evaluated in float32.  These
// share one kernel instantiation per shape class and select the function
// with a wave-uniform switch; definitions and the derivative conventions at
// kinks are PyTorch's.  `p` is the leaky slope, or alpha of ELU / CELU.
// FAST = false uses the accurate device exp / tanh / log1p / expm1 and
// IEEE division; FAST = true (16-bit outputs, as for GELU) builds them from
// the hardware exp2 / log2 / reciprocal instructions: relative error a few
// float32 ulps (1e-6 for |z| <= 20), or an absolute error near 1e-7 where a
// result cancels towards 0 (tanh, expm1 and log1p of tiny arguments) --
// far below a 16-bit ulp of the tensor's scale.
constexpr float kSeluScale = 1.0507009873554804934f;
constexpr float kSeluAlpha = 1.6732632423543772848f;
constexpr float kLog2e = 1.4426950408889634074f;
constexpr float kLn2 = 0.69314718055994530942f;

template <bool FAST> __device__ __forceinline__ float exp_f(float z) {
    if constexpr (FAST) return __builtin_amdgcn_exp2f(z * kLog2e);
    else return expf(z);
}
template <bool FAST> __device__ __forceinline__ float expm1_f(float z) {
    if constexpr (FAST) return __builtin_amdgcn_exp2f(z * kLog2e) - 1.0f;
    else return expm1f(z);
}
template <bool FAST> __device__ __forceinline__ float recip_f(float v) {
    if constexpr (FAST) return __builtin_amdgcn_rcpf(v);
    else return 1.0f / v;
}
// log(1 + e^-|z|) for the softplus family: the argument lies in (0, 1].
template <bool FAST> __device__ __forceinline__ float log1p_exp_neg_abs(float z) {
    const float e = exp_f<FAST>(-fabsf(z));
    if constexpr (FAST) return __builtin_amdgcn_logf(1.0f + e) * kLn2;
    else return log1pf(e);
}
template <bool FAST> __device__ __forceinline__ float sigmoid_f(float z) {
    return recip_f<FAST>(1.0f + exp_f<FAST>(-z));
}
template <bool FAST> __device__ __forceinline__ float tanh_f(float z) {
    if constexpr (FAST) {
        const float e = __builtin_amdgcn_exp2f(fabsf(z) * (-2.0f * kLog2e));
        return copysignf((1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e), z);
    } else {
        return tanhf(z);
    }
}
// softplus(z) = max(z, 0) + log(1 + e^-|z|), the identity above 20.
template <bool FAST> __device__ __forceinline__ float softplus_f(float z) {
    return z > 20.0f ? z : fmaxf(z, 0.0f) + log1p_exp_neg_abs<FAST>(z);
}

template <bool FAST = false>
__device__ inline float act_fwd_rt(int act, float p, float z) {
    switch (act) {
    case kActRelu: return z > 0.0f ? z : 0.0f;
    case kActGelu: return 0.5f * z * (1.0f + erff(z * kInvSqrt2));
    case kActSigmoid: return sigmoid_f<FAST>(z);
    case kActTanh: return tanh_f<FAST>(z);
    case kActSilu: return z * sigmoid_f<FAST>(z);
    case kActMish: return z * tanh_f<FAST>(softplus_f<FAST>(z));
    case kActLeakyRelu: return z > 0.0f ? z : p * z;
    case kActElu: return z > 0.0f ? z : p * expm1_f<FAST>(z);
    case kActSelu: return kSeluScale * (z > 0.0f ? z : kSeluAlpha * expm1_f<FAST>(z));
    case kActCelu: return z > 0.0f ? z : p * expm1_f<FAST>(z * recip_f<FAST>(p));
    case kActSoftplus: return softplus_f<FAST>(z);
    case kActRelu6: return fminf(fmaxf(z, 0.0f), 6.0f);
    case kActHardsigmoid: return z <= -3.0f ? 0.0f : (z >= 3.0f ? 1.0f : z * (1.0f / 6.0f) + 0.5f);
    case kActHardswish: return z <= -3.0f ? 0.0f : (z >= 3.0f ? z : z * (z + 3.0f) * (1.0f / 6.0f));
    default: return z;
    }
}

template <bool FAST = false>
__device__ inline float act_grad_rt(int act, float p, float z) {
    switch (act) {
    case kActRelu: return z > 0.0f ? 1.0f : 0.0f;
    case kActGelu: return act_grad<kActGelu, false>(z);
    case kActSigmoid: { const float s = sigmoid_f<FAST>(z); return s * (1.0f - s); }
    case kActTanh: { const float t = tanh_f<FAST>(z); return 1.0f - t * t; }
    case kActSilu: { const float s = sigmoid_f<FAST>(z); return s * (1.0f + z * (1.0f - s)); }
    case kActMish: {
        const float t = tanh_f<FAST>(softplus_f<FAST>(z));
        return t + z * sigmoid_f<FAST>(z) * (1.0f - t * t);
    }
    case kActLeakyRelu: return z > 0.0f ? 1.0f : p;
    case kActElu: return z > 0.0f ? 1.0f : p * exp_f<FAST>(z);
    case kActSelu: return kSeluScale * (z > 0.0f ? 1.0f : kSeluAlpha * exp_f<FAST>(z));
    case kActCelu: return z > 0.0f ? 1.0f : exp_f<FAST>(z * recip_f<FAST>(p));
    case kActSoftplus: return z > 20.0f ? 1.0f : sigmoid_f<FAST>(z);
    case kActRelu6: return (z > 0.0f && z < 6.0f) ? 1.0f : 0.0f;
    case kActHardsigmoid: return (z > -3.0f && z < 3.0f) ? (1.0f / 6.0f) : 0.0f;
    case kActHardswish: return z <= -3.0f ? 0.0f : (z < 3.0f ? z * (1.0f / 3.0f) + 0.5f : 1.0f);
    default: return 1.0f;
    }
}

// Compile-time activation, or the run-time one for ACT == kActGeneric.
template <int ACT, bool FAST>
__device__ __forceinline__ float act_fwd_any(float z, int act_rt, float p) {
    if constexpr (ACT == kActGeneric) return act_fwd_rt<FAST>(act_rt, p, z);
    else return act_fwd<ACT, FAST>(z);
}
// Forward activation for I/O type T: bf16 takes the fast forms; fp16 the
// exact ones, except GELU, which takes gelu_fast_rel; float32 the exact ones.
template <typename T, int ACT>
__device__ __forceinline__ float act_fwd_io(float z, int act_rt, float p) {
    if constexpr (std::is_same<T, bf16_t>::value) return act_fwd_any<ACT, true>(z, act_rt, p);
    else if constexpr (std::is_same<T, f16_t>::value && ACT == kActGelu) return gelu_fast_rel(z);
    else return act_fwd_any<ACT, false>(z, act_rt, p);
}
template <int ACT, bool FAST>
__device__ __forceinline__ float act_grad_any(float z, int act_rt, float p) {
    if constexpr (ACT == kActGeneric) return act_grad_rt<FAST>(act_rt, p, z);
    else return act_grad<ACT, FAST>(z);
}

}  // namespace mi355norm
