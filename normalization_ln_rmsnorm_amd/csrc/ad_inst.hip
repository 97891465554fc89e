// ad_inst.hip -- activation + dropout launchers for one I/O dtype
// (MI355NORM_AD_IO: 0 float32, 1 bf16, 2 fp16), compiled once per dtype.
#include "ad_kernels.hpp"

#ifndef MI355NORM_AD_IO
#error "MI355NORM_AD_IO must be 0 (float32), 1 (bf16) or 2 (fp16)"
#endif

namespace mi355norm {

#if MI355NORM_AD_IO == 0
using IoT = float;
#elif MI355NORM_AD_IO == 1
using IoT = bf16_t;
#else
using IoT = f16_t;
#endif

// Workgroups for a.n elements at V per vector and `unroll` vectors per thread
// per pass.  The forward takes half as many workgroups as chunks, so every
// thread makes two grid-stride passes: on the bf16 GELU dropout forward two
// passes measured 3-7% faster than one from 2^25 elements up (2^28: 175.5 ->
// 164.9 us), and the same at 2^24.  The backward takes one workgroup per
// chunk.  Both are capped at 2^22 workgroups, past which the grid-stride
// loop takes over.
static dim3 ad_grid(const AdArgs &a, int V, int unroll, bool fwd) {
    const int64_t nvec = a.n / V;
    const int64_t want = ceil_div(nvec > 0 ? nvec : 1, (int64_t)kAdBlock * unroll);
    int64_t g = fwd ? (want + 1) / 2 : want;
    if (g > ((int64_t)1 << 22)) g = (int64_t)1 << 22;
    return dim3((unsigned)g);
}

template <typename T, int V, bool DROP>
static auto fwd_kernel(int act) {
    switch (act) {
    case NORM_ACT_NONE: return act_dropout_fwd_kernel<T, V, kActNone, DROP>;
    case NORM_ACT_RELU: return act_dropout_fwd_kernel<T, V, kActRelu, DROP>;
    case NORM_ACT_GELU: return act_dropout_fwd_kernel<T, V, kActGelu, DROP>;
    default: return act_dropout_fwd_kernel<T, V, kActGeneric, DROP>;
    }
}

template <typename T, int V, bool DROP>
static auto bwd_kernel(int act) {
    switch (act) {
    case NORM_ACT_NONE: return act_dropout_bwd_kernel<T, V, kActNone, DROP>;
    case NORM_ACT_RELU: return act_dropout_bwd_kernel<T, V, kActRelu, DROP>;
    case NORM_ACT_GELU: return act_dropout_bwd_kernel<T, V, kActGelu, DROP>;
    default: return act_dropout_bwd_kernel<T, V, kActGeneric, DROP>;
    }
}

template <typename T, int V>
norm_status ad_launch_fwd(const AdArgs &a, const void *x, void *y, hipStream_t s) {
    auto fn = a.thresh > 0 ? fwd_kernel<T, V, true>(a.act_rt) : fwd_kernel<T, V, false>(a.act_rt);
    launch("act_dropout_fwd_kernel", true, fn, ad_grid(a, V, kAdUnrollFwd, true), dim3(kAdBlock), 0, s, (const T *)x, (T *)y, a);
    return launch_status();
}

template <typename T, int V>
norm_status ad_launch_bwd(const AdArgs &a, const void *dy, const void *x, void *dx, hipStream_t s) {
    auto fn = a.thresh > 0 ? bwd_kernel<T, V, true>(a.act_rt) : bwd_kernel<T, V, false>(a.act_rt);
    launch("act_dropout_bwd_kernel", true, fn, ad_grid(a, V, kAdUnrollBwd, false), dim3(kAdBlock), 0, s, (const T *)dy,
           (const T *)x, (T *)dx, a);
    return launch_status();
}

constexpr int kVW = 16 / (int)sizeof(IoT);
template norm_status ad_launch_fwd<IoT, kVW>(const AdArgs &, const void *, void *, hipStream_t);
template norm_status ad_launch_fwd<IoT, 1>(const AdArgs &, const void *, void *, hipStream_t);
template norm_status ad_launch_bwd<IoT, kVW>(const AdArgs &, const void *, const void *, void *, hipStream_t);
template norm_status ad_launch_bwd<IoT, 1>(const AdArgs &, const void *, const void *, void *, hipStream_t);

}  // namespace mi355norm
