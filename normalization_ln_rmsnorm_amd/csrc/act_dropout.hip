// act_dropout.hip -- entry points of the fused activation + dropout
// (argument checks, the Philox key / counter / threshold set-up); kernels in
// ad_kernels.hpp.
//
// Page (by title):
//   [ActPage] "Operator fusion in practice: attorch's activation and
//             dropout fusion kernels", sections 3-5.
#include <hip/hip_runtime.h>

#include <math.h>

#include "ad_kernels.hpp"

namespace mi355norm {

// Drop threshold on an element's 16 generator bits: round(p * 2^16), 0 for
// p = 0 and 2^16 (drop everything) for p = 1.
static uint32_t drop_threshold(float p) {
    const double d = (double)p;
    if (!(d > 0.0)) return 0u;
    if (d >= 1.0) return 1u << 16;
    return (uint32_t)floor(d * 65536.0 + 0.5);
}

static norm_status check_ad(norm_dtype dt, int64_t n, norm_act act, float act_param, float drop_p,
                            uint64_t offset) {
    if (!dtype_ok(dt)) return NORM_ERR_DTYPE;
    if (n < 0) return NORM_ERR_SHAPE;
    if (!act_ok(act)) return NORM_ERR_ACT;
    if (!act_param_ok(act, act_param)) return NORM_ERR_ARG;
    if (!(drop_p >= 0.0f && drop_p <= 1.0f)) return NORM_ERR_ARG;
    if (offset % 8 != 0) return NORM_ERR_ARG;
    if (offset > UINT64_MAX - (uint64_t)n) return NORM_ERR_ARG;
    return NORM_OK;
}

static AdArgs make_args(int64_t n, norm_act act, float act_param, float drop_p, uint64_t seed,
                        uint64_t offset) {
    AdArgs a;
    a.n = n;
    a.k0 = (uint32_t)seed;
    a.k1 = (uint32_t)(seed >> 32);
    a.blk0 = offset >> 3;
    a.thresh = drop_threshold(drop_p);
    a.scale = drop_p < 1.0f ? 1.0f / (1.0f - drop_p) : 0.0f;
    a.act_rt = (int)act;
    a.act_p = act_param;
    return a;
}

}  // namespace mi355norm

using namespace mi355norm;

extern "C" norm_status act_dropout_fwd(norm_dtype dt, int64_t n, norm_act act, float act_param, float drop_p,
                                       uint64_t seed, uint64_t offset, const void *x, void *y, void *stream) {
    CallScope scope;
    const norm_status s = check_ad(dt, n, act, act_param, drop_p, offset);
    if (s != NORM_OK) return s;
    if (n == 0) return NORM_OK;
    if (!x || !y) return NORM_ERR_NULL;
    const AdArgs a = make_args(n, act, act_param, drop_p, seed, offset);
    const bool vec = aligned16(x) && aligned16(y);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return with_io_type(dt, [&](auto tag) {
        using T = typename decltype(tag)::type;
        constexpr int VW = 16 / (int)sizeof(T);
        return vec ? ad_launch_fwd<T, VW>(a, x, y, st) : ad_launch_fwd<T, 1>(a, x, y, st);
    });
}

extern "C" norm_status act_dropout_bwd(norm_dtype dt, int64_t n, norm_act act, float act_param, float drop_p,
                                       uint64_t seed, uint64_t offset, const void *dy, const void *x, void *dx,
                                       void *stream) {
    CallScope scope;
    const norm_status s = check_ad(dt, n, act, act_param, drop_p, offset);
    if (s != NORM_OK) return s;
    if (n == 0) return NORM_OK;
    if (!dy || !x || !dx) return NORM_ERR_NULL;
    const AdArgs a = make_args(n, act, act_param, drop_p, seed, offset);
    const bool vec = aligned16(dy) && aligned16(x) && aligned16(dx);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return with_io_type(dt, [&](auto tag) {
        using T = typename decltype(tag)::type;
        constexpr int VW = 16 / (int)sizeof(T);
        return vec ? ad_launch_bwd<T, VW>(a, dy, x, dx, st) : ad_launch_bwd<T, 1>(a, dy, x, dx, st);
    });
}
