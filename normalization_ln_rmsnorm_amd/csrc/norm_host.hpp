// norm_host.hpp -- host-side helpers shared by the entry points: status
// handling, device properties, the optional kernel-timing hook, and launch
// error mapping.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "../../include/mi355norm.h"
#include "norm_device.hpp"

namespace mi355norm {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t dtype_size(norm_dtype dt) { return dt == NORM_F32 ? 4 : 2; }
inline bool dtype_ok(norm_dtype dt) { return dt == NORM_F32 || dt == NORM_BF16 || dt == NORM_F16; }

// Calls f(type_tag<T>{}) with T the element type of a (checked) I/O dtype.
template <typename T> struct type_tag { using type = T; };

template <typename F>
inline auto with_io_type(norm_dtype dt, F &&f) {
    switch (dt) {
    case NORM_F32: return f(type_tag<float>{});
    case NORM_BF16: return f(type_tag<bf16_t>{});
    default: return f(type_tag<f16_t>{});
    }
}

// Compute units of the current device (cached per device id).
int device_cu_count();

// Per-call kernel bookkeeping behind norm_arm_kernel_events: every entry
// point opens a CallScope; every kernel goes through launch(), which
// attaches the armed event pair (if any) to that kernel's dispatch and
// records whether the runtime accepted the launch.
void call_begin();
void call_end();
bool kernel_events(const char *name, bool is_main, hipEvent_t *start, hipEvent_t *stop);
void note_launch(hipError_t rc);
bool call_launch_failed();

struct CallScope {
    CallScope() { call_begin(); }
    ~CallScope() { call_end(); }
};

// Enqueues fn<<<grid, block, shmem, s>>>(args...).  The arguments are
// converted to the kernel's own parameter types first (the runtime copies
// them by address), and the launch's own return code is kept for this
// call's status: the thread's sticky last error, which may hold a failure
// of something the caller did earlier, is neither read nor cleared.
template <typename... P, typename... A>
inline void launch(const char *name, bool is_main, void (*fn)(P...), dim3 grid, dim3 block, size_t shmem,
                   hipStream_t s, A... args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> conv(static_cast<P>(args)...);
    void *argv[sizeof...(P) > 0 ? sizeof...(P) : 1] = {};
    std::apply([&argv](auto &...a) {
        int i = 0;
        ((argv[i++] = static_cast<void *>(&a)), ...);
    }, conv);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const void *f = reinterpret_cast<const void *>(fn);
    hipError_t rc;
    if (kernel_events(name, is_main, &e0, &e1))
        rc = hipExtLaunchKernel(f, grid, block, argv, shmem, s, e0, e1, 0);
    else
        rc = hipLaunchKernel(f, grid, block, argv, shmem, s);
    note_launch(rc);
}

// Status of the kernels this call has enqueued so far.
inline norm_status launch_status() { return call_launch_failed() ? NORM_ERR_HIP : NORM_OK; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Activation argument checks shared by the entry points: a known
// activation, and a finite parameter (nonzero for CELU, which divides by it).
inline bool act_ok(norm_act a) { return (int)a >= 0 && (int)a < kActCount; }
inline bool act_param_ok(norm_act a, float p) {
    if (!(p == p) || p == __builtin_inff() || p == -__builtin_inff()) return false;
    return !(a == NORM_ACT_CELU && p == 0.0f);
}

}  // namespace mi355norm
