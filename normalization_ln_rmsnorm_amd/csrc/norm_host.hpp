// norm_host.hpp -- host-side helpers shared by the entry points: status
// handling, device properties, the optional kernel-timing hook, and launch
// error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mi355norm.h"

namespace mi355norm {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t dtype_size(norm_dtype dt) { return dt == NORM_BF16 ? 2 : 4; }
inline bool dtype_ok(norm_dtype dt) { return dt == NORM_F32 || dt == NORM_BF16; }

// Compute units of the current device (cached per device id).
int device_cu_count();

// Timing hook (see norm_arm_kernel_events): called around the main kernel.
void hook_before(hipStream_t s, const char *kernel_name);
void hook_after(hipStream_t s);

// Map the launch status of the kernels just enqueued.
inline norm_status launch_status() {
    return hipGetLastError() == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace mi355norm
