// api_common.hip -- status strings, device properties and the kernel-timing
// hook shared by every entry point of libmi355norm.
#include <hip/hip_runtime.h>

#include <mutex>

#include "norm_host.hpp"

namespace mi355norm {

namespace {
struct ArmedEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
thread_local ArmedEvents g_armed;
thread_local const char *g_last_kernel = "";

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices] = {0};
std::mutex g_cu_mutex;
}  // namespace

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    if (g_cu_count[dev] > 0) return g_cu_count[dev];
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    g_cu_count[dev] = n;
    return n;
}

void hook_before(hipStream_t s, const char *kernel_name) {
    g_last_kernel = kernel_name;
    if (g_armed.start) (void)hipEventRecord(g_armed.start, s);
}

void hook_after(hipStream_t s) {
    if (g_armed.stop) (void)hipEventRecord(g_armed.stop, s);
    g_armed.start = nullptr;
    g_armed.stop = nullptr;
}

}  // namespace mi355norm

extern "C" const char *norm_status_str(norm_status s) {
    switch (s) {
    case NORM_OK: return "ok";
    case NORM_ERR_NULL: return "a required pointer is NULL";
    case NORM_ERR_SHAPE: return "unsupported or invalid shape";
    case NORM_ERR_DTYPE: return "unknown dtype";
    case NORM_ERR_ACT: return "unknown activation";
    case NORM_ERR_ARG: return "invalid argument (eps < 0, momentum outside [0,1], or fewer than 2 values per channel)";
    case NORM_ERR_WORKSPACE: return "workspace missing or too small";
    case NORM_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

extern "C" void norm_arm_kernel_events(void *start_event, void *stop_event) {
    mi355norm::g_armed.start = static_cast<hipEvent_t>(start_event);
    mi355norm::g_armed.stop = static_cast<hipEvent_t>(stop_event);
}

extern "C" const char *norm_last_kernel_name(void) { return mi355norm::g_last_kernel; }
