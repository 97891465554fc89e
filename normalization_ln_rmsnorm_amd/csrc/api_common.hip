// api_common.hip -- status strings, device properties and the kernel-timing
// hook shared by every entry point of libmi355norm.
#include <hip/hip_runtime.h>

#include <mutex>

#include "norm_host.hpp"

namespace mi355norm {

namespace {
constexpr int kMaxKernelsPerCall = 16;
struct CallState {
    hipEvent_t events[2 * kMaxKernelsPerCall] = {};
    int armed_pairs = 0;           // pairs armed for the current / next call
    int count = 0;                 // kernels launched by the current / last call
    int main_index = -1;
    bool launch_failed = false;    // a launch of the current call was rejected
    const char *names[kMaxKernelsPerCall] = {};
};
thread_local CallState g_call;

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

void call_begin() {
    g_call.count = 0;
    g_call.main_index = -1;
    g_call.launch_failed = false;
}

void note_launch(hipError_t rc) {
    if (rc != hipSuccess) g_call.launch_failed = true;
}

bool call_launch_failed() { return g_call.launch_failed; }

void call_end() { g_call.armed_pairs = 0; }

bool kernel_events(const char *name, bool is_main, hipEvent_t *start, hipEvent_t *stop) {
    const int i = g_call.count;
    if (i < kMaxKernelsPerCall) {
        g_call.names[i] = name;
        g_call.count = i + 1;
    }
    if (is_main) g_call.main_index = i;
    if (i < g_call.armed_pairs && (g_call.events[2 * i] || g_call.events[2 * i + 1])) {
        *start = g_call.events[2 * i];
        *stop = g_call.events[2 * i + 1];
        return true;
    }
    return false;
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

extern "C" void norm_arm_kernel_events(void *const *events, int n_pairs) {
    using namespace mi355norm;
    if (!events || n_pairs <= 0) {
        g_call.armed_pairs = 0;
        return;
    }
    if (n_pairs > kMaxKernelsPerCall) n_pairs = kMaxKernelsPerCall;
    for (int i = 0; i < 2 * n_pairs; ++i) g_call.events[i] = static_cast<hipEvent_t>(events[i]);
    g_call.armed_pairs = n_pairs;
}

extern "C" int norm_last_kernel_count(void) {
    return mi355norm::g_call.count < mi355norm::kMaxKernelsPerCall ? mi355norm::g_call.count
                                                                   : mi355norm::kMaxKernelsPerCall;
}

extern "C" const char *norm_last_kernel_name(int i) {
    if (i < 0 || i >= norm_last_kernel_count()) return "";
    return mi355norm::g_call.names[i] ? mi355norm::g_call.names[i] : "";
}

extern "C" int norm_last_main_kernel(void) { return mi355norm::g_call.main_index; }
