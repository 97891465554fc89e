// row_common.hpp -- declarations shared by the LayerNorm / RMSNorm entry
// points (rownorm.hip) and the kernel instantiations (row_inst.hip): the
// launch plan and the launchers, instantiated once per I/O dtype.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "norm_device.hpp"
#include "norm_host.hpp"

namespace mi355norm {

constexpr int kMaxBwdBlocksPerCU = 8;  // cap on persistent backward blocks per CU

struct RowPlan {
    int vec = 1;    // elements per vector access
    int it = 1;     // vectors per thread
    int tpr = 1;    // threads per row
    int block = 64; // threads per block
    int grid = 1;   // persistent blocks
};

// Launchers (row_kernels.hpp).  Each returns NORM_ERR_SHAPE for a plan no
// kernel instance covers.
template <typename T, bool RMS, int V>
norm_status row_launch_fwd(const RowPlan &p, hipStream_t s, const void *x, const void *w, const void *b,
                           void *y, float *mean, float *rstd, int64_t M, int N, float eps);
template <typename T, bool RMS, int V>
norm_status row_launch_bwd(const RowPlan &p, hipStream_t s, const void *dy, const void *x, const void *w,
                           const float *mean, const float *rstd, void *dx, float *part_w, float *part_b,
                           void *dw_out, void *db_out, int64_t M, int N);
// dw / db from the partial rows (fixed order, float64); either may be NULL.
template <typename T>
void row_launch_colsum(hipStream_t s, const float *part_w, const float *part_b, int parts, int N, void *dw,
                       void *db);
// out[0:n] = 0 (a kernel rather than a memset, so the call stays safe
// under stream capture).
template <typename T>
void row_launch_zero(hipStream_t s, void *out, int n);

}  // namespace mi355norm
