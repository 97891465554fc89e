// row_inst.hip -- explicit instantiation of the LayerNorm / RMSNorm
// launchers for one I/O dtype (MI355NORM_ROW_IO: 0 float32, 1 bf16, 2 fp16)
// and one operation (MI355NORM_ROW_RMS: 0 LayerNorm, 1 RMSNorm).  The build
// compiles this file once per pair, in parallel.
#include "row_kernels.hpp"

#if !defined(MI355NORM_ROW_IO) || !defined(MI355NORM_ROW_RMS)
#error "MI355NORM_ROW_IO (0 float32, 1 bf16, 2 fp16) and MI355NORM_ROW_RMS (0 / 1) must be set"
#endif

namespace mi355norm {

#if MI355NORM_ROW_IO == 0
using IoT = float;
#elif MI355NORM_ROW_IO == 1
using IoT = bf16_t;
#else
using IoT = f16_t;
#endif
constexpr int kVW = 16 / (int)sizeof(IoT);
constexpr bool kRms = MI355NORM_ROW_RMS != 0;

#define MI355NORM_ROW_INST(V)                                                                               \
    template norm_status row_launch_fwd<IoT, kRms, V>(const RowPlan &, hipStream_t, const void *,          \
                                                      const void *, const void *, void *, float *, float *, \
                                                      int64_t, int, float);                                 \
    template norm_status row_launch_bwd<IoT, kRms, V>(const RowPlan &, hipStream_t, const void *,          \
                                                      const void *, const void *, const float *,            \
                                                      const float *, void *, float *, float *, void *,   \
                                                      void *, int64_t, int);

MI355NORM_ROW_INST(kVW)
MI355NORM_ROW_INST(1)

// The column sum and zero fill depend on the dtype only: the LayerNorm unit
// of each dtype provides them.
#if !MI355NORM_ROW_RMS
template void row_launch_colsum<IoT>(hipStream_t, const float *, const float *, int, int, void *, void *);
template void row_launch_zero<IoT>(hipStream_t, void *, int);
#endif

}  // namespace mi355norm
