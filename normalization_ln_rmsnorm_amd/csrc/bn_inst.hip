// bn_inst.hip -- explicit instantiation of the BatchNorm launchers for one
// I/O dtype, chosen by MI355NORM_BN_IO (0 float32, 1 bf16, 2 fp16).  The
// build compiles this file once per dtype, in parallel.
#include "bn_cols.hpp"
#include "bn_plane.hpp"

#ifndef MI355NORM_BN_IO
#error "MI355NORM_BN_IO must be 0 (float32), 1 (bf16) or 2 (fp16)"
#endif

namespace mi355norm {

#if MI355NORM_BN_IO == 0
using IoT = float;
#elif MI355NORM_BN_IO == 1
using IoT = bf16_t;
#else
using IoT = f16_t;
#endif
constexpr int kVW = 16 / (int)sizeof(IoT);

#define MI355NORM_INST(V)                                                          \
    template norm_status bn_plane_fwd_train<IoT, V>(const BnGeom &, const BnArgs &); \
    template norm_status bn_plane_fwd_eval<IoT, V>(const BnGeom &, const BnArgs &);  \
    template norm_status bn_plane_bwd<IoT, V>(const BnGeom &, const BnArgs &);       \
    template norm_status bn_col_fwd_train<IoT, V>(const BnColGeom &, const BnColGeom &, const BnArgs &); \
    template norm_status bn_col_fwd_eval<IoT, V>(const BnColGeom &, const BnArgs &); \
    template norm_status bn_col_bwd<IoT, V>(const BnColGeom &, const BnColGeom &, const BnArgs &);

MI355NORM_INST(kVW)
MI355NORM_INST(1)

}  // namespace mi355norm
