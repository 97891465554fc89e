// batchnorm.hip -- BatchNorm entry points (training forward, eval forward,
// backward) with an optional fused residual add and activation: argument
// checks, the choice of data path, and the workspace layout.  The kernels
// live in bn_plane.hpp (long planes) and bn_cols.hpp (short planes,
// BatchNorm1d), instantiated per I/O dtype in bn_inst.hip.
//
// Pages (by title):
//   [NormPage] "How attorch implements LayerNorm, BatchNorm and RMSNorm:
//               the three normalization Triton kernels explained"
//   [MathPage] "Building custom GPU operators quickly with attorch.math:
//               an operator-fusion guide for advanced developers"
//   [ActPage]  "Operator fusion in practice: attorch's activation and
//               dropout fusion kernels"
//
// Layout.  x is [Nb][C][HW] (NCHW, or BatchNorm1d's (N, C) with HW = 1 and
// (N, C, L) with HW = L).
//
// Path choice (a function of dtype, C and HW only, so the workspace query
// and the call agree):
//   plane path    planes of at least 1 KiB that split into 128-bit vectors:
//                 each workgroup streams whole planes of one channel;
//   column path   otherwise, when a sample's C * HW values split into
//                 128-bit vectors (or the planes are short anyway): each
//                 workgroup streams a band of columns down the samples.
// norm_bn_force_path() pins one path for the whole process (tests of both
// paths on the same shapes); the workspace query follows it.  A library
// built with -DMI355NORM_TUNING also reads MI355NORM_BN_TILE (plane-path
// values per workgroup) and MI355NORM_BN_COL_PLAN ("rows_per_tile,
// vectors_per_row_slice"), once per process, for tuning sweeps; the regular
// build has no run-time knobs.
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <utility>
#include <initializer_list>

#include "bn_common.hpp"

namespace mi355norm {

constexpr int64_t kBnTileBytes = 16384;     // plane path: input bytes per workgroup
constexpr int64_t kBnPlaneMinBytes = 1024;  // shortest plane the plane path takes
constexpr int64_t kBnColMinBlocks = 512;    // column path: workgroups to aim for

enum BnPath { kPathPlane = 0, kPathCols = 1 };

// Plane path tile: 16 KiB of input per workgroup (4096 float32 or 8192
// 16-bit values, rounded up to whole planes), the best of a sweep over the
// two BatchNorm2d workloads.  MI355NORM_BN_TILE (values) overrides it.
static int64_t tile_elems(norm_dtype dt) {
#ifdef MI355NORM_TUNING
    static const long long over = [] {
        const char *e = getenv("MI355NORM_BN_TILE");
        const long long v = (e && *e) ? atoll(e) : 0;
        return (v >= 256 && v <= (1LL << 26)) ? v : 0;
    }();
    if (over) return over;
#endif
    return kBnTileBytes / (int64_t)dtype_size(dt);
}

static BnGeom make_geom(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW) {
    BnGeom g;
    g.Nb = Nb;
    g.HW = HW;
    g.C = (int)C;
    int64_t ppb = HW > 0 ? ceil_div(tile_elems(dt), HW) : 1;
    if (ppb > Nb) ppb = Nb > 0 ? Nb : 1;
    if (ppb < 1) ppb = 1;
    g.ppb = (int)ppb;
    g.tiles = (int)(Nb > 0 ? ceil_div(Nb, ppb) : 1);
    return g;
}

// 0: automatic; 1: plane path; 2: column path (norm_bn_force_path).
static std::atomic<int> g_forced_path{0};

static BnPath choose_path(norm_dtype dt, int64_t C, int64_t HW) {
    const int forced = g_forced_path.load(std::memory_order_relaxed);
    if (forced == 1) return kPathPlane;
    if (forced == 2) return kPathCols;
    const int64_t es = (int64_t)dtype_size(dt), v = 16 / es;
    const bool long_plane = HW * es >= kBnPlaneMinBytes;
    if (long_plane && HW % v == 0) return kPathPlane;
    if ((C * HW) % v == 0) return kPathCols;
    return long_plane ? kPathPlane : kPathCols;
}

// Column path rows per tile: 1 KiB of each column per tile (256 float32 or
// 512 16-bit rows), halved (down to 16 rows) while the grid would have
// fewer than kBnColMinBlocks workgroups.  Long row bands in about 512
// workgroups measured faster than more, shorter ones on the BatchNorm1d
// workloads (8192 x 2048 float32, 2048 x 512 x 32 bf16), and they keep the
// float64 per-(tile, column) sums small.  The reduction passes (statistics,
// backward sums) span 64 vectors of a row per workgroup (one wave's width,
// 1 KiB); the streaming passes (apply, dx), whose geometry fixes no
// workspace layout, span 128 (two waves side by side over 2 KiB of each
// row, two row slices), which measured faster there (bf16 2048 x 512 x 32
// dx 51.6 -> 47.1 us, float32 8192 x 2048 dx 33.3 -> 32.4 us) but slower for
// the reductions (their finalize merges twice the tiles).
static BnColGeom make_col_geom(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW, int V, bool stream = false) {
    BnColGeom g;
    const int64_t es = (int64_t)dtype_size(dt);
    g.Nb = Nb;
    g.C = (int)C;
    g.HW = HW;
    g.K = C * HW;
    g.KV = g.K / V;
    int ov_rt = 0, ov_cv = 0;
#ifdef MI355NORM_TUNING
    static const std::pair<int, int> over = [] {
        int rt = 0, cv = 0;
        const char *e = getenv("MI355NORM_BN_COL_PLAN");
        if (e && *e && sscanf(e, "%d,%d", &rt, &cv) == 2) {
            if (rt < 1 || rt > (1 << 20)) rt = 0;
            if (cv != 16 && cv != 32 && cv != 64 && cv != 128 && cv != 256) cv = 0;
        }
        return std::make_pair(rt, cv);
    }();
    ov_rt = over.first;
    ov_cv = over.second;
#endif
    const int64_t cv_cap = stream ? 2 * kWave : kWave;
    const int64_t cv_max = ov_cv ? ov_cv : cv_cap;
    g.CV = (int)(g.KV < cv_max ? (g.KV > 0 ? g.KV : 1) : cv_max);
    g.RPP = kBnBlock / g.CV;
    g.NCH = (int)ceil_div(g.KV > 0 ? g.KV : 1, g.CV);
    // The row tiling depends on the nominal (vector) width only, so the
    // workspace size does not depend on pointer alignment.
    const int64_t kv_nom = ceil_div(g.K, 16 / es);
    const int64_t nch_nom = ceil_div(kv_nom > 0 ? kv_nom : 1, cv_max);
    int64_t rt = 1024 / es;
    while (rt > 16 && nch_nom * ceil_div(Nb, rt) < kBnColMinBlocks) rt >>= 1;
    if (ov_rt) rt = ov_rt;
    g.RT = (int)rt;
    g.T = (int)(Nb > 0 ? ceil_div(Nb, rt) : 1);
    return g;
}

static norm_status check_bn(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW) {
    if (!dtype_ok(dt)) return NORM_ERR_DTYPE;
    if (Nb < 0 || C < 0 || HW < 0) return NORM_ERR_SHAPE;
    if (C > (int64_t)1 << 24 || Nb > (int64_t)1 << 31 || HW > (int64_t)1 << 40) return NORM_ERR_SHAPE;
    if (C > 0 && Nb > 0 && HW > 0 && Nb * C > ((int64_t)1 << 31) - 1) return NORM_ERR_SHAPE;
    if (C > 0 && HW > 0 && choose_path(dt, C, HW) == kPathCols) {
        // Column-path grids: chunks x row tiles must fit one launch.
        for (bool stream : {false, true}) {
            const BnColGeom g = make_col_geom(dt, Nb, C, HW, 1, stream);
            if ((int64_t)g.NCH * g.T >= ((int64_t)1 << 31)) return NORM_ERR_SHAPE;
        }
    }
    return NORM_OK;
}

static bool vec_ok(norm_dtype dt, int64_t span, std::initializer_list<const void *> ptrs) {
    if ((span * (int64_t)dtype_size(dt)) % 16 != 0) return false;
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return false;
    return true;
}

// Workspace.  Plane path: one float64 triple per (channel, tile) -- the
// forward's (count, mean, M2) or the backward's three sums.  Column path:
// up to three float64 sums per (row tile, column), then float32 [C][4] dx
// coefficients.
static size_t ws_layout(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW) {
    if (choose_path(dt, C, HW) == kPathPlane) {
        const BnGeom g = make_geom(dt, Nb, C, HW);
        return (size_t)C * g.tiles * 3 * sizeof(double);
    }
    const BnColGeom g = make_col_geom(dt, Nb, C, HW, 1);
    return col_part_bytes_host(g) + (size_t)C * 4 * sizeof(float);
}

enum BnOp { kOpTrain, kOpEval, kOpBwd };

// Launch one operation on the chosen path with the widest vector width the
// shape and pointers allow.
static norm_status run(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW, BnOp op, const BnArgs &a,
                       std::initializer_list<const void *> streamed) {
    const BnPath path = choose_path(dt, C, HW);
    const bool vec = vec_ok(dt, path == kPathPlane ? HW : C * HW, streamed);
    return with_io_type(dt, [&](auto tag) {
        using T = typename decltype(tag)::type;
        constexpr int VW = 16 / (int)sizeof(T);
        if (path == kPathPlane) {
            const BnGeom g = make_geom(dt, Nb, C, HW);
            switch (op) {
            case kOpTrain: return vec ? bn_plane_fwd_train<T, VW>(g, a) : bn_plane_fwd_train<T, 1>(g, a);
            case kOpEval: return vec ? bn_plane_fwd_eval<T, VW>(g, a) : bn_plane_fwd_eval<T, 1>(g, a);
            default: return vec ? bn_plane_bwd<T, VW>(g, a) : bn_plane_bwd<T, 1>(g, a);
            }
        }
        const BnColGeom g = make_col_geom(dt, Nb, C, HW, vec ? VW : 1);
        const BnColGeom gs = make_col_geom(dt, Nb, C, HW, vec ? VW : 1, true);
        switch (op) {
        case kOpTrain: return vec ? bn_col_fwd_train<T, VW>(g, gs, a) : bn_col_fwd_train<T, 1>(g, gs, a);
        case kOpEval: return vec ? bn_col_fwd_eval<T, VW>(gs, a) : bn_col_fwd_eval<T, 1>(gs, a);
        default: return vec ? bn_col_bwd<T, VW>(g, gs, a) : bn_col_bwd<T, 1>(g, gs, a);
        }
    });
}

}  // namespace mi355norm

using namespace mi355norm;

extern "C" size_t bn_workspace_bytes(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW) {
    if (check_bn(dt, Nb, C, HW) != NORM_OK) return 0;
    return ws_layout(dt, Nb, C, HW);
}

extern "C" norm_status bn_fwd_train(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW, float eps, float momentum,
                                    norm_act act, float act_param, const void *x, const void *res, const void *w,
                                    const void *b, float *running_mean, float *running_var, float *save_mean,
                                    float *save_rstd, void *y, void *ws, size_t ws_bytes, void *stream) {
    CallScope scope;
    norm_status s = check_bn(dt, Nb, C, HW);
    if (s != NORM_OK) return s;
    if (!act_ok(act)) return NORM_ERR_ACT;
    if (!(eps >= 0.0f) || !(momentum >= 0.0f && momentum <= 1.0f)) return NORM_ERR_ARG;
    if (!act_param_ok(act, act_param)) return NORM_ERR_ARG;
    if (C == 0) return NORM_OK;
    if (Nb * HW < 2) return NORM_ERR_ARG;  // the unbiased running variance needs n >= 2
    if (!x || !y || !save_mean || !save_rstd) return NORM_ERR_NULL;
    if (!ws || ws_bytes < ws_layout(dt, Nb, C, HW)) return NORM_ERR_WORKSPACE;
    BnArgs a{};
    a.st = static_cast<hipStream_t>(stream);
    a.act = act; a.act_p = act_param; a.eps = eps; a.momentum = momentum;
    a.x = x; a.res = res; a.w = w; a.b = b;
    a.rm = running_mean; a.rv = running_var; a.sm = save_mean; a.sr = save_rstd;
    a.y = y; a.ws = ws;
    return run(dt, Nb, C, HW, kOpTrain, a, {x, res, y});
}

extern "C" norm_status bn_fwd_eval(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW, float eps, norm_act act,
                                   float act_param, const void *x, const void *res, const void *w, const void *b,
                                   const float *running_mean, const float *running_var, void *y, void *stream) {
    CallScope scope;
    norm_status s = check_bn(dt, Nb, C, HW);
    if (s != NORM_OK) return s;
    if (!act_ok(act)) return NORM_ERR_ACT;
    if (!(eps >= 0.0f) || !act_param_ok(act, act_param)) return NORM_ERR_ARG;
    if (C == 0 || Nb * HW == 0) return NORM_OK;
    if (!x || !y || !running_mean || !running_var) return NORM_ERR_NULL;
    BnArgs a{};
    a.st = static_cast<hipStream_t>(stream);
    a.act = act; a.act_p = act_param; a.eps = eps;
    a.x = x; a.res = res; a.w = w; a.b = b;
    // Eval only reads the running statistics.
    a.rm = const_cast<float *>(running_mean); a.rv = const_cast<float *>(running_var);
    a.y = y;
    return run(dt, Nb, C, HW, kOpEval, a, {x, res, y});
}

extern "C" norm_status bn_bwd(norm_dtype dt, int64_t Nb, int64_t C, int64_t HW, norm_act act, float act_param,
                              const void *dy, const void *x, const void *res, const void *w, const void *b,
                              const float *save_mean, const float *save_rstd, void *dx, void *dres, void *dw,
                              void *db, void *ws, size_t ws_bytes, void *stream) {
    CallScope scope;
    norm_status s = check_bn(dt, Nb, C, HW);
    if (s != NORM_OK) return s;
    if (!act_ok(act)) return NORM_ERR_ACT;
    if (!act_param_ok(act, act_param)) return NORM_ERR_ARG;
    if (C == 0) return NORM_OK;
    if (Nb * HW < 2) return NORM_ERR_ARG;
    if (!dy || !x || !dx || !save_mean || !save_rstd) return NORM_ERR_NULL;
    if (res && !dres) return NORM_ERR_NULL;
    if (!ws || ws_bytes < ws_layout(dt, Nb, C, HW)) return NORM_ERR_WORKSPACE;
    BnArgs a{};
    a.st = static_cast<hipStream_t>(stream);
    a.act = act; a.act_p = act_param;
    a.dy = dy; a.x = x; a.res = res; a.w = w; a.b = b;
    a.sm = const_cast<float *>(save_mean); a.sr = const_cast<float *>(save_rstd);
    a.dx = dx; a.dres = dres; a.dw = dw; a.db = db; a.ws = ws;
    return run(dt, Nb, C, HW, kOpBwd, a, {dy, x, res, dx, dres});
}

extern "C" int norm_bn_force_path(int path) {
    if (path < 0 || path > 2) return -1;
    return g_forced_path.exchange(path);
}
