// rownorm.hip -- LayerNorm and RMSNorm entry points: argument checks, the
// launch planner and the workspace layout.  The kernels and their design
// notes are in row_kernels.hpp, instantiated per I/O dtype in row_inst.hip.
//
// Pages (by title):
//   [NormPage] "How attorch implements LayerNorm, BatchNorm and RMSNorm:
//               the three normalization Triton kernels explained"
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "row_common.hpp"

namespace mi355norm {

constexpr int64_t kDirectRowGroups = 8;  // backward: one block (no column-sum kernel) up to this
constexpr size_t kScratchBytes = NORM_NOALLOC_SCRATCH_BYTES;  // static scratch of rms_bwd_noalloc

// ---------------------------------------------------------------- planning


static const int kVecIts[] = {1, 2, 3, 4, 6, 8};
static const int kScalarIts[] = {1, 2, 4, 8, 16, 32, 64};

// Tuning override for sweeps, compiled only into a library built with
// -DMI355NORM_TUNING (the regular build has no run-time knobs):
// MI355NORM_ROW_PLAN="tpr,it,blocks_per_cu[,block_threads]", read once per
// process.
static bool env_override(int *tpr, int *it, int *bpc, int *block) {
#ifdef MI355NORM_TUNING
    static const struct Parsed {
        int n = 0, a = 0, b = 0, c = 0, d = 0;
        Parsed() {
            const char *s = getenv("MI355NORM_ROW_PLAN");
            if (s && *s) n = sscanf(s, "%d,%d,%d,%d", &a, &b, &c, &d);
        }
    } plan;
    if (plan.n < 3) return false;
    *tpr = plan.a; *it = plan.b; *bpc = plan.c; *block = plan.n == 4 ? plan.d : 0;
    return true;
#else
    (void)tpr; (void)it; (void)bpc; (void)block;
    return false;
#endif
}

static bool make_plan(norm_dtype dt, int64_t M, int64_t N, bool vec_ok, bool backward, RowPlan *p) {
    const int es = (int)dtype_size(dt);
    p->vec = vec_ok ? 16 / es : 1;
    const int64_t nv = N / p->vec;
    const int *its = vec_ok ? kVecIts : kScalarIts;
    const int n_its = vec_ok ? 6 : 7;
    int best_tpr = -1, best_it = -1;
    int64_t best_waste = INT64_MAX;
    // Smallest idle-slot count; ties go to more vectors per thread (fewer,
    // longer-running threads).  Vectors per thread are capped at 4 (16 for
    // the scalar path) while any tiling fits: holding more of the row costs
    // more registers than it buys (measured on the RMSNorm 16384 x 4096 and
    // ViT LayerNorm shapes).
    const int it_cap = vec_ok ? 4 : 16;
    for (int pass = 0; pass < 2 && best_tpr < 0; ++pass) {
        for (int tpr = 1; tpr <= 1024; tpr *= 2) {
            for (int i = 0; i < n_its; ++i) {
                const int it = its[i];
                if (pass == 0 && it > it_cap) continue;
                if ((int64_t)tpr * it < nv) continue;
                const int64_t waste = (int64_t)tpr * it - nv;
                if (waste < best_waste || (waste == best_waste && it > best_it)) {
                    best_waste = waste; best_tpr = tpr; best_it = it;
                }
            }
        }
    }
    if (best_tpr < 0) return false;
    // Blocks per CU.  The forward runs one block per row group (a grid up to
    // 64 blocks per CU, i.e. not persistent): it measured 2-3 % faster than
    // persistent grids on the RMSNorm 16384 x 4096 and ViT LayerNorm shapes.
    // The backward is persistent with 2 blocks per CU, because every block
    // adds a partial row for dw / db.
    int bpc = backward ? 2 : 64;
    int block = 256;
    int otpr, oit, obpc, oblock;
    if (env_override(&otpr, &oit, &obpc, &oblock) && otpr >= 1 && otpr <= 1024 && (otpr & (otpr - 1)) == 0 &&
        (int64_t)otpr * oit >= nv && obpc >= 1 && obpc <= (backward ? kMaxBwdBlocksPerCU : 4096)) {
        bool it_ok = false;
        for (int i = 0; i < n_its; ++i) it_ok |= its[i] == oit;
        if (it_ok) {
            best_tpr = otpr; best_it = oit; bpc = obpc;
            if (oblock == 64 || oblock == 128 || oblock == 256 || oblock == 512 || oblock == 1024) block = oblock;
        }
    }
    p->tpr = best_tpr;
    p->it = best_it;
    p->block = best_tpr >= block ? best_tpr : block;
    const int rpb = p->block / p->tpr;
    // The backward writes one partial row of dw (and db) per block, so a
    // block should cover at least two row groups; the forward has no
    // partials and takes one block per row group.  A backward of at most
    // kDirectRowGroups row groups runs as one block that writes dw / db
    // itself: a few extra row iterations cost less than the column-sum
    // kernel and its launch.
    const int64_t groups = ceil_div(M, rpb);
    // (Widening that block to 1024 threads to cut its row passes measured
    // 2.8x slower on LayerNorm 64 x 256; one row group per block where the
    // grid would still fit measured 13.0 -> 17.0 us on LayerNorm 4096 x 1000
    // bf16: the second group is what the next-row prefetch overlaps; a grid
    // trimmed so every block runs the same number of iterations measured
    // 25.4 -> 26.2 us on LayerNorm 25216 x 768 bf16: 451 blocks leave 61
    // CUs at half occupancy for the whole kernel, which costs more than a
    // last iteration run by a sixth of the grid.)
    const bool direct = backward && groups <= kDirectRowGroups;
    const int64_t needed = direct ? 1 : backward ? ceil_div(M, 2 * (int64_t)rpb) : groups;
    const int64_t cap = (int64_t)device_cu_count() * bpc;
    p->grid = (int)(needed < cap ? needed : cap);
    if (p->grid < 1) p->grid = 1;
    return true;
}

// The backward grid (= number of partial rows) never exceeds
// CUs * kMaxBwdBlocksPerCU nor M, so that bounds the workspace.
static int64_t max_partial_rows(int64_t M) {
    const int64_t cap = (int64_t)device_cu_count() * kMaxBwdBlocksPerCU;
    return M < cap ? (M > 0 ? M : 1) : cap;
}

static bool row_vec_ok(norm_dtype dt, int64_t N, std::initializer_list<const void *> ptrs) {
    if ((N * (int64_t)dtype_size(dt)) % 16 != 0) return false;
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return false;
    return true;
}

static norm_status check_rows(norm_dtype dt, int64_t M, int64_t N) {
    if (!dtype_ok(dt)) return NORM_ERR_DTYPE;
    if (M < 0 || N < 1) return NORM_ERR_SHAPE;
    if (N > (dt == NORM_F32 ? NORM_MAX_N_F32 : NORM_MAX_N_16)) return NORM_ERR_SHAPE;
    if (M > (int64_t)1 << 40) return NORM_ERR_SHAPE;
    return NORM_OK;
}

template <bool RMS>
static norm_status fwd_entry(norm_dtype dt, int64_t M, int64_t N, float eps, const void *x,
                             const void *w, const void *b, void *y, float *mean, float *rstd,
                             void *stream) {
    CallScope scope;
    norm_status st = check_rows(dt, M, N);
    if (st != NORM_OK) return st;
    if (!(eps >= 0.0f)) return NORM_ERR_ARG;
    if (M == 0) return NORM_OK;
    if (!x || !y) return NORM_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool vec = row_vec_ok(dt, N, {x, w, b, y});
    RowPlan p;
    if (!make_plan(dt, M, N, vec, false, &p)) return NORM_ERR_SHAPE;
    const int n = (int)N;
    return with_io_type(dt, [&](auto tag) {
        using T = typename decltype(tag)::type;
        constexpr int VW = 16 / (int)sizeof(T);
        return vec ? row_launch_fwd<T, RMS, VW>(p, s, x, w, b, y, mean, rstd, M, n, eps)
                   : row_launch_fwd<T, RMS, 1>(p, s, x, w, b, y, mean, rstd, M, n, eps);
    });
}

// ------------------------------------------------- static scratch (device)
// The no-allocation backward keeps its partial rows in this file-scope
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy (zero at load) until the process ends.  Host code must
// never pass the array's name to a kernel: on the host it is only a
// stand-in for the symbol.  The device address is taken once per device
// with hipGetSymbolAddress and used everywhere instead.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mutex;
}  // namespace

// The address of `scratch` on the device the stream `s` belongs to (the
// current device for the null stream); nullptr if the runtime fails.  The
// first use on a device takes the address with that device current and
// restores the caller's current device afterwards.
static void *static_scratch(hipStream_t s) {
    int dev = -1;
    if (s) {
        hipDevice_t d;
        if (hipStreamGetDevice(s, &d) != hipSuccess) return nullptr;
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return nullptr;
    }
    if (dev < 0 || dev >= kScratchDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void *addr = nullptr;
        const bool ok = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) == hipSuccess && addr;
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
        if (!ok) return nullptr;
        g_scratch_ptr[dev].store(addr, std::memory_order_release);
        p = addr;
    }
    return p;
}

static size_t bwd_ws_bytes(norm_dtype dt, int64_t M, int64_t N, int nparts) {
    if (check_rows(dt, M, N) != NORM_OK) return 0;
    return (size_t)max_partial_rows(M) * (size_t)N * sizeof(float) * (size_t)nparts;
}

// Where the backward's partial rows go: the caller's workspace (sized by
// the *_bwd_workspace_bytes query), or the library's static scratch (the
// no-allocation entry point), which must hold what the plan actually uses.
struct BwdScratch {
    bool is_static = false;
};

template <bool RMS>
static norm_status bwd_entry(norm_dtype dt, int64_t M, int64_t N, const void *dy, const void *x,
                             const void *w, const float *mean, const float *rstd, void *dx,
                             void *dw, void *db, void *ws, size_t ws_bytes, void *stream,
                             BwdScratch scratch_mode = {}) {
    CallScope scope;
    norm_status st = check_rows(dt, M, N);
    if (st != NORM_OK) return st;
    if (!dy || !x || !rstd || !dx || (!RMS && !mean)) {
        if (M == 0 && !(dw || db)) return NORM_OK;
        if (M > 0) return NORM_ERR_NULL;
    }
    const bool want = dw || db;
    if (!scratch_mode.is_static) {
        const size_t need = want ? bwd_ws_bytes(dt, M, N, RMS ? 1 : 2) : 0;
        if (want && (ws == nullptr || ws_bytes < need)) return NORM_ERR_WORKSPACE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int n = (int)N;
    if (M == 0) {
        // Empty batch: the parameter gradients are sums over no rows.
        if (!want) return NORM_OK;
        for (void *out : {dw, db}) {
            if (!out) continue;
            with_io_type(dt, [&](auto tag) {
                row_launch_zero<typename decltype(tag)::type>(s, out, n);
                return 0;
            });
        }
        return launch_status();
    }
    const bool vec = row_vec_ok(dt, N, {dy, x, w, dx});
    RowPlan p;
    if (!make_plan(dt, M, N, vec, true, &p)) return NORM_ERR_SHAPE;
    // One block: it writes dw / db directly.  Otherwise float32 partial
    // rows in the workspace, added by the column-sum kernel.
    const bool direct = p.grid == 1;
    size_t part_stride = (size_t)max_partial_rows(M) * N;  // floats from part_w to part_b
    if (scratch_mode.is_static) {
        // The static scratch holds exactly the partial rows this plan
        // writes; a shape that needs more is refused before anything runs.
        part_stride = (size_t)p.grid * N;
        const size_t used = (want && !direct) ? part_stride * sizeof(float) * (RMS ? 1 : 2) : 0;
        if (used > kScratchBytes) return NORM_ERR_WORKSPACE;
        if (used) {
            ws = static_scratch(s);
            if (!ws) return NORM_ERR_HIP;
        }
    }
    float *part_w = (dw && !direct) ? static_cast<float *>(ws) : nullptr;
    float *part_b = (!RMS && db && !direct) ? static_cast<float *>(ws) + part_stride : nullptr;
    void *dw_out = direct ? dw : nullptr;
    void *db_out = (direct && !RMS) ? db : nullptr;
    return with_io_type(dt, [&](auto tag) {
        using T = typename decltype(tag)::type;
        constexpr int VW = 16 / (int)sizeof(T);
        norm_status r = vec ? row_launch_bwd<T, RMS, VW>(p, s, dy, x, w, mean, rstd, dx, part_w, part_b,
                                                         dw_out, db_out, M, n)
                            : row_launch_bwd<T, RMS, 1>(p, s, dy, x, w, mean, rstd, dx, part_w, part_b,
                                                        dw_out, db_out, M, n);
        if (r != NORM_OK || !want || direct) return r;
        row_launch_colsum<T>(s, part_w, part_b, p.grid, n, dw, db);
        return launch_status();
    });
}

}  // namespace mi355norm

using namespace mi355norm;

extern "C" norm_status ln_fwd(norm_dtype dt, int64_t M, int64_t N, float eps, const void *x,
                              const void *w, const void *b, void *y, float *mean, float *rstd,
                              void *stream) {
    return fwd_entry<false>(dt, M, N, eps, x, w, b, y, mean, rstd, stream);
}

extern "C" size_t ln_bwd_workspace_bytes(norm_dtype dt, int64_t M, int64_t N) {
    return bwd_ws_bytes(dt, M, N, 2);
}

extern "C" norm_status ln_bwd(norm_dtype dt, int64_t M, int64_t N, const void *dy, const void *x,
                              const void *w, const float *mean, const float *rstd, void *dx,
                              void *dw, void *db, void *ws, size_t ws_bytes, void *stream) {
    return bwd_entry<false>(dt, M, N, dy, x, w, mean, rstd, dx, dw, db, ws, ws_bytes, stream);
}

extern "C" norm_status rms_fwd(norm_dtype dt, int64_t M, int64_t N, float eps, const void *x,
                               const void *w, void *y, float *rstd, void *stream) {
    return fwd_entry<true>(dt, M, N, eps, x, w, nullptr, y, nullptr, rstd, stream);
}

extern "C" size_t rms_bwd_workspace_bytes(norm_dtype dt, int64_t M, int64_t N) {
    return bwd_ws_bytes(dt, M, N, 1);
}

extern "C" norm_status rms_bwd(norm_dtype dt, int64_t M, int64_t N, const void *dy, const void *x,
                               const void *w, const float *rstd, void *dx, void *dw, void *ws,
                               size_t ws_bytes, void *stream) {
    return bwd_entry<true>(dt, M, N, dy, x, w, nullptr, rstd, dx, dw, nullptr, ws, ws_bytes, stream);
}

extern "C" norm_status rms_bwd_noalloc(norm_dtype dt, int64_t M, int64_t N, const void *dy, const void *x,
                                       const void *w, const float *rstd, void *dx, void *dw, void *stream) {
    return bwd_entry<true>(dt, M, N, dy, x, w, nullptr, rstd, dx, dw, nullptr, nullptr, 0, stream,
                           BwdScratch{true});
}
