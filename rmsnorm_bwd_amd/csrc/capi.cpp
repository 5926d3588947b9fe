// capi.cpp - the library's C ABI: argument validation (before any HIP call),
// launch planning, and dispatch to the kernels on the caller's stream.
//
// Pages cited, by title:
//   [I769] FlyDSL issue #769, "[Feature] Add rmsnorm backward (+ forward saves
//          rstd) to enable training / downstream (quack) integration"
//   [P800] FlyDSL PR #800, "[rmsnorm] Add fused-add / residual backward
//          (PR 2/3, #769)" - review-fix commit (shape/contiguity checks,
//          device guard) and fused-add commit (one dtype for all operands).
// The LayerNorm entry points follow [I769]'s PR sequence and status updates
// (forward saving mean and rstd, backward with dbias; weight and bias length
// checks and fp32 statistics).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "launch.h"
#include "plan.h"
#include "rmsnorm_mi355x.h"

namespace {

using rmsn::RowPlan;

bool dtype_ok(int d) { return d == RMSN_F32 || d == RMSN_F16 || d == RMSN_BF16; }
int esize(int d) { return d == RMSN_F32 ? 4 : 2; }
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(int64_t M, int64_t N) {
    if (M < 0 || M > INT32_MAX || N < 1 || N > RMSN_MAX_N) return RMSN_ERR_SHAPE;
    return RMSN_OK;
}

int check_eps(float eps) {
    if (!(eps >= 0.0f) || std::isinf(eps)) return RMSN_ERR_EPS;
    return RMSN_OK;
}

int check_flags(unsigned flags) {
    if (flags & ~7u) return RMSN_ERR_FLAGS;
    return RMSN_OK;
}

// Row strides: every row tensor that is present has N <= ld <= RMSN_MAX_LD.
struct Rows {
    const void *p;
    int64_t ld;
};

int check_strides(int64_t N, std::initializer_list<Rows> rows) {
    for (const Rows &r : rows)
        if (r.p && (r.ld < N || r.ld > RMSN_MAX_LD)) return RMSN_ERR_SHAPE;
    return RMSN_OK;
}

// The 16-byte vector path needs every row of every row tensor to start on a
// 16-byte boundary: the base and the row stride in bytes.
bool rows_vector_ok(std::initializer_list<Rows> rows, int es) {
    for (const Rows &r : rows)
        if (r.p && (!aligned(r.p, 16) || (r.ld * es) % 16 != 0)) return false;
    return true;
}

bool all_aligned(std::initializer_list<const void *> ptrs, uintptr_t a) {
    for (const void *p : ptrs)
        if (p && !aligned(p, a)) return false;
    return true;
}

// The pointer-only checks the pages' device guard stood for: each non-null
// pointer must be device memory of the current device.
int check_device(std::initializer_list<const void *> ptrs) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return RMSN_ERR_HIP;
    }
    for (const void *p : ptrs) {
        if (!p) continue;
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
            (void)hipGetLastError();
            return RMSN_ERR_DEVICE;
        }
        if (attr.type != hipMemoryTypeDevice || attr.device != dev) return RMSN_ERR_DEVICE;
    }
    return RMSN_OK;
}

static_assert(rmsn::DM_AUTO == RMSN_DGAMMA_AUTO && rmsn::DM_DETERMINISTIC == RMSN_DGAMMA_DETERMINISTIC &&
                  rmsn::DM_ATOMIC == RMSN_DGAMMA_ATOMIC && rmsn::DM_ONE_BLOCK == RMSN_DGAMMA_ONE_BLOCK,
              "dgamma mode values");

size_t workspace_for(int64_t M, int64_t N, int dtype, unsigned flags, bool vector_ok, int narrays) {
    RowPlan p;
    if (!rmsn::plan_rows(N, esize(dtype), vector_ok, &p)) return 0;
    return rmsn::bwd_workspace(M, N, p, flags & 3u, narrays);
}

// The public workspace query: alignment is not known here, so it answers for
// whichever row plan needs more.
size_t workspace_query(int64_t M, int64_t N, int dtype, unsigned flags, int narrays) {
    if (!dtype_ok(dtype) || check_shape(M, N) || check_flags(flags)) return 0;
    size_t a = workspace_for(M, N, dtype, flags, true, narrays);
    size_t b = workspace_for(M, N, dtype, flags, false, narrays);
    return a > b ? a : b;
}

// Backward of RMSNorm (mean == NULL) or LayerNorm (mean != NULL, with
// dbeta_f32 / dbeta).
int bwd_common(const void *x, int64_t ldx, const void *gamma, const void *dy, int64_t lddy, const void *dres,
               int64_t lddres, const float *mean, const float *rstd, void *dx, int64_t lddx, float *dgamma_f32,
               void *dgamma, float *dbeta_f32, void *dbeta, void *workspace, size_t workspace_bytes, int64_t M,
               int64_t N, int dtype, unsigned flags, void *stream, bool layer, bool own_scratch = false) {
    if (!dtype_ok(dtype)) return RMSN_ERR_DTYPE;
    if (int st = check_shape(M, N)) return st;
    if (int st = check_flags(flags)) return st;
    if (!gamma || !dgamma_f32 || !workspace) return RMSN_ERR_NULL;
    if (layer && !dbeta_f32) return RMSN_ERR_NULL;
    if (M > 0 && (!x || !dy || !rstd || !dx)) return RMSN_ERR_NULL;
    if (layer && M > 0 && !mean) return RMSN_ERR_NULL;
    if (M > 0) {
        if (int st = check_strides(N, {{x, ldx}, {dy, lddy}, {dres, lddres}, {dx, lddx}})) return st;
    }
    const int es = esize(dtype);
    if (!all_aligned({x, gamma, dy, dres, dx, dgamma, dbeta}, es) ||
        !all_aligned({rstd, mean, dgamma_f32, dbeta_f32}, 4) || !aligned(workspace, 256))
        return RMSN_ERR_ALIGN;
    const bool vector_ok =
        aligned(gamma, 16) && rows_vector_ok({{x, ldx}, {dy, lddy}, {dres, lddres}, {dx, lddx}}, es);
    RowPlan p;
    if (!rmsn::plan_rows(N, es, vector_ok, &p)) return RMSN_ERR_SHAPE;
    const int64_t grid = rmsn::bwd_blocks(M, N, p, !layer && dres != nullptr, flags & 3u);
    const int mode = rmsn::resolve_mode(flags & 3u, grid);
    // the public query's answer, whatever plan the pointers select, so a
    // buffer sized by the query is always accepted and nothing less is
    if (workspace_bytes < workspace_query(M, N, dtype, flags, layer ? 2 : 1)) return RMSN_ERR_WORKSPACE;
    if (flags & RMSN_CHECK_DEVICE) {
        // the library's own scratch is on the current device by construction
        if (int st = check_device({x, gamma, dy, dres, mean, rstd, dx, dgamma_f32, dgamma, dbeta_f32, dbeta,
                                   own_scratch ? nullptr : workspace}))
            return st;
    }
    rmsn::BwdArgs a;
    a.x = x;
    a.gamma = gamma;
    a.dy = dy;
    a.dres = layer ? nullptr : dres;
    a.rstd = rstd;
    a.mean = layer ? mean : nullptr;
    a.dx = dx;
    a.partials = nullptr;
    a.dgamma_f32 = dgamma_f32;
    a.dgamma = dgamma;
    a.dbeta_f32 = layer ? dbeta_f32 : nullptr;
    a.dbeta = layer ? dbeta : nullptr;
    a.layer = layer;
    a.M = M;
    a.N = (int)N;
    a.ldx = ldx;
    a.lddy = lddy;
    a.lddres = lddres;
    a.lddx = lddx;
    a.mode = mode;
    hipError_t e = rmsn::launch_bwd(dtype, p, a, (int)grid, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RMSN_OK : RMSN_ERR_HIP;
}


// Forward of RMSNorm (plain or fused-add) or, with `layer`, LayerNorm (beta
// nullable, mean saved).
int fwd_common(const void *x, int64_t ldx, const void *residual, int64_t ldres, const void *gamma,
               const void *beta, void *y, int64_t ldy, void *residual_out, int64_t ldres_out, float *mean,
               float *rstd, int64_t M, int64_t N, float eps, int dtype, void *stream, bool fused, bool layer) {
    if (!dtype_ok(dtype)) return RMSN_ERR_DTYPE;
    if (int st = check_shape(M, N)) return st;
    if (int st = check_eps(eps)) return st;
    if (!gamma) return RMSN_ERR_NULL;
    if (M > 0 && (!x || !y || !rstd)) return RMSN_ERR_NULL;
    if (fused && M > 0 && (!residual || !residual_out)) return RMSN_ERR_NULL;
    if (layer && M > 0 && !mean) return RMSN_ERR_NULL;
    if (!fused) residual = residual_out = nullptr;
    if (M > 0) {
        if (int st = check_strides(N, {{x, ldx}, {residual, ldres}, {y, ldy}, {residual_out, ldres_out}}))
            return st;
    }
    const int es = esize(dtype);
    if (!all_aligned({x, residual, gamma, beta, y, residual_out}, es) || !all_aligned({rstd, mean}, 4))
        return RMSN_ERR_ALIGN;
    const bool vector_ok = all_aligned({gamma, beta}, 16) &&
                           rows_vector_ok({{x, ldx}, {residual, ldres}, {y, ldy}, {residual_out, ldres_out}}, es);
    RowPlan p;
    if (!rmsn::plan_rows(N, es, vector_ok, &p)) return RMSN_ERR_SHAPE;
    rmsn::FwdArgs a;
    a.x = x;
    a.residual = fused ? residual : nullptr;
    a.gamma = gamma;
    a.beta = layer ? beta : nullptr;
    a.y = y;
    a.residual_out = fused ? residual_out : nullptr;
    a.mean = layer ? mean : nullptr;
    a.rstd = rstd;
    a.M = M;
    a.N = (int)N;
    a.ldx = ldx;
    a.ldres = ldres;
    a.ldy = ldy;
    a.ldres_out = ldres_out;
    a.eps = eps;
    hipError_t e = rmsn::launch_fwd(dtype, p, a, (int)rmsn::fwd_blocks(M, N, p, fused && !layer),
                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RMSN_OK : RMSN_ERR_HIP;
}

}  // namespace

extern "C" {

int rmsnorm_fwd_rstd(const void *x, const void *gamma, void *y, float *rstd, int64_t M, int64_t N, float eps,
                     int dtype, void *stream) {
    return fwd_common(x, N, nullptr, N, gamma, nullptr, y, N, nullptr, N, nullptr, rstd, M, N, eps, dtype, stream,
                      false, false);
}

int rmsnorm_fwd_rstd_strided(const void *x, int64_t ldx, const void *gamma, void *y, int64_t ldy, float *rstd,
                             int64_t M, int64_t N, float eps, int dtype, void *stream) {
    return fwd_common(x, ldx, nullptr, N, gamma, nullptr, y, ldy, nullptr, N, nullptr, rstd, M, N, eps, dtype,
                      stream, false, false);
}

int fused_add_rmsnorm_fwd_rstd(const void *x, const void *residual, const void *gamma, void *out,
                               void *residual_out, float *rstd, int64_t M, int64_t N, float eps, int dtype,
                               void *stream) {
    return fwd_common(x, N, residual, N, gamma, nullptr, out, N, residual_out, N, nullptr, rstd, M, N, eps, dtype,
                      stream, true, false);
}

int fused_add_rmsnorm_fwd_rstd_strided(const void *x, int64_t ldx, const void *residual, int64_t ldres,
                                       const void *gamma, void *out, int64_t ldout, void *residual_out,
                                       int64_t ldres_out, float *rstd, int64_t M, int64_t N, float eps, int dtype,
                                       void *stream) {
    return fwd_common(x, ldx, residual, ldres, gamma, nullptr, out, ldout, residual_out, ldres_out, nullptr, rstd,
                      M, N, eps, dtype, stream, true, false);
}

size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, unsigned flags) {
    return workspace_query(M, N, dtype, flags, 1);
}

int rmsnorm_bwd(const void *x, const void *gamma, const void *dy, const float *rstd, void *dx,
                float *dgamma_f32, void *dgamma, void *workspace, size_t workspace_bytes, int64_t M, int64_t N,
                int dtype, unsigned flags, void *stream) {
    return bwd_common(x, N, gamma, dy, N, nullptr, N, nullptr, rstd, dx, N, dgamma_f32, dgamma, nullptr, nullptr,
                      workspace, workspace_bytes, M, N, dtype, flags, stream, false);
}

int rmsnorm_bwd_no_alloc(const void *x, const void *gamma, const void *dy, const float *rstd, void *dx,
                         float *dgamma_f32, void *dgamma, int64_t M, int64_t N, int dtype, unsigned flags,
                         void *stream) {
    // 0 for arguments rmsnorm_bwd rejects: it then reports which, before any
    // HIP call (its dtype, shape and flags checks come first)
    const size_t need = workspace_query(M, N, dtype, flags, 1);
    if (need > (size_t)RMSN_NO_ALLOC_SCRATCH_BYTES) return RMSN_ERR_SCRATCH;
    void *scratch = nullptr;
    if (need != 0 && rmsn::device_scratch(&scratch) != hipSuccess) return RMSN_ERR_HIP;
    return bwd_common(x, N, gamma, dy, N, nullptr, N, nullptr, rstd, dx, N, dgamma_f32, dgamma, nullptr, nullptr,
                      scratch, RMSN_NO_ALLOC_SCRATCH_BYTES, M, N, dtype, flags, stream, false, true);
}

int rmsnorm_bwd_strided(const void *x, int64_t ldx, const void *gamma, const void *dy, int64_t lddy,
                        const float *rstd, void *dx, int64_t lddx, float *dgamma_f32, void *dgamma,
                        void *workspace, size_t workspace_bytes, int64_t M, int64_t N, int dtype, unsigned flags,
                        void *stream) {
    return bwd_common(x, ldx, gamma, dy, lddy, nullptr, N, nullptr, rstd, dx, lddx, dgamma_f32, dgamma, nullptr,
                      nullptr, workspace, workspace_bytes, M, N, dtype, flags, stream, false);
}

int fused_add_rmsnorm_bwd(const void *added, const void *gamma, const void *dy, const void *dresidual_out,
                          const float *rstd, void *dx, float *dgamma_f32, void *dgamma, void *workspace,
                          size_t workspace_bytes, int64_t M, int64_t N, int dtype, unsigned flags,
                          void *stream) {
    return bwd_common(added, N, gamma, dy, N, dresidual_out, N, nullptr, rstd, dx, N, dgamma_f32, dgamma, nullptr,
                      nullptr, workspace, workspace_bytes, M, N, dtype, flags, stream, false);
}

int fused_add_rmsnorm_bwd_strided(const void *added, int64_t ldadded, const void *gamma, const void *dy,
                                  int64_t lddy, const void *dresidual_out, int64_t lddres, const float *rstd,
                                  void *dx, int64_t lddx, float *dgamma_f32, void *dgamma, void *workspace,
                                  size_t workspace_bytes, int64_t M, int64_t N, int dtype, unsigned flags,
                                  void *stream) {
    return bwd_common(added, ldadded, gamma, dy, lddy, dresidual_out, lddres, nullptr, rstd, dx, lddx, dgamma_f32,
                      dgamma, nullptr, nullptr, workspace, workspace_bytes, M, N, dtype, flags, stream, false);
}

int layernorm_fwd_stats(const void *x, const void *gamma, const void *beta, void *y, float *mean, float *rstd,
                        int64_t M, int64_t N, float eps, int dtype, void *stream) {
    return fwd_common(x, N, nullptr, N, gamma, beta, y, N, nullptr, N, mean, rstd, M, N, eps, dtype, stream, false,
                      true);
}

int layernorm_fwd_stats_strided(const void *x, int64_t ldx, const void *gamma, const void *beta, void *y,
                                int64_t ldy, float *mean, float *rstd, int64_t M, int64_t N, float eps, int dtype,
                                void *stream) {
    return fwd_common(x, ldx, nullptr, N, gamma, beta, y, ldy, nullptr, N, mean, rstd, M, N, eps, dtype, stream,
                      false, true);
}

size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, unsigned flags) {
    return workspace_query(M, N, dtype, flags, 2);
}

int layernorm_bwd(const void *x, const void *gamma, const void *dy, const float *mean, const float *rstd,
                  void *dx, float *dgamma_f32, float *dbeta_f32, void *dgamma, void *dbeta, void *workspace,
                  size_t workspace_bytes, int64_t M, int64_t N, int dtype, unsigned flags, void *stream) {
    return bwd_common(x, N, gamma, dy, N, nullptr, N, mean, rstd, dx, N, dgamma_f32, dgamma, dbeta_f32, dbeta,
                      workspace, workspace_bytes, M, N, dtype, flags, stream, true);
}

int layernorm_bwd_strided(const void *x, int64_t ldx, const void *gamma, const void *dy, int64_t lddy,
                          const float *mean, const float *rstd, void *dx, int64_t lddx, float *dgamma_f32,
                          float *dbeta_f32, void *dgamma, void *dbeta, void *workspace, size_t workspace_bytes,
                          int64_t M, int64_t N, int dtype, unsigned flags, void *stream) {
    return bwd_common(x, ldx, gamma, dy, lddy, nullptr, N, mean, rstd, dx, lddx, dgamma_f32, dgamma, dbeta_f32,
                      dbeta, workspace, workspace_bytes, M, N, dtype, flags, stream, true);
}

const char *rmsn_status_string(int status) {
    switch (status) {
    case RMSN_OK: return "ok";
    case RMSN_ERR_NULL: return "a required pointer is NULL";
    case RMSN_ERR_SHAPE: return "M or N out of range";
    case RMSN_ERR_DTYPE: return "unknown dtype";
    case RMSN_ERR_EPS: return "eps must be finite and >= 0";
    case RMSN_ERR_WORKSPACE: return "workspace missing or too small";
    case RMSN_ERR_FLAGS: return "unknown flags";
    case RMSN_ERR_DEVICE: return "pointer is not on the current device";
    case RMSN_ERR_HIP: return "HIP runtime error";
    case RMSN_ERR_ALIGN: return "pointer not aligned to its element size";
    case RMSN_ERR_SCRATCH: return "the call needs more scratch than the library's static array holds";
    default: return "unknown status";
    }
}

}  // extern "C"
