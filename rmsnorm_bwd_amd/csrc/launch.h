// launch.h - kernel argument blocks and the launchers the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace rmsn {

struct BwdArgs {
    const void *x;       // x, or `added` for the fused variant (M, N)
    const void *gamma;   // (N)
    const void *dy;      // (M, N)
    const void *dres;    // dresidual_out (M, N), or null
    const float *rstd;   // (M)
    const float *mean;   // (M) for LayerNorm, else null (RMSNorm)
    void *dx;            // (M, N)
    float *partials;     // tiled fp32 block partials (partial mode), set by the launcher
    float *dgamma_f32;   // (N)
    void *dgamma;        // (N) in the dtype, or null
    float *dbeta_f32;    // (N), LayerNorm only
    void *dbeta;         // (N) in the dtype, or null; LayerNorm only
    int64_t M;
    int N;
    int64_t ldx, lddy, lddres, lddx;  // row strides in elements (N for contiguous rows)
    int mode;            // DG_DIRECT / DG_PARTIAL / DG_ATOMIC
    bool layer;          // LayerNorm (mean, dbeta) rather than RMSNorm
};

struct FwdArgs {
    const void *x;         // (M, N)
    const void *residual;  // (M, N), or null for the plain forward
    const void *gamma;     // (N)
    const void *beta;      // (N) LayerNorm bias, or null (zeros)
    void *y;               // (M, N)
    void *residual_out;    // (M, N) when residual is given
    float *mean;           // (M) for LayerNorm, else null (RMSNorm)
    float *rstd;           // (M)
    int64_t M;
    int N;
    int64_t ldx, ldres, ldy, ldres_out;  // row strides in elements (N for contiguous rows)
    float eps;
};

// Enqueue the backward on stream s: the main kernel with `grid` blocks, plus
// the dgamma finalize, zero-fill or cast kernels its mode needs.
hipError_t launch_bwd(int dtype, const RowPlan &p, const BwdArgs &a, int grid, void *workspace,
                      hipStream_t s);

// Device address, on the current device, of the static scratch array of
// rmsnorm_bwd_no_alloc (looked up once per device, then remembered).
hipError_t device_scratch(void **ptr);

// Enqueue the forward on stream s with `grid` blocks.
hipError_t launch_fwd(int dtype, const RowPlan &p, const FwdArgs &a, int grid, hipStream_t s);

// The main pass of the backward, and the forward, for long rows
// (p.long_row): long_rows.hip.
hipError_t launch_bwd_long(int dtype, const RowPlan &p, const BwdArgs &a, int grid, hipStream_t s);
hipError_t launch_fwd_long(int dtype, const RowPlan &p, const FwdArgs &a, int grid, hipStream_t s);
// The fused (a.dres set) or LayerNorm (a.layer) backward of 16-bit rows on
// 16-byte chunks, four a thread of 512 (at most 16384 elements), by the
// long-row kernel that loads a block's next row during the current one:
// long_rows.hip. Other calls fail with hipErrorInvalidValue.
hipError_t launch_bwd_next_row(int dtype, const BwdArgs &a, int grid, hipStream_t s);

}  // namespace rmsn
