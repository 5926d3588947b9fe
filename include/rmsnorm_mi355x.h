/*
 * rmsnorm_mi355x.h - C ABI of the MI355X (gfx950) RMSNorm library: the
 * forward passes that save a per-row rstd, and the backward passes (dx and the
 * weight gradient dgamma), plain and fused-add (prenorm residual); and the
 * LayerNorm forward (saving mean and rstd) and backward (dx, dgamma, dbeta).
 *
 * Pages cited, by title:
 *   [I769] FlyDSL issue #769, "[Feature] Add rmsnorm backward (+ forward saves
 *          rstd) to enable training / downstream (quack) integration"
 *   [P800] FlyDSL PR #800, "[rmsnorm] Add fused-add / residual backward
 *          (PR 2/3, #769)"
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer on the calling thread's current
 *     HIP device. The caller owns every buffer, the workspace included. The
 *     library allocates nothing, frees nothing and never synchronises (the
 *     one exception, rmsnorm_bwd_no_alloc's scratch, is a static array of
 *     the loaded library, not an allocation made by a call).
 *   - Row tensors are (M, N), row-major and contiguous (row stride N
 *     elements); gamma, beta and the weight-gradient outputs have N
 *     elements; rstd and mean have M. Each entry point has a *_strided twin
 *     that takes a row stride ld (elements) per row tensor, N <= ld <=
 *     RMSN_MAX_LD: row i of that tensor starts ld * i elements after its
 *     base, elements inside a row stay contiguous, and the gaps between
 *     rows are neither read nor written. Other arguments, results and
 *     errors are those of the contiguous entry point (a stride out of range
 *     is RMSN_ERR_SHAPE); rows take the 16-byte vector path only if every
 *     row of every row tensor starts on a 16-byte boundary.
 *   - One element dtype (rmsn_dtype_t) covers every row tensor, gamma and
 *     beta. rstd, mean, dgamma_f32 and dbeta_f32 are always float32.
 *   - Pointers need only element alignment. Rows whose start is not 16-byte
 *     aligned, or N that is not a multiple of the 16-byte vector, take a
 *     slower element-wise path with identical results.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the null stream). A status of RMSN_OK means the launch was enqueued.
 *     Only kernels are enqueued (no memset or copy nodes, no allocation),
 *     so calls may be captured into a HIP graph and replayed; the workspace
 *     carries no state from one call to the next.
 *   - Arguments are validated before anything is enqueued; a rejected call
 *     writes nothing. Inputs and outputs must not overlap, except where an
 *     entry point says so.
 *   - Limits: 0 <= M <= 2^31 - 1, 1 <= N <= RMSN_MAX_N. Rows of up to 16384
 *     elements stay in registers between the passes over them; longer rows
 *     are read once by the forwards and twice by the backwards (the second
 *     read mostly from the caches), with identical results.
 */
#ifndef RMSNORM_MI355X_H
#define RMSNORM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMSN_MAX_N 32768
/* Largest row stride, in elements, of the *_strided entry points. */
#define RMSN_MAX_LD (1LL << 24)

typedef enum { RMSN_F32 = 0, RMSN_F16 = 1, RMSN_BF16 = 2 } rmsn_dtype_t;

typedef enum {
    RMSN_OK = 0,
    RMSN_ERR_NULL = 1,      /* a required pointer is NULL */
    RMSN_ERR_SHAPE = 2,     /* M < 0, M too large, N < 1 or N > RMSN_MAX_N */
    RMSN_ERR_DTYPE = 3,     /* unknown dtype code */
    RMSN_ERR_EPS = 4,       /* eps is negative, NaN or infinite */
    RMSN_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the query */
    RMSN_ERR_FLAGS = 6,     /* unknown flag bits */
    RMSN_ERR_DEVICE = 7,    /* a pointer is not on the current device */
    RMSN_ERR_HIP = 8,       /* the HIP runtime reported an error */
    RMSN_ERR_ALIGN = 9,     /* a pointer is not aligned to its element size */
    RMSN_ERR_SCRATCH = 10   /* rmsnorm_bwd_no_alloc: the call needs more scratch
                               than the library's static array holds */
} rmsn_status_t;

/* Flags of the backward entry points. The low two bits choose how dgamma's
 * per-workgroup fp32 partials are combined across workgroups:
 *   RMSN_DGAMMA_AUTO           the library's measured default: one workgroup
 *                              writing the gradients itself for small
 *                              problems (N <= 1024 and M * N <= 8192, or
 *                              M <= 2 and N <= 8192), the deterministic
 *                              two-stage sum otherwise;
 *   RMSN_DGAMMA_DETERMINISTIC  partials go to the workspace and a second
 *                              kernel sums them in a fixed order: the same
 *                              inputs give the same bits on every call;
 *   RMSN_DGAMMA_ATOMIC         partials are added with fp32 atomics into
 *                              dgamma_f32; the sum order, so the last bits of
 *                              dgamma, may vary from call to call. These are
 *                              the hardware fp32 adds of device memory:
 *                              dgamma_f32 (and dbeta_f32) must be ordinary
 *                              device allocations (hipMalloc), not host,
 *                              managed or fine-grained memory, where such
 *                              adds do not take effect;
 *   RMSN_DGAMMA_ONE_BLOCK      the whole backward in one workgroup, which
 *                              writes the gradients itself: one launch,
 *                              deterministic, meant for problems of a few
 *                              short rows (one CU does all the work).
 * An explicit mode is honoured at every size. RMSN_CHECK_DEVICE
 * additionally checks, with the HIP runtime, that every pointer belongs to
 * the current device (the fault the pages' device guard fixed: [P800]
 * review-fix commit). */
enum {
    RMSN_DGAMMA_AUTO = 0,
    RMSN_DGAMMA_DETERMINISTIC = 1,
    RMSN_DGAMMA_ATOMIC = 2,
    RMSN_DGAMMA_ONE_BLOCK = 3,
    RMSN_CHECK_DEVICE = 4
};

/* RMSNorm forward that also saves rstd.
 * [I769] Scope/tasks, item 2, and Implementation plan (PR 1): the forward
 * already forms rrms = rsqrt(mean(x^2) + eps) per row; it now also stores it.
 * [P800] PR-1 commit: rstd is 1/RMS, fp32, shape (M,); eps is honoured
 * (review-fix commit).
 *   y[i,j]  = x[i,j] * rstd[i] * gamma[j], rounded once to the dtype
 *   rstd[i] = 1 / sqrt(sum_j x[i,j]^2 / N + eps), fp32
 * In: x (M,N), gamma (N). Out: y (M,N), rstd (M). eps >= 0 and finite. */
int rmsnorm_fwd_rstd(const void *x, const void *gamma, void *y, float *rstd,
                     int64_t M, int64_t N, float eps, int dtype, void *stream);

/* Fused-add (prenorm) forward that saves rstd. [P800] fused-add commit and
 * PR body: added = x + residual is returned as residual_out, normalised into
 * out, and its per-row rstd is saved.
 *   residual_out[i,j] = x[i,j] + residual[i,j] (fp32 sum, one rounding)
 *   rstd and out as in rmsnorm_fwd_rstd, taken over residual_out as stored.
 * In: x, residual (M,N), gamma (N). Out: out, residual_out (M,N), rstd (M).
 * residual_out may be the same buffer as residual (in-place update); no other
 * overlap is allowed. */
int fused_add_rmsnorm_fwd_rstd(const void *x, const void *residual, const void *gamma,
                               void *out, void *residual_out, float *rstd,
                               int64_t M, int64_t N, float eps, int dtype, void *stream);

/* Bytes of device workspace the backward entry points need for (M, N, dtype,
 * flags). The answer never exceeds 256 + 256 * N16 * 4 bytes, N16 being N
 * rounded up to a multiple of 16. The caller allocates at least this much,
 * 256-byte aligned, and passes it to rmsnorm_bwd / fused_add_rmsnorm_bwd.
 * Returns 0 for arguments the backward would reject. Makes no HIP call. */
size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, unsigned flags);

/* RMSNorm backward. [I769] Implementation plan, Math; [P800] PR-1 commit:
 * with x_hat = x * rstd and wdy = dy * gamma, per row
 *   c1       = (1/N) sum_j x_hat[j] * wdy[j]            (fp32)
 *   dx[i,j]  = (wdy[j] - x_hat[j] * c1) * rstd[i]        (rounded once)
 *   dgamma_f32[j] = sum_i dy[i,j] * x_hat[i,j]           (fp32, over all M rows)
 *   dgamma[j] = dgamma_f32[j] rounded to the dtype (only if dgamma != NULL)
 * In: x, dy (M,N); gamma (N); rstd (M, fp32, as saved by a forward).
 * Out: dx (M,N); dgamma_f32 (N, fp32, overwritten: the caller does not
 * zero it); dgamma (N, dtype, nullable). With M = 0, dgamma is all zeros.
 * workspace: device memory of at least rmsnorm_bwd_workspace_bytes(M, N,
 * dtype, flags) bytes, 256-byte aligned, for this call's exclusive use until
 * the call's work on `stream` completes; its contents on entry do not
 * matter. flags: one RMSN_DGAMMA_* mode, optionally | RMSN_CHECK_DEVICE. */
int rmsnorm_bwd(const void *x, const void *gamma, const void *dy, const float *rstd,
                void *dx, float *dgamma_f32, void *dgamma,
                void *workspace, size_t workspace_bytes,
                int64_t M, int64_t N, int dtype, unsigned flags, void *stream);

/* Fused-add (prenorm) RMSNorm backward. [P800] fused-add commit and PR body:
 * the plain backward taken over added (= residual_out of the forward), plus
 * the gradient arriving at residual_out:
 *   dx[i,j] = (wdy[j] - a_hat[j] * c1) * rstd[i] + dresidual_out[i,j]
 * Because added = x + residual, this one tensor is both the gradient of x
 * and of residual: it is stored once and the caller uses it for both.
 * dresidual_out may be NULL, which stands for zeros. dgamma is the plain
 * backward's dgamma over added. Other arguments as in rmsnorm_bwd. */
int fused_add_rmsnorm_bwd(const void *added, const void *gamma, const void *dy,
                          const void *dresidual_out, const float *rstd,
                          void *dx, float *dgamma_f32, void *dgamma,
                          void *workspace, size_t workspace_bytes,
                          int64_t M, int64_t N, int dtype, unsigned flags, void *stream);

/* LayerNorm forward that saves its statistics. [I769] PR sequence and status
 * updates: the LayerNorm follow-up's forward saves mean and rstd (fp32), with
 * weight and bias length checks. Taken as the textbook layer norm:
 *   mean[i] = (1/N) sum_j x[i,j]                         (fp32, stored)
 *   rstd[i] = 1/sqrt((1/N) sum_j (x[i,j] - mean[i])^2 + eps)   (fp32, stored)
 *   y[i,j]  = (x[i,j] - mean[i]) * rstd[i] * gamma[j] + beta[j]   (rounded once)
 * In: x (M,N); gamma (N); beta (N) or NULL for zeros. Out: y (M,N), mean (M),
 * rstd (M). Errors as rmsnorm_fwd_rstd. */
int layernorm_fwd_stats(const void *x, const void *gamma, const void *beta, void *y, float *mean,
                        float *rstd, int64_t M, int64_t N, float eps, int dtype, void *stream);

/* Bytes of workspace layernorm_bwd needs: as rmsnorm_bwd_workspace_bytes with
 * a second array of partials (dbeta); never more than 256 + 2 * 256 * N16 * 4.
 * Returns 0 for arguments the backward would reject. Makes no HIP call. */
size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, unsigned flags);

/* LayerNorm backward. [I769] PR sequence and status updates: the RMSNorm
 * backward's approach plus mean handling and the bias gradient. Per row,
 * with x_hat = (x - mean) * rstd and wdy = dy * gamma (fp32),
 *   c1 = (1/N) sum_j x_hat[j] * wdy[j],  c2 = (1/N) sum_j wdy[j]
 *   dx[i,j] = (wdy[j] - x_hat[j] * c1 - c2) * rstd[i]    (rounded once)
 *   dgamma_f32[j] = sum_i dy[i,j] * x_hat[i,j],  dbeta_f32[j] = sum_i dy[i,j]
 *   dgamma, dbeta = the fp32 sums rounded to the dtype (each nullable)
 * In: x, dy (M,N); gamma (N); mean, rstd (M, fp32, as saved by
 * layernorm_fwd_stats). Out: dx (M,N); dgamma_f32 and dbeta_f32 (N fp32,
 * overwritten); dgamma, dbeta (N, dtype, nullable). Workspace, flags, modes
 * and errors as rmsnorm_bwd (the modes govern both sums). */
int layernorm_bwd(const void *x, const void *gamma, const void *dy, const float *mean, const float *rstd,
                  void *dx, float *dgamma_f32, float *dbeta_f32, void *dgamma, void *dbeta,
                  void *workspace, size_t workspace_bytes, int64_t M, int64_t N, int dtype,
                  unsigned flags, void *stream);

/* Strided twins (row strides in elements; see the conventions above). The
 * gaps between rows are the caller's views, e.g. a slice of wider rows, a
 * column block of a packed tensor, or a transposed leading dimension; the
 * pages assert contiguity ([P800] review-fix commit), which these relax. */
int rmsnorm_fwd_rstd_strided(const void *x, int64_t ldx, const void *gamma, void *y, int64_t ldy,
                             float *rstd, int64_t M, int64_t N, float eps, int dtype, void *stream);
int fused_add_rmsnorm_fwd_rstd_strided(const void *x, int64_t ldx, const void *residual, int64_t ldres,
                                       const void *gamma, void *out, int64_t ldout, void *residual_out,
                                       int64_t ldres_out, float *rstd, int64_t M, int64_t N, float eps,
                                       int dtype, void *stream);
int rmsnorm_bwd_strided(const void *x, int64_t ldx, const void *gamma, const void *dy, int64_t lddy,
                        const float *rstd, void *dx, int64_t lddx, float *dgamma_f32, void *dgamma,
                        void *workspace, size_t workspace_bytes, int64_t M, int64_t N, int dtype,
                        unsigned flags, void *stream);
int fused_add_rmsnorm_bwd_strided(const void *added, int64_t ldadded, const void *gamma, const void *dy,
                                  int64_t lddy, const void *dresidual_out, int64_t lddres,
                                  const float *rstd, void *dx, int64_t lddx, float *dgamma_f32,
                                  void *dgamma, void *workspace, size_t workspace_bytes, int64_t M,
                                  int64_t N, int dtype, unsigned flags, void *stream);
int layernorm_fwd_stats_strided(const void *x, int64_t ldx, const void *gamma, const void *beta, void *y,
                                int64_t ldy, float *mean, float *rstd, int64_t M, int64_t N, float eps,
                                int dtype, void *stream);
int layernorm_bwd_strided(const void *x, int64_t ldx, const void *gamma, const void *dy, int64_t lddy,
                          const float *mean, const float *rstd, void *dx, int64_t lddx,
                          float *dgamma_f32, float *dbeta_f32, void *dgamma, void *dbeta,
                          void *workspace, size_t workspace_bytes, int64_t M, int64_t N, int dtype,
                          unsigned flags, void *stream);

/* Bytes of device memory the library holds on each GPU it runs on, for
 * rmsnorm_bwd_no_alloc: a 256-byte header and the fp32 dgamma partials of up
 * to 256 workgroups for rows of up to 8192 elements (8 MiB + 256 bytes). */
#define RMSN_NO_ALLOC_SCRATCH_BYTES (256 + 256 * 8192 * 4)

/* rmsnorm_bwd with no workspace argument, for callers that cannot allocate
 * device memory: code under HIP-graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It calls no allocating routine; its
 * scratch is a static device array of RMSN_NO_ALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (its address
 * is looked up once per device, on the first call with that device
 * current). Every call on one GPU shares that array and it keeps the last
 * call's contents: calls ordered on one stream are safe, but calls that
 * overlap on one GPU (other streams, other threads) race and give wrong
 * results. Nothing in it has to start at zero: a call writes every partial
 * it reads. A call whose workspace need (rmsnorm_bwd_workspace_bytes of the
 * same M, N, dtype and flags) exceeds RMSN_NO_ALLOC_SCRATCH_BYTES returns
 * RMSN_ERR_SCRATCH before anything is enqueued; only rows of more than 8192
 * elements in the default and deterministic modes can need that much (the
 * atomic mode and one-workgroup calls need only the header). Other
 * arguments, results and errors are those of rmsnorm_bwd, and for the same
 * arguments the results are bit for bit those of rmsnorm_bwd. */
int rmsnorm_bwd_no_alloc(const void *x, const void *gamma, const void *dy, const float *rstd,
                         void *dx, float *dgamma_f32, void *dgamma, int64_t M, int64_t N, int dtype,
                         unsigned flags, void *stream);

/* A static, human-readable name for a status code. */
const char *rmsn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MI355X_H */
