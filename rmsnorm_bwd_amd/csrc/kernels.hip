// kernels.hip - gfx950 kernels for RMSNorm forward (saving rstd) and backward,
// plain and fused-add, and their launchers.
//
// Pages cited, by title:
//   [I769] FlyDSL issue #769, "[Feature] Add rmsnorm backward (+ forward saves
//          rstd) to enable training / downstream (quack) integration"
//   [P800] FlyDSL PR #800, "[rmsnorm] Add fused-add / residual backward
//          (PR 2/3, #769)"
//
// Design. The work is bound by HBM bandwidth (about 7 flops per element
// against 6-8 bytes), so every kernel is built to move each byte once:
//   - rows are read with 16-byte loads (global_load_dwordx4) by consecutive
//     lanes, and each row stays in VGPRs between the reduction and the
//     output pass, so the backward reads x and dy from HBM exactly once;
//   - the next row's loads are issued before the current row is reduced, so
//     HBM requests stay in flight across the cross-lane sum;
//   - per-row sums use DPP and ds_swizzle inside a wavefront; rows wider than
//     64 threads add one LDS exchange;
//   - the backward is a persistent grid of at most 256 blocks, one per CU;
//     each block folds dy * x_hat for all of its rows into fp32 registers, so
//     dgamma leaves a block as a single (N,) fp32 partial rather than as M*N
//     atomics. A second, fixed-order kernel sums the partials (deterministic
//     mode), or the partials are added with fp32 atomics (atomic mode).
// The pages' design (one workgroup per row, a global fp32 atomic per element
// for dweight, a second read of the row for the output pass) is prior art for
// another code generator; it is not followed here.
#include "device.h"
#include "launch.h"
#include "plan.h"

namespace rmsn {

// ---------------------------------------------------------------------------
// Sum over the tpr threads of a row group. Every thread of the block calls it
// in uniform control flow (rows wider than a wavefront pass through a
// barrier). `slots` is LDS for 2 * rpb * (tpr / 64) floats; `parity`
// alternates between its halves so that one barrier per row suffices.
// ---------------------------------------------------------------------------
template <int TPR, int BLOCK>
__device__ __forceinline__ float row_sum(float v, float *slots, int parity) {
    if constexpr (TPR <= 64) {
        return group_sum<TPR>(v);
    } else {
        constexpr int WPR = TPR / 64;
        constexpr int RPB = BLOCK / TPR;
        v = group_sum<64>(v);
        const int wave = threadIdx.x >> 6;
        const int grp = threadIdx.x / TPR;
        float *s = slots + parity * (RPB * WPR) + grp * WPR;
        if (__lane_id() == 0) s[wave % WPR] = v;
        __syncthreads();
        float t = s[0];
#pragma unroll
        for (int w = 1; w < WPR; ++w) t += s[w];
        return t;
    }
}

// ---------------------------------------------------------------------------
// Backward, main pass. [I769] Implementation plan, Math; [P800] PR-1 and
// fused-add commits. Per row i (x is `added` for the fused variant):
//   x_hat = x * rstd_i, wdy = dy * gamma, c1 = (1/N) sum_j x_hat * wdy,
//   dx = (wdy - x_hat * c1) * rstd_i (+ dresidual_out), dgamma += dy * x_hat.
// ---------------------------------------------------------------------------
template <int DT, int VEC, int TPR, int K, int BLOCK>
__global__ __launch_bounds__(BLOCK) void bwd_main_kernel(BwdArgs a) {
    using P = Pack<DT, VEC>;
    constexpr int RPB = BLOCK / TPR;
    constexpr int WPR = TPR > 64 ? TPR / 64 : 1;
    extern __shared__ float lds[];
    float *slots = lds;
    float *comb = lds + 2 * RPB * WPR;

    const int N = a.N;
    const int nchunk = N / VEC;
    const int grp = threadIdx.x / TPR;
    const int lt = threadIdx.x % TPR;
    const bool has_dres = a.dres != nullptr;

    // gamma stays resident, packed, for the whole kernel
    P gp[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = lt + k * TPR;
        gp[k] = c < nchunk ? load_pack_cached<DT, VEC>(a.gamma, (int64_t)c * VEC) : zero_pack<DT, VEC>();
    }
    float acc[K][VEC];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[k][e] = 0.f;

    // Two x/dy row buffers: `cur` is reduced while `nxt` is in flight.
    // Chunks past the row end keep their zero fill and add nothing.
    P xc[K], dc[K], xn[K], dn[K], rc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) xc[k] = dc[k] = xn[k] = dn[k] = rc[k] = zero_pack<DT, VEC>();
    float r_cur = 0.f, r_nxt = 0.f;

    const int64_t M = a.M;
    const int64_t stride = (int64_t)gridDim.x * RPB;
    int64_t base = (int64_t)blockIdx.x * RPB;

    auto load_row = [&](int64_t row, P (&xv)[K], P (&dv)[K], float &r) {
        const int64_t off = row * N;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = lt + k * TPR;
            if (c < nchunk) {
                xv[k] = load_pack<DT, VEC>(a.x, off + (int64_t)c * VEC);
                dv[k] = load_pack<DT, VEC>(a.dy, off + (int64_t)c * VEC);
            }
        }
        r = a.rstd[row];
    };

    if (base + grp < M) load_row(base + grp, xc, dc, r_cur);
    int parity = 0;
    for (; base < M; base += stride) {
        const int64_t row = base + grp;
        const int64_t nrow = row + stride;
        const bool valid = row < M;
        // dresidual_out of this row is issued before the next row's x/dy so
        // that waiting for it does not wait for the prefetch (loads retire in
        // order)
        if (has_dres && valid) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int c = lt + k * TPR;
                if (c < nchunk) rc[k] = load_pack<DT, VEC>(a.dres, row * N + (int64_t)c * VEC);
            }
        }
        if (nrow < M) load_row(nrow, xn, dn, r_nxt);

        const float r = r_cur;
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float xh = elem(xc[k], e) * r;
                const float wdy = elem(dc[k], e) * elem(gp[k], e);
                part = fmaf(xh, wdy, part);
            }
        const float c1 = row_sum<TPR, BLOCK>(part, slots, parity) / (float)N;
        // Recompute x_hat and wdy from the packed row below instead of keeping
        // 2 * K * VEC fp32 values live across the sum.
#pragma unroll
        for (int k = 0; k < K; ++k) opaque(xc[k], dc[k]);

        if (valid) {
            const int64_t off = row * N;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int c = lt + k * TPR;
                if (c < nchunk) {
                    float o[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float dyv = elem(dc[k], e);
                        const float xh = elem(xc[k], e) * r;
                        const float wdy = dyv * elem(gp[k], e);
                        float d = fmaf(-xh, c1, wdy) * r;
                        if (has_dres) d += elem(rc[k], e);
                        o[e] = d;
                        acc[k][e] = fmaf(dyv, xh, acc[k][e]);
                    }
                    store_pack<DT, VEC>(a.dx, off + (int64_t)c * VEC, make_pack<DT, VEC>(o));
                }
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            xc[k] = xn[k];
            dc[k] = dn[k];
        }
        r_cur = r_nxt;
        parity ^= 1;
    }

    // ---- this block's dgamma partial ----
    auto emit = [&](int j, float v) {
        if (a.mode == DG_PARTIAL) {
            a.partials[(int64_t)blockIdx.x * N + j] = v;
        } else if (a.mode == DG_ATOMIC) {
            unsafeAtomicAdd(a.dgamma_f32 + j, v);
        } else {
            a.dgamma_f32[j] = v;
            if (a.dgamma) {
                if constexpr (DT == DT_F32) {
                    static_cast<float *>(a.dgamma)[j] = v;
                } else {
                    static_cast<uint16_t *>(a.dgamma)[j] = pack1<DT>(v);
                }
            }
        }
    };
    if constexpr (RPB == 1) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = lt + k * TPR;
            if (c < nchunk)
#pragma unroll
                for (int e = 0; e < VEC; ++e) emit(c * VEC + e, acc[k][e]);
        }
    } else {
        // fold the rpb row groups in a fixed order, then write the block's row
        for (int gi = 0; gi < RPB; ++gi) {
            if (grp == gi) {
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int c = lt + k * TPR;
                    if (c < nchunk)
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            comb[c * VEC + e] = gi == 0 ? acc[k][e] : comb[c * VEC + e] + acc[k][e];
                }
            }
            __syncthreads();
        }
        for (int j = threadIdx.x; j < N; j += BLOCK) emit(j, comb[j]);
    }
}

// ---------------------------------------------------------------------------
// Backward, dgamma finalize (deterministic mode): dgamma_f32[j] = sum over the
// G block partials in a fixed order, and its rounding to the dtype.
// 64 columns per block, each summed by 4 threads over interleaved partials,
// then combined in a fixed order.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const float *__restrict__ partials, int G,
                                                           int N, float *__restrict__ dgamma_f32,
                                                           void *__restrict__ dgamma) {
    __shared__ float red[4][64];
    const int l = threadIdx.x & 63;
    const int split = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + l;
    float s = 0.f;
    if (col < N) {
        int gi = split;
        for (; gi + 12 < G; gi += 16) {
            const float v0 = partials[(int64_t)gi * N + col];
            const float v1 = partials[(int64_t)(gi + 4) * N + col];
            const float v2 = partials[(int64_t)(gi + 8) * N + col];
            const float v3 = partials[(int64_t)(gi + 12) * N + col];
            s = (((s + v0) + v1) + v2) + v3;
        }
        for (; gi < G; gi += 4) s += partials[(int64_t)gi * N + col];
    }
    red[split][l] = s;
    __syncthreads();
    if (split == 0 && col < N) {
        const float t = ((red[0][l] + red[1][l]) + red[2][l]) + red[3][l];
        dgamma_f32[col] = t;
        if (dgamma) {
            if constexpr (DT == DT_F32) {
                static_cast<float *>(dgamma)[col] = t;
            } else {
                static_cast<uint16_t *>(dgamma)[col] = pack1<DT>(t);
            }
        }
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ p, int n) {
    for (int j = blockIdx.x * 256 + threadIdx.x; j < n; j += gridDim.x * 256) p[j] = 0.f;
}

template <int DT>
__global__ __launch_bounds__(256) void cast_kernel(const float *__restrict__ src, void *__restrict__ dst,
                                                   int n) {
    for (int j = blockIdx.x * 256 + threadIdx.x; j < n; j += gridDim.x * 256) {
        if constexpr (DT == DT_F32) {
            static_cast<float *>(dst)[j] = src[j];
        } else {
            static_cast<uint16_t *>(dst)[j] = pack1<DT>(src[j]);
        }
    }
}

// ---------------------------------------------------------------------------
// Forward that saves rstd, plain and fused-add. [I769] Scope/tasks item 2;
// [P800] PR-1 commit (rstd: fp32, one per row, eps honoured) and fused-add
// commit (added = x + residual is residual_out, rstd is that of added).
//   a = x, or round(x + residual) for the fused variant (fp32 sum, one RNE)
//   rstd = 1 / sqrt(sum a^2 / N + eps);   y = a * rstd * gamma
// ---------------------------------------------------------------------------
template <int DT, int VEC, int TPR, int K, int BLOCK>
__global__ __launch_bounds__(BLOCK) void fwd_kernel(FwdArgs a) {
    using P = Pack<DT, VEC>;
    constexpr int RPB = BLOCK / TPR;
    extern __shared__ float lds[];

    const int N = a.N;
    const int nchunk = N / VEC;
    const int grp = threadIdx.x / TPR;
    const int lt = threadIdx.x % TPR;
    const bool fused = a.residual != nullptr;

    float g[K][VEC];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = lt + k * TPR;
        P gp = c < nchunk ? load_pack_cached<DT, VEC>(a.gamma, (int64_t)c * VEC) : zero_pack<DT, VEC>();
#pragma unroll
        for (int e = 0; e < VEC; ++e) g[k][e] = elem(gp, e);
    }

    P xc[K], rc[K], xn[K], rn[K];
#pragma unroll
    for (int k = 0; k < K; ++k) xc[k] = rc[k] = xn[k] = rn[k] = zero_pack<DT, VEC>();

    const int64_t M = a.M;
    const int64_t stride = (int64_t)gridDim.x * RPB;
    int64_t base = (int64_t)blockIdx.x * RPB;

    auto load_row = [&](int64_t row, P (&xv)[K], P (&rv)[K]) {
        const int64_t off = row * N;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = lt + k * TPR;
            if (c < nchunk) {
                xv[k] = load_pack<DT, VEC>(a.x, off + (int64_t)c * VEC);
                if (fused) rv[k] = load_pack<DT, VEC>(a.residual, off + (int64_t)c * VEC);
            }
        }
    };

    if (base + grp < M) load_row(base + grp, xc, rc);
    int parity = 0;
    for (; base < M; base += stride) {
        const int64_t row = base + grp;
        const int64_t nrow = row + stride;
        if (nrow < M) load_row(nrow, xn, rn);
        const bool valid = row < M;

        float v[K][VEC];
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float t = elem(xc[k], e);
                if (fused) t = round_trip<DT>(t + elem(rc[k], e));
                v[k][e] = t;
                part = fmaf(t, t, part);
            }
        const float ms = row_sum<TPR, BLOCK>(part, lds, parity) / (float)N;
        const float r = 1.0f / sqrtf(ms + a.eps);

        if (valid) {
            const int64_t off = row * N;
            if (lt == 0) a.rstd[row] = r;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int c = lt + k * TPR;
                if (c < nchunk) {
                    float o[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) o[e] = v[k][e] * r * g[k][e];
                    store_pack<DT, VEC>(a.y, off + (int64_t)c * VEC, make_pack<DT, VEC>(o));
                    if (fused) store_pack<DT, VEC>(a.residual_out, off + (int64_t)c * VEC,
                                                   make_pack<DT, VEC>(v[k]));
                }
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            xc[k] = xn[k];
            rc[k] = rn[k];
        }
        parity ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

template <int TPR> constexpr int block_of() { return TPR > 256 ? TPR : 256; }

template <int DT, int VEC, int TPR, int K>
static hipError_t launch_bwd_cfg(const BwdArgs &a, int grid, hipStream_t s) {
    constexpr int BLOCK = block_of<TPR>();
    constexpr int RPB = BLOCK / TPR;
    constexpr int WPR = TPR > 64 ? TPR / 64 : 1;
    const size_t lds = (size_t)(2 * RPB * WPR + (RPB > 1 ? TPR * K * VEC : 0)) * sizeof(float);
    hipLaunchKernelGGL((bwd_main_kernel<DT, VEC, TPR, K, BLOCK>), dim3(grid), dim3(BLOCK), lds, s, a);
    return hipGetLastError();
}

template <int DT, int VEC, int TPR, int K>
static hipError_t launch_fwd_cfg(const FwdArgs &a, int grid, hipStream_t s) {
    constexpr int BLOCK = block_of<TPR>();
    constexpr int RPB = BLOCK / TPR;
    constexpr int WPR = TPR > 64 ? TPR / 64 : 1;
    const size_t lds = (size_t)(2 * RPB * WPR) * sizeof(float);
    hipLaunchKernelGGL((fwd_kernel<DT, VEC, TPR, K, BLOCK>), dim3(grid), dim3(BLOCK), lds, s, a);
    return hipGetLastError();
}

// Dispatch a row plan to its kernel instance. Every (vec, tpr, k) that
// plan_rows can return has an instance here; anything else is a bug and is
// reported as hipErrorInvalidValue without launching.
#define RMSN_DISPATCH(LAUNCH, ARGS, GRID, STREAM)                                              \
    do {                                                                                       \
        constexpr int VW = 16 / ElemSize<DT>::value;                                           \
        if (p.vec == VW) {                                                                     \
            if (p.tpr == 16 && p.k == 1) return LAUNCH<DT, VW, 16, 1>(ARGS, GRID, STREAM);     \
            if (p.tpr == 16 && p.k == 2) return LAUNCH<DT, VW, 16, 2>(ARGS, GRID, STREAM);     \
            if (p.k == 4) {                                                                    \
                switch (p.tpr) {                                                               \
                case 16: return LAUNCH<DT, VW, 16, 4>(ARGS, GRID, STREAM);                     \
                case 32: return LAUNCH<DT, VW, 32, 4>(ARGS, GRID, STREAM);                     \
                case 64: return LAUNCH<DT, VW, 64, 4>(ARGS, GRID, STREAM);                     \
                case 128: return LAUNCH<DT, VW, 128, 4>(ARGS, GRID, STREAM);                   \
                case 256: return LAUNCH<DT, VW, 256, 4>(ARGS, GRID, STREAM);                   \
                case 512: return LAUNCH<DT, VW, 512, 4>(ARGS, GRID, STREAM);                   \
                case 1024:                                                                     \
                    if constexpr (VW == 4) return LAUNCH<DT, VW, 1024, 4>(ARGS, GRID, STREAM); \
                    break;                                                                     \
                default: break;                                                                \
                }                                                                              \
            }                                                                                  \
        } else if (p.vec == 1) {                                                               \
            if (p.tpr == 64 && p.k == 4) return LAUNCH<DT, 1, 64, 4>(ARGS, GRID, STREAM);      \
            if (p.tpr == 64 && p.k == 8) return LAUNCH<DT, 1, 64, 8>(ARGS, GRID, STREAM);      \
            if (p.tpr == 64 && p.k == 16) return LAUNCH<DT, 1, 64, 16>(ARGS, GRID, STREAM);    \
            if (p.tpr == 256 && p.k == 16) return LAUNCH<DT, 1, 256, 16>(ARGS, GRID, STREAM);  \
            if (p.tpr == 1024 && p.k == 16) return LAUNCH<DT, 1, 1024, 16>(ARGS, GRID, STREAM); \
        }                                                                                      \
        return hipErrorInvalidValue;                                                           \
    } while (0)

template <int DT>
static hipError_t dispatch_bwd(const RowPlan &p, const BwdArgs &a, int grid, hipStream_t s) {
    RMSN_DISPATCH(launch_bwd_cfg, a, grid, s);
}

template <int DT>
static hipError_t dispatch_fwd(const RowPlan &p, const FwdArgs &a, int grid, hipStream_t s) {
    RMSN_DISPATCH(launch_fwd_cfg, a, grid, s);
}

template <int DT>
static hipError_t launch_bwd_dt(const RowPlan &p, const BwdArgs &args, int grid, void *workspace,
                                hipStream_t s) {
    BwdArgs a = args;
    hipError_t e;
    if (a.M == 0) {
        // no rows: dgamma is zero
        hipLaunchKernelGGL(fill_zero_kernel, dim3((a.N + 255) / 256), dim3(256), 0, s, a.dgamma_f32, a.N);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (a.dgamma) {
            hipLaunchKernelGGL(cast_kernel<DT>, dim3((a.N + 255) / 256), dim3(256), 0, s, a.dgamma_f32,
                               a.dgamma, a.N);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    if (a.mode == DG_PARTIAL) {
        a.partials = reinterpret_cast<float *>(static_cast<char *>(workspace) + WS_HEADER);
        if ((e = dispatch_bwd<DT>(p, a, grid, s)) != hipSuccess) return e;
        hipLaunchKernelGGL(bwd_finalize_kernel<DT>, dim3((a.N + 63) / 64), dim3(256), 0, s, a.partials, grid,
                           a.N, a.dgamma_f32, a.dgamma);
        return hipGetLastError();
    }
    if (a.mode == DG_ATOMIC) {
        hipLaunchKernelGGL(fill_zero_kernel, dim3((a.N + 255) / 256), dim3(256), 0, s, a.dgamma_f32, a.N);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = dispatch_bwd<DT>(p, a, grid, s)) != hipSuccess) return e;
        if (a.dgamma) {
            hipLaunchKernelGGL(cast_kernel<DT>, dim3((a.N + 255) / 256), dim3(256), 0, s, a.dgamma_f32,
                               a.dgamma, a.N);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    return dispatch_bwd<DT>(p, a, grid, s);  // DG_DIRECT: one block writes dgamma itself
}

hipError_t launch_bwd(int dtype, const RowPlan &p, const BwdArgs &a, int grid, void *workspace,
                      hipStream_t s) {
    switch (dtype) {
    case DT_F32: return launch_bwd_dt<DT_F32>(p, a, grid, workspace, s);
    case DT_F16: return launch_bwd_dt<DT_F16>(p, a, grid, workspace, s);
    case DT_BF16: return launch_bwd_dt<DT_BF16>(p, a, grid, workspace, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd(int dtype, const RowPlan &p, const FwdArgs &a, int grid, hipStream_t s) {
    if (a.M == 0) return hipSuccess;
    switch (dtype) {
    case DT_F32: return dispatch_fwd<DT_F32>(p, a, grid, s);
    case DT_F16: return dispatch_fwd<DT_F16>(p, a, grid, s);
    case DT_BF16: return dispatch_fwd<DT_BF16>(p, a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rmsn
