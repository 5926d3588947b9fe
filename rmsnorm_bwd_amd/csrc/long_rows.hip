// long_rows.hip - forward and backward for rows of more than 16384
// elements (up to MAX_N), where a row no longer fits the register-resident
// window ring of kernels.hip next to the weight-gradient accumulators.
//
// Pages cited, by title:
//   [I769] FlyDSL issue #769, "[Feature] Add rmsnorm backward (+ forward saves
//          rstd) to enable training / downstream (quack) integration" -
//          Implementation plan (Math), PR sequence and status updates
//          (LayerNorm: forward saving mean and rstd, backward with dbias).
//   [P800] FlyDSL PR #800, "[rmsnorm] Add fused-add / residual backward
//          (PR 2/3, #769)" - PR-1 and fused-add commits; the second pass of
//          the backward re-reads the row, as the review-fix commit notes the
//          pages' own backward does for every row.
//   [P854] FlyDSL PR #854, "[Test] Expand RMSNorm backward configs, cache
//          reuse, and Torch benchmarks" - Summary (generic-path coverage of
//          rows longer than the fast paths).
//
// One row per block of 512 threads at a time; each thread owns the chunks t,
// t + 512, ... (K of them, VEC elements each, K * VEC = 64), so a row of up
// to 32768 elements is covered. Persistent grid: block b takes rows b, b + G,
// ... Row tensors go through buffer descriptors whose range is the row, so
// chunks past the row end read as zero and are not stored.
//
// Forward: the row stays in registers (64 values a thread, packed), so x (and
// residual) are read once: RMSNorm takes one row sum, LayerNorm two (the mean,
// then the centred variance), and the outputs are formed from the registers.
// The fused forward's residual_out may be residual itself: nothing is read
// after it is written.
//
// Backward: in registers the row (x and dy, and dresidual_out) would leave
// too little room for the 64 (LayerNorm: 128) fp32 weight-gradient
// accumulators, so the row is read twice: the first pass forms the row sums
// (sum x*wdy; for LayerNorm also sum wdy), the second re-reads x, dy and
// dresidual_out (mostly from the caches: a block re-reads what it read one
// pass earlier), writes dx and folds dy * x_hat (and dy) into the
// accumulators. gamma is re-read with the row (it stays in the caches).
#include "device.h"
#include "launch.h"
#include "plan.h"

namespace rmsn {
namespace {

constexpr int LB = 512;           // threads per block
constexpr int LWAVES = LB / 64;   // wavefronts per block
constexpr int LGROUP = 4;         // chunks loaded together
constexpr int OPL_RMS = 0, OPL_FUSED = 1, OPL_LN = 2;

// Sums of NV values over the block (one row): DPP inside each wavefront, then
// one LDS exchange; `slots` holds 2 * NV * LWAVES floats and `parity`
// alternates between its halves so one barrier per sum suffices.
template <int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float *slots, int &parity) {
    const int wave = threadIdx.x >> 6;
    float *s = slots + parity * (NV * LWAVES);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        v[i] = group_sum<64>(v[i]);
        if (__lane_id() == 0) s[i * LWAVES + wave] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        float t = s[i * LWAVES];
#pragma unroll
        for (int w = 1; w < LWAVES; ++w) t += s[i * LWAVES + w];
        v[i] = t;
    }
    parity ^= 1;
}

// ---------------------------------------------------------------------------
// Forward, long rows.
// ---------------------------------------------------------------------------
template <int DT, int VEC, int OP>
__global__ __launch_bounds__(LB) void fwd_long_kernel(FwdArgs a) {
    using P = Pack<DT, VEC>;
    constexpr int K = 64 / VEC;
    constexpr bool FUSED = OP == OPL_FUSED, LN = OP == OPL_LN;
    constexpr int ES = ElemSize<DT>::value;
    __shared__ float slots[2 * 2 * LWAVES];
    const int N = a.N;
    const int64_t M = a.M;
    const uint32_t row_bytes = (uint32_t)N * ES;
    const int nchunk = N / VEC;
    uint32_t coff[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = threadIdx.x + k * LB;
        coff[k] = c < nchunk ? (uint32_t)c * (VEC * ES) : OOB;
    }
    const rsrc_t rg = make_rsrc(a.gamma, row_bytes);
    const rsrc_t rb = make_rsrc(a.beta, LN && a.beta ? row_bytes : 0u);
    const float inv_n = 1.0f / (float)N;
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const rsrc_t rx = window_rsrc<ES>(a.x, row, a.ldx, 1, row_bytes);
        P av[K];  // the row (for the fused variant, added = x + residual rounded)
#pragma unroll
        for (int k = 0; k < K; ++k) av[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rx, coff[k]);
        if constexpr (FUSED) {
            const rsrc_t rr = window_rsrc<ES>(a.residual, row, a.ldres, 1, row_bytes);
            const rsrc_t ro = window_rsrc<ES>(a.residual_out, row, a.ldres_out, 1, row_bytes);
#pragma unroll
            for (int k0 = 0; k0 < K; k0 += LGROUP) {
                P rv[LGROUP];
#pragma unroll
                for (int j = 0; j < LGROUP; ++j) rv[j] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rr, coff[k0 + j]);
#pragma unroll
                for (int j = 0; j < LGROUP; ++j) {
                    float t[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) t[e] = elem(av[k0 + j], e) + elem(rv[j], e);
                    av[k0 + j] = make_pack<DT, VEC>(t);  // rounded once
                }
            }
            // every residual read is done before residual_out (which may be
            // residual itself) is written
#pragma unroll
            for (int k = 0; k < K; ++k) buf_store<DT, VEC, AUX_STREAM_STORE>(ro, coff[k], av[k]);
        }
        float r, mu = 0.f;
        if constexpr (LN) {
            float s1[1] = {0.f};
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) s1[0] += elem(av[k], e);
            block_sum<1>(s1, slots, parity);
            mu = s1[0] * inv_n;
            float s2[1] = {0.f};
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float d = coff[k] == OOB ? 0.f : elem(av[k], e) - mu;  // chunks past the row end
                    s2[0] = fmaf(d, d, s2[0]);
                }
            block_sum<1>(s2, slots, parity);
            r = 1.0f / sqrtf(s2[0] * inv_n + a.eps);
        } else {
            float ss[1] = {0.f};
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) ss[0] = fmaf(elem(av[k], e), elem(av[k], e), ss[0]);
            block_sum<1>(ss, slots, parity);
            r = 1.0f / sqrtf(ss[0] * inv_n + a.eps);
        }
        if (threadIdx.x == 0) {
            buf_store_f32(make_rsrc(at(a.rstd, row, 4), 4u), 0u, r);
            if constexpr (LN) buf_store_f32(make_rsrc(at(a.mean, row, 4), 4u), 0u, mu);
        }
        const rsrc_t ry = window_rsrc<ES>(a.y, row, a.ldy, 1, row_bytes);
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += LGROUP) {
            P gv[LGROUP], bv[LN ? LGROUP : 1];
#pragma unroll
            for (int j = 0; j < LGROUP; ++j) {
                gv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rg, coff[k0 + j]);
                if constexpr (LN) bv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rb, coff[k0 + j]);
            }
#pragma unroll
            for (int j = 0; j < LGROUP; ++j) {
                float o[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    if constexpr (LN)
                        o[e] = fmaf((elem(av[k0 + j], e) - mu) * r, elem(gv[j], e), elem(bv[j], e));
                    else
                        o[e] = elem(av[k0 + j], e) * r * elem(gv[j], e);
                }
                buf_store<DT, VEC, FUSED ? AUX_STREAM_STORE : AUX_SINGLE_STORE>(ry, coff[k0 + j],
                                                                               make_pack<DT, VEC>(o));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Backward, long rows: two passes over each row (see the file comment).
// ---------------------------------------------------------------------------
template <int DT, int VEC, int OP>
__global__ __launch_bounds__(LB) void bwd_long_kernel(BwdArgs a) {
    using P = Pack<DT, VEC>;
    constexpr int K = 64 / VEC;
    constexpr bool FUSED = OP == OPL_FUSED, LN = OP == OPL_LN;
    constexpr int NA = LN ? 2 : 1;
    constexpr int ES = ElemSize<DT>::value;
    __shared__ float slots[2 * 2 * LWAVES];
    const int N = a.N;
    const int64_t M = a.M;
    const int G = gridDim.x;
    const uint32_t row_bytes = (uint32_t)N * ES;
    const int nchunk = N / VEC;
    const float inv_n = 1.0f / (float)N;
    uint32_t coff[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = threadIdx.x + k * LB;
        coff[k] = c < nchunk ? (uint32_t)c * (VEC * ES) : OOB;
    }
    const rsrc_t rg = make_rsrc(a.gamma, row_bytes);
    float acc[NA][K][VEC];
#pragma unroll
    for (int q = 0; q < NA; ++q)
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[q][k][e] = 0.f;
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += G) {
        const rsrc_t rx = window_rsrc<ES>(a.x, row, a.ldx, 1, row_bytes);
        const rsrc_t rd = window_rsrc<ES>(a.dy, row, a.lddy, 1, row_bytes);
        const float r = buf_load_f32(make_rsrc(at(a.rstd, row, 4), 4u), 0u);
        const float mu = LN ? buf_load_f32(make_rsrc(at(a.mean, row, 4), 4u), 0u) : 0.f;
        // pass 1: the row sums
        float s[2] = {0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += LGROUP) {
            P xv[LGROUP], dv[LGROUP], gv[LGROUP];
#pragma unroll
            for (int j = 0; j < LGROUP; ++j) {
                xv[j] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rx, coff[k0 + j]);
                dv[j] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rd, coff[k0 + j]);
                gv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rg, coff[k0 + j]);
            }
#pragma unroll
            for (int j = 0; j < LGROUP; ++j)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float wd = elem(dv[j], e) * elem(gv[j], e);
                    s[0] = fmaf(elem(xv[j], e) - mu, wd, s[0]);
                    if constexpr (LN) s[1] += wd;
                }
        }
        float b, d = 0.f;
        if constexpr (LN) {
            block_sum<2>(s, slots, parity);
            b = r * r * (s[0] * r * inv_n);  // r^2 c1, c1 = r sum (x - mu) wdy / N
            d = r * (s[1] * inv_n);          // r c2, c2 = sum wdy / N
        } else {
            float t[1] = {s[0]};
            block_sum<1>(t, slots, parity);
            b = r * r * (t[0] * r * inv_n);
        }
        // pass 2: dx, and the weight-gradient terms
        const rsrc_t rz = window_rsrc<ES>(a.dres, row, a.lddres, FUSED ? 1u : 0u, row_bytes);
        const rsrc_t rw = window_rsrc<ES>(a.dx, row, a.lddx, 1, row_bytes);
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += LGROUP) {
            P xv[LGROUP], dv[LGROUP], gv[LGROUP], zv[FUSED ? LGROUP : 1];
#pragma unroll
            for (int j = 0; j < LGROUP; ++j) {
                xv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rx, coff[k0 + j]);
                dv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rd, coff[k0 + j]);
                gv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rg, coff[k0 + j]);
                if constexpr (FUSED) zv[j] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rz, coff[k0 + j]);
            }
#pragma unroll
            for (int j = 0; j < LGROUP; ++j) {
                float o[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float xc = elem(xv[j], e) - mu;
                    const float dyv = elem(dv[j], e);
                    float dd = fmaf(-b, xc, r * (dyv * elem(gv[j], e)));
                    if constexpr (LN) dd -= d;
                    if constexpr (FUSED) dd += elem(zv[j], e);
                    o[e] = dd;
                    acc[0][k0 + j][e] = fmaf(dyv, xc * r, acc[0][k0 + j][e]);
                    if constexpr (LN) acc[NA - 1][k0 + j][e] += dyv;
                }
                buf_store<DT, VEC, FUSED ? AUX_STREAM_STORE : AUX_SINGLE_STORE>(rw, coff[k0 + j],
                                                                               make_pack<DT, VEC>(o));
            }
        }
    }

    // this block's weight-gradient sums: a partial (two-stage sum), fp32
    // atomics, or, with one block, the gradients themselves
    const int64_t pstride = (int64_t)((N + FIN_TILE - 1) / FIN_TILE) * FIN_TILE * G;
#pragma unroll
    for (int q = 0; q < NA; ++q) {
        float *out32 = q ? a.dbeta_f32 : a.dgamma_f32;
        void *outT = q ? a.dbeta : a.dgamma;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = threadIdx.x + k * LB;
            if (c >= nchunk) continue;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int j = c * VEC + e;
                const float v = acc[q][k][e];
                if (a.mode == DG_PARTIAL) {
                    a.partials[q * pstride + partial_index(j, blockIdx.x, G)] = v;
                } else if (a.mode == DG_ATOMIC) {
                    unsafeAtomicAdd(out32 + j, v);
                } else {
                    out32[j] = v;
                    if (outT) {
                        if constexpr (DT == DT_F32)
                            static_cast<float *>(outT)[j] = v;
                        else
                            static_cast<uint16_t *>(outT)[j] = pack1<DT>(v);
                    }
                }
            }
        }
    }
}

template <int DT, int VEC>
hipError_t fwd_long_vec(const FwdArgs &a, int grid, hipStream_t s) {
    if (a.mean)
        hipLaunchKernelGGL((fwd_long_kernel<DT, VEC, OPL_LN>), dim3(grid), dim3(LB), 0, s, a);
    else if (a.residual)
        hipLaunchKernelGGL((fwd_long_kernel<DT, VEC, OPL_FUSED>), dim3(grid), dim3(LB), 0, s, a);
    else
        hipLaunchKernelGGL((fwd_long_kernel<DT, VEC, OPL_RMS>), dim3(grid), dim3(LB), 0, s, a);
    return hipGetLastError();
}

template <int DT, int VEC>
hipError_t bwd_long_vec(const BwdArgs &a, int grid, hipStream_t s) {
    if (a.layer)
        hipLaunchKernelGGL((bwd_long_kernel<DT, VEC, OPL_LN>), dim3(grid), dim3(LB), 0, s, a);
    else if (a.dres)
        hipLaunchKernelGGL((bwd_long_kernel<DT, VEC, OPL_FUSED>), dim3(grid), dim3(LB), 0, s, a);
    else
        hipLaunchKernelGGL((bwd_long_kernel<DT, VEC, OPL_RMS>), dim3(grid), dim3(LB), 0, s, a);
    return hipGetLastError();
}

template <int DT>
hipError_t fwd_long_dt(const RowPlan &p, const FwdArgs &a, int grid, hipStream_t s) {
    constexpr int VW = 16 / ElemSize<DT>::value;
    if (p.vec == VW && p.k * VW == 64) return fwd_long_vec<DT, VW>(a, grid, s);
    if (p.vec == 1 && p.k == 64) return fwd_long_vec<DT, 1>(a, grid, s);
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t bwd_long_dt(const RowPlan &p, const BwdArgs &a, int grid, hipStream_t s) {
    constexpr int VW = 16 / ElemSize<DT>::value;
    if (p.vec == VW && p.k * VW == 64) return bwd_long_vec<DT, VW>(a, grid, s);
    if (p.vec == 1 && p.k == 64) return bwd_long_vec<DT, 1>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_long(int dtype, const RowPlan &p, const FwdArgs &a, int grid, hipStream_t s) {
    switch (dtype) {
    case DT_F32: return fwd_long_dt<DT_F32>(p, a, grid, s);
    case DT_F16: return fwd_long_dt<DT_F16>(p, a, grid, s);
    case DT_BF16: return fwd_long_dt<DT_BF16>(p, a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_long(int dtype, const RowPlan &p, const BwdArgs &a, int grid, hipStream_t s) {
    switch (dtype) {
    case DT_F32: return bwd_long_dt<DT_F32>(p, a, grid, s);
    case DT_F16: return bwd_long_dt<DT_F16>(p, a, grid, s);
    case DT_BF16: return bwd_long_dt<DT_BF16>(p, a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rmsn
