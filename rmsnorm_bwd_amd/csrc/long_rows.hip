// long_rows.hip - forward and backward for rows of more than 16384
// elements (up to MAX_N), where a row no longer fits the register-resident
// window ring of kernels.hip next to the weight-gradient accumulators; also
// the fused and (mostly) the LayerNorm backward of 16-bit rows of
// 12296-16384 elements, where that ring holds only one window.
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
// to 32768 elements is covered (fewer chunks where the plan gives fewer:
// six for 16-bit rows of at most 24576 elements, four for the fused and
// LayerNorm rows of at most 16384). Persistent grid: block b takes rows b, b + G,
// ... Row tensors go through buffer descriptors whose range is the row, so
// chunks past the row end read as zero and are not stored.
//
// Forward: the row stays in registers (64 values a thread, packed), so x (and
// residual) are read once: RMSNorm takes one row sum, LayerNorm two (the mean,
// then the centred variance), and the outputs are formed from the registers.
// The fused forward's residual_out may be residual itself: nothing is read
// after it is written.
//
// Backward on 16-byte chunks (RMSNorm plain and fused; LayerNorm for 16-bit
// types): the row (x, dy, dresidual_out) stays in registers and each
// thread's 64 fp32 dgamma accumulators live in LDS (128 KiB a block: a
// thread's own slots, so no barrier guards them), so each row is read once.
// gamma is re-read from the caches or held in registers, and for 16-bit
// RMSNorm the block's next row is loaded during the current one (the modes
// of long_mode in plan.h). LayerNorm's dbeta accumulators (a second array
// would not fit the LDS) stay in registers, which leaves room beside them
// for a 16-bit row and gamma only, or for two rows at four chunks a thread
// (the rows of at most 16384 elements this kernel takes from kernels.hip).
// Each thread's sums leave as 16-byte partial stores (or, when one block
// runs the call, as the gradients themselves, four columns a store where
// the outputs are aligned for it). dx is stored non-temporally (NT) by every
// variant here, where the main kernel's plain and LayerNorm dx use SC1:
// measured on MI355X, µs per call, NT against SC1, bf16: plain 1024 x
// 16400 32.9 -> 28.2, 1024 x 32768 54.5 -> 49.6, 4096 x 24576 124.6 ->
// 113.5, 8192 x 32768 308 -> 298; LayerNorm 2048 x 32768 108.5 -> 97.4;
// fp32 4096 x 20000 183.4 -> 179.0; the rest within 1%.
//
// Backward in two passes (LayerNorm on fp32 rows, and every variant on
// single elements, where N or the pointers are not 16-byte aligned): the
// first pass forms the row sums (sum (x - mean)*wdy, and sum wdy for
// LayerNorm), the second re-reads x and dy (mostly from the caches: the
// block read them one pass earlier), writes dx and folds dy * x_hat (and
// dy) into the accumulators.
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
    auto off = [&](int k) -> uint32_t {
        const int c = threadIdx.x + k * LB;
        return c < nchunk ? (uint32_t)c * (VEC * ES) : OOB;
    };
    const rsrc_t rg = make_rsrc(a.gamma, row_bytes);
    const rsrc_t rb = make_rsrc(a.beta, LN && a.beta ? row_bytes : 0u);
    const float inv_n = 1.0f / (float)N;
    // On 16-byte chunks gamma (and beta) stay in registers for the whole
    // kernel, and the fused variant loads its residual row at once: no load
    // is then issued after a row's first stores, so nothing waits on a store
    // (loads and stores retire through one in-order counter). Measured on
    // MI355X against loading gamma per group of chunks, two runs on two
    // boxes: plain 8192 x 20000 bf16 -5.1 / -4.8%, plain fp32 4096 x 24576
    // -5.7 / -2.5%, fused 4096 x 32768 bf16 -3.2 / +1.4%, LayerNorm 8192 x
    // 20000 bf16 -0.6 / +0.5%. Single elements (64 registers of gamma a
    // thread) keep the per-group loads.
    constexpr bool GRES = VEC > 1;
    P gres[GRES ? K : 1], bres[GRES && LN ? K : 1];
    if constexpr (GRES) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            gres[k] = buf_load<DT, VEC, AUX_DEFAULT>(rg, off(k));
            if constexpr (LN) bres[k] = buf_load<DT, VEC, AUX_DEFAULT>(rb, off(k));
        }
    }
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const rsrc_t rx = window_rsrc<ES>(a.x, row, a.ldx, 1, row_bytes);
        P av[K];  // the row (for the fused variant, added = x + residual rounded)
#pragma unroll
        for (int k = 0; k < K; ++k) av[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rx, off(k));
        if constexpr (FUSED) {
            const rsrc_t rr = window_rsrc<ES>(a.residual, row, a.ldres, 1, row_bytes);
            const rsrc_t ro = window_rsrc<ES>(a.residual_out, row, a.ldres_out, 1, row_bytes);
            constexpr int RG = GRES ? K : LGROUP;  // residual chunks loaded together
#pragma unroll
            for (int k0 = 0; k0 < K; k0 += RG) {
                P rv[RG];
#pragma unroll
                for (int j = 0; j < RG; ++j) rv[j] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rr, off(k0 + j));
#pragma unroll
                for (int j = 0; j < RG; ++j) {
                    float t[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) t[e] = elem(av[k0 + j], e) + elem(rv[j], e);
                    av[k0 + j] = make_pack<DT, VEC>(t);  // rounded once
                }
            }
            // every residual read is done before residual_out (which may be
            // residual itself) is written
#pragma unroll
            for (int k = 0; k < K; ++k) buf_store<DT, VEC, AUX_STREAM_STORE>(ro, off(k), av[k]);
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
                    const float d = off(k) == OOB ? 0.f : elem(av[k], e) - mu;  // chunks past the row end
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
                if constexpr (GRES) {
                    gv[j] = gres[k0 + j];
                    if constexpr (LN) bv[j] = bres[LN ? k0 + j : 0];
                } else {
                    gv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rg, off(k0 + j));
                    if constexpr (LN) bv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rb, off(k0 + j));
                }
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
                buf_store<DT, VEC, AUX_FWD_STORE>(ry, off(k0 + j), make_pack<DT, VEC>(o));
            }
        }
    }
}

// One weight-gradient sum of this block for column j of array q (0 dgamma,
// 1 dbeta): a partial (the two-stage sum), an fp32 atomic add, or, when one
// block runs the call, the gradient itself and its dtype copy.
template <int DT>
__device__ __forceinline__ void emit_long(const BwdArgs &a, int q, int j, float v, int G, int64_t pstride) {
    float *out32 = q ? a.dbeta_f32 : a.dgamma_f32;
    void *outT = q ? a.dbeta : a.dgamma;
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

typedef float lf32x4 __attribute__((ext_vector_type(4)));
constexpr int NSLOT = 64 / 4;  // float4 dgamma accumulator slots a thread (64 elements)

// Whether one block writing the gradients itself may store four columns at
// once: the fp32 outputs 16-byte aligned, their dtype copies aligned for four
// values (8 bytes, 16 for fp32).
template <int DT>
__device__ __forceinline__ bool direct_vec_ok(const BwdArgs &a, bool ln) {
    constexpr uintptr_t TA = DT == DT_F32 ? 15 : 7;
    const bool g = ((reinterpret_cast<uintptr_t>(a.dgamma_f32) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(a.dgamma) & TA) == 0);
    const bool b = !ln || (((reinterpret_cast<uintptr_t>(a.dbeta_f32) & 15) == 0) &&
                           ((reinterpret_cast<uintptr_t>(a.dbeta) & TA) == 0));
    return g && b;
}

// Columns j..j+3 of array q (0 dgamma, 1 dbeta) written by the one block that
// runs the call: the fp32 sums in one 16-byte store, their dtype copy in one
// more.
template <int DT>
__device__ __forceinline__ void emit_direct4(const BwdArgs &a, int q, int j, lf32x4 v) {
    typedef uint32_t lu32x2 __attribute__((ext_vector_type(2)));
    float *out32 = q ? a.dbeta_f32 : a.dgamma_f32;
    void *outT = q ? a.dbeta : a.dgamma;
    *reinterpret_cast<lf32x4 *>(out32 + j) = v;
    if (outT) {
        if constexpr (DT == DT_F32)
            *reinterpret_cast<lf32x4 *>(static_cast<float *>(outT) + j) = v;
        else
            *reinterpret_cast<lu32x2 *>(static_cast<uint16_t *>(outT) + j) =
                lu32x2{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
    }
}

// A thread's sums of array q for its chunk c (VEC columns from c * VEC):
// partials in 16-byte stores (four consecutive columns, a multiple of 4 from
// the row start, lie in one partial tile), the gradients of a one-block call
// four columns at a time where the outputs are aligned for it (a single CU
// storing element by element is what bounds such a call), else one column
// at a time.
template <int DT, int VEC, int K, bool LN>
__device__ __forceinline__ void emit_chunk(const BwdArgs &a, int t, int c, int k, const lf32x4 (*acc)[LB],
                                           const float (&accb)[LN ? K : 1][LN ? VEC : 1], int G,
                                           int64_t pstride) {
    if constexpr (VEC % 4 == 0) {
        if (a.mode == DG_PARTIAL) {
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                const int i = k * VEC + e;
                const int64_t p = partial_index(c * VEC + e, blockIdx.x, G);
                *reinterpret_cast<lf32x4 *>(a.partials + p) = acc[i / 4][t];
                if constexpr (LN)
                    *reinterpret_cast<lf32x4 *>(a.partials + pstride + p) =
                        lf32x4{accb[k][e], accb[k][e + 1], accb[k][e + 2], accb[k][e + 3]};
            }
            return;
        }
        if (a.mode == DG_DIRECT && direct_vec_ok<DT>(a, LN)) {
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                const int i = k * VEC + e;
                emit_direct4<DT>(a, 0, c * VEC + e, acc[i / 4][t]);
                if constexpr (LN)
                    emit_direct4<DT>(a, 1, c * VEC + e,
                                     lf32x4{accb[k][e], accb[k][e + 1], accb[k][e + 2], accb[k][e + 3]});
            }
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const int i = k * VEC + e;
        emit_long<DT>(a, 0, c * VEC + e, acc[i / 4][t][i % 4], G, pstride);
        if constexpr (LN) emit_long<DT>(a, 1, c * VEC + e, accb[k][e], G, pstride);
    }
}

// ---------------------------------------------------------------------------
// Backward, long rows, on 16-byte chunks, one read of each row: the row in
// registers, the dgamma accumulators in LDS (LayerNorm's dbeta accumulators
// in registers). MODE (LM_* in plan.h) says where gamma lives and whether
// the block's next row is loaded during this one.
// ---------------------------------------------------------------------------
template <int DT, int VEC, int K, int OP, int MODE>
__global__ __launch_bounds__(LB) void bwd_long_1pass_kernel(BwdArgs a) {
    using P = Pack<DT, VEC>;
    constexpr int LG = K % LGROUP == 0 ? LGROUP : 2;  // chunks handled together
    constexpr int NSL = K * VEC / 4;                  // float4 dgamma accumulator slots a thread
    constexpr bool FUSED = OP == OPL_FUSED, LN = OP == OPL_LN;
    constexpr int ES = ElemSize<DT>::value;
    constexpr bool GRES = MODE != LM_RELOAD;  // gamma resident in registers
    // two rows fit beside gamma for 16-bit types, beside LayerNorm's dbeta
    // accumulators too at four chunks a thread
    static_assert(MODE != LM_PREFETCH || (ES == 2 && (!LN || K * VEC <= 32)), "two rows do not fit");
    static_assert((LG * VEC) % 4 == 0 && K % LG == 0, "whole accumulator slots per group");
    static_assert(K % 2 == 0, "gamma fenced in pairs of chunks");
    // slot s of thread t at acc_lds[s][t]: consecutive lanes, consecutive 16 bytes
    __shared__ lf32x4 acc_lds[NSL][LB];
    __shared__ float slots[2 * (LN ? 2 : 1) * LWAVES];
    const int N = a.N;
    const int64_t M = a.M;
    const int G = gridDim.x;
    const int t = threadIdx.x;
    const uint32_t row_bytes = (uint32_t)N * ES;
    const int nchunk = N / VEC;
    const float inv_n = 1.0f / (float)N;
    auto off = [&](int k) -> uint32_t {
        const int c = t + k * LB;
        return c < nchunk ? (uint32_t)c * (VEC * ES) : OOB;
    };
#pragma unroll
    for (int q = 0; q < NSL; ++q) acc_lds[q][t] = lf32x4{0.f, 0.f, 0.f, 0.f};
    float accb[LN ? K : 1][LN ? VEC : 1];  // dbeta, LayerNorm
#pragma unroll
    for (int k = 0; k < (LN ? K : 1); ++k)
#pragma unroll
        for (int e = 0; e < (LN ? VEC : 1); ++e) accb[k][e] = 0.f;
    const rsrc_t rg = make_rsrc(a.gamma, row_bytes);
    P gres[GRES ? K : 1];
    if constexpr (GRES) {
#pragma unroll
        for (int k = 0; k < K; ++k) gres[k] = buf_load<DT, VEC, AUX_DEFAULT>(rg, off(k));
    }
    auto gamma_group = [&](int k0, P (&gv)[LG]) {
#pragma unroll
        for (int j = 0; j < LG; ++j) {
            if constexpr (GRES)
                gv[j] = gres[k0 + j];
            else
                gv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rg, off(k0 + j));
        }
    };
    // With gamma resident, an empty asm statement that "rewrites" the packed
    // registers keeps the compiler from holding their unpacked fp32 values
    // across the row sum or from one row to the next (that spills).
    auto fence_gamma = [&]() {
        if constexpr (GRES) {
#pragma unroll
            for (int k = 0; k < K; k += 2) opaque(gres[k], gres[k + 1]);
        }
    };
    // nr = 0 (a row past the end, loaded ahead) makes every access fall
    // outside the descriptors: no memory is touched and the values are 0.
    auto load_row = [&](int64_t row, uint32_t nr, P (&xv)[K], P (&dv)[K]) {
        const rsrc_t rx = window_rsrc<ES>(a.x, row, a.ldx, nr, row_bytes);
        const rsrc_t rd = window_rsrc<ES>(a.dy, row, a.lddy, nr, row_bytes);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            xv[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rx, off(k));
            dv[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rd, off(k));
        }
    };
    auto load_rstd = [&](int64_t row, uint32_t nr) -> float {
        return buf_load_f32(make_rsrc(at(a.rstd, row, 4), nr * 4u), 0u);
    };
    auto load_mean = [&](int64_t row, uint32_t nr) -> float {
        if constexpr (LN) return buf_load_f32(make_rsrc(at(a.mean, row, 4), nr * 4u), 0u);
        return 0.f;
    };
    auto load_dres = [&](int64_t row, P (&zv)[FUSED ? K : 1]) {
        if constexpr (FUSED) {
            const rsrc_t rz = window_rsrc<ES>(a.dres, row, a.lddres, 1, row_bytes);
#pragma unroll
            for (int k = 0; k < K; ++k) zv[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rz, off(k));
        }
    };
    int parity = 0;
    // RMSNorm: c1 = r sum x wdy / N, dx = r wdy - r^2 c1 x. LayerNorm, with
    // xc = x - mean: c1 = r sum xc wdy / N, c2 = sum wdy / N, dx = r wdy -
    // r^2 c1 xc - r c2.
    auto process = [&](int64_t row, P (&xv)[K], P (&dv)[K], P (&zv)[FUSED ? K : 1], float r, float mu) {
        fence_gamma();
        float s[LN ? 2 : 1] = {};
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += LG) {
            P gv[LG];
            gamma_group(k0, gv);
#pragma unroll
            for (int j = 0; j < LG; ++j)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float wd = elem(dv[k0 + j], e) * elem(gv[j], e);
                    s[0] = fmaf(elem(xv[k0 + j], e) - mu, wd, s[0]);
                    if constexpr (LN) s[1] += wd;
                }
        }
        block_sum<LN ? 2 : 1>(s, slots, parity);
        if constexpr (GRES) {
#pragma unroll
            for (int k = 0; k < K; ++k) opaque(xv[k], dv[k]);
            fence_gamma();
        }
        const float b = r * r * (s[0] * r * inv_n);  // r^2 c1
        const float d = LN ? r * (s[LN ? 1 : 0] * inv_n) : 0.f;  // r c2
        const rsrc_t rw = window_rsrc<ES>(a.dx, row, a.lddx, 1, row_bytes);
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += LG) {
            P gv[LG];
            gamma_group(k0, gv);
            float tv[LG * VEC];  // this group's dy * x_hat terms
#pragma unroll
            for (int j = 0; j < LG; ++j) {
                const int k = k0 + j;
                float o[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float xe = elem(xv[k], e) - mu;
                    const float dyv = elem(dv[k], e);
                    float dd = fmaf(-b, xe, r * (dyv * elem(gv[j], e)));
                    if constexpr (LN) dd -= d;
                    if constexpr (FUSED) dd += elem(zv[k], e);
                    o[e] = dd;
                    tv[j * VEC + e] = dyv * (xe * r);
                    if constexpr (LN) accb[k][e] += dyv;
                }
                buf_store<DT, VEC, AUX_STREAM_STORE>(rw, off(k), make_pack<DT, VEC>(o));
            }
#pragma unroll
            for (int q = 0; q < LG * VEC / 4; ++q) {
                lf32x4 v = acc_lds[k0 * VEC / 4 + q][t];
                v += lf32x4{tv[4 * q], tv[4 * q + 1], tv[4 * q + 2], tv[4 * q + 3]};
                acc_lds[k0 * VEC / 4 + q][t] = v;
            }
        }
    };
    if constexpr (MODE == LM_PREFETCH) {
        // Two register sets, a and b, alternate: while one row is computed
        // the next row of the block arrives in the other set. The next row's
        // loads are issued after this row's dresidual_out loads and before
        // its stores, so waiting for either never waits for the other row.
        P xa[K], da[K], xb[K], db[K], z[FUSED ? K : 1];
        int64_t row = blockIdx.x;  // < M: the grid has at most M blocks
        load_row(row, 1u, xa, da);
        float ra = load_rstd(row, 1u), rb;
        float ma = load_mean(row, 1u), mb;
        for (;;) {
            const uint32_t nb = row + G < M ? 1u : 0u;
            load_dres(row, z);
            load_row(row + G, nb, xb, db);
            rb = load_rstd(row + G, nb);
            mb = load_mean(row + G, nb);
            process(row, xa, da, z, ra, ma);
            row += G;
            if (row >= M) break;
            const uint32_t na = row + G < M ? 1u : 0u;
            load_dres(row, z);
            load_row(row + G, na, xa, da);
            ra = load_rstd(row + G, na);
            ma = load_mean(row + G, na);
            process(row, xb, db, z, rb, mb);
            row += G;
            if (row >= M) break;
        }
    } else {
        for (int64_t row = blockIdx.x; row < M; row += G) {
            P xv[K], dv[K], zv[FUSED ? K : 1];
            load_row(row, 1u, xv, dv);
            load_dres(row, zv);
            const float r = load_rstd(row, 1u);
            process(row, xv, dv, zv, r, load_mean(row, 1u));
        }
    }
    // this block's weight-gradient sums (dgamma from its own LDS slots: no
    // barrier needed)
    const int64_t pstride = (int64_t)((N + FIN_TILE - 1) / FIN_TILE) * FIN_TILE * G;
    // the thread index passes through an empty asm here, so that the address
    // arithmetic of these stores is not hoisted into the row loop, where its
    // registers would spill
    int te = t;
    asm volatile("" : "+v"(te));
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = te + k * LB;
        if (c < nchunk) emit_chunk<DT, VEC, K, LN>(a, te, c, k, acc_lds, accb, G, pstride);
    }
}

// ---------------------------------------------------------------------------
// Backward, long rows, two passes over each row (see the file comment):
// LayerNorm, and RMSNorm on single elements (16-byte chunks do not fit the
// row or the pointers). dgamma accumulators in LDS; LayerNorm's dbeta
// accumulators in registers.
// ---------------------------------------------------------------------------
template <int DT, int VEC, int OP>
__global__ __launch_bounds__(LB) void bwd_long_2pass_kernel(BwdArgs a) {
    using P = Pack<DT, VEC>;
    constexpr int K = 64 / VEC;
    constexpr bool FUSED = OP == OPL_FUSED, LN = OP == OPL_LN;
    constexpr int ES = ElemSize<DT>::value;
    static_assert((LGROUP * VEC) % 4 == 0, "whole accumulator slots per group");
    __shared__ lf32x4 acc_lds[NSLOT][LB];
    __shared__ float slots[2 * 2 * LWAVES];
    const int N = a.N;
    const int64_t M = a.M;
    const int G = gridDim.x;
    const int t = threadIdx.x;
    const uint32_t row_bytes = (uint32_t)N * ES;
    const int nchunk = N / VEC;
    const float inv_n = 1.0f / (float)N;
    auto off = [&](int k) -> uint32_t {
        const int c = t + k * LB;
        return c < nchunk ? (uint32_t)c * (VEC * ES) : OOB;
    };
#pragma unroll
    for (int q = 0; q < NSLOT; ++q) acc_lds[q][t] = lf32x4{0.f, 0.f, 0.f, 0.f};
    float accb[LN ? K : 1][LN ? VEC : 1];  // dbeta, LayerNorm
#pragma unroll
    for (int k = 0; k < (LN ? K : 1); ++k)
#pragma unroll
        for (int e = 0; e < (LN ? VEC : 1); ++e) accb[k][e] = 0.f;
    const rsrc_t rg = make_rsrc(a.gamma, row_bytes);
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += G) {
        const rsrc_t rx = window_rsrc<ES>(a.x, row, a.ldx, 1, row_bytes);
        const rsrc_t rd = window_rsrc<ES>(a.dy, row, a.lddy, 1, row_bytes);
        const float r = buf_load_f32(make_rsrc(at(a.rstd, row, 4), 4u), 0u);
        float mu = 0.f;
        if constexpr (LN) mu = buf_load_f32(make_rsrc(at(a.mean, row, 4), 4u), 0u);
        // pass 1: the row sums
        float s[2] = {0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += LGROUP) {
            P xv[LGROUP], dv[LGROUP], gv[LGROUP];
#pragma unroll
            for (int j = 0; j < LGROUP; ++j) {
                xv[j] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rx, off(k0 + j));
                dv[j] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rd, off(k0 + j));
                gv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rg, off(k0 + j));
            }
#pragma unroll
            for (int j = 0; j < LGROUP; ++j)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float wd = elem(dv[j], e) * elem(gv[j], e);
                    s[0] = fmaf(elem(xv[j], e) - mu, wd, s[0]);
                    if constexpr (LN) s[1] += wd;
                }
            // single elements: one group's loads in flight at a time, or the
            // unrolled pass hoists all 64 chunks' loads and spills
            if constexpr (VEC == 1) asm volatile("" ::: "memory");
        }
        float b, d = 0.f;
        if constexpr (LN) {
            block_sum<2>(s, slots, parity);
            b = r * r * (s[0] * r * inv_n);  // r^2 c1, c1 = r sum (x - mu) wdy / N
            d = r * (s[1] * inv_n);          // r c2, c2 = sum wdy / N
        } else {
            float t1[1] = {s[0]};
            block_sum<1>(t1, slots, parity);
            b = r * r * (t1[0] * r * inv_n);
        }
        // pass 2: dx, and the weight-gradient terms
        const rsrc_t rz = window_rsrc<ES>(a.dres, row, a.lddres, FUSED ? 1u : 0u, row_bytes);
        const rsrc_t rw = window_rsrc<ES>(a.dx, row, a.lddx, 1, row_bytes);
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += LGROUP) {
            P xv[LGROUP], dv[LGROUP], gv[LGROUP], zv[FUSED ? LGROUP : 1];
#pragma unroll
            for (int j = 0; j < LGROUP; ++j) {
                xv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rx, off(k0 + j));
                dv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rd, off(k0 + j));
                gv[j] = buf_load<DT, VEC, AUX_DEFAULT>(rg, off(k0 + j));
                if constexpr (FUSED) zv[j] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rz, off(k0 + j));
            }
            float tv[LGROUP * VEC];
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
                    tv[j * VEC + e] = dyv * (xc * r);
                    if constexpr (LN) accb[k0 + j][e] += dyv;
                }
                buf_store<DT, VEC, AUX_STREAM_STORE>(rw, off(k0 + j),
                                                                               make_pack<DT, VEC>(o));
            }
#pragma unroll
            for (int q = 0; q < LGROUP * VEC / 4; ++q) {
                lf32x4 v = acc_lds[k0 * VEC / 4 + q][t];
                v += lf32x4{tv[4 * q], tv[4 * q + 1], tv[4 * q + 2], tv[4 * q + 3]};
                acc_lds[k0 * VEC / 4 + q][t] = v;
            }
            if constexpr (VEC == 1) asm volatile("" ::: "memory");
        }
    }
    // this block's weight-gradient sums
    const int64_t pstride = (int64_t)((N + FIN_TILE - 1) / FIN_TILE) * FIN_TILE * G;
    // the thread index passes through an empty asm here, so that the address
    // arithmetic of these stores is not hoisted into the row loop, where its
    // registers would spill
    int te = t;
    asm volatile("" : "+v"(te));
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = te + k * LB;
        if (c < nchunk) emit_chunk<DT, VEC, K, LN>(a, te, c, k, acc_lds, accb, G, pstride);
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

// The RMSNorm long-row backward on 16-byte chunks in the mode long_mode
// picks (plan.h); only the modes an element size and variant can run are
// instantiated.
template <int DT, int VEC, int K, int OP>
hipError_t bwd_long_rms(const BwdArgs &a, int grid, hipStream_t s) {
    constexpr int ES = ElemSize<DT>::value;
    constexpr int FAST = ES == 2 ? LM_PREFETCH : (OP == OPL_FUSED ? LM_RELOAD : LM_RESIDENT);
    // six chunks a thread only for 16-bit rows of at most LONG6_N elements,
    // which long_mode always runs with the next row loaded ahead
    static_assert(K * VEC == 64 || FAST == LM_PREFETCH, "six-chunk rows are 16-bit");
    if constexpr (FAST != LM_RELOAD) {
        if (K * VEC < 64 || long_mode(ES, OP == OPL_FUSED, a.M, a.N) == FAST) {
            hipLaunchKernelGGL((bwd_long_1pass_kernel<DT, VEC, K, OP, FAST>), dim3(grid), dim3(LB), 0, s, a);
            return hipGetLastError();
        }
    }
    if constexpr (K * VEC == 64)
        hipLaunchKernelGGL((bwd_long_1pass_kernel<DT, VEC, K, OP, LM_RELOAD>), dim3(grid), dim3(LB), 0, s, a);
    return hipGetLastError();
}

template <int DT, int VEC, int K>
hipError_t bwd_long_vec(const BwdArgs &a, int grid, hipStream_t s) {
    if (a.layer) {
        // 16-bit rows on 16-byte chunks fit the registers beside the dbeta
        // accumulators and gamma: one read of each row; fp32 rows and single
        // elements take two passes
        if constexpr (ElemSize<DT>::value == 2 && VEC > 1)
            hipLaunchKernelGGL((bwd_long_1pass_kernel<DT, VEC, K, OPL_LN, LM_RESIDENT>), dim3(grid), dim3(LB), 0,
                               s, a);
        else
            hipLaunchKernelGGL((bwd_long_2pass_kernel<DT, VEC, OPL_LN>), dim3(grid), dim3(LB), 0, s, a);
    } else if constexpr (VEC == 1) {
        if (a.dres)
            hipLaunchKernelGGL((bwd_long_2pass_kernel<DT, 1, OPL_FUSED>), dim3(grid), dim3(LB), 0, s, a);
        else
            hipLaunchKernelGGL((bwd_long_2pass_kernel<DT, 1, OPL_RMS>), dim3(grid), dim3(LB), 0, s, a);
    } else if (a.dres) {
        return bwd_long_rms<DT, VEC, K, OPL_FUSED>(a, grid, s);
    } else {
        return bwd_long_rms<DT, VEC, K, OPL_RMS>(a, grid, s);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t fwd_long_dt(const RowPlan &p, const FwdArgs &a, int grid, hipStream_t s) {
    constexpr int VW = 16 / ElemSize<DT>::value;
    // the forward holds 64 elements a thread whatever the backward's chunk count
    if (p.vec == VW && (p.k * VW == 64 || (VW == 8 && p.k == 6))) return fwd_long_vec<DT, VW>(a, grid, s);
    if (p.vec == 1 && p.k == 64) return fwd_long_vec<DT, 1>(a, grid, s);
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t bwd_long_dt(const RowPlan &p, const BwdArgs &a, int grid, hipStream_t s) {
    constexpr int VW = 16 / ElemSize<DT>::value;
    if (p.vec == VW && p.k * VW == 64) return bwd_long_vec<DT, VW, 64 / VW>(a, grid, s);
    if constexpr (VW == 8) {
        if (p.vec == 8 && p.k == 6) return bwd_long_vec<DT, 8, 6>(a, grid, s);
    }
    if (p.vec == 1 && p.k == 64) return bwd_long_vec<DT, 1, 64>(a, grid, s);
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

template <int DT>
hipError_t bwd_next_row_dt(const BwdArgs &a, int grid, hipStream_t s) {
    if (a.layer) {
        hipLaunchKernelGGL((bwd_long_1pass_kernel<DT, 8, 4, OPL_LN, LM_PREFETCH>), dim3(grid), dim3(LB), 0, s, a);
        return hipGetLastError();
    }
    if (a.dres) return bwd_long_rms<DT, 8, 4, OPL_FUSED>(a, grid, s);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_next_row(int dtype, const BwdArgs &a, int grid, hipStream_t s) {
    switch (dtype) {
    case DT_F16: return bwd_next_row_dt<DT_F16>(a, grid, s);
    case DT_BF16: return bwd_next_row_dt<DT_BF16>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rmsn
