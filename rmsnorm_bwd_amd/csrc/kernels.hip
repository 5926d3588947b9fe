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
//   - rows are read with 16-byte loads (buffer_load_dwordx4 through buffer
//     descriptors) by consecutive lanes, and each row stays in VGPRs between
//     the reduction and the output pass, so the backward reads x and dy from
//     HBM exactly once;
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
#include <atomic>
#include <mutex>

#include "device.h"
#include "launch.h"
#include "plan.h"
#include "rmsnorm_mi355x.h"

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

// Sums of two values over the tpr threads of a row group, with the same
// one-barrier exchange as row_sum; `slots` then holds 4 * rpb * (tpr / 64)
// floats.
template <int TPR, int BLOCK>
__device__ __forceinline__ void row_sum2(float &u, float &v, float *slots, int parity) {
    if constexpr (TPR <= 64) {
        u = group_sum<TPR>(u);
        v = group_sum<TPR>(v);
    } else {
        constexpr int WPR = TPR / 64;
        constexpr int RPB = BLOCK / TPR;
        u = group_sum<64>(u);
        v = group_sum<64>(v);
        const int wave = threadIdx.x >> 6;
        const int grp = threadIdx.x / TPR;
        float *s = slots + 2 * (parity * (RPB * WPR) + grp * WPR);
        if (__lane_id() == 0) {
            s[2 * (wave % WPR)] = u;
            s[2 * (wave % WPR) + 1] = v;
        }
        __syncthreads();
        float a = s[0], b = s[1];
#pragma unroll
        for (int w = 1; w < WPR; ++w) {
            a += s[2 * w];
            b += s[2 * w + 1];
        }
        u = a;
        v = b;
    }
}

// Store of a dgamma partial: plain (the default), so that the partials stay
// in the caches for the finalize that reads them right after, or
// non-temporal with RMSN_PARTIAL_NT. Measured on MI355X: plain stores take
// 4096 x 4096 bf16 from 22.05 to 20.9 us.
#ifndef RMSN_PARTIAL_NT
#define RMSN_PARTIAL_NT 0
#endif
template <class V>
__device__ __forceinline__ void partial_store(V v, V *p) {
#if RMSN_PARTIAL_NT
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// The operation a row kernel instance computes.
enum : int { OP_RMS = 0, OP_RMS_FUSED = 1, OP_LN = 2 };

// ---------------------------------------------------------------------------
// Backward, main pass. [I769] Implementation plan, Math; [P800] PR-1 and
// fused-add commits. Per row i (x is `added` for the fused variant):
//   x_hat = x * rstd_i, wdy = dy * gamma, c1 = (1/N) sum_j x_hat * wdy,
//   dx = (wdy - x_hat * c1) * rstd_i (+ dresidual_out), dgamma += dy * x_hat.
//
// Block b owns the row windows b*rpb + t*gridDim*rpb (t = 0, 1, ...), each
// window rpb consecutive rows, one per row group. A ring of DEPTH windows is
// in flight: after a window is reduced and stored, its registers receive the
// loads of the window DEPTH steps ahead. All row traffic goes through buffer
// descriptors whose range is the window's existing rows, so rows past M and
// chunks past the row end read as zero and are not stored, without branches;
// that keeps the compiler's memory-counter waits exact, so a window's use
// never waits on the loads of the windows behind it.
// ---------------------------------------------------------------------------
// Pause between the ring's first windows, in units of 64 cycles (s_sleep).
#ifndef RMSN_PROLOGUE_PAUSE
#define RMSN_PROLOGUE_PAUSE 8
#endif

// Row groups a block folds pairwise rather than one after another, and the
// exchange slots the fold needs.
constexpr int FOLD_TREE_MIN = 8;
constexpr int fold_slots(int rpb) { return rpb >= FOLD_TREE_MIN ? rpb / 2 : 1; }

template <int DT, int VEC, int TPR, int K, int BLOCK, int DEPTH, int OP>
__global__ __launch_bounds__(BLOCK) void bwd_main_kernel(BwdArgs a) {
    using P = Pack<DT, VEC>;
    constexpr bool FUSED = OP == OP_RMS_FUSED;
    constexpr bool LN = OP == OP_LN;
    constexpr int NA = LN ? 2 : 1;  // weight-gradient arrays: dgamma, and dbeta for LayerNorm
    constexpr int ES = ElemSize<DT>::value;
    constexpr int RPB = BLOCK / TPR;
    constexpr int WPR = TPR > 64 ? TPR / 64 : 1;
    extern __shared__ float lds[];
    float *slots = lds;
    float *comb = lds + 2 * NA * RPB * WPR;

    const int N = a.N;
    const float inv_n = 1.0f / (float)N;  // one rounding: a multiply, not a divide per row
    const int64_t M = a.M;
    const uint32_t row_bytes = (uint32_t)N * ES;
    const int nchunk = N / VEC;
    const int grp = threadIdx.x / TPR;
    const int lt = threadIdx.x % TPR;
    // byte offset of the thread's row in a window, per row tensor (zero with
    // one row a window)
    const uint32_t gx = (uint32_t)(grp * a.ldx * ES), gd = (uint32_t)(grp * a.lddy * ES);
    const uint32_t gz = (uint32_t)(grp * a.lddres * ES), gw = (uint32_t)(grp * a.lddx * ES);

    // byte offset of each owned chunk inside a row; chunks past the row end
    // get an offset outside every descriptor range
    uint32_t coff[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = lt + k * TPR;
        coff[k] = c < nchunk ? (uint32_t)c * (VEC * ES) : OOB;
    }

    // gamma stays resident, packed, for the whole kernel
    P gp[K];
    {
        const rsrc_t rg = make_rsrc(a.gamma, row_bytes);
#pragma unroll
        for (int k = 0; k < K; ++k) gp[k] = buf_load<DT, VEC, AUX_DEFAULT>(rg, coff[k]);
    }
    // acc[0] folds dy * x_hat (dgamma), acc[1] dy (dbeta, LayerNorm)
    float acc[NA][K][VEC];
#pragma unroll
    for (int q = 0; q < NA; ++q)
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[q][k][e] = 0.f;

    P xs[DEPTH][K], ds[DEPTH][K], rs[DEPTH][FUSED ? K : 1];
    float rr[DEPTH], mr[DEPTH];  // rstd, and the mean for LayerNorm

    const int64_t wstride = (int64_t)gridDim.x * RPB;
    const int64_t w0 = (int64_t)blockIdx.x * RPB;

    auto load_window = [&](int64_t wb, P (&xv)[K], P (&dv)[K], P (&rv)[FUSED ? K : 1], float &r, float &mu) {
        const uint32_t nr = rows_in<RPB>(wb, M);
        const rsrc_t rx = window_rsrc<ES>(a.x, wb, a.ldx, nr, row_bytes);
        const rsrc_t rd = window_rsrc<ES>(a.dy, wb, a.lddy, nr, row_bytes);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            xv[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rx, gx + coff[k]);
            dv[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rd, gd + coff[k]);
        }
        if constexpr (FUSED) {
            const rsrc_t rz = window_rsrc<ES>(a.dres, wb, a.lddres, nr, row_bytes);
#pragma unroll
            for (int k = 0; k < K; ++k) rv[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rz, gz + coff[k]);
        }
        const rsrc_t rt = make_rsrc(at(a.rstd, wb, 4), rows_in<RPB>(wb, M) * 4u);
        r = buf_load_f32(rt, (uint32_t)grp * 4u);
        if constexpr (LN) {
            const rsrc_t rm = make_rsrc(at(a.mean, wb, 4), rows_in<RPB>(wb, M) * 4u);
            mu = buf_load_f32(rm, (uint32_t)grp * 4u);
        } else {
            mu = 0.f;
        }
    };

    // The same arithmetic as the definition, with the per-row factors pulled
    // out of the per-element work. RMSNorm: sum x_hat*wdy = r * sum x*wdy,
    // and dx = (wdy - x_hat*c1) * r = r*wdy - (r*r*c1)*x. LayerNorm, with
    // xc = x - mean: c1 = r * sum xc*wdy / N, c2 = sum wdy / N (both sums in
    // one exchange), dx = (wdy - x_hat*c1 - c2) * r = r*wdy - (r*r*c1)*xc -
    // r*c2. Every row sum flips `parity`. The window's dx is packed into
    // `out`; the caller issues the next window's loads before the stores (see
    // the loop below).
    //
    // A thread whose share of the row is at most 16 values keeps x (centred
    // for LayerNorm) and wdy from the first pass in fp32 registers for the
    // second; with a larger share the second pass recomputes them from the
    // packed row, since keeping 2 * K * VEC fp32 values live across the sum
    // spills (measured on MI355X: keeping them takes fused 1024 x 8192 bf16
    // from 19.0 to 18.5 us and leaves 4096 x 4096 unchanged or faster, while at
    // 32 values a thread 1024 x 16384 goes from 27.4 to 36.7 us).
    constexpr bool KEEP = K * VEC <= 16;
    //
    // acc_on = false leaves the weight-gradient accumulators alone (the last
    // group's terms are added beforehand by `accumulate`, below).
    auto compute = [&](P (&xv)[K], P (&dv)[K], P (&rv)[FUSED ? K : 1], float r, float mu, int &parity,
                       P (&out)[K], bool acc_on) {
        float b, d = 0.f;
        float xk[KEEP ? K : 1][KEEP ? VEC : 1], wk[KEEP ? K : 1][KEEP ? VEC : 1];
        if constexpr (LN) {
            float p1 = 0.f, p2 = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float xc = elem(xv[k], e) - mu;
                    const float wd = elem(dv[k], e) * elem(gp[k], e);
                    if constexpr (KEEP) {
                        xk[k][e] = xc;
                        wk[k][e] = wd;
                    }
                    p1 = fmaf(xc, wd, p1);
                    p2 += wd;
                }
            row_sum2<TPR, BLOCK>(p1, p2, slots, parity);
            parity ^= 1;
            const float c1 = p1 * r * inv_n;
            b = r * r * c1;
            d = r * (p2 * inv_n);
        } else {
            float part = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float wd = elem(dv[k], e) * elem(gp[k], e);
                    if constexpr (KEEP) {
                        xk[k][e] = elem(xv[k], e);
                        wk[k][e] = wd;
                    }
                    part = fmaf(elem(xv[k], e), wd, part);
                }
            const float c1 = row_sum<TPR, BLOCK>(part, slots, parity) * r * inv_n;
            parity ^= 1;
            b = r * r * c1;
        }
        if constexpr (!KEEP) {
#pragma unroll
            for (int k = 0; k < K; ++k) opaque(xv[k], dv[k]);
        }
        // The same for rstd (and the mean). Passing its ring register through
        // an in-place asm also keeps the register allocator from moving the
        // slot's next rstd into a different register, which would need a
        // copy, and a wait for that load, at the loop's back edge.
        float r2 = r, mu2 = mu;
        asm volatile("" : "+v"(r2));
        if constexpr (LN) asm volatile("" : "+v"(mu2));
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float xv_e = KEEP ? xk[k][e] : (LN ? elem(xv[k], e) - mu2 : elem(xv[k], e));
                const float dyv = elem(dv[k], e);
                const float wd = KEEP ? wk[k][e] : dyv * elem(gp[k], e);
                float dd = fmaf(-b, xv_e, r2 * wd);
                if constexpr (LN) dd -= d;
                if constexpr (FUSED) dd += elem(rv[k], e);
                o[e] = dd;
                if (acc_on) {
                    acc[0][k][e] = fmaf(dyv, xv_e * r2, acc[0][k][e]);
                    if constexpr (LN) acc[NA - 1][k][e] += dyv;
                }
            }
            out[k] = make_pack<DT, VEC>(o);
        }
    };
    // dx: NT for the fused backward, on the element path (single elements:
    // 4096 x 12289 bf16 104.0 -> 92.7 us, 600 x 6001 16.4 -> 14.3 us,
    // LayerNorm 4096 x 4097 45.2 -> 42.3 us) and on rows of 512 threads that
    // hold 16 or more elements each for LayerNorm (bf16 1024 x 8192 19.0 ->
    // 17.6 us, 32768 x 8192 266 -> 255 us), 32 or more 16-bit elements for
    // the plain backward (bf16 16384 x 16384 306 -> 295 us, 1024 x 16384
    // 27.6 -> 25.8 us); SC1 on the other 16-byte chunks (NT lost there:
    // plain 16384 x 8192 120 -> 132 us, LayerNorm 131072 x 256 37.0 -> 39.1
    // us, plain fp32 4096 x 16384 136.5 -> 138.5 us)
    constexpr bool ROW_NT =
        TPR == RMSN_TPR_MAX && (LN ? K * VEC >= 16 : ES == 2 && K * VEC >= 32);
    constexpr int DX_STORE = FUSED || VEC == 1 || ROW_NT ? AUX_STREAM_STORE : AUX_SINGLE_STORE;
    auto store_dx = [&](int64_t wb, const P (&out)[K]) {
        const rsrc_t rw = window_rsrc<ES>(a.dx, wb, a.lddx, rows_in<RPB>(wb, M), row_bytes);
#pragma unroll
        for (int k = 0; k < K; ++k) buf_store<DT, VEC, DX_STORE>(rw, gw + coff[k], out[k]);
    };

    // Block b takes the windows b, b + G, b + 2G, ... (G blocks in the grid).
    // The first windows' loads, in window order: the fence keeps the
    // scheduler from sinking a window's rstd load below later windows' row
    // loads, which would make the memory counter's sequence on entering the
    // loop differ from the one on its back edge; the compiler then merges
    // the two pessimistically and waits for windows a step does not use.
    // When the block's ring fills, a short pause (512 cycles) after each
    // window but the last lets the memory system return the first window
    // before the rest, so the first dx stores start earlier: measured on
    // MI355X, 4096 x 4096 bf16 21.4 -> 20.9-21.2 us and 1024 x 4096 10.3 ->
    // 9.9 us; the fused backward is unchanged, and longer pauses lose again.
    // A block with fewer windows (one row: a latency-bound call) does not
    // pause. The test is made once: a test per window costs 0.25 us at
    // 4096 x 4096, and two copies of the prologue cost more.
    const bool full_ring = w0 + (DEPTH - 1) * wstride < M;
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
        load_window(w0 + s * wstride, xs[s], ds[s], rs[s], rr[s], mr[s]);
        asm volatile("" ::: "memory");
        if (s + 1 < DEPTH && full_ring) __builtin_amdgcn_s_sleep(RMSN_PROLOGUE_PAUSE);
    }
    int parity = 0;
    // Steady state: groups of DEPTH windows that all hold rows, with no
    // branch in the body, so every wait counts exactly the loads it
    // needs. Loads and stores retire through one in-order counter, so
    // each window's stores are issued after the loads that refill its
    // ring slot: waiting for a load then never means waiting for a store
    // issued after it (in particular, the loads of windows past the last
    // row, issued in the final group, never hold up the end of the kernel
    // behind the last stores).
    int64_t base = w0;
    for (; base + (DEPTH - 1) * wstride < M; base += DEPTH * wstride) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
            const int64_t wb = base + s * wstride;
            P out[K];
            compute(xs[s], ds[s], rs[s], rr[s], mr[s], parity, out, true);
            settle(out);
            load_window(wb + DEPTH * wstride, xs[s], ds[s], rs[s], rr[s], mr[s]);
            store_dx(wb, out);
        }
    }
    // Take delivery of every load still in flight into the ring, in one
    // wait that only covers stores issued at least a window earlier.
    // After it no load is pending, so the branches of the last, partial
    // group cannot make a later wait conservative (with one in-order
    // counter for loads and stores, a conservative wait would also wait
    // for every store).
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
#pragma unroll
        for (int k = 0; k < K; ++k) {
            consume(xs[s][k]);
            consume(ds[s][k]);
            if constexpr (FUSED) consume(rs[s][k]);
        }
    // ---- this block's weight-gradient partials (dgamma; dbeta for LayerNorm) ----
    // Partials go to the workspace in 16-byte stores where the columns allow;
    // array q of the tiled partials starts q * pstride floats in.
    auto emit_partials = [&]() {
        const int64_t pstride = (int64_t)((N + FIN_TILE - 1) / FIN_TILE) * FIN_TILE * gridDim.x;
        auto emit1 = [&](int q, int j, float v) {
            float *out32 = q ? a.dbeta_f32 : a.dgamma_f32;
            void *outT = q ? a.dbeta : a.dgamma;
            if (a.mode == DG_PARTIAL) {
                partial_store(v, a.partials + q * pstride + partial_index(j, blockIdx.x, gridDim.x));
            } else if (a.mode == DG_ATOMIC) {
                unsafeAtomicAdd(out32 + j, v);
            } else {
                out32[j] = v;
                if (outT) {
                    if constexpr (DT == DT_F32) {
                        static_cast<float *>(outT)[j] = v;
                    } else {
                        static_cast<uint16_t *>(outT)[j] = pack1<DT>(v);
                    }
                }
            }
        };
        // One block writing the gradients itself stores four columns at once (a
        // 16-byte store of the fp32 sums, an 8- or 16-byte store of their dtype
        // copy) where every output is aligned for it: scattered element stores
        // from a single CU are what bound a one-block call (measured on MI355X,
        // one row of 8192 bf16 columns: 8.1 us with element stores).
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        constexpr uintptr_t TA = DT == DT_F32 ? 15 : 7;  // alignment mask of a 4-column dtype copy
        constexpr bool USES_EMIT4 = RPB > 1 || VEC % 4 == 0;  // else only element stores are made
        const bool direct_vec =
            USES_EMIT4 && a.mode == DG_DIRECT && ((reinterpret_cast<uintptr_t>(a.dgamma_f32) & 15) == 0) &&
            ((reinterpret_cast<uintptr_t>(a.dgamma) & TA) == 0) &&
            (NA == 1 || (((reinterpret_cast<uintptr_t>(a.dbeta_f32) & 15) == 0) &&
                         ((reinterpret_cast<uintptr_t>(a.dbeta) & TA) == 0)));
        // four consecutive columns j..j+3 (j a multiple of 4, all < N) lie in one
        // partial tile, so one 16-byte store writes them
        auto emit4 = [&](int q, int j, float v0, float v1, float v2, float v3) {
            if (a.mode == DG_PARTIAL) {
                f32x4 v = {v0, v1, v2, v3};
                partial_store(v, reinterpret_cast<f32x4 *>(a.partials + q * pstride +
                                                           partial_index(j, blockIdx.x, gridDim.x)));
            } else if (direct_vec) {
                float *out32 = q ? a.dbeta_f32 : a.dgamma_f32;
                void *outT = q ? a.dbeta : a.dgamma;
                *reinterpret_cast<f32x4 *>(out32 + j) = f32x4{v0, v1, v2, v3};
                if (outT) {
                    if constexpr (DT == DT_F32) {
                        *reinterpret_cast<f32x4 *>(static_cast<float *>(outT) + j) = f32x4{v0, v1, v2, v3};
                    } else {
                        *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(outT) + j) =
                            u32x2{pack2<DT>(v0, v1), pack2<DT>(v2, v3)};
                    }
                }
            } else {
                emit1(q, j, v0);
                emit1(q, j + 1, v1);
                emit1(q, j + 2, v2);
                emit1(q, j + 3, v3);
            }
        };
        if constexpr (RPB == 1) {
#pragma unroll
            for (int q = 0; q < NA; ++q)
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int c = lt + k * TPR;
                    if (c < nchunk) {
                        if constexpr (VEC % 4 == 0) {
#pragma unroll
                            for (int e = 0; e < VEC; e += 4)
                                emit4(q, c * VEC + e, acc[q][k][e], acc[q][k][e + 1], acc[q][k][e + 2],
                                      acc[q][k][e + 3]);
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) emit1(q, c * VEC + e, acc[q][k][e]);
                        }
                    }
                }
        } else {
            // Fold the rpb row groups in a fixed order and leave the block's total
            // in slot 0, from which all threads write it out. With 8 or more
            // groups, pairwise: in the round of half-width h (rpb/2, rpb/4, ...,
            // 1) groups h..2h-1 leave their sums in exchange slot g - h and groups
            // 0..h-1 add them (group 0 ends with ((g0 + g8) + (g4 + g12)) + ...),
            // 2 log2(rpb) barriers instead of one a group; with fewer groups, one
            // group after another into slot 0. Measured on MI355X (GPU time per
            // call): 16 groups, 8 x 256 fp32 7.1 -> 4.2 us, 32 x 256 bf16 6.1 ->
            // 4.5 us, 16384 x 512 bf16 18.1 -> 14.1 us, 32768 x 256 bf16 14.3 ->
            // 12.5 us; 4 groups are 0.1 us faster one after another.
            constexpr int CS = TPR * K * VEC;  // floats of one array in a slot
            auto slot_io = [&](int s, bool add) {
                float *sl = comb + s * (NA * CS);
#pragma unroll
                for (int q = 0; q < NA; ++q)
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        const int c = lt + k * TPR;
                        if (c < nchunk)
#pragma unroll
                            for (int e = 0; e < VEC; ++e) {
                                float *p = sl + q * CS + c * VEC + e;
                                if (add)
                                    acc[q][k][e] += *p;
                                else
                                    *p = acc[q][k][e];
                            }
                    }
            };
            if constexpr (RPB >= FOLD_TREE_MIN) {
#pragma unroll
                for (int h = RPB / 2; h >= 1; h >>= 1) {
                    if (grp >= h && grp < 2 * h) slot_io(grp - h, false);
                    __syncthreads();
                    if (grp < h) {
                        slot_io(grp, true);
                        if (h == 1) slot_io(0, false);
                    }
                    __syncthreads();
                }
            } else {
                for (int gi = 0; gi < RPB; ++gi) {
                    if (grp == gi) {
#pragma unroll
                        for (int q = 0; q < NA; ++q)
#pragma unroll
                            for (int k = 0; k < K; ++k) {
                                const int c = lt + k * TPR;
                                if (c < nchunk)
#pragma unroll
                                    for (int e = 0; e < VEC; ++e) {
                                        float *cq = comb + q * CS + c * VEC + e;
                                        *cq = gi == 0 ? acc[q][k][e] : *cq + acc[q][k][e];
                                    }
                            }
                    }
                    __syncthreads();
                }
            }
            const int n4 = N & ~3;
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const float *cq = comb + q * CS;  // slot 0
                for (int j = threadIdx.x * 4; j < n4; j += BLOCK * 4)
                    emit4(q, j, cq[j], cq[j + 1], cq[j + 2], cq[j + 3]);
                for (int j = n4 + threadIdx.x; j < N; j += BLOCK) emit1(q, j, cq[j]);
            }
        }
    };

    // A window's weight-gradient terms, as `compute` forms them.
    auto accumulate = [&](const P (&xv)[K], const P (&dv)[K], float r, float mu) {
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float xv_e = LN ? elem(xv[k], e) - mu : elem(xv[k], e);
                const float dyv = elem(dv[k], e);
                acc[0][k][e] = fmaf(dyv, xv_e * r, acc[0][k][e]);
                if constexpr (LN) acc[NA - 1][k][e] += dyv;
            }
    };
    // The last, partial group (block-uniform tests): its rows are loaded.
    // With one row a window its weight-gradient terms, which need the saved
    // statistics but not the row sums, are added first and the block's
    // partials go out before the group's row sums and dx, overlapping them
    // instead of trailing the last dx stores. The sums take the same rows in
    // the same order either way, so the results are bit-identical. Measured
    // on MI355X, bf16, µs per call: fused 1024 x 8192 17.9-18.0 -> 17.3-17.5,
    // LayerNorm 4096 x 4096 23.0-23.6 -> 22.8, plain 512 x 8192 11.8 -> 11.1,
    // 128 x 4096 6.45 -> 6.2-6.3; 4096 x 4096, 16384 x 4096 and 32768 x 8192
    // unchanged. Blocks of several rows, whose fold across row groups takes
    // barriers, lost 2-5% with it (128 x 1024 6.3 -> 6.5-6.6, fused 512 x
    // 2048 7.4 -> 7.6) and store after the group, as does a block whose
    // windows fill whole groups (it has no partial group).
    if (RPB == 1 && base < M) {
#pragma unroll
        for (int s = 0; s < DEPTH - 1; ++s)
            if (base + s * wstride < M) accumulate(xs[s], ds[s], rr[s], mr[s]);
        emit_partials();
#pragma unroll
        for (int s = 0; s < DEPTH - 1; ++s) {
            const int64_t wb = base + s * wstride;
            if (wb < M) {
                P out[K];
                compute(xs[s], ds[s], rs[s], rr[s], mr[s], parity, out, false);
                store_dx(wb, out);
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < DEPTH - 1; ++s) {
            const int64_t wb = base + s * wstride;
            if (wb < M) {
                P out[K];
                compute(xs[s], ds[s], rs[s], rr[s], mr[s], parity, out, true);
                store_dx(wb, out);
            }
        }
        emit_partials();
    }
}

// ---------------------------------------------------------------------------
// Backward, dgamma finalize (deterministic mode): dgamma_f32[j] = sum over the
// G block partials in a fixed order, and its rounding to the dtype.
// The partials are stored in tiles of FIN_TILE columns (16 by default):
// tile t is a [G][FIN_TILE] block of floats, one contiguous run of
// G * FIN_TILE * 4 bytes. One 256-thread block reduces one tile: thread i
// owns column i % FIN_TILE and rows i / FIN_TILE + FIN_RS k (k = 0, 1, ...;
// FIN_RS = 256 / FIN_TILE), issuing all its loads before the first add (for
// each k the block reads 1 KiB contiguously), then the FIN_RS per-thread sums
// of a column are added in row order through LDS. Measured on MI355X, wider
// tiles (whole 128-byte lines per block row of a tile) do not pay:
// 4096 x 4096 bf16 20.6-20.7 us at 16 columns, 21.1 at 32, 21.8 at 64.
// ---------------------------------------------------------------------------
constexpr int FIN_RS = 256 / FIN_TILE;  // partial rows one pass of the block covers
constexpr int FIN_LOADS = (BWD_MAX_BLOCKS + FIN_RS - 1) / FIN_RS;

template <int DT>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const float *__restrict__ partials, int G, int N,
                                                           float *__restrict__ dgamma_f32,
                                                           void *__restrict__ dgamma,
                                                           float *__restrict__ dbeta_f32,
                                                           void *__restrict__ dbeta) {
    // blockIdx.y selects the partial array: 0 dgamma, 1 dbeta (LayerNorm)
    __shared__ float red[FIN_RS][FIN_TILE];
    const int c = threadIdx.x % FIN_TILE;
    const int r0 = threadIdx.x / FIN_TILE;
    const int64_t pstride = (int64_t)((N + FIN_TILE - 1) / FIN_TILE) * FIN_TILE * G;
    const float *tile = partials + blockIdx.y * pstride + (int64_t)blockIdx.x * G * FIN_TILE;
    float *out32 = blockIdx.y ? dbeta_f32 : dgamma_f32;
    void *outT = blockIdx.y ? dbeta : dgamma;
    float v[FIN_LOADS];
#pragma unroll
    for (int k = 0; k < FIN_LOADS; ++k) {
        const int g = r0 + FIN_RS * k;
        v[k] = g < G ? tile[g * FIN_TILE + c] : 0.f;
    }
    float t = v[0];
#pragma unroll
    for (int k = 1; k < FIN_LOADS; ++k) t += v[k];
    red[r0][c] = t;
    __syncthreads();
    const int col = blockIdx.x * FIN_TILE + c;
    if (r0 == 0 && col < N) {
        float sum = red[0][c];
#pragma unroll
        for (int w = 1; w < FIN_RS; ++w) sum += red[w][c];
        out32[col] = sum;
        if (outT) {
            if constexpr (DT == DT_F32) {
                static_cast<float *>(outT)[col] = sum;
            } else {
                static_cast<uint16_t *>(outT)[col] = pack1<DT>(sum);
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
// LayerNorm ([I769] PR sequence and status updates: the forward saves mean
// and rstd), in two row sums over the row held in registers:
//   mean = sum x / N, rstd = 1 / sqrt(sum (x - mean)^2 / N + eps),
//   y = (x - mean) * rstd * gamma + beta
// Same windows, ring and buffer descriptors as the backward.
// ---------------------------------------------------------------------------
template <int DT, int VEC, int TPR, int K, int BLOCK, int DEPTH, int OP>
__global__ __launch_bounds__(BLOCK) void fwd_kernel(FwdArgs a) {
    using P = Pack<DT, VEC>;
    constexpr bool FUSED = OP == OP_RMS_FUSED;
    constexpr bool LN = OP == OP_LN;
    constexpr int ES = ElemSize<DT>::value;
    constexpr int RPB = BLOCK / TPR;
    extern __shared__ float lds[];

    const int N = a.N;
    const int64_t M = a.M;
    const uint32_t row_bytes = (uint32_t)N * ES;
    const int nchunk = N / VEC;
    const int grp = threadIdx.x / TPR;
    const int lt = threadIdx.x % TPR;
    // byte offset of the thread's row in a window, per row tensor
    const uint32_t gx = (uint32_t)(grp * a.ldx * ES), gr = (uint32_t)(grp * a.ldres * ES);
    const uint32_t gy = (uint32_t)(grp * a.ldy * ES), go = (uint32_t)(grp * a.ldres_out * ES);

    uint32_t coff[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = lt + k * TPR;
        coff[k] = c < nchunk ? (uint32_t)c * (VEC * ES) : OOB;
    }
    P gp[K], bp[LN ? K : 1];
    {
        const rsrc_t rg = make_rsrc(a.gamma, row_bytes);
#pragma unroll
        for (int k = 0; k < K; ++k) gp[k] = buf_load<DT, VEC, AUX_DEFAULT>(rg, coff[k]);
        if constexpr (LN) {
            // a null beta gets an empty range: its loads read zeros
            const rsrc_t rb = make_rsrc(a.beta, a.beta ? row_bytes : 0u);
#pragma unroll
            for (int k = 0; k < K; ++k) bp[k] = buf_load<DT, VEC, AUX_DEFAULT>(rb, coff[k]);
        }
    }

    P xs[DEPTH][K], rs[DEPTH][FUSED ? K : 1];
    const int64_t wstride = (int64_t)gridDim.x * RPB;
    const int64_t w0 = (int64_t)blockIdx.x * RPB;
    // the row's rstd is written by thread 0 of its group
    const uint32_t rstd_off = lt == 0 ? (uint32_t)grp * 4u : OOB;

    auto load_window = [&](int64_t wb, P (&xv)[K], P (&rv)[FUSED ? K : 1]) {
        const uint32_t nr = rows_in<RPB>(wb, M);
        const rsrc_t rx = window_rsrc<ES>(a.x, wb, a.ldx, nr, row_bytes);
#pragma unroll
        for (int k = 0; k < K; ++k) xv[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rx, gx + coff[k]);
        if constexpr (FUSED) {
            const rsrc_t rz = window_rsrc<ES>(a.residual, wb, a.ldres, nr, row_bytes);
#pragma unroll
            for (int k = 0; k < K; ++k) rv[k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(rz, gr + coff[k]);
        }
    };

    // Computes the window's outputs (y packed into `yo`, added into `av`)
    // and stores rstd (and the mean); y and residual_out are stored by the
    // caller after it has issued the loads that refill the ring slot. Every
    // row sum flips `parity`.
    auto compute = [&](int64_t wb, P (&xv)[K], P (&rv)[FUSED ? K : 1], int &parity, P (&av)[K], P (&yo)[K]) {
        const uint32_t nr = rows_in<RPB>(wb, M);
        if constexpr (LN) {
            float s1 = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) s1 += elem(xv[k], e);
            const float mu = row_sum<TPR, BLOCK>(s1, lds, parity) / (float)N;
            parity ^= 1;
            float s2 = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    // chunks past the row end hold zeros but are not part of it
                    const float dv = coff[k] == OOB ? 0.f : elem(xv[k], e) - mu;
                    s2 = fmaf(dv, dv, s2);
                }
            const float var = row_sum<TPR, BLOCK>(s2, lds, parity) / (float)N;
            parity ^= 1;
            const float r = 1.0f / sqrtf(var + a.eps);
            buf_store_f32(make_rsrc(at(a.rstd, wb, 4), nr * 4u), rstd_off, r);
            buf_store_f32(make_rsrc(at(a.mean, wb, 4), nr * 4u), rstd_off, mu);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float o[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    o[e] = fmaf((elem(xv[k], e) - mu) * r, elem(gp[k], e), elem(bp[k], e));
                yo[k] = make_pack<DT, VEC>(o);
                av[k] = xv[k];
            }
            return;
        }
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if constexpr (FUSED) {
                float t[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) t[e] = elem(xv[k], e) + elem(rv[k], e);
                av[k] = make_pack<DT, VEC>(t);  // added, rounded once to the dtype
            } else {
                av[k] = xv[k];
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float v = elem(av[k], e);
                part = fmaf(v, v, part);
            }
        }
        const float ms = row_sum<TPR, BLOCK>(part, lds, parity) / (float)N;
        parity ^= 1;
        const float r = 1.0f / sqrtf(ms + a.eps);
        buf_store_f32(make_rsrc(at(a.rstd, wb, 4), nr * 4u), rstd_off, r);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = elem(av[k], e) * r * elem(gp[k], e);
            yo[k] = make_pack<DT, VEC>(o);
        }
    };
    // y: NT for the fused forward and where a thread holds 16 or more
    // elements of a row, SC1 below (the measurements are at the cache-policy
    // bits in device.h)
    constexpr int Y_STORE = FUSED || K * VEC >= 16 ? AUX_FWD_STORE : AUX_FWD_SHORT_STORE;
    auto store_rows = [&](int64_t wb, const P (&av)[K], const P (&yo)[K]) {
        const uint32_t nr = rows_in<RPB>(wb, M);
        const rsrc_t ry = window_rsrc<ES>(a.y, wb, a.ldy, nr, row_bytes);
#pragma unroll
        for (int k = 0; k < K; ++k) buf_store<DT, VEC, Y_STORE>(ry, gy + coff[k], yo[k]);
        if constexpr (FUSED) {
            const rsrc_t ro = window_rsrc<ES>(a.residual_out, wb, a.ldres_out, nr, row_bytes);
#pragma unroll
            for (int k = 0; k < K; ++k) buf_store<DT, VEC, AUX_STREAM_STORE>(ro, go + coff[k], av[k]);
        }
    };

    const bool full_ring = w0 + (DEPTH - 1) * wstride < M;
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
        load_window(w0 + s * wstride, xs[s], rs[s]);
        asm volatile("" ::: "memory");  // window order, as in the backward
        // the backward's prologue pause; measured on MI355X it takes the plain
        // forward at 4096 x 4096 bf16 from 13.25 to 13.0 us and at 16384 x
        // 4096 from 42.9 to 42.1 us, and does nothing for the fused forward
        if constexpr (!FUSED) {
            if (s + 1 < DEPTH && full_ring) __builtin_amdgcn_s_sleep(RMSN_PROLOGUE_PAUSE);
        }
    }
    int parity = 0;
    // As in the backward: full groups without branches, and each window's
    // stores issued after the loads that refill its ring slot.
    int64_t base = w0;
    for (; base + (DEPTH - 1) * wstride < M; base += DEPTH * wstride) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
            const int64_t wb = base + s * wstride;
            P av[K], yo[K];
            compute(wb, xs[s], rs[s], parity, av, yo);
            settle(yo);
            load_window(wb + DEPTH * wstride, xs[s], rs[s]);
            store_rows(wb, av, yo);
        }
    }
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
#pragma unroll
        for (int k = 0; k < K; ++k) {
            consume(xs[s][k]);
            if constexpr (FUSED) consume(rs[s][k]);
        }
#pragma unroll
    for (int s = 0; s < DEPTH - 1; ++s) {
        const int64_t wb = base + s * wstride;
        if (wb < M) {
            P av[K], yo[K];
            compute(wb, xs[s], rs[s], parity, av, yo);
            store_rows(wb, av, yo);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

template <int TPR> constexpr int block_of() { return block_threads(TPR); }

// Windows in flight per row group: as many as fit RMSN_RING_VGPRS registers
// of ring, at most RMSN_DEPTH and at least one. A window costs, per row array
// (2, or 3 for the fused variant), 8 registers per 16-byte chunk on the vector
// path and 2 per element on the element path (the loaded bytes plus the
// unpacked values the arithmetic keeps live). LayerNorm's second set of
// accumulators (dbeta, one register per element held) comes out of the same
// budget. With blocks of up to 512 threads a wave may use 256 VGPRs; the
// budget leaves room for gamma, the accumulators and the arithmetic, so that
// no vector-path instance spills.
template <int VEC, int TPR, int K, int OP> constexpr int ring_depth() {
    static_assert(block_of<TPR>() <= 512, "blocks of at most 512 threads");
    constexpr int per_window = (OP == OP_RMS_FUSED ? 3 : 2) * (VEC == 1 ? 2 * K : 8 * K);
    constexpr int budget = RMSN_RING_VGPRS - (OP == OP_LN ? K * VEC : 0);
    constexpr int d = budget / per_window;
    return d < 1 ? 1 : (d > RMSN_DEPTH ? RMSN_DEPTH : d);
}

// PLAIN = false and LAYER = false leave the plain and the LayerNorm backward
// out (for a plan that only the others take); a call that would need it then
// fails with hipErrorInvalidValue.
template <int DT, int VEC, int TPR, int K, bool PLAIN = true, bool LAYER = true>
static hipError_t launch_bwd_cfg(const BwdArgs &a, int grid, hipStream_t s) {
    constexpr int BLOCK = block_of<TPR>();
    constexpr int RPB = BLOCK / TPR;
    constexpr int WPR = TPR > 64 ? TPR / 64 : 1;
    constexpr int DF = ring_depth<VEC, TPR, K, OP_RMS_FUSED>();
    constexpr int DP = ring_depth<VEC, TPR, K, OP_RMS>();
    constexpr int DL = ring_depth<VEC, TPR, K, OP_LN>();
    // LDS: the row-sum slots (two values a row for LayerNorm), then, when a
    // block holds several rows, the exchange slots of the row-group fold, one
    // combine area per weight-gradient array each (at most 32 KiB)
    const int na = a.layer ? 2 : 1;
    const size_t lds = (size_t)(2 * na * RPB * WPR + (RPB > 1 ? fold_slots(RPB) * na * TPR * K * VEC : 0)) *
                       sizeof(float);
    if (a.layer) {
        if constexpr (LAYER)
            hipLaunchKernelGGL((bwd_main_kernel<DT, VEC, TPR, K, BLOCK, DL, OP_LN>), dim3(grid), dim3(BLOCK), lds, s,
                               a);
        else
            return hipErrorInvalidValue;
    } else if (a.dres)
        hipLaunchKernelGGL((bwd_main_kernel<DT, VEC, TPR, K, BLOCK, DF, OP_RMS_FUSED>), dim3(grid), dim3(BLOCK), lds,
                           s, a);
    else if constexpr (PLAIN)
        hipLaunchKernelGGL((bwd_main_kernel<DT, VEC, TPR, K, BLOCK, DP, OP_RMS>), dim3(grid), dim3(BLOCK), lds, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// The forward's ring holds fewer row arrays than the backward's: x (plain,
// LayerNorm) or x and residual (fused), with no dy. Counting its own arrays
// lets rows of four or more chunks a thread keep a deeper ring (measured on
// MI355X against the backward's count, µs per call: fused 16384 x 12288 bf16
// 290.4 -> 273.5, LayerNorm 8192 x 16384 bf16 100.3 -> 92.7, plain 8192 x
// 16384 bf16 92.2 -> 88.9, fused 8192 x 8192 fp32 195.8 -> 188.5, plain
// 4096 x 12289 bf16 (element path) 71.5 -> 68.5). LayerNorm's element path
// keeps the backward's count: its 32-element rows would spill otherwise.
template <int VEC, int TPR, int K, int OP> constexpr int fwd_ring_depth() {
    if constexpr (OP == OP_LN && VEC == 1) {
        return ring_depth<VEC, TPR, K, OP>();
    } else {
        constexpr int per_window = (OP == OP_RMS_FUSED ? 2 : 1) * (VEC == 1 ? 2 * K : 8 * K);
        constexpr int d = RMSN_RING_VGPRS / per_window;
        return d < 1 ? 1 : (d > RMSN_DEPTH ? RMSN_DEPTH : d);
    }
}

template <int DT, int VEC, int TPR, int K>
static hipError_t launch_fwd_cfg(const FwdArgs &a, int grid, hipStream_t s) {
    constexpr int BLOCK = block_of<TPR>();
    constexpr int RPB = BLOCK / TPR;
    constexpr int WPR = TPR > 64 ? TPR / 64 : 1;
    constexpr int DF = fwd_ring_depth<VEC, TPR, K, OP_RMS_FUSED>();
    constexpr int DP = fwd_ring_depth<VEC, TPR, K, OP_RMS>();
    constexpr int DL = fwd_ring_depth<VEC, TPR, K, OP_LN>();
    const size_t lds = (size_t)(2 * RPB * WPR) * sizeof(float);
    if (a.mean)
        hipLaunchKernelGGL((fwd_kernel<DT, VEC, TPR, K, BLOCK, DL, OP_LN>), dim3(grid), dim3(BLOCK), lds, s, a);
    else if (a.residual)
        hipLaunchKernelGGL((fwd_kernel<DT, VEC, TPR, K, BLOCK, DF, OP_RMS_FUSED>), dim3(grid), dim3(BLOCK), lds, s, a);
    else
        hipLaunchKernelGGL((fwd_kernel<DT, VEC, TPR, K, BLOCK, DP, OP_RMS>), dim3(grid), dim3(BLOCK), lds, s, a);
    return hipGetLastError();
}

// Dispatch of (vec, tpr, k) to a kernel instance. Every plan plan_rows can
// return has an instance; anything else is reported as hipErrorInvalidValue
// without a launch.
template <template <int, int, int, int> class L, int DT, int VW, int K, class A>
static hipError_t by_tpr(int tpr, const A &a, int grid, hipStream_t s) {
    switch (tpr) {
    case 16: return L<DT, VW, 16, K>::go(a, grid, s);
    case 32: return L<DT, VW, 32, K>::go(a, grid, s);
    case 64: return L<DT, VW, 64, K>::go(a, grid, s);
    case 128: return L<DT, VW, 128, K>::go(a, grid, s);
    case 256: return L<DT, VW, 256, K>::go(a, grid, s);
    case 512: return L<DT, VW, 512, K>::go(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

template <template <int, int, int, int> class L, int DT, class A>
static hipError_t dispatch(const RowPlan &p, const A &a, int grid, hipStream_t s) {
    constexpr int VW = 16 / ElemSize<DT>::value;
    static_assert(RMSN_TPR_MAX == 512 || RMSN_TPR_MAX == 256, "row thread cap");
    if (p.vec == VW) {
        if (p.tpr == 16) {  // short rows inside one wavefront
            if (p.k == 1) return L<DT, VW, 16, 1>::go(a, grid, s);
            if (p.k == 2) return L<DT, VW, 16, 2>::go(a, grid, s);
            if (p.k == 4) return L<DT, VW, 16, 4>::go(a, grid, s);
        }
        if (p.k == RMSN_K_MIN && p.tpr < RMSN_TPR_MAX) return by_tpr<L, DT, VW, RMSN_K_MIN>(p.tpr, a, grid, s);
        if (p.tpr == RMSN_TPR_MAX) {
            switch (p.k) {
            case 1: return L<DT, VW, RMSN_TPR_MAX, 1>::go(a, grid, s);
            case 2: return L<DT, VW, RMSN_TPR_MAX, 2>::go(a, grid, s);
            case 4: return L<DT, VW, RMSN_TPR_MAX, 4>::go(a, grid, s);
            case 8:  // only fp32 rows are long enough
                if constexpr (VW == 4) return L<DT, VW, RMSN_TPR_MAX, 8>::go(a, grid, s);
                break;
            default: break;
            }
        }
    } else if (p.vec == 1) {
        if (p.tpr == 64 && p.k == 4) return L<DT, 1, 64, 4>::go(a, grid, s);
        if (p.tpr == 64 && p.k == 8) return L<DT, 1, 64, 8>::go(a, grid, s);
        if (p.tpr == 64 && p.k == 16) return L<DT, 1, 64, 16>::go(a, grid, s);
        if (p.tpr == 256 && p.k == 8) return L<DT, 1, 256, 8>::go(a, grid, s);
        if (p.tpr == 256 && p.k == 16) return L<DT, 1, 256, 16>::go(a, grid, s);
        if (p.tpr == 512 && p.k == 16) return L<DT, 1, 512, 16>::go(a, grid, s);
        if (p.tpr == 512 && p.k == 32) return L<DT, 1, 512, 32>::go(a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <int DT, int VEC, int TPR, int K> struct BwdLaunch {
    static hipError_t go(const BwdArgs &a, int grid, hipStream_t s) {
        return launch_bwd_cfg<DT, VEC, TPR, K>(a, grid, s);
    }
};
template <int DT, int VEC, int TPR, int K> struct FwdLaunch {
    static hipError_t go(const FwdArgs &a, int grid, hipStream_t s) {
        return launch_fwd_cfg<DT, VEC, TPR, K>(a, grid, s);
    }
};

// Rows of four 16-byte chunks a thread on 512-thread groups leave the fused
// backward (dresidual_out in its ring) and LayerNorm's (its dbeta
// accumulators) one window in flight; bwd_route (plan.h) hands them to
// other kernels:
// - three chunks a thread, for rows of at most 1536 chunks (8200-12288
//   16-bit or 4100-6144 fp32 elements), which leaves room for two windows.
//   Measured on MI355X, µs per call: fused bf16 16384 x 10240 286.9 ->
//   225.7, 16384 x 12288 310.5 -> 271.1, 4096 x 12288 86.9 -> 74.3; fused
//   fp32 16384 x 6144 281.6 -> 263.4, 4096 x 5120 68.8 -> 59.4; LayerNorm
//   bf16 16384 x 12288 230.3 -> 211.9, 4096 x 10240 65.3 -> 54.1. LayerNorm
//   fp32 was mixed (16384 x 6144 200.5 -> 209.0, 4096 x 5120 48.6 -> 47.4)
//   and the plain backward, two windows at four chunks already, slower (bf16
//   16384 x 12288 202.0 -> 222.5): both keep four.
// - the long-row kernel, for 16-bit rows of 1537-2048 chunks (12296-16384
//   elements): it keeps its dgamma accumulators in LDS and so holds the
//   block's next row in flight while it computes the current one. Measured,
//   µs per call: fused bf16 16384 x 14336 359.2 -> 315.1, 4096 x 12296
//   94.9 -> 84.8, 2048 x 16384 58.3 -> 55.1, 512 x 16384 22.2 -> 20.4;
//   LayerNorm bf16 4096 x 14336 80.1 -> 72.6, 16384 x 12296 287.2 -> 271.4,
//   1024 x 16384 36.5 -> 34.3, f16 4096 x 16384 88.9 -> 81.4. LayerNorm rows
//   of exactly 16384 elements lost there at many rows (6144 x 16384 124.0
//   -> 128.4, 16384 x 16384 297 -> 324) and keep this kernel above 2^26
//   elements a call; the plain backward gains nothing (16384 x 16384 298 ->
//   310, 4096 x 14336 63.5 -> 62.4) and stays.
template <int DT>
static hipError_t dispatch_bwd(const RowPlan &p, const BwdArgs &a, int grid, hipStream_t s) {
    if (p.long_row) return launch_bwd_long(DT, p, a, grid, s);
    constexpr int VW = 16 / ElemSize<DT>::value;
    constexpr bool B16 = VW == 8;  // 16-bit elements
    switch (bwd_route(ElemSize<DT>::value, a.dres != nullptr, a.layer, p, a.M, a.N)) {
    case BR_THREE_CHUNKS: return launch_bwd_cfg<DT, VW, RMSN_TPR_MAX, 3, false, B16>(a, grid, s);
    case BR_NEXT_ROW: return launch_bwd_next_row(DT, a, grid, s);
    default: return dispatch<BwdLaunch, DT>(p, a, grid, s);
    }
}

// The forward's route for 16-bit rows whose plan leaves chunk slots empty
// (fwd_route in plan.h, with its measurements): three chunks a thread on 512
// threads, on 256-thread groups two rows a block, on 128-thread groups four
// rows a block, on one wavefront a row (four rows a block), on 32-thread
// groups (eight rows a block) or with three chunks instead of four on the
// plan's 16-thread groups; every other forward takes its row plan.
template <int DT>
static hipError_t dispatch_fwd(const RowPlan &p, const FwdArgs &a, int grid, hipStream_t s) {
    if (p.long_row) return launch_fwd_long(DT, p, a, grid, s);
    constexpr int VW = 16 / ElemSize<DT>::value;
    switch (fwd_route(ElemSize<DT>::value, a.residual != nullptr, a.mean != nullptr, p, a.M, a.N)) {
    case FR_THREE_CHUNKS:  // 16-bit rows only
        if constexpr (VW == 8) return launch_fwd_cfg<DT, VW, RMSN_TPR_MAX, 3>(a, grid, s);
        break;
    case FR_HALF_ROWS:  // 16-bit rows only
        if constexpr (VW == 8) return launch_fwd_cfg<DT, VW, RMSN_TPR_MAX / 2, 3>(a, grid, s);
        break;
    case FR_QUARTER_ROWS: return launch_fwd_cfg<DT, VW, RMSN_TPR_MAX / 4, 3>(a, grid, s);
    case FR_WAVE_ROWS: return launch_fwd_cfg<DT, VW, 64, 3>(a, grid, s);
    case FR_NARROW_ROWS: return launch_fwd_cfg<DT, VW, 32, 3>(a, grid, s);
    case FR_SHORT_ROWS:  // 16-bit rows only
        if constexpr (VW == 8) return launch_fwd_cfg<DT, VW, 16, 3>(a, grid, s);
        break;
    default: break;
    }
    return dispatch<FwdLaunch, DT>(p, a, grid, s);
}

template <int DT>
static hipError_t launch_bwd_dt(const RowPlan &p, const BwdArgs &args, int grid, void *workspace,
                                hipStream_t s) {
    BwdArgs a = args;
    const int na = a.layer ? 2 : 1;  // weight-gradient arrays: dgamma, and dbeta for LayerNorm
    float *out32[2] = {a.dgamma_f32, a.dbeta_f32};
    void *outT[2] = {a.dgamma, a.dbeta};
    const dim3 vec_grid((a.N + 255) / 256);
    // zero (and, with `cast`, round to the dtype) every weight-gradient array
    auto zero_all = [&](bool cast) -> hipError_t {
        for (int q = 0; q < na; ++q) {
            hipLaunchKernelGGL(fill_zero_kernel, vec_grid, dim3(256), 0, s, out32[q], a.N);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            if (cast && outT[q]) {
                hipLaunchKernelGGL(cast_kernel<DT>, vec_grid, dim3(256), 0, s, out32[q], outT[q], a.N);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
        }
        return hipSuccess;
    };
    hipError_t e;
    if (a.M == 0) return zero_all(true);  // no rows: the weight gradients are zero
    if (a.mode == DG_PARTIAL) {
        a.partials = reinterpret_cast<float *>(static_cast<char *>(workspace) + WS_HEADER);
        if ((e = dispatch_bwd<DT>(p, a, grid, s)) != hipSuccess) return e;
        hipLaunchKernelGGL(bwd_finalize_kernel<DT>, dim3((a.N + FIN_TILE - 1) / FIN_TILE, na), dim3(256), 0, s,
                           a.partials, grid, a.N, a.dgamma_f32, a.dgamma, a.dbeta_f32, a.dbeta);
        return hipGetLastError();
    }
    if (a.mode == DG_ATOMIC) {
        if ((e = zero_all(false)) != hipSuccess) return e;
        if ((e = dispatch_bwd<DT>(p, a, grid, s)) != hipSuccess) return e;
        for (int q = 0; q < na; ++q)
            if (outT[q]) {
                hipLaunchKernelGGL(cast_kernel<DT>, vec_grid, dim3(256), 0, s, out32[q], outT[q], a.N);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
        return hipSuccess;
    }
    return dispatch_bwd<DT>(p, a, grid, s);  // DG_DIRECT: one block writes the gradients itself
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

// ---------------------------------------------------------------------------
// Scratch of rmsnorm_bwd_no_alloc: one static array per GPU, the workspace of
// callers that cannot allocate. In host code `scratch` names a host-side
// stand-in, not device memory; the kernels get its device address, looked up
// once per device with that device current and remembered here.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[RMSN_NO_ALLOC_SCRATCH_BYTES];
static_assert(RMSN_NO_ALLOC_SCRATCH_BYTES >= WS_HEADER, "the scratch holds at least the header");

constexpr int SCRATCH_DEVICES = 64;
static std::atomic<void *> scratch_addr[SCRATCH_DEVICES];
static std::mutex scratch_mu;

hipError_t device_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_DEVICES) return hipErrorInvalidDevice;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr) {
                (void)hipGetLastError();
                return e != hipSuccess ? e : hipErrorInvalidSymbol;
            }
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
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
