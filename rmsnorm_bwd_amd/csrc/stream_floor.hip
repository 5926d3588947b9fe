// stream_floor.hip - a measuring kernel, not part of the C ABI: the
// backward's row traffic without its arithmetic. It moves exactly the row
// bytes the backward moves (two or three (M, N) tensors read, one written)
// through the same row plan, grid, row windows, buffer descriptors, ring of
// windows in flight, prologue pause and cache-policy bits as the backward's
// main kernel, with out = a + b (+ c) in place of the row reduction, the dx
// formula and the weight-gradient partials. What it reaches at a shape is
// what the window ring itself delivers there, the floor the backward is
// measured against. Built into its own library, loaded only by the
// benchmark.
#include "device.h"
#include "plan.h"

namespace rmsn {

struct StreamArgs {
    const void *in[3];  // two or three (M, N) row tensors, contiguous
    void *out;          // (M, N)
    int64_t M;
    int N;
};

template <int DT, int VEC, int TPR, int K, int BLOCK, int DEPTH, int NR>
__global__ __launch_bounds__(BLOCK) void stream_kernel(StreamArgs a) {
    using P = Pack<DT, VEC>;
    constexpr int ES = ElemSize<DT>::value;
    constexpr int RPB = BLOCK / TPR;
    // the backward's dx policy: system-coherent stores with two row reads,
    // non-temporal with three
    constexpr int STORE_AUX = NR == 3 ? AUX_STREAM_STORE : AUX_SINGLE_STORE;
    const int N = a.N;
    const int64_t M = a.M;
    const uint32_t row_bytes = (uint32_t)N * ES;
    const int nchunk = N / VEC;
    const int grp = threadIdx.x / TPR;
    const int lt = threadIdx.x % TPR;
    const uint32_t goff = (uint32_t)(grp * N * ES);
    uint32_t coff[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = lt + k * TPR;
        coff[k] = c < nchunk ? (uint32_t)c * (VEC * ES) : OOB;
    }
    P v[DEPTH][NR][K];
    const int64_t wstride = (int64_t)gridDim.x * RPB;
    const int64_t w0 = (int64_t)blockIdx.x * RPB;

    auto load_window = [&](int64_t wb, P (&w)[NR][K]) {
        const uint32_t nr = rows_in<RPB>(wb, M);
#pragma unroll
        for (int q = 0; q < NR; ++q) {
            const rsrc_t r = window_rsrc<ES>(a.in[q], wb, N, nr, row_bytes);
#pragma unroll
            for (int k = 0; k < K; ++k) w[q][k] = buf_load<DT, VEC, AUX_STREAM_LOAD>(r, goff + coff[k]);
        }
    };
    auto compute = [&](P (&w)[NR][K], P (&o)[K]) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float f[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float t = elem(w[0][k], e) + elem(w[1][k], e);
                if constexpr (NR == 3) t += elem(w[2][k], e);
                f[e] = t;
            }
            o[k] = make_pack<DT, VEC>(f);
        }
    };
    auto store = [&](int64_t wb, const P (&o)[K]) {
        const rsrc_t r = window_rsrc<ES>(a.out, wb, N, rows_in<RPB>(wb, M), row_bytes);
#pragma unroll
        for (int k = 0; k < K; ++k) buf_store<DT, VEC, STORE_AUX>(r, goff + coff[k], o[k]);
    };

    // the backward's prologue: the ring's first windows in order, with its
    // pause when the ring fills
    const bool full_ring = w0 + (DEPTH - 1) * wstride < M;
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
        load_window(w0 + s * wstride, v[s]);
        asm volatile("" ::: "memory");
        if (s + 1 < DEPTH && full_ring) __builtin_amdgcn_s_sleep(8);
    }
    int64_t base = w0;
    for (; base + (DEPTH - 1) * wstride < M; base += DEPTH * wstride) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
            const int64_t wb = base + s * wstride;
            P o[K];
            compute(v[s], o);
            settle(o);
            load_window(wb + DEPTH * wstride, v[s]);
            store(wb, o);
        }
    }
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
#pragma unroll
        for (int q = 0; q < NR; ++q)
#pragma unroll
            for (int k = 0; k < K; ++k) consume(v[s][q][k]);
#pragma unroll
    for (int s = 0; s < DEPTH - 1; ++s) {
        const int64_t wb = base + s * wstride;
        if (wb < M) {
            P o[K];
            compute(v[s], o);
            store(wb, o);
        }
    }
}

// The backward's ring depth for this many row arrays (two reads, or three for
// the fused variant), from the same register budget.
template <int VEC, int K, int NR> constexpr int stream_depth() {
    constexpr int d = RMSN_RING_VGPRS / (NR * (VEC == 1 ? 2 * K : 8 * K));
    return d < 1 ? 1 : (d > RMSN_DEPTH ? RMSN_DEPTH : d);
}

template <int DT, int VEC, int TPR, int K>
static hipError_t go(const StreamArgs &a, int nr, int grid, hipStream_t s) {
    constexpr int BLOCK = block_threads(TPR);
    if (nr == 3)
        hipLaunchKernelGGL((stream_kernel<DT, VEC, TPR, K, BLOCK, stream_depth<VEC, K, 3>(), 3>), dim3(grid),
                           dim3(BLOCK), 0, s, a);
    else
        hipLaunchKernelGGL((stream_kernel<DT, VEC, TPR, K, BLOCK, stream_depth<VEC, K, 2>(), 2>), dim3(grid),
                           dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t dispatch(const RowPlan &p, const StreamArgs &a, int nr, int grid, hipStream_t s) {
    constexpr int VW = 16 / ElemSize<DT>::value;
    if (p.vec != VW) return hipErrorInvalidValue;
    if (p.tpr == 16) {
        if (p.k == 1) return go<DT, VW, 16, 1>(a, nr, grid, s);
        if (p.k == 2) return go<DT, VW, 16, 2>(a, nr, grid, s);
        if (p.k == 4) return go<DT, VW, 16, 4>(a, nr, grid, s);
        return hipErrorInvalidValue;
    }
    if (p.k == 1) {
        switch (p.tpr) {
        case 32: return go<DT, VW, 32, 1>(a, nr, grid, s);
        case 64: return go<DT, VW, 64, 1>(a, nr, grid, s);
        case 128: return go<DT, VW, 128, 1>(a, nr, grid, s);
        case 256: return go<DT, VW, 256, 1>(a, nr, grid, s);
        case 512: return go<DT, VW, 512, 1>(a, nr, grid, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (p.tpr != 512) return hipErrorInvalidValue;
    switch (p.k) {
    case 2: return go<DT, VW, 512, 2>(a, nr, grid, s);
    case 4: return go<DT, VW, 512, 4>(a, nr, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rmsn

// Streams out = a + b (+ c) over (M, N) contiguous rows of `dtype` (0 fp32,
// 1 fp16, 2 bf16) on `stream`, with the grid the backward would launch for
// the same rows. c may be NULL (two reads). Every pointer 16-byte aligned and
// N a multiple of 16 bytes' worth of elements. Returns 0 when enqueued, 1 for
// arguments outside that (nothing launched), 2 for a HIP error.
extern "C" int rmsn_stream_floor(const void *a, const void *b, const void *c, void *out, int64_t M, int64_t N,
                                 int dtype, void *stream) {
    using namespace rmsn;
    if (dtype < 0 || dtype > 2 || M < 1 || M > INT32_MAX || !a || !b || !out) return 1;
    const int es = dtype == 0 ? 4 : 2;
    for (const void *p : {a, b, c, static_cast<const void *>(out)})
        if (p && reinterpret_cast<uintptr_t>(p) % 16) return 1;
    RowPlan p;
    if (!plan_rows(N, es, true, &p) || p.vec * es != 16) return 1;
    const int nr = c ? 3 : 2;
    const int grid = (int)bwd_blocks(M, N, p, nr == 3, DM_DETERMINISTIC);
    StreamArgs args{{a, b, c}, out, M, (int)N};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (dtype) {
    case 0: e = dispatch<DT_F32>(p, args, nr, grid, s); break;
    case 1: e = dispatch<DT_F16>(p, args, nr, grid, s); break;
    default: e = dispatch<DT_BF16>(p, args, nr, grid, s); break;
    }
    if (e == hipErrorInvalidValue) return 1;
    return e == hipSuccess ? 0 : 2;
}
