// autograd_ext.cpp - the autograd nodes of rmsnorm(x, weight, eps),
// fused_add_rmsnorm(x, residual, weight, eps) and layer_norm(x, weight, bias,
// eps) as torch C++ autograd Functions over the library's C ABI.
//
// Marshalling only, as the Python binding: each node allocates its outputs
// with torch, finds the current HIP stream, and calls the C entry point; all
// arithmetic runs in the library's kernels. Written in C++ so that torch's
// autograd engine calls the backward without entering Python: through a
// Python autograd.Function the engine's hand-off to the interpreter and the
// binding's own checks cost more host time per backward than the kernels of
// a small problem take.
//
// Pages cited, by title:
//   [I769] FlyDSL issue #769, "[Feature] Add rmsnorm backward (+ forward saves
//          rstd) to enable training / downstream (quack) integration" - Scope /
//          tasks items 3-4 (an autograd function whose forward saves x, the
//          weight and rstd and whose backward calls the backward kernel; the
//          gradient of residual_out on the fused path); PR sequence and status
//          updates (the LayerNorm follow-up: forward saving mean and rstd,
//          backward with the bias gradient).
//   [P800] FlyDSL PR #800, "[rmsnorm] Add fused-add / residual backward (PR
//          2/3, #769)" - PR-1 commit (rmsnorm(x, weight, eps) over inputs of
//          any rank, rows on the last dimension); fused-add commit (the
//          prenorm form returns (out, residual_out); one gradient serves x
//          and residual).
#include <torch/extension.h>

#include <c10/core/DeviceGuard.h>
#include <c10/hip/HIPStream.h>
#include <hip/hip_runtime_api.h>

#include <list>
#include <mutex>
#include <utility>
#include <vector>

#include "rmsnorm_mi355x.h"

namespace {

using torch::Tensor;
using torch::autograd::AutogradContext;
using torch::autograd::variable_list;

int dtype_code(const Tensor &t) {
    switch (t.scalar_type()) {
    case at::kFloat: return RMSN_F32;
    case at::kHalf: return RMSN_F16;
    case at::kBFloat16: return RMSN_BF16;
    default: TORCH_CHECK_TYPE(false, "rmsnorm_bwd_amd: unsupported dtype ", t.scalar_type());
    }
    return -1;
}

void check_status(int status, const char *fn) {
    TORCH_CHECK(status == RMSN_OK, fn, ": status ", status, " (", rmsn_status_string(status), ")");
}

// (M, ld) of a row tensor whose last dimension holds a row's N elements at
// unit stride and whose leading dimensions collapse into one row stride ld;
// false for any other layout (the caller then copies it).
bool row_view(const Tensor &t, int64_t N, int64_t &M, int64_t &ld) {
    if (t.dim() == 0 || t.size(-1) != N) return false;
    if (t.is_contiguous()) {
        M = t.numel() / N;
        ld = N;
        return true;
    }
    if (N > 1 && t.stride(-1) != 1) return false;
    std::vector<std::pair<int64_t, int64_t>> lead;
    for (int64_t d = 0; d + 1 < t.dim(); ++d)
        if (t.size(d) != 1) lead.emplace_back(t.size(d), t.stride(d));
    M = 1;
    for (const auto &p : lead) M *= p.first;
    if (lead.empty()) {
        ld = N;
        return true;
    }
    for (size_t i = 0; i + 1 < lead.size(); ++i)
        if (lead[i].second != lead[i + 1].second * lead[i + 1].first) return false;
    ld = lead.back().second;
    return ld >= N;
}

// The tensor itself when the library can read it in place, else a copy.
Tensor rows_of(const Tensor &t, int64_t N, int64_t &M, int64_t &ld) {
    if (row_view(t, N, M, ld)) return t;
    Tensor c = t.contiguous();
    M = c.numel() / N;
    ld = N;
    return c;
}

void *ptr(const Tensor &t) { return t.defined() ? t.data_ptr() : nullptr; }

hipStream_t current_stream(const Tensor &t) {
    return c10::hip::getCurrentHIPStream(t.device().index()).stream();
}

// One backward workspace per (device, stream), at most 16 streams, the least
// recently used dropped first; calls on one stream run in order, so they
// never share one concurrently, and torch's allocator hands a dropped buffer
// only to later work of the stream that used it. A call on a stream that is
// being captured into a graph never uses the cache: the graph keeps the
// workspace's address for its replays, so it gets a buffer of its own from
// the graph's memory pool, which lives as long as the graph.
struct WorkspaceCache {
    struct Entry {
        int device;
        hipStream_t stream;
        Tensor buf;
    };
    std::mutex mu;
    std::list<Entry> lru;  // most recent first
    static constexpr size_t kStreams = 16;

    Tensor get(const Tensor &like, hipStream_t s, size_t need) {
        const size_t bytes = need < 256 ? 256 : need;
        auto opts = like.options().dtype(at::kByte);
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
            (void)hipGetLastError();
            cs = hipStreamCaptureStatusNone;
        }
        if (cs != hipStreamCaptureStatusNone) return torch::empty({(int64_t)bytes}, opts);
        const int dev = like.device().index();
        std::lock_guard<std::mutex> lock(mu);
        for (auto it = lru.begin(); it != lru.end(); ++it) {
            if (it->device == dev && it->stream == s) {
                if ((size_t)it->buf.numel() < bytes) it->buf = torch::empty({(int64_t)bytes}, opts);
                lru.splice(lru.begin(), lru, it);
                return lru.front().buf;
            }
        }
        lru.push_front(Entry{dev, s, torch::empty({(int64_t)bytes}, opts)});
        while (lru.size() > kStreams) lru.pop_back();
        return lru.front().buf;
    }
};

WorkspaceCache &workspaces() {
    static WorkspaceCache *c = new WorkspaceCache();  // never destroyed: lives past interpreter teardown
    return *c;
}

// The weight's gradient in its dtype: the fp32 sum for fp32 weights, else
// the library's round-to-nearest-even copy.
Tensor weight_grad(const Tensor &weight, const Tensor &g32, const Tensor &gT) {
    return weight.scalar_type() == at::kFloat ? g32 : gT;
}

void check_operands(const Tensor &x, const Tensor &weight, const char *fn) {
    TORCH_CHECK_VALUE(x.is_cuda(), fn, ": tensors must be on a GPU");
    TORCH_CHECK_VALUE(weight.dim() == 1 && x.dim() >= 1 && x.size(-1) == weight.size(0), fn,
                      ": x.shape[-1] must equal the weight's length");
    TORCH_CHECK_TYPE(x.scalar_type() == weight.scalar_type(), fn, ": x and weight must share one dtype");
    TORCH_CHECK_VALUE(x.device() == weight.device(), fn, ": tensors on different devices");
}

// ---------------------------------------------------------------------------
// rmsnorm: y = x * rstd * weight, rstd = 1/sqrt(mean(x^2) + eps) per row
// ---------------------------------------------------------------------------
struct RMSNormFn : public torch::autograd::Function<RMSNormFn> {
    static Tensor forward(AutogradContext *ctx, Tensor x, Tensor weight, double eps) {
        check_operands(x, weight, "rmsnorm");
        const int64_t N = weight.size(0);
        weight = weight.contiguous();
        int64_t M, ldx;
        x = rows_of(x, N, M, ldx);
        c10::DeviceGuard guard(x.device());
        Tensor y = torch::empty(x.sizes(), x.options());
        Tensor rstd = torch::empty({M}, x.options().dtype(at::kFloat));
        const int dt = dtype_code(x);
        void *s = current_stream(x);
        const int st = ldx == N ? rmsnorm_fwd_rstd(ptr(x), ptr(weight), ptr(y), rstd.data_ptr<float>(), M, N,
                                                   (float)eps, dt, s)
                                : rmsnorm_fwd_rstd_strided(ptr(x), ldx, ptr(weight), ptr(y), N,
                                                           rstd.data_ptr<float>(), M, N, (float)eps, dt, s);
        check_status(st, "rmsnorm_fwd_rstd");
        ctx->save_for_backward({x, weight, rstd});
        return y;
    }

    static variable_list backward(AutogradContext *ctx, variable_list grads) {
        const auto saved = ctx->get_saved_variables();
        const Tensor &x = saved[0], &weight = saved[1], &rstd = saved[2];
        const int64_t N = weight.size(0), M = rstd.size(0);
        int64_t Mx, ldx, Md, lddy;
        row_view(x, N, Mx, ldx);
        Tensor dy = rows_of(grads[0], N, Md, lddy);
        c10::DeviceGuard guard(x.device());
        Tensor dx = torch::empty(x.sizes(), x.options());
        Tensor dg32 = torch::empty({N}, x.options().dtype(at::kFloat));
        Tensor dgT = weight.scalar_type() == at::kFloat ? Tensor() : torch::empty_like(weight);
        const int dt = dtype_code(x);
        hipStream_t s = current_stream(x);
        Tensor ws = workspaces().get(x, s, rmsnorm_bwd_workspace_bytes(M, N, dt, RMSN_DGAMMA_AUTO));
        const int st =
            ldx == N && lddy == N
                ? rmsnorm_bwd(ptr(x), ptr(weight), ptr(dy), rstd.data_ptr<float>(), ptr(dx), dg32.data_ptr<float>(),
                              ptr(dgT), ptr(ws), (size_t)ws.numel(), M, N, dt, RMSN_DGAMMA_AUTO, s)
                : rmsnorm_bwd_strided(ptr(x), ldx, ptr(weight), ptr(dy), lddy, rstd.data_ptr<float>(), ptr(dx), N,
                                      dg32.data_ptr<float>(), ptr(dgT), ptr(ws), (size_t)ws.numel(), M, N, dt,
                                      RMSN_DGAMMA_AUTO, s);
        check_status(st, "rmsnorm_bwd");
        return {dx, weight_grad(weight, dg32, dgT), Tensor()};
    }
};

// ---------------------------------------------------------------------------
// fused_add_rmsnorm: residual_out = x + residual (one rounding),
// out = rmsnorm(residual_out); returns (out, residual_out)
// ---------------------------------------------------------------------------
struct FusedAddRMSNormFn : public torch::autograd::Function<FusedAddRMSNormFn> {
    static variable_list forward(AutogradContext *ctx, Tensor x, Tensor residual, Tensor weight, double eps) {
        check_operands(x, weight, "fused_add_rmsnorm");
        TORCH_CHECK_VALUE(residual.sizes() == x.sizes(), "fused_add_rmsnorm: residual must have x's shape");
        TORCH_CHECK_TYPE(residual.scalar_type() == x.scalar_type(), "fused_add_rmsnorm: one dtype for all operands");
        TORCH_CHECK_VALUE(residual.device() == x.device(), "fused_add_rmsnorm: tensors on different devices");
        const int64_t N = weight.size(0);
        weight = weight.contiguous();
        int64_t M, ldx, Mr, ldr;
        x = rows_of(x, N, M, ldx);
        residual = rows_of(residual, N, Mr, ldr);
        c10::DeviceGuard guard(x.device());
        Tensor out = torch::empty(x.sizes(), x.options());
        Tensor added = torch::empty(x.sizes(), x.options());
        Tensor rstd = torch::empty({M}, x.options().dtype(at::kFloat));
        const int dt = dtype_code(x);
        void *s = current_stream(x);
        const int st =
            ldx == N && ldr == N
                ? fused_add_rmsnorm_fwd_rstd(ptr(x), ptr(residual), ptr(weight), ptr(out), ptr(added),
                                             rstd.data_ptr<float>(), M, N, (float)eps, dt, s)
                : fused_add_rmsnorm_fwd_rstd_strided(ptr(x), ldx, ptr(residual), ldr, ptr(weight), ptr(out), N,
                                                     ptr(added), N, rstd.data_ptr<float>(), M, N, (float)eps, dt, s);
        check_status(st, "fused_add_rmsnorm_fwd_rstd");
        ctx->save_for_backward({added, weight, rstd});
        return {out, added};
    }

    static variable_list backward(AutogradContext *ctx, variable_list grads) {
        const auto saved = ctx->get_saved_variables();
        const Tensor &added = saved[0], &weight = saved[1], &rstd = saved[2];
        const int64_t N = weight.size(0), M = rstd.size(0);
        int64_t Md, lddy = N, Mr, lddres = N;
        // no gradient reached `out`: its gradient is zeros; none reached
        // residual_out: the library takes a NULL dresidual_out as zeros
        Tensor dy = grads[0].defined() ? rows_of(grads[0], N, Md, lddy) : torch::zeros_like(added);
        Tensor dres = grads[1].defined() ? rows_of(grads[1], N, Mr, lddres) : Tensor();
        c10::DeviceGuard guard(added.device());
        Tensor dx = torch::empty(added.sizes(), added.options());
        Tensor dg32 = torch::empty({N}, added.options().dtype(at::kFloat));
        Tensor dgT = weight.scalar_type() == at::kFloat ? Tensor() : torch::empty_like(weight);
        const int dt = dtype_code(added);
        hipStream_t s = current_stream(added);
        Tensor ws = workspaces().get(added, s, rmsnorm_bwd_workspace_bytes(M, N, dt, RMSN_DGAMMA_AUTO));
        const int st =
            lddy == N && lddres == N
                ? fused_add_rmsnorm_bwd(ptr(added), ptr(weight), ptr(dy), ptr(dres), rstd.data_ptr<float>(),
                                        ptr(dx), dg32.data_ptr<float>(), ptr(dgT), ptr(ws), (size_t)ws.numel(), M,
                                        N, dt, RMSN_DGAMMA_AUTO, s)
                : fused_add_rmsnorm_bwd_strided(ptr(added), N, ptr(weight), ptr(dy), lddy, ptr(dres), lddres,
                                                rstd.data_ptr<float>(), ptr(dx), N, dg32.data_ptr<float>(),
                                                ptr(dgT), ptr(ws), (size_t)ws.numel(), M, N, dt, RMSN_DGAMMA_AUTO,
                                                s);
        check_status(st, "fused_add_rmsnorm_bwd");
        // x and residual enter only through their sum: one gradient for both
        return {dx, dx, weight_grad(weight, dg32, dgT), Tensor()};
    }
};

// ---------------------------------------------------------------------------
// layer_norm: y = (x - mean) * rstd * weight + bias
// ---------------------------------------------------------------------------
struct LayerNormFn : public torch::autograd::Function<LayerNormFn> {
    static Tensor forward(AutogradContext *ctx, Tensor x, Tensor weight, Tensor bias, double eps) {
        check_operands(x, weight, "layer_norm");
        const int64_t N = weight.size(0);
        const bool has_bias = bias.defined();
        if (has_bias) {
            TORCH_CHECK_VALUE(bias.dim() == 1 && bias.size(0) == N, "layer_norm: bias must have N elements");
            TORCH_CHECK_TYPE(bias.scalar_type() == x.scalar_type(), "layer_norm: one dtype for all operands");
            bias = bias.contiguous();
        }
        weight = weight.contiguous();
        int64_t M, ldx;
        x = rows_of(x, N, M, ldx);
        c10::DeviceGuard guard(x.device());
        Tensor y = torch::empty(x.sizes(), x.options());
        Tensor mean = torch::empty({M}, x.options().dtype(at::kFloat));
        Tensor rstd = torch::empty({M}, x.options().dtype(at::kFloat));
        const int dt = dtype_code(x);
        void *s = current_stream(x);
        const int st = ldx == N ? layernorm_fwd_stats(ptr(x), ptr(weight), ptr(bias), ptr(y), mean.data_ptr<float>(),
                                                      rstd.data_ptr<float>(), M, N, (float)eps, dt, s)
                                : layernorm_fwd_stats_strided(ptr(x), ldx, ptr(weight), ptr(bias), ptr(y), N,
                                                              mean.data_ptr<float>(), rstd.data_ptr<float>(), M, N,
                                                              (float)eps, dt, s);
        check_status(st, "layernorm_fwd_stats");
        ctx->save_for_backward({x, weight, mean, rstd});
        ctx->saved_data["has_bias"] = has_bias;
        return y;
    }

    static variable_list backward(AutogradContext *ctx, variable_list grads) {
        const auto saved = ctx->get_saved_variables();
        const Tensor &x = saved[0], &weight = saved[1], &mean = saved[2], &rstd = saved[3];
        const bool has_bias = ctx->saved_data["has_bias"].toBool();
        const int64_t N = weight.size(0), M = rstd.size(0);
        int64_t Mx, ldx, Md, lddy;
        row_view(x, N, Mx, ldx);
        Tensor dy = rows_of(grads[0], N, Md, lddy);
        c10::DeviceGuard guard(x.device());
        const bool half = weight.scalar_type() != at::kFloat;
        Tensor dx = torch::empty(x.sizes(), x.options());
        Tensor dg32 = torch::empty({N}, x.options().dtype(at::kFloat));
        Tensor db32 = torch::empty({N}, x.options().dtype(at::kFloat));
        Tensor dgT = half ? torch::empty_like(weight) : Tensor();
        Tensor dbT = half && has_bias ? torch::empty_like(weight) : Tensor();
        const int dt = dtype_code(x);
        hipStream_t s = current_stream(x);
        Tensor ws = workspaces().get(x, s, layernorm_bwd_workspace_bytes(M, N, dt, RMSN_DGAMMA_AUTO));
        const int st =
            ldx == N && lddy == N
                ? layernorm_bwd(ptr(x), ptr(weight), ptr(dy), mean.data_ptr<float>(), rstd.data_ptr<float>(), ptr(dx),
                                dg32.data_ptr<float>(), db32.data_ptr<float>(), ptr(dgT), ptr(dbT), ptr(ws),
                                (size_t)ws.numel(), M, N, dt, RMSN_DGAMMA_AUTO, s)
                : layernorm_bwd_strided(ptr(x), ldx, ptr(weight), ptr(dy), lddy, mean.data_ptr<float>(),
                                        rstd.data_ptr<float>(), ptr(dx), N, dg32.data_ptr<float>(),
                                        db32.data_ptr<float>(), ptr(dgT), ptr(dbT), ptr(ws), (size_t)ws.numel(), M, N,
                                        dt, RMSN_DGAMMA_AUTO, s);
        check_status(st, "layernorm_bwd");
        Tensor dbias = has_bias ? (half ? dbT : db32) : Tensor();
        return {dx, weight_grad(weight, dg32, dgT), dbias, Tensor()};
    }
};

}  // namespace

PYBIND11_MODULE(_autograd_ext, m) {
    m.doc() = "torch autograd nodes of rmsnorm, fused_add_rmsnorm and layer_norm over the library's C ABI";
    m.def("rmsnorm", [](const Tensor &x, const Tensor &weight, double eps) {
        return RMSNormFn::apply(x, weight, eps);
    });
    m.def("fused_add_rmsnorm", [](const Tensor &x, const Tensor &residual, const Tensor &weight, double eps) {
        auto outs = FusedAddRMSNormFn::apply(x, residual, weight, eps);
        return std::make_tuple(outs[0], outs[1]);
    });
    m.def("layer_norm", [](const Tensor &x, const Tensor &weight, const c10::optional<Tensor> &bias, double eps) {
        return LayerNormFn::apply(x, weight, bias.has_value() ? *bias : Tensor(), eps);
    });
}
