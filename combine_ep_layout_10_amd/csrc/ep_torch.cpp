// Compiled torch binding of the hot entry points of include/ep.h: argument
// marshalling only. Each function checks its tensors (device, contiguity,
// dtype, shape against the handle's or config's sizes, so no kernel can
// index past a caller's buffer), turns them into pointers and calls the C
// ABI; every step of the path runs in the HIP kernels behind libep.so, which
// this module links. It exists because the same checks written in Python
// cost the host 2-3 us per call, as much as the kernel launch itself on
// launch-bound shapes (decode). ops.py owns allocation and the handle
// objects; configs and handles arrive as the addresses of their C structs.
#include <torch/extension.h>

#include <initializer_list>
#include <stdexcept>
#include <string>

#include "../../include/ep.h"

namespace {

void ok(ep_status s, const char* where) {
    if (s != EP_OK)
        throw std::runtime_error(std::string(where) + " failed: " + ep_status_string(s) + ": " +
                                 ep_last_error_message());
}

// Device pointer of a contiguous tensor of dtype dt on device dev.
void* ptr(const at::Tensor& t, const char* name, at::ScalarType dt, int64_t dev) {
    if (!t.is_cuda()) throw std::invalid_argument(std::string(name) + " must be a device tensor");
    if (t.get_device() != dev)
        throw std::invalid_argument(std::string(name) + " is on device " + std::to_string(t.get_device()) +
                                    ", not on the current device " + std::to_string(dev));
    if (!t.is_contiguous()) throw std::invalid_argument(std::string(name) + " must be contiguous");
    if (t.scalar_type() != dt)
        throw std::invalid_argument(std::string(name) + " has dtype " + std::string(c10::toString(t.scalar_type())) +
                                    ", expected " + std::string(c10::toString(dt)));
    return t.data_ptr();
}

void* opt_ptr(const c10::optional<at::Tensor>& t, const char* name, at::ScalarType dt, int64_t dev) {
    return t.has_value() ? ptr(*t, name, dt, dev) : nullptr;
}

void shape(const at::Tensor& t, std::initializer_list<int64_t> want, const char* name) {
    bool same = t.dim() == (int64_t)want.size();
    int i = 0;
    for (int64_t w : want) same = same && t.size(i++) == w;
    if (!same) {
        std::string s = "(";
        for (int64_t w : want) s += std::to_string(w) + ",";
        throw std::invalid_argument(std::string(name) + " has shape " + c10::str(t.sizes()) + ", expected " + s +
                                    ")");
    }
}

void opt_shape(const c10::optional<at::Tensor>& t, std::initializer_list<int64_t> want, const char* name) {
    if (t.has_value()) shape(*t, want, name);
}

const ep_config* cfg_of(int64_t addr) { return reinterpret_cast<const ep_config*>(addr); }
ep_handle* handle_of(int64_t addr) { return reinterpret_cast<ep_handle*>(addr); }

int64_t rows_bound(const ep_config* c) {
    const int64_t r = ep_recv_rows_bound(c);
    if (r < 0) ok(EP_ERR_INVALID_ARG, "ep_recv_rows_bound");
    return r;
}

at::ScalarType idx_type(const ep_config* c) { return c->idx_bits == 64 ? at::kLong : at::kInt; }

void* stream_of(int64_t s) { return reinterpret_cast<void*>(s); }

// ---------------------------------------------------------------- calls

void layout(int64_t cfg, const at::Tensor& topk_idx, const c10::optional<at::Tensor>& topk_w,
            const at::Tensor& workspace, int64_t handle, int64_t stream, int64_t dev) {
    const ep_config* c = cfg_of(cfg);
    const int64_t T = topk_idx.dim() == 2 ? topk_idx.size(0) : -1;
    shape(topk_idx, {T, c->num_topk}, "topk_idx");
    opt_shape(topk_w, {T, c->num_topk}, "topk_w");
    ok(ep_layout(c, (int32_t)T, ptr(topk_idx, "topk_idx", idx_type(c), dev),
                 (const float*)opt_ptr(topk_w, "topk_w", at::kFloat, dev),
                 ptr(workspace, "workspace", at::kByte, dev), (size_t)workspace.numel(), handle_of(handle),
                 stream_of(stream)),
       "ep_layout");
}

void dispatch_forward(int64_t cfg, const at::Tensor& topk_idx, const c10::optional<at::Tensor>& topk_w,
                      const at::Tensor& workspace, int64_t dtype, const at::Tensor& x,
                      const c10::optional<at::Tensor>& x_scales, const at::Tensor& recv,
                      const c10::optional<at::Tensor>& recv_scales, int64_t handle, int64_t stream, int64_t dev) {
    const ep_config* c = cfg_of(cfg);
    const int64_t T = topk_idx.dim() == 2 ? topk_idx.size(0) : -1;
    const int64_t H = c->hidden, R = rows_bound(c);
    const bool fp8 = dtype != EP_BF16, pre = dtype == EP_FP8_PREQUANT;
    shape(topk_idx, {T, c->num_topk}, "topk_idx");
    opt_shape(topk_w, {T, c->num_topk}, "topk_w");
    shape(x, {T, H}, "x");
    if (pre) opt_shape(x_scales, {T, H / 128}, "x_scales");
    shape(recv, {R, H}, "recv");
    if (fp8) opt_shape(recv_scales, {R, H / 128}, "recv_scales");
    ok(ep_dispatch_forward(c, (int32_t)T, ptr(topk_idx, "topk_idx", idx_type(c), dev),
                           (const float*)opt_ptr(topk_w, "topk_w", at::kFloat, dev),
                           ptr(workspace, "workspace", at::kByte, dev), (size_t)workspace.numel(), (int32_t)dtype,
                           ptr(x, "x", pre ? at::kByte : at::kBFloat16, dev),
                           (const float*)opt_ptr(x_scales, "x_scales", at::kFloat, dev),
                           ptr(recv, "recv", fp8 ? at::kByte : at::kBFloat16, dev),
                           (float*)opt_ptr(recv_scales, "recv_scales", at::kFloat, dev), handle_of(handle),
                           stream_of(stream)),
       "ep_dispatch_forward");
}

// ep_dispatch (pair_w absent) and ep_combine_backward (pair_w = topk_w):
// both move a [T, H] input (with its 1x128 scales when pre-quantised) into
// the receive rows of the handle.
void dispatch_like(int64_t handle, int64_t dtype, const at::Tensor& x, const c10::optional<at::Tensor>& x_scales,
                   const c10::optional<at::Tensor>& pair_w, const at::Tensor& recv,
                   const c10::optional<at::Tensor>& recv_scales, bool backward, int64_t stream, int64_t dev) {
    const ep_handle* h = handle_of(handle);
    const ep_config* c = &h->cfg;
    const int64_t T = h->num_tokens, H = c->hidden, R = rows_bound(c);
    const bool fp8 = dtype != EP_BF16, pre = dtype == EP_FP8_PREQUANT;
    shape(x, {T, H}, backward ? "grad_out" : "x");
    if (pre) opt_shape(x_scales, {T, H / 128}, backward ? "grad_out_scales" : "x_scales");
    opt_shape(pair_w, {T, c->num_topk}, "topk_w");
    shape(recv, {R, H}, backward ? "grad_y" : "recv");
    if (fp8) opt_shape(recv_scales, {R, H / 128}, backward ? "grad_y_scales" : "recv_scales");
    void* px = ptr(x, backward ? "grad_out" : "x", pre ? at::kByte : at::kBFloat16, dev);
    void* pr = ptr(recv, backward ? "grad_y" : "recv", fp8 ? at::kByte : at::kBFloat16, dev);
    float* prs = (float*)opt_ptr(recv_scales, backward ? "grad_y_scales" : "recv_scales", at::kFloat, dev);
    const float* pxs = (const float*)opt_ptr(x_scales, backward ? "grad_out_scales" : "x_scales", at::kFloat, dev);
    if (backward)
        ok(ep_combine_backward(h, (int32_t)dtype, px, pxs, (const float*)opt_ptr(pair_w, "topk_w", at::kFloat, dev),
                               pr, prs, stream_of(stream)),
           "ep_combine_backward");
    else
        ok(ep_dispatch(h, (int32_t)dtype, px, pxs, pr, prs, stream_of(stream)), "ep_dispatch");
}

void dispatch(int64_t handle, int64_t dtype, const at::Tensor& x, const c10::optional<at::Tensor>& x_scales,
              const at::Tensor& recv, const c10::optional<at::Tensor>& recv_scales, int64_t stream, int64_t dev) {
    dispatch_like(handle, dtype, x, x_scales, c10::nullopt, recv, recv_scales, false, stream, dev);
}

void combine_backward(int64_t handle, int64_t dtype, const at::Tensor& grad_out,
                      const c10::optional<at::Tensor>& grad_out_scales, const c10::optional<at::Tensor>& topk_w,
                      const at::Tensor& grad_y, const c10::optional<at::Tensor>& grad_y_scales, int64_t stream,
                      int64_t dev) {
    dispatch_like(handle, dtype, grad_out, grad_out_scales, topk_w, grad_y, grad_y_scales, true, stream, dev);
}

// ep_combine (weights optional) and ep_dispatch_backward (no weights): a
// [rows, H] input reduced into [T, H], with the optional per-row values
// gathered to [T, k].
void combine_like(int64_t handle, const at::Tensor& y, const c10::optional<at::Tensor>& topk_w,
                  const at::Tensor& out, const c10::optional<at::Tensor>& row_vals,
                  const c10::optional<at::Tensor>& out_vals, bool backward, int64_t stream, int64_t dev) {
    const ep_handle* h = handle_of(handle);
    const ep_config* c = &h->cfg;
    const int64_t T = h->num_tokens, H = c->hidden, k = c->num_topk, R = rows_bound(c);
    shape(y, {R, H}, backward ? "grad_recv" : "y");
    opt_shape(topk_w, {T, k}, "topk_w");
    shape(out, {T, H}, backward ? "grad_x" : "out");
    opt_shape(row_vals, {R}, backward ? "grad_row_w" : "row_vals");
    opt_shape(out_vals, {T, k}, backward ? "grad_topk_w" : "out_vals");
    const void* py = ptr(y, backward ? "grad_recv" : "y", at::kBFloat16, dev);
    void* po = ptr(out, backward ? "grad_x" : "out", at::kBFloat16, dev);
    const float* prv = (const float*)opt_ptr(row_vals, backward ? "grad_row_w" : "row_vals", at::kFloat, dev);
    float* pov = (float*)opt_ptr(out_vals, backward ? "grad_topk_w" : "out_vals", at::kFloat, dev);
    if (backward)
        ok(ep_dispatch_backward(h, py, prv, po, pov, stream_of(stream)), "ep_dispatch_backward");
    else
        ok(ep_combine(h, py, (const float*)opt_ptr(topk_w, "topk_w", at::kFloat, dev), po, prv, pov,
                      stream_of(stream)),
           "ep_combine");
}

void combine(int64_t handle, const at::Tensor& y, const c10::optional<at::Tensor>& topk_w, const at::Tensor& out,
             const c10::optional<at::Tensor>& row_vals, const c10::optional<at::Tensor>& out_vals, int64_t stream,
             int64_t dev) {
    combine_like(handle, y, topk_w, out, row_vals, out_vals, false, stream, dev);
}

void dispatch_backward(int64_t handle, const at::Tensor& grad_recv, const c10::optional<at::Tensor>& grad_row_w,
                       const at::Tensor& grad_x, const c10::optional<at::Tensor>& grad_topk_w, int64_t stream,
                       int64_t dev) {
    combine_like(handle, grad_recv, c10::nullopt, grad_x, grad_row_w, grad_topk_w, true, stream, dev);
}

}  // namespace

PYBIND11_MODULE(TORCH_EXTENSION_NAME, m) {
    m.doc() = "Compiled torch binding of include/ep.h (argument checks and the C calls)";
    m.def("layout", &layout);
    m.def("dispatch_forward", &dispatch_forward);
    m.def("dispatch", &dispatch);
    m.def("combine_backward", &combine_backward);
    m.def("combine", &combine);
    m.def("dispatch_backward", &dispatch_backward);
}
