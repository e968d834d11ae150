// Host side of the C ABI declared in include/ep.h: argument checks, the
// workspace map, handle construction and kernel launches on the caller's
// stream. No device memory is allocated here.
#include <stdarg.h>
#include <atomic>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep_internal.h"

namespace {

thread_local char g_msg[512] = "";

ep_status fail(ep_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return s;
}

ep_status hip_fail(hipError_t e, const char* what) {
    return fail(EP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kMaxHidden = 1 << 24;

// Byte offsets of every region of a workspace (256-byte aligned regions).
struct WsMap {
    size_t flags, cnt, pad, eoff, doff, dtok, slot, rsrc, rw, bpart, dpart, fpart, total;
    int nblk_max;
};

int64_t rows_bound(const ep_config& c) {
    if (c.mode == EP_MODE_FIXED) return (int64_t)c.num_experts * c.capacity;
    return (int64_t)c.max_tokens * c.num_topk + (int64_t)c.num_experts * (c.expert_alignment - 1);
}

ep_status check_config(const ep_config* c) {
    if (c == nullptr) return fail(EP_ERR_INVALID_ARG, "config is NULL");
    if (c->mode != EP_MODE_COMPACT && c->mode != EP_MODE_FIXED)
        return fail(EP_ERR_INVALID_ARG, "mode %d is not EP_MODE_COMPACT or EP_MODE_FIXED", c->mode);
    if (c->num_experts < 1 || c->num_experts > ep::kMaxExperts)
        return fail(EP_ERR_INVALID_ARG, "num_experts %d outside [1, %d]", c->num_experts, ep::kMaxExperts);
    if (c->num_topk < 1 || c->num_topk > ep::kMaxTopk)
        return fail(EP_ERR_INVALID_ARG, "num_topk %d outside [1, %d]", c->num_topk, ep::kMaxTopk);
    if (c->num_dests < 1 || c->num_experts % c->num_dests != 0)
        return fail(EP_ERR_INVALID_ARG, "num_dests %d must divide num_experts %d", c->num_dests, c->num_experts);
    if (c->max_tokens < 0 || (int64_t)c->max_tokens * c->num_topk >= (1ll << 31))
        return fail(EP_ERR_INVALID_ARG, "max_tokens %d out of range", c->max_tokens);
    if (c->hidden < 8 || c->hidden % 8 != 0)
        return fail(EP_ERR_INVALID_ARG, "hidden %d must be a positive multiple of 8", c->hidden);
    // Row stores go through buffer resources whose size and offsets are
    // 32-bit byte counts: a bf16 row (2 * hidden bytes) must stay far below 2^32.
    if (c->hidden > kMaxHidden) return fail(EP_ERR_INVALID_ARG, "hidden %d exceeds %d", c->hidden, kMaxHidden);
    if (c->idx_bits != 32 && c->idx_bits != 64)
        return fail(EP_ERR_INVALID_ARG, "idx_bits %d must be 32 or 64", c->idx_bits);
    if (c->mode == EP_MODE_COMPACT && c->expert_alignment < 1)
        return fail(EP_ERR_INVALID_ARG, "expert_alignment %d must be >= 1", c->expert_alignment);
    if (c->mode == EP_MODE_FIXED && (c->capacity < 1 || c->expert_alignment != 1))
        return fail(EP_ERR_INVALID_ARG, "FIXED mode needs capacity >= 1 (got %d) and expert_alignment 1 (got %d)",
                    c->capacity, c->expert_alignment);
    if (rows_bound(*c) >= (1ll << 31)) return fail(EP_ERR_INVALID_ARG, "receive rows bound exceeds 2^31");
    if ((c->flags & ~EP_FLAG_NO_ZERO_PAD) != 0) return fail(EP_ERR_INVALID_ARG, "unknown flags 0x%x", c->flags);
    return EP_OK;
}

WsMap ws_map(const ep_config& c) {
    WsMap m;
    const size_t E = c.num_experts, D = c.num_dests;
    const size_t P = (size_t)c.max_tokens * c.num_topk;
    const size_t R = (size_t)rows_bound(c);
    m.nblk_max = (int)((P + ep::kLayoutPairsPerBlock - 1) / ep::kLayoutPairsPerBlock);
    if (m.nblk_max < 1) m.nblk_max = 1;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = round_up(o + (bytes ? bytes : 4), 256);
        return at;
    };
    m.flags = take(4);
    m.cnt = take(4 * E);
    m.pad = take(4 * E);
    m.eoff = take(4 * (E + 1));
    m.doff = take(4 * (D + 1));
    m.dtok = take(4 * D);
    m.slot = take(4 * P);
    m.rsrc = take(4 * R);
    m.rw = take(4 * R);
    m.bpart = take(4 * E * (size_t)m.nblk_max);
    m.dpart = take(4 * D * (size_t)m.nblk_max);
    m.fpart = take(4 * (size_t)m.nblk_max);
    m.total = o;
    return m;
}

ep_status check_handle(const ep_handle* h) {
    if (h == nullptr) return fail(EP_ERR_INVALID_ARG, "handle is NULL");
    ep_status s = check_config(&h->cfg);
    if (s != EP_OK) return s;
    if (h->num_tokens < 0 || h->num_tokens > h->cfg.max_tokens)
        return fail(EP_ERR_INVALID_ARG, "handle num_tokens %d outside [0, %d]", h->num_tokens, h->cfg.max_tokens);
    if (h->slot == nullptr || h->cnt == nullptr || h->expert_off == nullptr || h->pad == nullptr)
        return fail(EP_ERR_INVALID_ARG, "handle has NULL arrays (not built by ep_layout?)");
    return EP_OK;
}

// Checks a dispatch and fills its kernel arguments; enqueues nothing.
// `names`: what the caller calls its input, scales, output and output scales
// (ep_dispatch's, or ep_combine_backward's), for the error messages.
struct DispatchNames {
    const char *x, *x_scales, *recv, *recv_scales;
};
constexpr DispatchNames kDispatchNames = {"x", "x_scales", "recv", "recv_scales"};
constexpr DispatchNames kCombineBackwardNames = {"grad_out", "grad_out_scales", "grad_y", "grad_y_scales"};

ep_status prepare_dispatch(const ep_handle* h, int32_t dtype, const void* x, const float* x_scales,
                           const float* pair_w, void* recv, float* recv_scales, ep::DispatchArgs* out, int* kind,
                           const DispatchNames& n = kDispatchNames) {
    ep_status s = check_handle(h);
    if (s != EP_OK) return s;
    const ep_config& c = h->cfg;
    const int T = h->num_tokens;
    if (dtype != EP_BF16 && dtype != EP_FP8_QUANTIZE && dtype != EP_FP8_PREQUANT)
        return fail(EP_ERR_INVALID_ARG, "dtype %d unknown", (int)dtype);
    const bool fp8 = dtype != EP_BF16;
    if (fp8 && c.hidden % 128 != 0)
        return fail(EP_ERR_INVALID_ARG, "FP8 dispatch needs hidden %% 128 == 0 (hidden %d)", c.hidden);
    if (pair_w != nullptr && dtype == EP_FP8_PREQUANT)
        return fail(EP_ERR_UNSUPPORTED, "per-pair weights need EP_BF16 or EP_FP8_QUANTIZE");
    if (T > 0 && (x == nullptr || !aligned(x, 16)))
        return fail(EP_ERR_INVALID_ARG, "%s must be non-NULL and 16-byte aligned", n.x);
    if (recv == nullptr || !aligned(recv, 16))
        return fail(EP_ERR_INVALID_ARG, "%s must be non-NULL and 16-byte aligned", n.recv);
    if (fp8 && (recv_scales == nullptr || !aligned(recv_scales, 4)))
        return fail(EP_ERR_INVALID_ARG, "%s (4-byte aligned) is required for an FP8 output", n.recv_scales);
    if (dtype == EP_FP8_PREQUANT && T > 0 && (x_scales == nullptr || !aligned(x_scales, 4)))
        return fail(EP_ERR_INVALID_ARG, "%s (4-byte aligned) is required for EP_FP8_PREQUANT", n.x_scales);
    ep::DispatchArgs& a = *out;
    a.x = x;
    a.x_scales = x_scales;
    a.recv = recv;
    a.recv_scales = recv_scales;
    a.slot = h->slot;
    a.pair_w = pair_w;
    a.cnt = h->cnt;
    a.pad = h->pad;
    a.expert_off = h->expert_off;
    a.T = T;
    a.H = c.hidden;
    a.k = c.num_topk;
    a.E = c.num_experts;
    a.zero_pad = (c.mode == EP_MODE_COMPACT && !(c.flags & EP_FLAG_NO_ZERO_PAD)) ? 1 : 0;
    a.pad_rows_max = a.zero_pad ? c.expert_alignment - 1 : 0;
    ep::set_pad_pieces(a, ep::kPadRowsPerPiece);  // the single-launch path sets its own
    if (dtype == EP_BF16)
        *kind = pair_w ? ep::kDispatchBf16Weighted : ep::kDispatchBf16;
    else if (dtype == EP_FP8_QUANTIZE)
        *kind = pair_w ? ep::kDispatchFp8QuantWeighted : ep::kDispatchFp8Quant;
    else
        *kind = ep::kDispatchFp8Copy;
    return EP_OK;
}

ep_status do_dispatch(const ep_handle* h, int32_t dtype, const void* x, const float* x_scales, const float* pair_w,
                      void* recv, float* recv_scales, hipStream_t stream, const DispatchNames& n = kDispatchNames) {
    ep::DispatchArgs a;
    int kind = 0;
    ep_status s = prepare_dispatch(h, dtype, x, x_scales, pair_w, recv, recv_scales, &a, &kind, n);
    if (s != EP_OK) return s;
    hipError_t e = ep::launch_dispatch(kind, a, stream);
    if (e != hipSuccess) return hip_fail(e, "dispatch launch");
    return EP_OK;
}

ep_status do_combine(const ep_handle* h, const void* y, const float* w, void* out, const float* row_vals,
                     float* out_vals, hipStream_t stream) {
    ep_status s = check_handle(h);
    if (s != EP_OK) return s;
    const int T = h->num_tokens;
    if (y == nullptr || !aligned(y, 16)) return fail(EP_ERR_INVALID_ARG, "y must be non-NULL and 16-byte aligned");
    if (T > 0 && (out == nullptr || !aligned(out, 16)))
        return fail(EP_ERR_INVALID_ARG, "out must be non-NULL and 16-byte aligned");
    if ((row_vals == nullptr) != (out_vals == nullptr))
        return fail(EP_ERR_INVALID_ARG, "row_vals and out_vals must be given together");
    ep::CombineArgs a;
    a.y = (const uint16_t*)y;
    a.w = w;
    a.out = (uint16_t*)out;
    a.slot = h->slot;
    a.row_vals = row_vals;
    a.out_vals = out_vals;
    a.T = T;
    a.H = h->cfg.hidden;
    a.k = h->cfg.num_topk;
    hipError_t e = ep::launch_combine(a, stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return EP_OK;
}

// Bytes of the multi-block layout's per-block partials for one call
// (counts [nblk][E], distinct tokens [nblk][D], error bits [nblk]; regions
// 256-byte aligned), and their offsets from the start of that scratch.
struct PartMap {
    size_t bpart, dpart, fpart, total;
};

PartMap part_map(const ep_config& c, int64_t pairs) {
    int64_t nblk = (pairs + ep::kLayoutPairsPerBlock - 1) / ep::kLayoutPairsPerBlock;
    if (nblk < 1) nblk = 1;
    PartMap p;
    p.bpart = 0;
    p.dpart = round_up(4 * (size_t)c.num_experts * nblk, 256);
    p.fpart = p.dpart + round_up(4 * (size_t)c.num_dests * nblk, 256);
    p.total = p.fpart + round_up(4 * (size_t)nblk, 256);
    return p;
}

// Checks a layout, builds its handle and kernel arguments; enqueues nothing.
// scratch == nullptr: the per-block partials live in the workspace (which
// must hold ep_workspace_bytes); otherwise they live at `scratch` (checked
// by the caller to hold part_map(...).total bytes) and the workspace needs
// only the handle's arrays.
ep_status prepare_layout(const ep_config* cfg, int32_t num_tokens, const void* topk_idx, const float* topk_w,
                         void* workspace, size_t workspace_bytes, ep_handle* out, ep::LayoutArgs* args, bool* small_out,
                         char* scratch = nullptr) {
    ep_status s = check_config(cfg);
    if (s != EP_OK) return s;
    if (num_tokens < 0 || num_tokens > cfg->max_tokens)
        return fail(EP_ERR_INVALID_ARG, "num_tokens %d outside [0, %d]", num_tokens, cfg->max_tokens);
    if (num_tokens > 0 && (topk_idx == nullptr || !aligned(topk_idx, cfg->idx_bits / 8)))
        return fail(EP_ERR_INVALID_ARG, "topk_idx must be non-NULL and aligned to its element size");
    if (topk_w != nullptr && !aligned(topk_w, 4)) return fail(EP_ERR_INVALID_ARG, "topk_w must be 4-byte aligned");
    const WsMap m = ws_map(*cfg);
    if (workspace == nullptr || !aligned(workspace, 256))
        return fail(EP_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
    const size_t need = scratch ? m.bpart : m.total;
    if (workspace_bytes < need)
        return fail(EP_ERR_WORKSPACE, "workspace has %zu bytes, the config needs %zu", workspace_bytes, need);
    char* ws = (char*)workspace;
    ep_handle h;
    memset(&h, 0, sizeof h);
    h.cfg = *cfg;
    h.num_tokens = num_tokens;
    h.err_flags = (uint32_t*)(ws + m.flags);
    h.cnt = (int32_t*)(ws + m.cnt);
    h.pad = (int32_t*)(ws + m.pad);
    h.expert_off = (int32_t*)(ws + m.eoff);
    h.dest_off = (int32_t*)(ws + m.doff);
    h.dest_tokens = (int32_t*)(ws + m.dtok);
    h.slot = (int32_t*)(ws + m.slot);
    h.row_src = (int32_t*)(ws + m.rsrc);
    h.row_w = (float*)(ws + m.rw);
    h.internal = scratch ? (void*)scratch : (void*)(ws + m.bpart);
    h.topk_idx = num_tokens > 0 ? topk_idx : nullptr;

    const int64_t P = (int64_t)num_tokens * cfg->num_topk;
    const bool small = P <= ep::kSmallMaxPairs && cfg->num_experts <= ep::kSmallMaxExperts;
    int nblk = (int)((P + ep::kLayoutPairsPerBlock - 1) / ep::kLayoutPairsPerBlock);
    if (nblk < 1) nblk = 1;  // a layout of zero pairs still writes zero counts
    h.num_blocks = small ? 1 : nblk;

    ep::LayoutArgs& a = *args;
    a.idx = topk_idx;
    a.w = topk_w;
    a.idx_bits = cfg->idx_bits;
    a.T = num_tokens;
    a.E = cfg->num_experts;
    a.k = cfg->num_topk;
    a.A = cfg->mode == EP_MODE_COMPACT ? cfg->expert_alignment : 1;
    a.D = cfg->num_dests;
    a.C = cfg->mode == EP_MODE_FIXED ? cfg->capacity : 0;
    a.mode = cfg->mode;
    int nbits = 1;
    while ((1 << nbits) < cfg->num_experts) ++nbits;
    a.nbits = nbits;
    a.epd = cfg->num_experts / cfg->num_dests;
    a.nblk = nblk;
    a.cnt = h.cnt;
    a.pad = h.pad;
    a.expert_off = h.expert_off;
    a.dest_off = h.dest_off;
    a.dest_tokens = h.dest_tokens;
    a.slot = h.slot;
    a.row_src = h.row_src;
    a.row_w = h.row_w;
    a.err_flags = h.err_flags;
    if (scratch) {
        const PartMap pm = part_map(*cfg, (int64_t)num_tokens * cfg->num_topk);
        a.bpart = (int32_t*)(scratch + pm.bpart);
        a.dpart = (int32_t*)(scratch + pm.dpart);
        a.fpart = (uint32_t*)(scratch + pm.fpart);
    } else {
        a.bpart = (int32_t*)(ws + m.bpart);
        a.dpart = (int32_t*)(ws + m.dpart);
        a.fpart = (uint32_t*)(ws + m.fpart);
    }
    *small_out = small;
    *out = h;
    return EP_OK;
}

// The multi-block layout's per-block partials for
// ep_dispatch_forward_static_scratch: a library-held device array instead
// of the caller's workspace, for callers that cannot allocate. Every entry a
// call reads is written earlier in the same call (each layout block writes
// its own counts, distinct-token counts and error bits before any block
// reads them), so nothing needs clearing between calls.
constexpr size_t kStaticScratchBytes = 1u << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device with hipGetSymbolAddress (host code must never pass the array's
// name itself to a kernel: on the host it is only a stand-in).
ep_status static_scratch_address(char** out) {
    static std::atomic<void*> addr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(EP_ERR_UNSUPPORTED, "device %d: at most 64 devices", dev);
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr) return fail(EP_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        addr[dev].store(p, std::memory_order_release);
    }
    *out = (char*)p;
    return EP_OK;
}

// ep_dispatch_forward, with the layout's partials in `scratch` when given.
ep_status dispatch_forward_impl(const ep_config* cfg, int32_t num_tokens, const void* topk_idx, const float* topk_w,
                                void* workspace, size_t workspace_bytes, int32_t dtype, const void* x,
                                const float* x_scales, void* recv, float* recv_scales, ep_handle* out, void* stream,
                                char* scratch) {
    ep_handle h;
    ep::LayoutArgs la;
    bool small = false;
    ep_status s = check_config(cfg);
    if (s != EP_OK) return s;
    if (out == nullptr) return fail(EP_ERR_INVALID_ARG, "out handle is NULL");
    s = prepare_layout(cfg, num_tokens, topk_idx, topk_w, workspace, workspace_bytes, &h, &la, &small, scratch);
    if (s != EP_OK) return s;
    ep::DispatchArgs da;
    int kind = 0;
    s = prepare_dispatch(&h, dtype, x, x_scales, nullptr, recv, recv_scales, &da, &kind);
    if (s != EP_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    // the single launch addresses the handle's arrays by 32-bit offsets
    // from the workspace base
    const bool offsets32 = ws_map(*cfg).bpart <= 0xFFFFFFFFull;
    bool fused = false;
    if (small && offsets32) {
        e = ep::fused_layout_dispatch_fits(la, da, &fused);
        if (e != hipSuccess) return hip_fail(e, "device query");
    }
    if (fused) {
        e = ep::launch_layout_dispatch_small(kind, la, da, (char*)workspace, st);
        if (e != hipSuccess) return hip_fail(e, "layout + dispatch launch");
    } else {
        e = ep::launch_layout(la, small, st);
        if (e != hipSuccess) return hip_fail(e, "layout launch");
        e = ep::launch_dispatch(kind, da, st);
        if (e != hipSuccess) return hip_fail(e, "dispatch launch");
    }
    *out = h;
    return EP_OK;
}

}  // namespace

namespace ep {

namespace {

// A positive integer from the environment, or 0 when unset or malformed.
int env_int(const char* name) {
    const char* v = getenv(name);
    if (v == nullptr || *v == 0) return 0;
    char* end = nullptr;
    const long n = strtol(v, &end, 10);
    return (*end == 0 && n > 0 && n <= (1 << 30)) ? (int)n : 0;
}

}  // namespace

bool launch_debug() { return env_int("EP_BUFFER_DEBUG") == 1; }

void launch_debug_print(const char* kernel, dim3 grid, dim3 block, const char* fmt, ...) {
    char extra[256] = "";
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(extra, sizeof extra, fmt, ap);
    va_end(ap);
    fprintf(stderr, "[ep] %s grid %u block %u %s\n", kernel, grid.x, block.x, extra);
}

hipError_t device_cu_count(int* out) {
    const int forced = env_int("EP_LAUNCH_CUS");
    if (forced >= 1 && forced <= 4096) {
        *out = forced;
        return hipSuccess;
    }
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (n <= 0) return hipErrorInvalidDevice;
        cached[dev].store(n, std::memory_order_relaxed);  // every thread stores the same value
    }
    *out = n;
    return hipSuccess;
}

}  // namespace ep

extern "C" {

size_t ep_workspace_bytes(const ep_config* cfg) {
    if (check_config(cfg) != EP_OK) return 0;
    return ws_map(*cfg).total;
}

int64_t ep_recv_rows_bound(const ep_config* cfg) {
    if (check_config(cfg) != EP_OK) return -1;
    return rows_bound(*cfg);
}

ep_status ep_layout(const ep_config* cfg, int32_t num_tokens, const void* topk_idx, const float* topk_w,
                    void* workspace, size_t workspace_bytes, ep_handle* out, void* stream) {
    ep_handle h;
    ep::LayoutArgs a;
    bool small = false;
    ep_status s = check_config(cfg);
    if (s != EP_OK) return s;
    if (out == nullptr) return fail(EP_ERR_INVALID_ARG, "out handle is NULL");
    s = prepare_layout(cfg, num_tokens, topk_idx, topk_w, workspace, workspace_bytes, &h, &a, &small);
    if (s != EP_OK) return s;
    hipError_t e = ep::launch_layout(a, small, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "layout launch");
    *out = h;
    return EP_OK;
}

ep_status ep_dispatch_forward(const ep_config* cfg, int32_t num_tokens, const void* topk_idx, const float* topk_w,
                              void* workspace, size_t workspace_bytes, int32_t dtype, const void* x,
                              const float* x_scales, void* recv, float* recv_scales, ep_handle* out, void* stream) {
    return dispatch_forward_impl(cfg, num_tokens, topk_idx, topk_w, workspace, workspace_bytes, dtype, x, x_scales,
                                 recv, recv_scales, out, stream, nullptr);
}

ep_status ep_dispatch_forward_static_scratch(const ep_config* cfg, int32_t num_tokens, const void* topk_idx,
                                             const float* topk_w, void* workspace, size_t workspace_bytes,
                                             int32_t dtype, const void* x, const float* x_scales, void* recv,
                                             float* recv_scales, ep_handle* out, void* stream) {
    ep_status s = check_config(cfg);
    if (s != EP_OK) return s;
    if (num_tokens < 0 || num_tokens > cfg->max_tokens)
        return fail(EP_ERR_INVALID_ARG, "num_tokens %d outside [0, %d]", num_tokens, cfg->max_tokens);
    const PartMap pm = part_map(*cfg, (int64_t)num_tokens * cfg->num_topk);
    if (pm.total > kStaticScratchBytes)
        return fail(EP_ERR_WORKSPACE,
                    "the layout's per-block partials need %zu bytes, more than the library's %zu-byte static scratch "
                    "(ep_dispatch_forward takes them from the workspace instead)",
                    pm.total, (size_t)kStaticScratchBytes);
    char* scr = nullptr;
    s = static_scratch_address(&scr);
    if (s != EP_OK) return s;
    return dispatch_forward_impl(cfg, num_tokens, topk_idx, topk_w, workspace, workspace_bytes, dtype, x, x_scales,
                                 recv, recv_scales, out, stream, scr);
}

ep_status ep_dispatch(const ep_handle* h, int32_t dtype, const void* x, const float* x_scales, void* recv,
                      float* recv_scales, void* stream) {
    return do_dispatch(h, dtype, x, x_scales, nullptr, recv, recv_scales, (hipStream_t)stream);
}

ep_status ep_combine(const ep_handle* h, const void* y, const float* topk_w, void* out, const float* row_vals,
                     float* out_vals, void* stream) {
    return do_combine(h, y, topk_w, out, row_vals, out_vals, (hipStream_t)stream);
}

ep_status ep_dispatch_backward(const ep_handle* h, const void* grad_recv, const float* grad_row_w, void* grad_x,
                               float* grad_topk_w, void* stream) {
    return do_combine(h, grad_recv, nullptr, grad_x, grad_row_w, grad_topk_w, (hipStream_t)stream);
}

ep_status ep_combine_backward(const ep_handle* h, int32_t dtype, const void* grad_out, const float* grad_out_scales,
                              const float* topk_w, void* grad_y, float* grad_y_scales, void* stream) {
    if (topk_w != nullptr && dtype == EP_FP8_PREQUANT)
        return fail(EP_ERR_UNSUPPORTED, "weighted combine_backward needs EP_BF16 or EP_FP8_QUANTIZE");
    return do_dispatch(h, dtype, grad_out, grad_out_scales, topk_w, grad_y, grad_y_scales, (hipStream_t)stream,
                       kCombineBackwardNames);
}

ep_status ep_combine_weight_grad(const ep_handle* h, const void* grad_out, const void* y, float* grad_topk_w,
                                 void* stream) {
    ep_status s = check_handle(h);
    if (s != EP_OK) return s;
    const int T = h->num_tokens;
    if (T > 0 && (grad_out == nullptr || !aligned(grad_out, 16)))
        return fail(EP_ERR_INVALID_ARG, "grad_out must be non-NULL and 16-byte aligned");
    if (T > 0 && (y == nullptr || !aligned(y, 16)))
        return fail(EP_ERR_INVALID_ARG, "y must be non-NULL and 16-byte aligned");
    if (T > 0 && (grad_topk_w == nullptr || !aligned(grad_topk_w, 4)))
        return fail(EP_ERR_INVALID_ARG, "grad_topk_w must be non-NULL and 4-byte aligned");
    ep::WeightGradArgs a;
    a.grad_out = (const uint16_t*)grad_out;
    a.y = (const uint16_t*)y;
    a.slot = h->slot;
    a.grad_w = grad_topk_w;
    a.T = T;
    a.H = h->cfg.hidden;
    a.k = h->cfg.num_topk;
    hipError_t e = ep::launch_weight_grad(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "weight gradient launch");
    return EP_OK;
}

ep_status ep_grouped_gemm_fp8(const ep_handle* h, const void* a, const float* a_scales, const void* b,
                              const float* b_scales, int32_t n, void* out, void* stream) {
    ep_status s = check_handle(h);
    if (s != EP_OK) return s;
    const ep_config& c = h->cfg;
    if (c.hidden % 128 != 0) return fail(EP_ERR_UNSUPPORTED, "grouped GEMM needs hidden %% 128 == 0 (hidden %d)", c.hidden);
    if (n < 128 || n % 128 != 0) return fail(EP_ERR_INVALID_ARG, "n %d must be a positive multiple of 128", n);
    if (c.mode == EP_MODE_COMPACT && c.expert_alignment % 128 != 0)
        return fail(EP_ERR_UNSUPPORTED, "grouped GEMM needs expert_alignment %% 128 == 0 (got %d)", c.expert_alignment);
    if (c.mode == EP_MODE_FIXED && c.capacity % 128 != 0)
        return fail(EP_ERR_UNSUPPORTED, "grouped GEMM needs capacity %% 128 == 0 (got %d)", c.capacity);
    if (a == nullptr || !aligned(a, 16) || a_scales == nullptr || !aligned(a_scales, 4))
        return fail(EP_ERR_INVALID_ARG, "a must be 16-byte aligned and a_scales non-NULL");
    if (b == nullptr || !aligned(b, 16) || b_scales == nullptr || !aligned(b_scales, 4))
        return fail(EP_ERR_INVALID_ARG, "b must be 16-byte aligned and b_scales non-NULL");
    if (out == nullptr || !aligned(out, 16)) return fail(EP_ERR_INVALID_ARG, "out must be non-NULL and 16-byte aligned");
    ep::GemmArgs g;
    g.a = (const uint8_t*)a;
    g.sa = a_scales;
    g.b = (const uint8_t*)b;
    g.sb = b_scales;
    g.c = (uint16_t*)out;
    g.expert_off = h->expert_off;
    g.pad = h->pad;
    g.cnt = h->cnt;
    g.E = c.num_experts;
    g.K = c.hidden;
    g.N = n;
    g.mode = c.mode;
    g.C = c.capacity;
    hipError_t e = ep::launch_grouped_gemm_fp8(g, rows_bound(c), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "grouped GEMM launch");
    return EP_OK;
}

ep_status ep_handle_read_counts(const ep_handle* h, int32_t* cnt, int32_t* pad, int64_t* rows, void* stream) {
    ep_status s = check_handle(h);
    if (s != EP_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    const size_t E = h->cfg.num_experts;
    hipError_t e = hipSuccess;
    int32_t total = 0;
    if (cnt) e = hipMemcpyAsync(cnt, h->cnt, 4 * E, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess && pad) e = hipMemcpyAsync(pad, h->pad, 4 * E, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess && rows) e = hipMemcpyAsync(&total, h->expert_off + E, 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "read counts");
    if (rows) *rows = total;
    return EP_OK;
}

ep_status ep_handle_check(const ep_handle* h, uint32_t* flags, void* stream) {
    ep_status s = check_handle(h);
    if (s != EP_OK) return s;
    if (flags == nullptr) return fail(EP_ERR_INVALID_ARG, "flags is NULL");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(flags, h->err_flags, 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "read error flags");
    return EP_OK;
}

const char* ep_status_string(int32_t s) {
    switch (s) {
        case EP_OK: return "EP_OK";
        case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG";
        case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED";
        case EP_ERR_HIP: return "EP_ERR_HIP";
        case EP_ERR_WORKSPACE: return "EP_ERR_WORKSPACE";
    }
    return "EP_ERR_UNKNOWN";
}

const char* ep_last_error_message(void) { return g_msg; }

}  // extern "C"
