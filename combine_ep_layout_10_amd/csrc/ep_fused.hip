// Single-launch layout + dispatch for small batches — the DeepEP README's
// dispatch_forward (layout and copy in one call) on the decode-sized inputs
// of "Example use in inference decoding", where launch latency, not memory
// traffic, sets the time.
//
// The layout has a grid-wide dependency (a token's row depends on the
// counts of every expert before it), so instead of waiting on other blocks
// every block recomputes the whole layout of the batch in LDS (pairs <=
// 4096, E <= 512: a few KiB of ids read from L2 per block). Block 0 writes
// the handle's arrays; the next blocks zero-fill padding rows; the rest copy
// one token each, taking their slots from the lanes that ranked their pairs.
// No block waits on another, and the result equals ep_layout followed by
// ep_dispatch bit for bit (the same device code computes both).
#include "ep_internal.h"
#include "ep_layout_dev.h"
#include "ep_dispatch_dev.h"

namespace ep {

template <int IT, int KIND>
__global__ __launch_bounds__(1024) void k_layout_dispatch_small(LayoutArgs la, DispatchArgs da) {
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_slot[kMaxTopk];
    SmallLayout<IT> L;
    const bool lead = blockIdx.x == 0;
    small_layout<IT>(la, lds, lead, L);
    if (lead) {
        small_layout_publish<IT>(la, L);
        return;
    }
    const int b = (int)blockIdx.x - 1;
    if (b < da.npad_blocks) {
        const int e = b / da.pad_blocks_per_expert;
        const int part = b % da.pad_blocks_per_expert;
        const int r0 = L.s_off[e] + L.s_cnt[e] + part * kPadRowsPerBlock;
        const int r1 = min(r0 + kPadRowsPerBlock, L.s_off[e + 1]);
        dispatch_zero_rows<KIND>(da, r0, r1);
        return;
    }
    const int t = b - da.npad_blocks;
    const int lane = threadIdx.x & 63;
    const int64_t p0 = (int64_t)t * la.k;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t p = L.base + it * kWave + lane;
        if (p >= p0 && p < p0 + la.k) s_slot[p - p0] = small_layout_slot<IT>(la, L, it);
    }
    __syncthreads();
    const int my_s = lane < la.k ? s_slot[lane] : -1;
    dispatch_token<KIND>(da, t, my_s, 0.0f);
}

template <int KIND>
static void launch_fused_kind(const LayoutArgs& la, const DispatchArgs& da, int grid, size_t lds, hipStream_t s) {
    if ((int64_t)la.T * la.k <= 1024)
        hipLaunchKernelGGL((k_layout_dispatch_small<1, KIND>), dim3(grid), dim3(1024), lds, s, la, da);
    else
        hipLaunchKernelGGL((k_layout_dispatch_small<4, KIND>), dim3(grid), dim3(1024), lds, s, la, da);
}

bool fused_layout_dispatch_fits(int64_t pairs, int E) { return pairs <= kSmallMaxPairs && E <= kSmallMaxExperts; }

hipError_t launch_layout_dispatch_small(int kind, const LayoutArgs& la, const DispatchArgs& da, hipStream_t stream) {
    const int grid = 1 + da.npad_blocks + da.T;
    const size_t lds = small_layout_lds_bytes(la.E, la.D);
    switch (kind) {
        case kDispatchBf16: launch_fused_kind<kDispatchBf16>(la, da, grid, lds, stream); break;
        case kDispatchFp8Quant: launch_fused_kind<kDispatchFp8Quant>(la, da, grid, lds, stream); break;
        case kDispatchFp8Copy: launch_fused_kind<kDispatchFp8Copy>(la, da, grid, lds, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ep
