// Dispatch kernels: copy every token's hidden row into the receive rows of
// its k (token, expert) pairs — the DeepEP README's dispatch_forward (BF16 x,
// or FP8 x as (data, scale_factors)) and combine_backward (a dispatch that
// reuses the handle), for the receive rows of one GPU.
//
// Token-major: one block per token (the copy itself is dispatch_token in
// ep_dispatch_dev.h). Padding rows of the aligned layout are cleared by
// extra blocks placed first in the grid (at most kPadBlocksPerCU per CU,
// each looping over pieces of the experts' padding), so they overlap with
// the token blocks.
#include "ep_internal.h"
#include "ep_dispatch_dev.h"

namespace ep {

template <int KIND>
__global__ __launch_bounds__(1024) void k_dispatch(DispatchArgs a) {
    if ((int)blockIdx.x < a.npad_blocks) {
        // zero-fill pieces blockIdx.x, + npad_blocks, ...: up to
        // pad_rows_per_piece padding rows of one expert each
        for (int pc = blockIdx.x; pc < a.npad_pieces; pc += a.npad_blocks) {
            const int e = pc / a.pad_pieces_per_expert;
            const int part = pc % a.pad_pieces_per_expert;
            const int r0 = a.expert_off[e] + a.cnt[e] + part * a.pad_rows_per_piece;
            const int r1 = min(r0 + a.pad_rows_per_piece, a.expert_off[e] + a.pad[e]);
            dispatch_zero_rows<KIND>(a, r0, r1);
        }
        return;
    }
    const int t = (int)blockIdx.x - a.npad_blocks;
    const int lane = threadIdx.x & 63;
    int my_s = -1;
    float my_w = 0.0f;
    if (lane < a.k) {
        my_s = a.slot[(int64_t)t * a.k + lane];
        if (KIND == kDispatchBf16Weighted || KIND == kDispatchFp8QuantWeighted)
            my_w = a.pair_w[(int64_t)t * a.k + lane];
    }
    dispatch_token<KIND>(a, t, 0, dispatch_nvec<KIND>(a), my_s, my_w);
}

hipError_t launch_dispatch(int kind, const DispatchArgs& args, hipStream_t stream) {
    DispatchArgs a = args;
    int cus = 0;
    const hipError_t err = device_cu_count(&cus);
    if (err != hipSuccess) return err;
    a.npad_blocks = min(a.npad_pieces, kPadBlocksPerCU * cus);
    const bool fp8 = kind == kDispatchFp8Quant || kind == kDispatchFp8Copy || kind == kDispatchFp8QuantWeighted;
    const int nvec = fp8 ? a.H / 16 : a.H / 8;
    int threads = ((nvec + 63) / 64) * 64;
    if (threads > 1024) threads = 1024;
    if (threads < 64) threads = 64;
    const int64_t grid64 = (int64_t)a.npad_blocks + a.T;
    if (grid64 == 0) return hipSuccess;
    if (grid64 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const int grid = (int)grid64;
    if (launch_debug())
        launch_debug_print("k_dispatch", dim3(grid), dim3(threads),
                           "kind %d tokens %d zero-fill blocks %d pieces %d rows/piece %d", kind, a.T, a.npad_blocks,
                           a.npad_pieces, a.pad_rows_per_piece);
    switch (kind) {
        case kDispatchBf16:
            hipLaunchKernelGGL(k_dispatch<kDispatchBf16>, dim3(grid), dim3(threads), 0, stream, a);
            break;
        case kDispatchBf16Weighted:
            hipLaunchKernelGGL(k_dispatch<kDispatchBf16Weighted>, dim3(grid), dim3(threads), 0, stream, a);
            break;
        case kDispatchFp8Quant:
            hipLaunchKernelGGL(k_dispatch<kDispatchFp8Quant>, dim3(grid), dim3(threads), 0, stream, a);
            break;
        case kDispatchFp8Copy:
            hipLaunchKernelGGL(k_dispatch<kDispatchFp8Copy>, dim3(grid), dim3(threads), 0, stream, a);
            break;
        case kDispatchFp8QuantWeighted:
            hipLaunchKernelGGL(k_dispatch<kDispatchFp8QuantWeighted>, dim3(grid), dim3(threads), 0, stream, a);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ep
