// Combine kernel: reduce each token's k expert-output rows back into one
// BF16 row — the DeepEP README's combine_forward, and dispatch_backward (a
// combine without weights that also gathers per-row values back to the
// pairs), for the receive rows of one GPU.
//
// One block per piece of seg vectors of a token's row (pieces of about 128
// vectors for large batches; for batches too small to fill the chip, enough
// pieces to reach every CU); each lane owns 8 channels (one dwordx4 of bf16)
// of the output row. It issues the loads of all k source rows (up
// to 8 at a time) before any arithmetic, so k 16-byte loads per lane are in
// flight, then accumulates in binary32 with fused multiply-add in k order
// from +0, rounds to bf16 (nearest even) and writes one dwordx4.
#include "ep_internal.h"

namespace ep {

template <bool WEIGHTED>
__global__ __launch_bounds__(1024) void k_combine(CombineArgs a) {
    const int t = blockIdx.x / a.nsplit, part = blockIdx.x % a.nsplit;
    const int tid = threadIdx.x, lane = tid & 63;
    // Lane j < k of every wave holds pair j's slot and weight; the loops below
    // broadcast them with readlane, so no load sits between the row loads.
    int my_s = -1;
    float my_w = 0.0f;
    if (lane < a.k) {
        my_s = a.slot[(int64_t)t * a.k + lane];
        if (WEIGHTED) my_w = a.w[(int64_t)t * a.k + lane];
    }
    if (a.out_vals != nullptr && part == 0 && tid < a.k)
        a.out_vals[(int64_t)t * a.k + tid] = my_s >= 0 ? a.row_vals[my_s] : 0.0f;

    const int c1 = min((part + 1) * a.seg, a.H / 8);
    for (int c = part * a.seg + tid; c < c1; c += blockDim.x) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int j0 = 0; j0 < a.k; j0 += 8) {
            uint4 v[8];
            int s[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                s[u] = j0 + u < a.k ? __builtin_amdgcn_readlane(my_s, j0 + u) : -1;
                v[u] = make_uint4(0u, 0u, 0u, 0u);
                if (s[u] >= 0) v[u] = load_row_stream(a.y + (int64_t)s[u] * a.H, 2u * (uint32_t)a.H, 16u * c);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (s[u] < 0) continue;
                float f[8];
                f[0] = bf16_to_f32(v[u].x & 0xFFFFu);
                f[1] = bf16_to_f32(v[u].x >> 16);
                f[2] = bf16_to_f32(v[u].y & 0xFFFFu);
                f[3] = bf16_to_f32(v[u].y >> 16);
                f[4] = bf16_to_f32(v[u].z & 0xFFFFu);
                f[5] = bf16_to_f32(v[u].z >> 16);
                f[6] = bf16_to_f32(v[u].w & 0xFFFFu);
                f[7] = bf16_to_f32(v[u].w >> 16);
                if (WEIGHTED) {
                    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j0 + u));
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, f[i], acc[i]);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = acc[i] + f[i];
                }
            }
        }
        const uint4 o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        store_row_stream(a.out + (int64_t)t * a.H, 2u * (uint32_t)a.H, 16u * c, o);
    }
}

// Gradient of the weighted combine with respect to its weights: for every
// pair, grad_w[t, j] = sum_c grad_out[t, c] * y[slot[t, j], c], the dot
// product of the token's output gradient with the pair's expert-output row
// (0 for skipped pairs). One block per token, each lane owning 8 channels
// per vector as in the combine: the lane loads its grad_out vector once and
// the k row vectors (all issued before the arithmetic), accumulates one
// binary32 partial per pair with fused multiply-adds over its channels, in
// channel order and then over its vectors in order; the 64 lanes of a wave
// are summed by a butterfly (xor 32, 16, ..., 1), and the waves' sums are
// added by thread j in wave order. The order is fixed, so the result is
// deterministic; a product passes through at most
// 8 * ceil(vectors / threads) + 6 + waves - 1 binary32 additions.
__global__ __launch_bounds__(1024) void k_weight_grad(WeightGradArgs a) {
    __shared__ float red[16][kMaxTopk];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int my_s = -1;
    if (lane < a.k) my_s = a.slot[(int64_t)t * a.k + lane];
    const int nvec = a.H / 8;
    for (int j0 = 0; j0 < a.k; j0 += 8) {
        float acc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = 0.0f;
        for (int c = tid; c < nvec; c += blockDim.x) {
            const uint4 gv = ((const uint4*)(a.grad_out + (int64_t)t * a.H))[c];
            uint4 v[8];
            int s[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                s[u] = j0 + u < a.k ? __builtin_amdgcn_readlane(my_s, j0 + u) : -1;
                v[u] = make_uint4(0u, 0u, 0u, 0u);
                if (s[u] >= 0) v[u] = load_row_stream(a.y + (int64_t)s[u] * a.H, 2u * (uint32_t)a.H, 16u * c);
            }
            float g[8];
            g[0] = bf16_to_f32(gv.x & 0xFFFFu);
            g[1] = bf16_to_f32(gv.x >> 16);
            g[2] = bf16_to_f32(gv.y & 0xFFFFu);
            g[3] = bf16_to_f32(gv.y >> 16);
            g[4] = bf16_to_f32(gv.z & 0xFFFFu);
            g[5] = bf16_to_f32(gv.z >> 16);
            g[6] = bf16_to_f32(gv.w & 0xFFFFu);
            g[7] = bf16_to_f32(gv.w >> 16);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc[u] = __builtin_fmaf(g[0], bf16_to_f32(v[u].x & 0xFFFFu), acc[u]);
                acc[u] = __builtin_fmaf(g[1], bf16_to_f32(v[u].x >> 16), acc[u]);
                acc[u] = __builtin_fmaf(g[2], bf16_to_f32(v[u].y & 0xFFFFu), acc[u]);
                acc[u] = __builtin_fmaf(g[3], bf16_to_f32(v[u].y >> 16), acc[u]);
                acc[u] = __builtin_fmaf(g[4], bf16_to_f32(v[u].z & 0xFFFFu), acc[u]);
                acc[u] = __builtin_fmaf(g[5], bf16_to_f32(v[u].z >> 16), acc[u]);
                acc[u] = __builtin_fmaf(g[6], bf16_to_f32(v[u].w & 0xFFFFu), acc[u]);
                acc[u] = __builtin_fmaf(g[7], bf16_to_f32(v[u].w >> 16), acc[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) acc[u] += __shfl_xor(acc[u], off, kWave);
            if (lane == 0 && j0 + u < a.k) red[w][j0 + u] = acc[u];
        }
    }
    __syncthreads();
    if (tid < a.k) {
        const int nw = (blockDim.x + 63) >> 6;
        float sum = red[0][tid];
        for (int ww = 1; ww < nw; ++ww) sum += red[ww][tid];
        const int s = a.slot[(int64_t)t * a.k + tid];
        a.grad_w[(int64_t)t * a.k + tid] = s >= 0 ? sum : 0.0f;
    }
}

hipError_t launch_weight_grad(const WeightGradArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int nvec = a.H / 8;
    int threads = ((nvec + 63) / 64) * 64;
    if (threads > 1024) threads = 1024;
    if (launch_debug()) launch_debug_print("k_weight_grad", dim3(a.T), dim3(threads), "tokens %d", a.T);
    hipLaunchKernelGGL(k_weight_grad, dim3(a.T), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& args, hipStream_t stream) {
    if (args.T == 0) return hipSuccess;
    CombineArgs a = args;
    const int nvec = a.H / 8;
    int cus = 0;
    const hipError_t err = device_cu_count(&cus);
    if (err != hipSuccess) return err;
    const int target = kSplitBlocksPerCU * cus;
    // Batches with fewer tokens than about two per CU split each row into
    // pieces of at least 64 vectors, so that the gather reaches every CU.
    // Larger batches split rows into pieces of about kCombineSegLarge
    // vectors: small blocks refill the CUs' wave slots sooner than one
    // block per row (measured on MI355X at 8192 x 7168 x top-8: 128-thread
    // blocks 179 us against 184 us for 896-thread blocks).
    int nsplit = a.T < target ? (target + a.T - 1) / a.T : (nvec + kCombineSegLarge - 1) / kCombineSegLarge;
    nsplit = max(1, min(nsplit, nvec / 64));
    a.seg = (nvec + nsplit - 1) / nsplit;
    a.nsplit = (nvec + a.seg - 1) / a.seg;
    int threads = ((a.seg + 63) / 64) * 64;
    if (threads > 1024) threads = 1024;
    const dim3 grid((unsigned)a.T * a.nsplit);
    if (launch_debug())
        launch_debug_print(a.w != nullptr ? "k_combine<true>" : "k_combine<false>", grid, dim3(threads),
                           "tokens %d pieces/row %d vectors/piece %d", a.T, a.nsplit, a.seg);
    if (a.w != nullptr)
        hipLaunchKernelGGL(k_combine<true>, grid, dim3(threads), 0, stream, a);
    else
        hipLaunchKernelGGL(k_combine<false>, grid, dim3(threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ep
