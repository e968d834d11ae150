// Dispatch kernels: copy every token's hidden row into the receive rows of
// its k (token, expert) pairs — the DeepEP README's dispatch_forward (BF16 x,
// or FP8 x as (data, scale_factors)) and combine_backward (a dispatch that
// reuses the handle), for the receive rows of one GPU.
//
// Token-major: one block per token, so x is read once and written k times.
// Each lane moves one 16-byte vector per row (dwordx4 loads and stores); a
// wave covers 1 KiB of a row per instruction. The FP8 kind quantises on the
// fly: a lane holds 16 bf16 values (two dwordx4 loads), eight consecutive
// lanes hold one 1x128 block, the block's amax is reduced across those eight
// lanes with DPP, and the lane writes its 16 E4M3 codes as one dwordx4.
// Padding rows of the aligned layout are cleared by extra blocks placed
// first in the grid, so they overlap with the token blocks.
// Cache policy (measured on MI355X at the 8K x 7168 x top-8 shape): the k
// payload rows go out with streaming stores; x is read with plain loads and
// the 32-byte pieces of each scale row with plain stores, which L2 merges
// into whole lines (streaming either of them cost about 30 us per call).
#include "ep_internal.h"

namespace ep {

__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float f[8]) {
    f[0] = bf16_to_f32(v.x & 0xFFFFu);
    f[1] = bf16_to_f32(v.x >> 16);
    f[2] = bf16_to_f32(v.y & 0xFFFFu);
    f[3] = bf16_to_f32(v.y >> 16);
    f[4] = bf16_to_f32(v.z & 0xFFFFu);
    f[5] = bf16_to_f32(v.z >> 16);
    f[6] = bf16_to_f32(v.w & 0xFFFFu);
    f[7] = bf16_to_f32(v.w >> 16);
}

__device__ __forceinline__ uint4 pack_bf16x8(const float f[8]) {
    uint4 o;
    o.x = f32_to_bf16_rne(f[0]) | (f32_to_bf16_rne(f[1]) << 16);
    o.y = f32_to_bf16_rne(f[2]) | (f32_to_bf16_rne(f[3]) << 16);
    o.z = f32_to_bf16_rne(f[4]) | (f32_to_bf16_rne(f[5]) << 16);
    o.w = f32_to_bf16_rne(f[6]) | (f32_to_bf16_rne(f[7]) << 16);
    return o;
}

template <int KIND>
__global__ __launch_bounds__(1024) void k_dispatch(DispatchArgs a) {
    constexpr bool kFp8 = KIND == kDispatchFp8Quant || KIND == kDispatchFp8Copy;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int64_t row_out = kFp8 ? (int64_t)a.H : 2 * (int64_t)a.H;
    const int nb = a.H / 128;

    if ((int)blockIdx.x < a.npad_blocks) {
        // zero-fill up to kPadRowsPerBlock padding rows of one expert
        const int e = blockIdx.x / a.pad_blocks_per_expert;
        const int part = blockIdx.x % a.pad_blocks_per_expert;
        const int r0 = a.expert_off[e] + a.cnt[e] + part * kPadRowsPerBlock;
        const int r1 = min(r0 + kPadRowsPerBlock, a.expert_off[e] + a.pad[e]);
        const int nvec = (int)(row_out / 16);
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        for (int r = r0; r < r1; ++r) {
            uint4* dst = (uint4*)((char*)a.recv + (int64_t)r * row_out);
            for (int c = tid; c < nvec; c += nthreads) store_stream(dst + c, z);
            if (kFp8)
                for (int b = tid; b < nb; b += nthreads) a.recv_scales[(int64_t)r * nb + b] = 0.0f;
        }
        return;
    }

    const int t = (int)blockIdx.x - a.npad_blocks;
    // Lane j < k of every wave holds pair j's slot (and weight); the store
    // loops broadcast them with readlane, so no load waits between stores.
    const int lane = tid & 63;
    int my_s = -1;
    float my_w = 0.0f;
    if (lane < a.k) {
        my_s = a.slot[(int64_t)t * a.k + lane];
        if (KIND == kDispatchBf16Weighted) my_w = a.pair_w[(int64_t)t * a.k + lane];
    }

    if (KIND == kDispatchBf16 || KIND == kDispatchBf16Weighted) {
        const uint4* src = (const uint4*)((const char*)a.x + (int64_t)t * 2 * a.H);
        const int nvec = a.H / 8;
        for (int c = tid; c < nvec; c += nthreads) {
            const uint4 v = src[c];
            float f[8];
            if (KIND == kDispatchBf16Weighted) unpack_bf16x8(v, f);
            for (int j = 0; j < a.k; ++j) {
                const int s = __builtin_amdgcn_readlane(my_s, j);
                if (s < 0) continue;
                uint4 o = v;
                if (KIND == kDispatchBf16Weighted) {
                    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
                    float g[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) g[i] = wj * f[i];
                    o = pack_bf16x8(g);
                }
                store_stream((uint4*)((char*)a.recv + (int64_t)s * row_out) + c, o);
            }
        }
    } else if (KIND == kDispatchFp8Quant) {
        const uint4* src = (const uint4*)((const char*)a.x + (int64_t)t * 2 * a.H);
        const int nvec = a.H / 16;  // 16 bf16 in, 16 codes out per lane
        // The loop bound is uniform so every lane of a wave takes part in the
        // DPP reduction; `act` only guards memory.
        for (int c0 = 0; c0 < nvec; c0 += nthreads) {
            const int c = c0 + tid;
            const bool act = c < nvec;
            uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
            if (act) {
                v0 = src[2 * c];
                v1 = src[2 * c + 1];
            }
            float f[16];
            unpack_bf16x8(v0, f);
            unpack_bf16x8(v1, f + 8);
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
            amax = max8_dpp(amax);
            const float scale = amax / 448.0f;
            uint32_t w4[4] = {0u, 0u, 0u, 0u};
            if (amax != 0.0f) {
#pragma unroll
                for (int i = 0; i < 16; ++i) w4[i >> 2] |= f32_to_e4m3_sat(f[i] / scale) << (8 * (i & 3));
            }
            const uint4 o = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            if (act) {
                for (int j = 0; j < a.k; ++j) {
                    const int s = __builtin_amdgcn_readlane(my_s, j);
                    if (s < 0) continue;
                    store_stream((uint4*)((char*)a.recv + (int64_t)s * row_out) + c, o);
                    if ((c & 7) == 0) a.recv_scales[(int64_t)s * nb + (c >> 3)] = scale;
                }
            }
        }
    } else {  // kDispatchFp8Copy
        const uint4* src = (const uint4*)((const char*)a.x + (int64_t)t * a.H);
        const int nvec = a.H / 16;
        for (int c = tid; c < nvec; c += nthreads) {
            const uint4 v = src[c];
            const bool scale_lane = (c & 7) == 0;
            const float sc = scale_lane ? a.x_scales[(int64_t)t * nb + (c >> 3)] : 0.0f;
            for (int j = 0; j < a.k; ++j) {
                const int s = __builtin_amdgcn_readlane(my_s, j);
                if (s < 0) continue;
                store_stream((uint4*)((char*)a.recv + (int64_t)s * row_out) + c, v);
                if (scale_lane) a.recv_scales[(int64_t)s * nb + (c >> 3)] = sc;
            }
        }
    }
}

hipError_t launch_dispatch(int kind, const DispatchArgs& a, hipStream_t stream) {
    const bool fp8 = kind == kDispatchFp8Quant || kind == kDispatchFp8Copy;
    const int nvec = fp8 ? a.H / 16 : a.H / 8;
    int threads = ((nvec + 63) / 64) * 64;
    if (threads > 1024) threads = 1024;
    if (threads < 64) threads = 64;
    const int grid = a.npad_blocks + a.T;
    if (grid == 0) return hipSuccess;
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
        default:
            hipLaunchKernelGGL(k_dispatch<kDispatchFp8Copy>, dim3(grid), dim3(threads), 0, stream, a);
            break;
    }
    return hipGetLastError();
}

}  // namespace ep
