// Device code of the dispatch shared by the dispatch kernel and the fused
// single-launch layout + dispatch (internal).
//
// One block per token: x is read once and written k times. Each lane moves
// one 16-byte vector per row (dwordx4 loads and stores); a wave covers 1 KiB
// of a row per instruction. The FP8 kind quantises on the fly: a lane holds
// 16 bf16 values (two dwordx4 loads), eight consecutive lanes hold one 1x128
// block, the block's amax is reduced across those eight lanes with DPP, and
// the lane writes its 16 E4M3 codes as one dwordx4.
// Cache policy (measured on MI355X at the 8K x 7168 x top-8 shape): the k
// payload rows go out with streaming stores; x is read with plain loads and
// the 32-byte pieces of each scale row with plain stores, which L2 merges
// into whole lines (streaming either of them cost about 30 us per call).
#pragma once

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

constexpr bool dispatch_is_fp8(int kind) { return kind == kDispatchFp8Quant || kind == kDispatchFp8Copy; }

// Zero-fills receive rows [r0, r1) (data and, for FP8, scales) with the
// whole block.
template <int KIND>
__device__ __forceinline__ void dispatch_zero_rows(const DispatchArgs& a, int r0, int r1) {
    constexpr bool kFp8 = dispatch_is_fp8(KIND);
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int64_t row_out = kFp8 ? (int64_t)a.H : 2 * (int64_t)a.H;
    const int nb = a.H / 128;
    const int nvec = (int)(row_out / 16);
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (int r = r0; r < r1; ++r) {
        uint4* dst = (uint4*)((char*)a.recv + (int64_t)r * row_out);
        for (int c = tid; c < nvec; c += nthreads) store_stream(dst + c, z);
        if (kFp8)
            for (int b = tid; b < nb; b += nthreads) a.recv_scales[(int64_t)r * nb + b] = 0.0f;
    }
}

// Copies token t's row into the receive rows of its k pairs with the whole
// block. Lane j < k of every wave holds pair j's row in my_s (-1 = skipped)
// and, for the weighted kind, its weight in my_w; the store loops broadcast
// them with readlane, so no load waits between stores.
template <int KIND>
__device__ __forceinline__ void dispatch_token(const DispatchArgs& a, int t, int my_s, float my_w) {
    constexpr bool kFp8 = dispatch_is_fp8(KIND);
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int64_t row_out = kFp8 ? (int64_t)a.H : 2 * (int64_t)a.H;
    const int nb = a.H / 128;
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

}  // namespace ep
