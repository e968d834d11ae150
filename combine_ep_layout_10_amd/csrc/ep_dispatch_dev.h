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
// payload rows and the zero padding rows go out with store_row_stream
// (buffer stores, sc0 sc1 nt); x is read with plain loads and the 32-byte
// pieces of each scale row with plain stores, which L2 merges into whole
// lines (streaming either of them cost about 30 us per call; plain payload
// stores cost 29-38 us).
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
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
}

constexpr bool dispatch_is_fp8(int kind) {
    return kind == kDispatchFp8Quant || kind == kDispatchFp8Copy || kind == kDispatchFp8QuantWeighted;
}

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
        char* dst = (char*)a.recv + (int64_t)r * row_out;
        for (int c = tid; c < nvec; c += nthreads) store_row_stream(dst, (uint32_t)row_out, 16u * c, z);
        if (kFp8)
            for (int b = tid; b < nb; b += nthreads) a.recv_scales[(int64_t)r * nb + b] = 0.0f;
    }
}

// What one lane holds of a token's row between the load and the stores.
// Raw: the loaded bytes (BF16: one 16-byte vector of 8 values; FP8 quantise:
// two vectors, 16 values; FP8 copy: one vector of 16 codes and its block's
// scale). Vec: what is stored (the vector, and the 1x128 scale for FP8).
struct DispatchRaw {
    uint4 v0, v1;
    float scale;
};
struct DispatchVec {
    uint4 v, v1;  // v1: second half of the 16 values (weighted FP8 only)
    float scale;
};

// Issues the loads of vector c of token t's row (no arithmetic, so callers
// can overlap them with other work).
template <int KIND>
__device__ __forceinline__ DispatchRaw dispatch_load(const DispatchArgs& a, int t, int c, bool act) {
    DispatchRaw r;
    r.v0 = make_uint4(0u, 0u, 0u, 0u);
    r.v1 = r.v0;
    r.scale = 0.0f;
    if (!act) return r;
    if (KIND == kDispatchBf16 || KIND == kDispatchBf16Weighted) {
        r.v0 = ((const uint4*)((const char*)a.x + (int64_t)t * 2 * a.H))[c];
    } else if (KIND == kDispatchFp8Quant || KIND == kDispatchFp8QuantWeighted) {
        const uint4* src = (const uint4*)((const char*)a.x + (int64_t)t * 2 * a.H);
        r.v0 = src[2 * c];
        r.v1 = src[2 * c + 1];
    } else {  // kDispatchFp8Copy
        r.v0 = ((const uint4*)((const char*)a.x + (int64_t)t * a.H))[c];
        if ((c & 7) == 0) r.scale = a.x_scales[(int64_t)t * (a.H / 128) + (c >> 3)];
    }
    return r;
}

// The amax of a 1x128 block held by eight consecutive lanes (16 values
// each): this lane's maximum magnitude, then a DPP reduction across the
// eight lanes. Every lane of the wave must call it (inactive lanes hold
// zeros).
__device__ __forceinline__ float block_amax16(const float f[16]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
    return max8_dpp(amax);
}

// Quantises this lane's 16 values of a 1x128 block whose amax (a bfloat16
// value: the largest magnitude in the block) is given: scale = amax / 448,
// codes = E4M3(x / scale) rounded to nearest even, x / scale being the IEEE
// binary32 quotient; an all-zero block gives scale 0 and zero codes.
//
// scale = fl(amax / 448) by div448_bf16. The quotient is taken as
// q = y - (y*scale - x) * r with r = 1/scale and y = x*r (one division per
// lane instead of 16; the residual y*scale - x is exact by FMA). No
// copysign is needed for -0: for x != 0 the FMA's exact value
// y - (y*scale - x)*r has x's sign, and rounding keeps it (a quotient that
// underflows is a zero of x's sign); for x = +-0 the residual is +0 and
// q = -(+0)*r + y = y, a zero of x's sign. Checked exhaustively on MI355X: for every pair of
// finite bf16 values |x| <= amax with scale >= 2^-80, q equals the IEEE
// quotient wherever |x / scale| >= 2^-10 (below that every code is a signed
// zero and both agree). Smaller scales (amax < 2^-71) take the IEEE
// division. The codes come from gfx950's v_cvt_pk_fp8_f32 (OCP E4M3, round
// to nearest even), checked against an integer round-to-nearest-even
// encoder on every binary32 of magnitude <= 448.0001; quotients never exceed
// 448 * (1 + 2^-23) because |x| <= amax.
__device__ __forceinline__ uint4 quantize16_amax(const float f[16], float amax, float& scale_out) {
    const float scale = div448_bf16(amax);
    float q[16];
    if (scale >= 0x1p-80f) {
        // 1/scale from the hardware reciprocal and one Newton step: checked on
        // MI355X against the IEEE quotient 1/scale for every scale this branch
        // can see (fl(a/448) for each of the 25,504 positive finite bfloat16 a
        // with a scale >= 2^-80): identical, so r is the correctly rounded
        // reciprocal.
        const float r0 = __builtin_amdgcn_rcpf(scale);
        const float r = __builtin_fmaf(__builtin_fmaf(-scale, r0, 1.0f), r0, r0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float y = f[i] * r;
            const float e = __builtin_fmaf(y, scale, -f[i]);
            q[i] = __builtin_fmaf(-e, r, y);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = amax != 0.0f ? f[i] / scale : 0.0f;
    }
    uint32_t w4[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * d], q[4 * d + 1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * d + 2], q[4 * d + 3], w, true);
        w4[d] = (uint32_t)w;
    }
    scale_out = scale;
    return make_uint4(w4[0], w4[1], w4[2], w4[3]);
}

// The 1x128 block quantiser on 16 bf16 values per lane (every lane of the
// wave must call it).
__device__ __forceinline__ uint4 quantize16(const float f[16], float& scale_out) {
    return quantize16_amax(f, block_amax16(f), scale_out);
}

// Turns loaded bytes into what is stored. FP8 quantise: the 1x128 block
// quantiser above; vectors must be grouped in aligned runs of eight. The
// weighted FP8 kind keeps the values: each pair is quantised at the store.
template <int KIND>
__device__ __forceinline__ DispatchVec dispatch_encode(const DispatchRaw& r) {
    DispatchVec d;
    d.v = r.v0;
    d.v1 = r.v1;
    d.scale = r.scale;
    if (KIND == kDispatchFp8Quant) {
        float f[16];
        unpack_bf16x8(r.v0, f);
        unpack_bf16x8(r.v1, f + 8);
        d.v = quantize16(f, d.scale);
    }
    return d;
}

// Stores vector c of a loaded row into the receive rows of the token's k
// pairs. Lane j < k of every wave holds pair j's row in my_s (-1 = skipped)
// and, for the weighted kind, its weight in my_w; the loop broadcasts them
// with readlane, so no load waits between stores.
template <int KIND>
__device__ __forceinline__ void dispatch_store(const DispatchArgs& a, const DispatchVec& d, int c, bool act,
                                               int my_s, float my_w) {
    constexpr bool kFp8 = dispatch_is_fp8(KIND);
    const int64_t row_out = kFp8 ? (int64_t)a.H : 2 * (int64_t)a.H;
    const int nb = a.H / 128;
    if (KIND == kDispatchFp8QuantWeighted) {
        // Each pair's copy is bf16(w * x), quantised with its own scales.
        // Rounding to binary32 and to bf16 is monotone and odd, so the
        // block amax of bf16(w * x) is bf16(|w| * amax(x)) exactly: the
        // block reduction over x runs once (every lane of the wave takes
        // part; `act` guards only the stores), not once per pair.
        float f[16];
        unpack_bf16x8(d.v, f);
        unpack_bf16x8(d.v1, f + 8);
        const float ax = block_amax16(f);
        for (int j = 0; j < a.k; ++j) {
            const int s = __builtin_amdgcn_readlane(my_s, j);
            if (s < 0) continue;
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
            // bf16(w * x) lands in the high half of a binary32 whose low
            // half is bf16(0) = 0: the rounded product as a binary32, one
            // conversion per value and no unpacking.
            float g[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) g[i] = __uint_as_float(pack_bf16x2(0.0f, wj * f[i]));
            const float ag = bf16_to_f32(pack_bf16x2(fabsf(wj) * ax, 0.0f) & 0xFFFFu);
            float scale;
            const uint4 o = quantize16_amax(g, ag, scale);
            if (act) {
                store_row_stream((char*)a.recv + (int64_t)s * row_out, (uint32_t)row_out, 16u * c, o);
                if ((c & 7) == 0) a.recv_scales[(int64_t)s * nb + (c >> 3)] = scale;
            }
        }
        return;
    }
    float f[8];
    if (KIND == kDispatchBf16Weighted) unpack_bf16x8(d.v, f);
    if (!act) return;
    for (int j = 0; j < a.k; ++j) {
        const int s = __builtin_amdgcn_readlane(my_s, j);
        if (s < 0) continue;
        uint4 o = d.v;
        if (KIND == kDispatchBf16Weighted) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
            float g[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) g[i] = wj * f[i];
            o = pack_bf16x8(g);
        }
        store_row_stream((char*)a.recv + (int64_t)s * row_out, (uint32_t)row_out, 16u * c, o);
        if (kFp8 && (c & 7) == 0) a.recv_scales[(int64_t)s * nb + (c >> 3)] = d.scale;
    }
}

// Vectors per row: 8 bf16 (BF16 kinds) or 16 codes (FP8 kinds) per vector.
template <int KIND>
__device__ __forceinline__ int dispatch_nvec(const DispatchArgs& a) {
    return dispatch_is_fp8(KIND) ? a.H / 16 : a.H / 8;
}

// Copies vectors [c0, c1) of token t's row into the receive rows of its k
// pairs with the whole block (c0 a multiple of 8 for the FP8 kinds). The
// loop bound is uniform across the block, so every lane of a wave takes part
// in the FP8 amax reduction; `act` only guards memory.
template <int KIND>
__device__ __forceinline__ void dispatch_token(const DispatchArgs& a, int t, int c0, int c1, int my_s,
                                               float my_w) {
    for (int cb = c0; cb < c1; cb += blockDim.x) {
        const int c = cb + threadIdx.x;
        const bool act = c < c1;
        const DispatchVec d = dispatch_encode<KIND>(dispatch_load<KIND>(a, t, c, act));
        dispatch_store<KIND>(a, d, c, act, my_s, my_w);
    }
}

}  // namespace ep
