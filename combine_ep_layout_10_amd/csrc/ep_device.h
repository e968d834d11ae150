// Device helpers shared by the gfx950 kernels of the dispatch/combine library.
// Wave64 only: every lane mask below is 64 bits wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// binary32 -> bfloat16 bits, round to nearest even. Inputs are finite: adding
// 0x7FFF plus the kept LSB carries into the kept half exactly when the
// discarded half is above one half, or equal to it with an odd kept LSB.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two binary32 -> packed bfloat16 (a in the low half), round to nearest even,
// by gfx950's v_cvt_pk_bf16_f32 (one instruction for both). Checked on
// MI355X against f32_to_bf16_rne on every non-NaN binary32 pattern,
// subnormals included: identical.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fl(a / 448) for a >= 0 that is a bfloat16 value: the product with
// c = fl(1/448) and one FMA correction (residual a - y * 448 is exact).
// Checked in exact rational arithmetic on every finite non-negative bfloat16
// value, subnormals included: equal to the IEEE quotient. Infinity passes
// through (inf / 448 = inf).
__device__ __forceinline__ float div448_bf16(float a) {
    constexpr float c = 1.0f / 448.0f;
    const float y = a * c;
    const float e = __builtin_fmaf(-y, 448.0f, a);
    const float s = __builtin_fmaf(e, c, y);
    return a < __builtin_inff() ? s : a;
}

// ---------------------------------------------------------------- memory

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte store into one row through a buffer resource, with the
// cache policy sc0 sc1 nt (LLVM's GLC | SLC | SCC bits, read by gfx950 as
// sc0, nt and sc1). Measured on MI355X on the dispatch's pattern (a 14 KiB
// row read, then written to 8 rows): 6.36 TB/s of total traffic against
// 5.83 TB/s with plain non-temporal global stores. `row` must be the same in
// every lane (it becomes the resource's base, in scalar registers); stores at
// or past `row_bytes` are dropped by the hardware. The resource's last word
// selects 32-bit data (0x00020000); with 0 the stores are dropped (checked).
constexpr int kBufferFlags = 0x00020000;
constexpr int kCpolStream = 1 | 2 | 16;

__device__ __forceinline__ void store_row_stream(void* row, uint32_t row_bytes, uint32_t off, uint4 v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(row, 0, (int)row_bytes, kBufferFlags);
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, kCpolStream);
}

// Streaming (nt) 16-byte load from one row through a buffer resource, for
// rows gathered once (the combine's expert-output rows): nt keeps single-use
// rows from displacing reusable lines in L2 and MALL, and the row's base sits
// in scalar registers, so a lane adds only its 32-bit offset. Measured on
// MI355X in the 8192 x 7168 x top-8 combine: 178.2-178.8 us against
// 180.2-181.4 us for non-temporal global loads with 64-bit per-lane
// addresses, three runs in alternation (sc0 nt, sc1 nt and sc0 sc1 nt the
// same within noise; without nt 191-193 us). `row` must be the same in every
// lane; loads at or past `row_bytes` return zeros.
constexpr int kCpolLoadStream = 2;

__device__ __forceinline__ uint4 load_row_stream(const void* row, uint32_t row_bytes, uint32_t off) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, (int)row_bytes, kBufferFlags);
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolLoadStream);
    return make_uint4(x.x, x.y, x.z, x.w);
}

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Lanes of the wave whose (active, key) equals this lane's: AND over the key's
// bits of "lanes that agree on this bit". nbits covers every key value.
__device__ __forceinline__ uint64_t match_peers(int key, bool active, int nbits) {
    uint64_t m = ballot64(active);
    for (int b = 0; b < nbits; ++b) {
        bool bit = (key >> b) & 1;
        uint64_t on = ballot64(active && bit);
        m &= bit ? on : ~on;
    }
    return m;
}

__device__ __forceinline__ uint64_t lanes_below(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Max over the 8 consecutive lanes of an aligned group (lane & ~7) with DPP:
// swap neighbours, swap pairs, then mirror inside each half-row of 8.
__device__ __forceinline__ float max8_dpp(float v) {
    int x = __float_as_int(v);
    int y = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v = fmaxf(v, __int_as_float(y));
    x = __float_as_int(v);
    y = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);       // quad_perm [2,3,0,1]
    v = fmaxf(v, __int_as_float(y));
    x = __float_as_int(v);
    y = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);      // row_half_mirror
    return fmaxf(v, __int_as_float(y));
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int n = __shfl_up(v, o, kWave);
        if (lane >= o) v += n;
    }
    return v;
}

// Exclusive prefix sum over a block of nthreads (multiple of 64, <= 1024).
// `tmp` is LDS of at least 17 ints. Every thread of the block must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nw = blockDim.x >> 6;
    int inc = wave_inclusive_scan(v);
    if (lane == 63) tmp[w] = inc;
    __syncthreads();
    if (w == 0) {
        int s = lane < nw ? tmp[lane] : 0;
        int si = wave_inclusive_scan(s);
        if (lane < nw) tmp[lane] = si - s;
        if (lane == nw - 1) tmp[16] = si;
    }
    __syncthreads();
    int out = inc - v + tmp[w];
    *total = tmp[16];
    __syncthreads();
    return out;
}

}  // namespace ep
