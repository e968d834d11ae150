// FP8 grouped GEMM over the aligned expert-major layout: the consumer the
// layout is built for (DeepEP README: per-expert received-token counts "for
// GEMM", rows padded to expert_alignment; "New features": EPv2's new GEMM
// layout). For every row r of expert e and output channel n:
//   C[r, n] = bf16( sum_kb sa[r, kb] * sb[e, n/128, kb]
//                          * sum_{k in block kb} A[r, k] * B[e, n, k] )
// with A the dispatched E4M3 codes [rows, K] and their 1x128 scales
// sa [rows, K/128], B[e] the expert's E4M3 weights [N, K] with 128x128 block
// scales sb[e] [N/128, K/128].
//
// Tiling (gfx950, wave64): a block of 4 waves computes a 128 x 128 tile of C;
// each wave owns a 64 x 64 quarter as 2 x 2 MFMA tiles of 32 x 32. The K loop
// runs over 128-wide scale blocks: the A and B tiles of one block (2 x 16 KiB)
// are staged in LDS (rows padded to 144 bytes so the 16-byte operand reads of
// 16 consecutive rows cover all 64 banks once), each wave issues
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales (two K steps of 64)
// into fresh fp32 partials, and the partials are promoted into the fp32
// accumulators with the row's 1x128 scale times the tile's 128x128 weight
// scale (one binary32 product, one FMA). The loads of the next K block are
// issued into registers before the MFMAs of the current one.
//
// MFMA operand layout (checked on MI355X): lane l holds row (l mod 32) of
// the A sub-tile and column (l mod 32) of the B sub-tile, each with 32 K
// values; A and B lanes with the same l / 32 must hold the same K values,
// in the same byte order (which K values they are does not matter for the
// product). Result: lane l, register i holds row 8(i/4) + 4(l/32) + (i mod 4),
// column l mod 32.
//
// Block order: logical block L enumerates experts in order, within an expert
// the 128-column tiles, within those the expert's 128-row tiles, so blocks
// sharing an A or B tile are adjacent; logical blocks are dealt to the 8 XCDs
// in contiguous ranges (hardware block b runs on XCD b mod 8), so the reuse
// happens inside one XCD's L2.
#include "ep_internal.h"

namespace ep {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kTile = 128;
constexpr int kLdsRow = kTile + 16;  // padded row stride (bytes)
constexpr int kXcds = 8;

// Rows of expert e that the GEMM covers and the first tile's row.
__device__ __forceinline__ void gemm_expert_tiles(const GemmArgs& a, int e, int& first_row, int& ntiles) {
    if (a.mode == EP_MODE_COMPACT) {
        first_row = a.expert_off[e];
        ntiles = (a.expert_off[e + 1] - first_row) / kTile;
    } else {
        first_row = e * a.C;
        ntiles = (a.pad[e] + kTile - 1) / kTile;
    }
}

__global__ __launch_bounds__(256) void k_grouped_gemm_fp8(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kTile * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint8_t s_b[kTile * kLdsRow];
    __shared__ float s_sa[kTile];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nt_n = a.N / kTile;

    // logical block: a contiguous range per XCD. Hardware block b runs on XCD
    // b mod 8 as its (b / 8)-th block; with total = 8q + r, XCDs below r take
    // q + 1 logical blocks and the others q, which maps blocks one to one.
    const int total = (int)gridDim.x;
    const int q = total / kXcds, r = total % kXcds;
    const int xcd = (int)blockIdx.x % kXcds, idx = (int)blockIdx.x / kXcds;
    const int L = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;

    // expert of L: COMPACT tiles are numbered by row / 128 (every expert range
    // is a whole number of tiles); FIXED experts own C / 128 tile slots each.
    int e, n_tile, row0;
    if (a.mode == EP_MODE_COMPACT) {
        int lo = 0, hi = a.E;  // largest e with expert_off[e] / 128 * nt_n <= L
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((a.expert_off[mid] / kTile) * nt_n <= L) lo = mid;
            else hi = mid - 1;
        }
        e = lo;
        if (e >= a.E) return;  // past the last row
        int first_row, ntiles;
        gemm_expert_tiles(a, e, first_row, ntiles);
        const int local = L - (first_row / kTile) * nt_n;
        if (ntiles == 0 || local >= ntiles * nt_n) return;
        n_tile = local / ntiles;
        row0 = first_row + (local % ntiles) * kTile;
    } else {
        const int slots = a.C / kTile;
        e = L / (slots * nt_n);
        const int local = L % (slots * nt_n);
        int first_row, ntiles;
        gemm_expert_tiles(a, e, first_row, ntiles);
        n_tile = local / slots;
        const int m = local % slots;
        if (m >= ntiles) return;
        row0 = first_row + m * kTile;
    }
    const int n0 = n_tile * kTile;
    const int KB = a.K / kTile;

    // staging: thread t moves 64 bytes of row t / 2 (A) and of column t / 2 (B)
    const int srow = tid >> 1, shalf = tid & 1;
    const uint8_t* ga = a.a + (int64_t)(row0 + srow) * a.K + shalf * 64;
    const uint8_t* gb = a.b + ((int64_t)e * a.N + n0 + srow) * a.K + shalf * 64;
    const float* gsa = a.sa + (int64_t)row0 * KB;
    const float* gsb = a.sb + ((int64_t)e * nt_n + n_tile) * KB;

    v4i_t ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;  // next K block's bytes (64 of A, 64 of B)
    float rsa = 0.0f;
    ra0 = ((const v4i_t*)ga)[0];
    ra1 = ((const v4i_t*)ga)[1];
    ra2 = ((const v4i_t*)ga)[2];
    ra3 = ((const v4i_t*)ga)[3];
    rb0 = ((const v4i_t*)gb)[0];
    rb1 = ((const v4i_t*)gb)[1];
    rb2 = ((const v4i_t*)gb)[2];
    rb3 = ((const v4i_t*)gb)[3];
    if (tid < kTile) rsa = gsa[(int64_t)tid * KB];

    const int wm = w >> 1, wn = w & 1;
    const int g = lane >> 5, r32 = lane & 31;
    v16f_t acc[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[s][t][i] = 0.0f;

    for (int kb = 0; kb < KB; ++kb) {
        __syncthreads();  // the previous block's operands have been read
        v4i_t* la = (v4i_t*)(s_a + srow * kLdsRow + shalf * 64);
        v4i_t* lb = (v4i_t*)(s_b + srow * kLdsRow + shalf * 64);
        la[0] = ra0;
        la[1] = ra1;
        la[2] = ra2;
        la[3] = ra3;
        lb[0] = rb0;
        lb[1] = rb1;
        lb[2] = rb2;
        lb[3] = rb3;
        if (tid < kTile) s_sa[tid] = rsa;
        const float sbv = gsb[kb];
        __syncthreads();
        if (kb + 1 < KB) {  // next block's loads go out before this block's MFMAs
            const int64_t off = (int64_t)(kb + 1) * kTile;
            const v4i_t* na = (const v4i_t*)(ga + off);
            const v4i_t* nb = (const v4i_t*)(gb + off);
            ra0 = na[0];
            ra1 = na[1];
            ra2 = na[2];
            ra3 = na[3];
            rb0 = nb[0];
            rb1 = nb[1];
            rb2 = nb[2];
            rb3 = nb[3];
            if (tid < kTile) rsa = gsa[(int64_t)tid * KB + kb + 1];
        }
        v16f_t part[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) part[s][t][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8i_t opa[2], opb[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint8_t* pa = s_a + (64 * wm + 32 * s + r32) * kLdsRow + 64 * ks + 32 * g;
                const uint8_t* pb = s_b + (64 * wn + 32 * s + r32) * kLdsRow + 64 * ks + 32 * g;
                const v4i_t a0 = *(const v4i_t*)pa, a1 = *(const v4i_t*)(pa + 16);
                const v4i_t b0 = *(const v4i_t*)pb, b1 = *(const v4i_t*)(pb + 16);
                opa[s] = (v8i_t){a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                opb[s] = (v8i_t){b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    part[s][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opa[s], opb[t], part[s][t], 0, 0, 0,
                                                                                127, 0, 127);
        }
        // promotion: acc += part * (sa[row] * sb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 64 * wm + 32 * s + 8 * (i >> 2) + 4 * g + (i & 3);
                const float f = s_sa[row] * sbv;
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[s][t][i] = __builtin_fmaf(part[s][t][i], f, acc[s][t][i]);
            }
    }

    // epilogue: bf16, round to nearest even
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = row0 + 64 * wm + 32 * s + 8 * (i >> 2) + 4 * g + (i & 3);
                const int col = n0 + 64 * wn + 32 * t + r32;
                a.c[(int64_t)row * a.N + col] = (uint16_t)f32_to_bf16_rne(acc[s][t][i]);
            }
}

hipError_t launch_grouped_gemm_fp8(const GemmArgs& a, int64_t rows_bound, hipStream_t stream) {
    const int nt_n = a.N / kTile;
    int64_t blocks;
    if (a.mode == EP_MODE_COMPACT)
        blocks = (rows_bound + kTile - 1) / kTile * nt_n;
    else
        blocks = (int64_t)a.E * (a.C / kTile) * nt_n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_grouped_gemm_fp8, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ep
