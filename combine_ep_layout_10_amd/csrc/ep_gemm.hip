// FP8 grouped GEMM over the aligned expert-major layout: the consumer the
// layout is built for (DeepEP README: per-expert received-token counts meant for
// the expert GEMM, rows padded to expert_alignment; "New features": EPv2's new GEMM
// layout). For every row r of expert e and output channel n:
//   C[r, n] = bf16( sum_kb sa[r, kb] * sb[e, n/128, kb]
//                          * sum_{k in block kb} A[r, k] * B[e, n, k] )
// with A the dispatched E4M3 codes [rows, K] and their 1x128 scales
// sa [rows, K/128], B[e] the expert's E4M3 weights [N, K] with 128x128 block
// scales sb[e] [N/128, K/128].
//
// Two kernels. For N % 256 == 0, k_grouped_gemm_fp8_dma (128 x 256 tiles fed
// by LDS DMA; described with it below). For any N % 128, k_grouped_gemm_fp8:
// (gfx950, wave64) a block of 4 waves computes a 128 x 128 tile of C;
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
// happens inside one XCD's L2. The ranges cover the tiles the layout uses:
// in COMPACT mode the grid is sized from the rows bound (the rows used are
// only known on the device), and dealing the whole grid put every unused
// block on the last XCDs (17.6 % of the grid on the V3 layout, one and a
// half XCDs idle: 4.07 against 3.51 ms). Round-robin dealing balances as
// well but spreads each A tile over all 8 L2s (14.4 against 11.2 GB
// fetched per launch).
#include "ep_internal.h"

namespace ep {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kTile = 128;
constexpr int kLdsRow = kTile + 16;  // padded row stride (bytes)
constexpr int kXcds = 8;
constexpr int kMaxGemmKBlocks = 512;  // K / 128 limit of the DMA kernel (two column halves' scales in LDS)

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

// Blocks that hold a tile: COMPACT numbers tiles by row / 128 up to the
// layout's expert_off[E]; FIXED gives every expert C / 128 tile slots.
__device__ __forceinline__ int gemm_used_blocks(const GemmArgs& a, int nt_n) {
    if (a.mode == EP_MODE_COMPACT) return min((a.expert_off[a.E] / kTile) * nt_n, (int)gridDim.x);
    return (int)gridDim.x;
}

__global__ __launch_bounds__(256) void k_grouped_gemm_fp8(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kTile * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint8_t s_b[kTile * kLdsRow];
    __shared__ float s_sa[kTile];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nt_n = a.N / kTile;

    // logical block: a contiguous range per XCD. Hardware block b runs on XCD
    // b mod 8 as its (b / 8)-th block; of the blocks below total = 8q + r,
    // XCDs below r take q + 1 and the others q, which maps them one to one
    // onto the logical blocks [0, total); blocks from total on have no tile.
    const int total = gemm_used_blocks(a, nt_n);
    if ((int)blockIdx.x >= total) return;
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

// ---------------------------------------------------------------- 128 x 256 tiles, LDS DMA
// For N % 256 == 0: a block of 8 waves computes a 128 x 256 tile (waves 2 x 4,
// each a 64 x 64 piece as above). Operands move global -> LDS by DMA
// (global_load_lds_dwordx4: lane i's 16 bytes land at the wave's LDS pointer
// + 16 i, checked on MI355X), into a ring of kStages LDS stages, issued two
// K blocks ahead, so up to 2 x 48 KiB per CU are in flight without staging
// registers. LDS rows are not padded: 16-byte chunk c of row r is stored at
// chunk position c ^ ((r / 2) mod 8) of its 128-byte row. A row covers half of
// the 64 banks (rows of one parity the same half), so any 16 consecutive rows
// read at one chunk hit all 64 banks exactly once. The row scales of a K block
// come by 4-byte DMA (lane i -> + 4 i) into a ring of their own. Every wave
// issues the same number of DMA loads per stage (waves 2..7 repeat a scale
// load into a scratch LDS slot), and past the last K block the pipeline
// re-issues the last stage's loads (the same bytes into the same buffer), so
// the wait before each K block is one constant vmcnt.

constexpr int kStages = 3;
constexpr int kScaleStages = 4;  // row scales are read one K block later than the operands
constexpr int kBN2 = 256;
constexpr int kDmaPerStage = 2 + 4 + 1;  // A, B, scale loads per wave and stage

// s_waitcnt with only the vector-memory count limited (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
#define EP_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// One global -> LDS DMA load per lane (16 or 4 bytes), written as inline
// assembly: the compiler cannot tell which LDS bytes a DMA load writes, so
// for the intrinsic it waits for every outstanding DMA load before any LDS
// read, which would drain the prefetch ring each K block. Here the waits are
// explicit (EP_WAIT_VMCNT + barrier before a stage is read). The source is a
// wave-uniform base (scalar register pair) plus a 32-bit per-lane byte
// offset, so that the per-lane part stays fixed over the K loop; `lds` is the
// wave's LDS destination (uniform), lane i's data lands at lds + size * i.
// The LDS address goes in through an m0 input operand: the compiler writes
// m0 itself and knows what it holds (the asm never writes it); the s_nop is
// the one wait state an m0 write needs before an LDS DMA reads it.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// a pointer that is the same in every lane, moved to scalar registers
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__global__ __launch_bounds__(512) void k_grouped_gemm_fp8_dma(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kStages][kTile * kTile];
    __shared__ __attribute__((aligned(16))) uint8_t s_b[kStages][kBN2 * kTile];
    __shared__ __attribute__((aligned(16))) float s_sa[kScaleStages][kTile];
    __shared__ __attribute__((aligned(16))) float s_dummy[64];
    __shared__ float s_sb[kMaxGemmKBlocks];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nt_n = a.N / kBN2;

    const int total = gemm_used_blocks(a, nt_n);  // dealt as in k_grouped_gemm_fp8
    if ((int)blockIdx.x >= total) return;
    const int q = total / kXcds, r = total % kXcds;
    const int xcd = (int)blockIdx.x % kXcds, idx = (int)blockIdx.x / kXcds;
    const int L = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;

    int e, n_tile, row0, live;  // live: rows of the tile that hold pairs (the rest are padding)
    if (a.mode == EP_MODE_COMPACT) {
        int lo = 0, hi = a.E;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((a.expert_off[mid] / kTile) * nt_n <= L) lo = mid;
            else hi = mid - 1;
        }
        e = lo;
        if (e >= a.E) return;
        int first_row, ntiles;
        gemm_expert_tiles(a, e, first_row, ntiles);
        const int local = L - (first_row / kTile) * nt_n;
        if (ntiles == 0 || local >= ntiles * nt_n) return;
        n_tile = local / ntiles;
        row0 = first_row + (local % ntiles) * kTile;
        live = a.cnt[e] - (row0 - first_row);
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
        live = a.pad[e] - m * kTile;
    }
    e = __builtin_amdgcn_readfirstlane(e);
    live = __builtin_amdgcn_readfirstlane(live);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    const int n0 = __builtin_amdgcn_readfirstlane(n_tile) * kBN2;
    const int KB = a.K / kTile;

    // weight-block scales of this column tile: all K blocks, once
    const float* gsb = a.sb + ((int64_t)e * (a.N / kTile) + n0 / kTile) * KB;
    const float* gsb2 = gsb + KB;  // the second 128-column half of the tile
    for (int i = tid; i < 2 * KB; i += blockDim.x) s_sb[i] = i < KB ? gsb[i] : gsb2[i - KB];
    EP_WAIT_VMCNT(0);
    __syncthreads();

    // DMA sources: tile bases (uniform) and per-lane offsets within K block 0;
    // K block kb adds kb * 128 bytes (kb * 4 for the row scales) to the bases.
    // Offsets fit 32 bits: at most 255 rows of K <= 32768 bytes.
    const int sub = lane >> 3, ch = lane & 7;
    const uint8_t* baseA = uniform_ptr(a.a + (int64_t)row0 * a.K);
    const uint8_t* baseB = uniform_ptr(a.b + ((int64_t)e * a.N + n0) * a.K);
    const float* baseS = uniform_ptr(a.sa + (int64_t)row0 * KB);
    uint32_t offA[2], offB[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = (w * 2 + j) * 8 + sub;
        offA[j] = (uint32_t)(m * a.K + ((ch ^ ((m >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = (w * 4 + j) * 8 + sub;
        offB[j] = (uint32_t)(n * a.K + ((ch ^ ((n >> 1) & 7)) << 4));
    }
    const uint32_t offS = (uint32_t)(((w & 1) * 64 + lane) * KB * 4);  // scale row this lane moves
    const uint32_t ldsA = lds_addr(&s_a[0][0]), ldsB = lds_addr(&s_b[0][0]);
    const uint32_t ldsS = w < 2 ? lds_addr(&s_sa[0][0]) + w * 256 : lds_addr(s_dummy);
    const uint32_t ldsS_step = w < 2 ? kTile * 4 : 0;

    auto issue = [&](int kb) {
        const int st = kb % kStages;
        const uint8_t* ga = uniform_ptr(baseA + (int64_t)kb * kTile);
        const uint8_t* gb = uniform_ptr(baseB + (int64_t)kb * kTile);
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(ga, offA[j], ldsA + st * (kTile * kTile) + (w * 2 + j) * 1024);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(gb, offB[j], ldsB + st * (kBN2 * kTile) + (w * 4 + j) * 1024);
        dma4(uniform_ptr(baseS + kb), offS, ldsS + (kb % kScaleStages) * ldsS_step);
    };
    issue(0);
    issue(min(1, KB - 1));
    issue(min(2, KB - 1));

    const int wm = w >> 2, wn = w & 3;
    const int g = lane >> 5, r32 = lane & 31;
    // 32-row pieces wholly past the expert's pairs are padding: their MFMAs
    // and promotion are skipped (the wave still loads and waits with the
    // block) and they are written as zeros, which is what zero padding rows
    // give. The SIMD's other wave then has the MFMA unit to itself.
    const bool live0 = 64 * wm < live, live1 = 64 * wm + 32 < live;
    v16f_t acc[2][2], part[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[s][t][i] = 0.0f;

    // LDS byte offsets of this lane's operand chunks within a stage, per K
    // step (64 wide) and chunk of the pair; the second 32-row (column) piece
    // is 32 rows = 4096 bytes further, with the same swizzle
    uint32_t rdA[2][2], rdB[2][2];
    {
        const int ra = 64 * wm + r32, rb = 64 * wn + r32;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                rdA[ks][j] = 16 * swz(ra, 4 * ks + 2 * g + j);
                rdB[ks][j] = 16 * swz(rb, 4 * ks + 2 * g + j);
            }
    }
    // operands of one K step (64 wide) of one stage: A rows and B columns of
    // this wave's two 32-row and two 32-column pieces
    auto read_ops = [&](int st, int ks, v8i_t opa[2], v8i_t opb[2]) {
        const uint8_t* la = &s_a[0][0] + st * (kTile * kTile);
        const uint8_t* lb = &s_b[0][0] + st * (kBN2 * kTile);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const v4i_t a0 = *(const v4i_t*)(la + rdA[ks][0] + 4096 * s);
            const v4i_t a1 = *(const v4i_t*)(la + rdA[ks][1] + 4096 * s);
            const v4i_t b0 = *(const v4i_t*)(lb + rdB[ks][0] + 4096 * s);
            const v4i_t b1 = *(const v4i_t*)(lb + rdB[ks][1] + 4096 * s);
            opa[s] = (v8i_t){a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            opb[s] = (v8i_t){b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        }
    };
    // The MFMAs take the B operand first, so each 32 x 32 piece comes out
    // transposed: lane r32 holds one output row, element i of the 16 holds
    // column 8 (i / 4) + 4 g + i % 4. The promotion factor (row scale x
    // column-block scale) is then one value per lane and piece row: this
    // wave's 64 columns lie in one 128-column scale block.
    // acc += part * (row scale * column scale) for the pieces of K block kb
    auto promote = [&](int kb, int s, int t, float f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[s][t][i] = __builtin_fmaf(part[s][t][i], f, acc[s][t][i]);
    };
    auto factor = [&](int kb, int s) {
        const float sbv = s_sb[(wn >> 1) * KB + kb];  // waves 0-1 and 2-3 of a row cover different halves
        return s_sa[kb % kScaleStages][64 * wm + 32 * s + r32] * sbv;
    };

    // Software pipeline over K blocks. On entry to K block kb both K steps'
    // operands of stage kb are in registers and `part` holds K block kb - 1.
    //  1. per 32 x 32 piece: promote its K block kb - 1 partial, then start
    //     its first MFMA of K block kb (the FMAs overlap the MFMAs in flight);
    //  2. barrier: every wave has finished reading stage kb (all its reads
    //     were issued in the previous K block) and stage kb + 1 has landed;
    //  3. DMA of stage kb + 3 into stage kb's buffer;
    //  4. read stage kb + 1's first K step into the registers just consumed,
    //     then the second MFMAs of K block kb, then stage kb + 1's second K
    //     step. Past the last K block the reads hit a valid, unused stage.
    // Row scales have a ring of 4: those of K block kb - 1 are read in step 1
    // of K block kb, before the barrier after which stage kb + 3's land in
    // that slot.
    EP_WAIT_VMCNT(2 * kDmaPerStage);
    __syncthreads();
    asm volatile("" ::"v"(&s_a[0][0]), "v"(&s_b[0][0]), "v"(&s_sa[0][0]) : "memory");
    v8i_t opa0[2], opb0[2], opa1[2], opb1[2];
    read_ops(0, 0, opa0, opb0);
    read_ops(0, 1, opa1, opb1);
    for (int kb = 0; kb < KB; ++kb) {
        float f[2] = {0.0f, 0.0f};
        if (kb > 0) {
            f[0] = factor(kb - 1, 0);
            f[1] = factor(kb - 1, 1);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (!(s == 0 ? live0 : live1)) continue;
                if (kb > 0) promote(kb - 1, s, t, f[s]);
                v16f_t z;
#pragma unroll
                for (int i = 0; i < 16; ++i) z[i] = 0.0f;
                part[s][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opb0[t], opa0[s], z, 0, 0, 0, 127, 0, 127);
            }
        // keep the scheduler from moving the MFMAs and FMAs above past the
        // barrier: they are meant to run while the wave waits at it
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): this wave's LDS reads are done
        EP_WAIT_VMCNT(kDmaPerStage);              // this wave's loads of stage kb + 1 are done
        __syncthreads();                          // ... and every other wave's
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::"v"(&s_a[0][0]), "v"(&s_b[0][0]), "v"(&s_sa[0][0]) : "memory");
        issue(min(kb + 3, KB - 1));
        const int nxt = (kb + 1) % kStages;
        read_ops(nxt, 0, opa0, opb0);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (s == 0 ? live0 : live1)
                    part[s][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opb1[t], opa1[s], part[s][t], 0, 0, 0,
                                                                                127, 0, 127);
        read_ops(nxt, 1, opa1, opb1);
    }
    {
        const float f0 = factor(KB - 1, 0), f1 = factor(KB - 1, 1);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (live0) promote(KB - 1, 0, t, f0);
            if (live1) promote(KB - 1, 1, t, f1);
        }
    }
    EP_WAIT_VMCNT(0);

    // epilogue: bf16, round to nearest even; four adjacent columns per store
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = row0 + 64 * wm + 32 * s + r32;
                const int col = n0 + 64 * wn + 32 * t + 8 * q + 4 * g;
                const uint2 v = make_uint2(pack_bf16x2(acc[s][t][4 * q], acc[s][t][4 * q + 1]),
                                           pack_bf16x2(acc[s][t][4 * q + 2], acc[s][t][4 * q + 3]));
                *(uint2*)(a.c + (int64_t)row * a.N + col) = v;
            }
}

hipError_t launch_grouped_gemm_fp8(const GemmArgs& a, int64_t rows_bound, hipStream_t stream) {
    const bool wide = a.N % kBN2 == 0 && a.K / kTile <= kMaxGemmKBlocks / 2;
    const int nt_n = a.N / (wide ? kBN2 : kTile);
    int64_t blocks;
    if (a.mode == EP_MODE_COMPACT)
        blocks = (rows_bound + kTile - 1) / kTile * nt_n;
    else
        blocks = (int64_t)a.E * (a.C / kTile) * nt_n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (launch_debug())
        launch_debug_print(wide ? "k_grouped_gemm_fp8_dma" : "k_grouped_gemm_fp8", dim3((unsigned)blocks),
                           dim3(wide ? 512 : 256), "n %d hidden %d", a.N, a.K);
    if (wide)
        hipLaunchKernelGGL(k_grouped_gemm_fp8_dma, dim3((unsigned)blocks), dim3(512), 0, stream, a);
    else
        hipLaunchKernelGGL(k_grouped_gemm_fp8, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ep
