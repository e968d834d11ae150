// Kernel argument blocks and launch entry points of the HIP library (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ep.h"
#include "ep_device.h"

namespace ep {

// Multi-block layout: waves per block, one group of 64 pairs per wave.
constexpr int kLayoutWaves = 16;
constexpr int kLayoutPairsPerBlock = kLayoutWaves * kWave;  // 1024
// Single-block layout limits.
constexpr int kSmallMaxPairs = 4096;
constexpr int kSmallMaxExperts = 512;
// Largest per-block count matrix (blocks x experts) that every assign block
// reduces on its own instead of waiting for a one-block scan launch.
constexpr int kInlineScanMaxCells = 32768;
// Limits checked by the host API.
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 32;

struct LayoutArgs {
    const void* idx;
    const float* w;
    int idx_bits;
    int T, E, k, A, D, C, mode;
    int nbits;  // bits needed to hold any expert id
    int epd;    // experts per destination
    int nblk;   // multi-block grid size
    int tpe;    // threads per expert column when reducing per-block counts
    int32_t* cnt;
    int32_t* pad;
    int32_t* expert_off;
    int32_t* dest_off;
    int32_t* dest_tokens;
    int32_t* slot;
    int32_t* row_src;
    float* row_w;
    uint32_t* err_flags;
    int32_t* bpart;   // [nblk][E] per-block counts, then per-block bases
    int32_t* dpart;   // [nblk][D] per-block distinct-token counts
    uint32_t* fpart;  // [nblk] per-block error bits
};

// kDispatchFp8QuantWeighted: combine_backward of a weighted combine with FP8
// output, each pair's copy bf16(w * x) quantised with its own 1x128 scales.
enum DispatchKind {
    kDispatchBf16 = 0,
    kDispatchBf16Weighted = 1,
    kDispatchFp8Quant = 2,
    kDispatchFp8Copy = 3,
    kDispatchFp8QuantWeighted = 4
};

struct DispatchArgs {
    const void* x;
    const float* x_scales;
    void* recv;
    float* recv_scales;
    const int32_t* slot;
    const float* pair_w;
    const int32_t* cnt;
    const int32_t* pad;
    const int32_t* expert_off;
    int T, H, k, E;
    int zero_pad;
    int pad_rows_max;        // most padding rows one expert can have (A - 1; 0 without zero-fill)
    int pad_rows_per_piece;     // padding rows of one zero-fill piece (of one expert's padding)
    int pad_pieces_per_expert;  // pieces per expert
    int npad_pieces;            // pad_pieces_per_expert * E
    int npad_blocks;            // blocks that clear them (piece i by block i % npad_blocks)
    // single-launch layout + dispatch only: each token's row is split into
    // nsplit blocks of seg vectors (seg <= 1024, a multiple of 8)
    int nsplit, seg;
};

struct CombineArgs {
    const uint16_t* y;
    const float* w;
    uint16_t* out;
    const int32_t* slot;
    const float* row_vals;
    float* out_vals;
    int T, H, k;
    int nsplit, seg;  // each token's row is split into nsplit blocks of seg vectors
};

// Combine splits the rows of batches smaller than this many tokens per CU so
// that about this many blocks per CU gather.
constexpr int kSplitBlocksPerCU = 2;
// Vectors per block piece of the combine for batches of at least
// kSplitBlocksPerCU tokens per CU.
constexpr int kCombineSegLarge = 128;
// Blocks of the single-launch layout + dispatch per CU. Every block redoes
// the small layout, so a second block on a CU competes with the first for
// its SIMDs (measured on MI355X at 128 x 7168 x top-8: one block per CU,
// two pieces per row, beats two blocks per CU by about 4 us).
constexpr int kFusedBlocksPerCU = 1;
// Compute units the launchers size grids for: the current device's count
// (queried once per device; the cache is atomic, so concurrent first calls
// are safe), or EP_LAUNCH_CUS when the environment sets it to 1..4096.
// Returns the failed query's error instead of guessing a count.
hipError_t device_cu_count(int* out);
// EP_BUFFER_DEBUG=1: launchers print the geometry they pick to stderr.
bool launch_debug();
void launch_debug_print(const char* kernel, dim3 grid, dim3 block, const char* fmt, ...);

struct WeightGradArgs {
    const uint16_t* grad_out;
    const uint16_t* y;
    const int32_t* slot;
    float* grad_w;
    int T, H, k;
};

struct GemmArgs {
    const uint8_t* a;
    const float* sa;
    const uint8_t* b;
    const float* sb;
    uint16_t* c;
    const int32_t* expert_off;
    const int32_t* pad;
    const int32_t* cnt;
    int E, K, N, mode, C;
};

// Padding rows per zero-fill piece (a piece of one expert's padding): in the
// dispatch kernel, and in the single-launch layout + dispatch, where every
// block also redoes the small layout and so should be few. In the dispatch
// kernel at most kPadBlocksPerCU blocks per CU clear the pieces, each looping
// over its share, so that pieces past an expert's padding cost a few loads
// instead of a launched block. Measured on MI355X at 8192 x 7168 x top-8,
// alignment 128 (zero-fill blocks first in the grid), weighted BF16 kind:
// one block per 16-row piece 225-228 us; per 4-row piece 218-223 us; 2-row
// pieces over 2,048 blocks 217.7-218.1 us (three runs in alternation).
constexpr int kPadRowsPerPiece = 2;
constexpr int kPadBlocksPerCU = 8;
constexpr int kFusedPadRowsPerPiece = 16;

// Sets the zero-fill work of a dispatch: pad_pieces_per_expert pieces of
// rows_per_piece rows for each expert (pieces past an expert's padding clear
// nothing), one block per piece (launchers may cap npad_blocks).
inline void set_pad_pieces(DispatchArgs& a, int rows_per_piece) {
    a.pad_rows_per_piece = rows_per_piece;
    a.pad_pieces_per_expert = (a.pad_rows_max + rows_per_piece - 1) / rows_per_piece;
    a.npad_pieces = a.pad_pieces_per_expert * a.E;
    a.npad_blocks = a.npad_pieces;
    if (a.pad_pieces_per_expert == 0) a.pad_pieces_per_expert = 1;  // never divided by when there are no pieces
}

hipError_t launch_layout(const LayoutArgs& a, bool small, hipStream_t stream);
hipError_t launch_dispatch(int kind, const DispatchArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_weight_grad(const WeightGradArgs& a, hipStream_t stream);
hipError_t launch_grouped_gemm_fp8(const GemmArgs& a, int64_t rows_bound, hipStream_t stream);
// Kernel arguments of the single-launch layout + dispatch, packed into the
// fields that kernel reads: the handle's arrays as 32-bit offsets from the
// workspace base, small sizes as 16-bit fields. A launch costs the host
// about 3 ns per byte of kernel arguments on this part (measured: 3.84 us
// for 320 bytes, 2.96 us for 12), and this launch sits on the decode path.
struct FusedArgs {
    const void* idx;
    const float* w;
    char* ws;  // the handle's arrays live at ws + o_*
    const void* x;
    const float* x_scales;
    void* recv;
    float* recv_scales;
    uint32_t o_cnt, o_pad, o_eoff, o_doff, o_dtok, o_slot, o_rsrc, o_rw, o_flags;
    int32_t T, H, A, C, pad_pieces_per_expert, npad_blocks;
    int16_t E, k, D, epd, nbits, idx_bits, mode, zero_pad, nsplit, seg, pad_rows_per_piece;
};

__host__ __device__ inline LayoutArgs fused_layout_args(const FusedArgs& f) {
    LayoutArgs a = {};
    a.idx = f.idx;
    a.w = f.w;
    a.idx_bits = f.idx_bits;
    a.T = f.T;
    a.E = f.E;
    a.k = f.k;
    a.A = f.A;
    a.D = f.D;
    a.C = f.C;
    a.mode = f.mode;
    a.nbits = f.nbits;
    a.epd = f.epd;
    a.cnt = (int32_t*)(f.ws + f.o_cnt);
    a.pad = (int32_t*)(f.ws + f.o_pad);
    a.expert_off = (int32_t*)(f.ws + f.o_eoff);
    a.dest_off = (int32_t*)(f.ws + f.o_doff);
    a.dest_tokens = (int32_t*)(f.ws + f.o_dtok);
    a.slot = (int32_t*)(f.ws + f.o_slot);
    a.row_src = (int32_t*)(f.ws + f.o_rsrc);
    a.row_w = (float*)(f.ws + f.o_rw);
    a.err_flags = (uint32_t*)(f.ws + f.o_flags);
    return a;
}

__host__ __device__ inline DispatchArgs fused_dispatch_args(const FusedArgs& f) {
    DispatchArgs d = {};
    d.x = f.x;
    d.x_scales = f.x_scales;
    d.recv = f.recv;
    d.recv_scales = f.recv_scales;
    d.slot = (const int32_t*)(f.ws + f.o_slot);
    d.cnt = (const int32_t*)(f.ws + f.o_cnt);
    d.pad = (const int32_t*)(f.ws + f.o_pad);
    d.expert_off = (const int32_t*)(f.ws + f.o_eoff);
    d.T = f.T;
    d.H = f.H;
    d.k = f.k;
    d.E = f.E;
    d.zero_pad = f.zero_pad;
    d.pad_rows_per_piece = f.pad_rows_per_piece;
    d.pad_pieces_per_expert = f.pad_pieces_per_expert;
    d.npad_blocks = f.npad_blocks;
    d.nsplit = f.nsplit;
    d.seg = f.seg;
    return d;
}

// Single-launch layout + dispatch (unweighted kinds) for small batches.
// Whether ep_dispatch_forward takes the single launch: pairs <= 4096,
// E <= 512, and its zero-fill blocks plus one block per token fit the
// resident blocks.
hipError_t fused_layout_dispatch_fits(const LayoutArgs& la, const DispatchArgs& da, bool* fits);
// ws: the workspace base that every handle array of `la` lies in.
hipError_t launch_layout_dispatch_small(int kind, const LayoutArgs& la, const DispatchArgs& da, char* ws,
                                        hipStream_t stream);

}  // namespace ep
