// Single-launch layout + dispatch for small batches — the DeepEP README's
// dispatch_forward (layout and copy in one call) on the decode-sized inputs
// of "Example use in inference decoding", where launch latency, not memory
// traffic, sets the time.
//
// The layout has a grid-wide dependency (a token's row depends on the
// counts of every expert before it), so instead of waiting on other blocks
// every block derives what it needs from all the ids of the batch (pairs <=
// 4096, E <= 512: a few KiB read from L2 per block). Where a pair's row
// follows from counts alone (FIXED capacity: e*C + the earlier pairs of its
// expert; the aligned layout with alignment 1: the pairs of smaller experts
// + the earlier pairs of its expert), a token block counts just those for its
// own pairs; with larger alignments every block recomputes the whole layout
// in LDS. With larger alignments the first blocks copy one piece (seg
// vectors) of one token's row each, the last ones zero-fill padding rows,
// and block 0 also writes the handle's arrays. Where rows follow from
// counts, each token block writes its own pairs' slots and rows, and block 0
// copies nothing: it only writes the counts and offsets, so that work runs
// beside the copies instead of after block 0's piece of a row. A token
// block issues the loads of its piece of x before the layout work, so both
// round trips overlap. Small batches have few tokens, so rows are split over
// several blocks to reach every CU, but the grid is kept to one block per CU:
// a block left for a second round would double the time, and two blocks on
// one CU slow each other's layout work. No block waits on another, and the
// result equals ep_layout followed by ep_dispatch bit for bit (the same
// device code computes both).
#include "ep_internal.h"
#include "ep_layout_dev.h"
#include "ep_dispatch_dev.h"

namespace ep {

// Layouts whose rows follow from counts alone (FIXED capacity, and the
// aligned layout with alignment 1), block 0's share: pairs per expert,
// distinct tokens per destination and the error bits, from the ids every
// block has loaded (this wave's IT groups of 64 pairs starting at `base`);
// writes cnt, pad, expert_off, dest_off, dest_tokens and the error word.
// FIXED: pad = min(cnt, C), expert_off = e*C. Alignment 1: pad = cnt,
// expert_off = the exclusive scan of cnt. Every thread of the block must
// call it.
template <int IT>
__device__ __forceinline__ void rank_layout_publish_counts(const LayoutArgs& a, const int ids[IT], const bool val[IT],
                                                           bool bad, int64_t base, int32_t* lds) {
    __shared__ int tmp[17];
    const int tid = threadIdx.x;
    const bool fixed = a.mode == EP_MODE_FIXED;
    int32_t* hist = lds;                 // [E]
    int32_t* dh = lds + a.E;             // [D]
    int32_t* off = lds + a.E + a.D;      // [E+1]
    for (int i = tid; i < a.E + a.D; i += blockDim.x) lds[i] = 0;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        if (val[it]) atomicAdd(&hist[ids[it]], 1);
        const int dd = val[it] ? ids[it] / a.epd : -1;
        if (first_in_dest(a, base + it * kWave, dd, val[it])) atomicAdd(&dh[dd], 1);
    }
    const bool any_bad = __syncthreads_or(bad);
    bool over = false;
    for (int e = tid; e < a.E; e += blockDim.x) {
        const int n = hist[e];
        a.cnt[e] = n;
        a.pad[e] = fixed ? (n < a.C ? n : a.C) : n;
        over |= fixed && n > a.C;
    }
    if (fixed) {
        for (int e = tid; e <= a.E; e += blockDim.x) a.expert_off[e] = e * a.C;
        for (int d = tid; d <= a.D; d += blockDim.x) a.dest_off[d] = d * a.epd * a.C;
    } else {  // E <= 512 < blockDim: one expert per thread
        int total;
        const int excl = block_exclusive_scan(tid < a.E ? hist[tid] : 0, tmp, &total);
        if (tid < a.E) off[tid] = excl;
        if (tid == 0) off[a.E] = total;
        __syncthreads();
        for (int e = tid; e <= a.E; e += blockDim.x) a.expert_off[e] = off[e];
        for (int d = tid; d <= a.D; d += blockDim.x) a.dest_off[d] = off[d * a.epd];
    }
    for (int d = tid; d < a.D; d += blockDim.x) a.dest_tokens[d] = dh[d];
    const bool any_over = __syncthreads_or(over);
    if (tid == 0) a.err_flags[0] = (any_bad ? EP_ERRFLAG_BAD_ID : 0u) | (any_over ? EP_ERRFLAG_OVERFLOW : 0u);
}

// The rows of token t's k pairs in a layout whose rows follow from counts.
// Pair p = t*k + j of expert e has rank r = the number of valid pairs
// p' < p with expert e (the stable order). FIXED: row e*C + r, or nowhere
// when r >= C. Alignment 1: row b + r, b = the number of valid pairs with an
// expert below e (the exclusive scan of the counts at e). So a token block
// needs only these 2k counts, not the whole layout. Lane j < k of every wave
// loads pair j's expert id; per chunk of eight pairs, each wave counts the
// matches among its loaded ids with one ballot per pair and group (the
// expert id broadcast with readlane) and lane 0 stores the eight counts to
// LDS as two 16-byte writes. After one barrier every wave adds the 16
// waves' counts itself: lane l takes pair l mod 8 of waves l/8 and l/8 + 8,
// and three lane exchanges (xor 8, 16, 32) finish the sum, so lane j ends
// up with pair j's count in a register and no second barrier is needed.
// Part 0 of the token also writes the pairs' slot, row_src and row_w.
// Returns the row of pair `lane` in lanes lane < k (-1 elsewhere). Every
// thread of the block must call it (`tok` is block-uniform); the block has
// kLayoutWaves waves.
template <int IT>
__device__ __forceinline__ int rank_layout_token_slots(const LayoutArgs& a, const int ids[IT], const bool val[IT],
                                                       int64_t base, bool tok, int t, int part) {
    __shared__ __align__(16) int32_t s_wc[kLayoutWaves][kMaxTopk];
    __shared__ __align__(16) int32_t s_wb[kLayoutWaves][kMaxTopk];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool fixed = a.mode == EP_MODE_FIXED;
    const int64_t p0 = (int64_t)t * a.k;
    int my_e = -1;  // lane j < k: pair j's expert (-1 when skipped)
    if (tok && lane < a.k) {
        bool v = false, b = false;
        const int e = load_id(a, p0 + lane, v, b);
        my_e = v ? e : -1;
    }
    if (tok) {
        for (int j0 = 0; j0 < a.k; j0 += 8) {  // uniform
            int n[8], nb[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = j0 + u < a.k ? __builtin_amdgcn_readlane(my_e, j0 + u) : -1;
                n[u] = 0;
                nb[u] = 0;
                if (e >= 0) {
#pragma unroll
                    for (int it = 0; it < IT; ++it) {
                        const int64_t p = base + it * kWave + lane;
                        n[u] += __popcll(ballot64(val[it] && ids[it] == e && p < p0 + j0 + u));
                        if (!fixed) nb[u] += __popcll(ballot64(val[it] && ids[it] < e));
                    }
                }
            }
            if (lane == 0) {
                *(int4*)&s_wc[w][j0] = make_int4(n[0], n[1], n[2], n[3]);
                *(int4*)&s_wc[w][j0 + 4] = make_int4(n[4], n[5], n[6], n[7]);
                if (!fixed) {
                    *(int4*)&s_wb[w][j0] = make_int4(nb[0], nb[1], nb[2], nb[3]);
                    *(int4*)&s_wb[w][j0 + 4] = make_int4(nb[4], nb[5], nb[6], nb[7]);
                }
            }
        }
    }
    __syncthreads();
    int my_s = -1;
    if (tok) {
        const int u = lane & 7, ww = lane >> 3;
        for (int j0 = 0; j0 < a.k; j0 += 8) {  // uniform
            int r = s_wc[ww][j0 + u] + s_wc[ww + 8][j0 + u];
            int b = fixed ? 0 : s_wb[ww][j0 + u] + s_wb[ww + 8][j0 + u];
            r += __shfl_xor(r, 8, kWave);
            r += __shfl_xor(r, 16, kWave);
            r += __shfl_xor(r, 32, kWave);
            if (!fixed) {
                b += __shfl_xor(b, 8, kWave);
                b += __shfl_xor(b, 16, kWave);
                b += __shfl_xor(b, 32, kWave);
            }
            // lane j in [j0, j0 + 8) holds pair j's totals (j0 is a multiple of 8)
            if (lane >= j0 && lane < j0 + 8 && lane < a.k && my_e >= 0)
                my_s = fixed ? (r < a.C ? my_e * a.C + r : -1) : b + r;
        }
        if (part == 0 && w == 0 && lane < a.k) {
            a.slot[p0 + lane] = my_s;
            if (my_s >= 0) {
                a.row_src[my_s] = (int32_t)(p0 + lane);
                if (a.w) a.row_w[my_s] = a.w[p0 + lane];
            }
        }
    }
    return my_s;
}

template <int IT, int KIND>
__global__ __launch_bounds__(1024) void k_layout_dispatch_small(FusedArgs f) {
    const LayoutArgs la = fused_layout_args(f);
    const DispatchArgs da = fused_dispatch_args(f);
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_slot[kMaxTopk];
    // Rows that follow from counts: block 0 only publishes the counts and
    // offsets, the token-piece blocks follow it. Otherwise the token-piece
    // blocks come first (block 0 also publishes) and zero-fill blocks last.
    const bool by_rank = la.mode == EP_MODE_FIXED || la.A == 1;  // uniform across the grid
    const int ntok = da.T * da.nsplit;
    const int tb = (int)blockIdx.x - (by_rank ? 1 : 0);        // token-piece index
    const bool tok = tb >= 0 && tb < ntok;
    const int t = tok ? tb / da.nsplit : 0;
    const int part = tok ? tb % da.nsplit : 0;
    const int c = part * da.seg + (int)threadIdx.x;
    const int c_end = min((part + 1) * da.seg, dispatch_nvec<KIND>(da));
    const bool act = tok && (int)threadIdx.x < da.seg && c < c_end;
    const DispatchRaw raw = dispatch_load<KIND>(da, t, c, act);

    if (by_rank) {
        const int lane = threadIdx.x & 63;
        const int64_t P = (int64_t)la.T * la.k;
        const int64_t base = (int64_t)(threadIdx.x >> 6) * (IT * kWave);
        int ids[IT];
        bool val[IT];
        bool bad = false;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int64_t p = base + it * kWave + lane;
            bool v = false, b = false;
            ids[it] = p < P ? load_id(la, p, v, b) : 0;
            val[it] = v;
            bad |= b;
        }
        const int my_s = rank_layout_token_slots<IT>(la, ids, val, base, tok, t, part);
        if (blockIdx.x == 0) rank_layout_publish_counts<IT>(la, ids, val, bad, base, lds);  // not a token block
        if (!tok || (int)threadIdx.x >= ((da.seg + 63) & ~63)) return;
        const DispatchVec d = dispatch_encode<KIND>(raw);
        dispatch_store<KIND>(da, d, c, act, my_s, 0.0f);
        return;
    }

    SmallLayout<IT> L;
    const bool lead = blockIdx.x == 0;
    small_layout<IT>(la, lds, lead, L);
    if (lead) small_layout_publish<IT>(la, L);
    if (!tok) {
        if (lead && ntok == 0 && da.npad_blocks == 0) return;  // an empty batch: the handle only
        const int pb = tb - ntok;
        if (pb >= da.npad_blocks) return;
        const int e = pb / da.pad_pieces_per_expert;
        const int pp = pb % da.pad_pieces_per_expert;
        const int r0 = L.s_off[e] + L.s_cnt[e] + pp * da.pad_rows_per_piece;
        const int r1 = min(r0 + da.pad_rows_per_piece, L.s_off[e + 1]);
        dispatch_zero_rows<KIND>(da, r0, r1);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int64_t p0 = (int64_t)t * la.k;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t p = L.base + it * kWave + lane;
        if (p >= p0 && p < p0 + la.k) s_slot[p - p0] = small_layout_slot<IT>(la, L, it);
    }
    __syncthreads();
    if ((int)threadIdx.x >= ((da.seg + 63) & ~63)) return;  // whole waves past the piece
    const int my_s = lane < la.k ? s_slot[lane] : -1;
    const DispatchVec d = dispatch_encode<KIND>(raw);
    dispatch_store<KIND>(da, d, c, act, my_s, 0.0f);
}

template <int KIND>
static void launch_fused_kind(const FusedArgs& f, int grid, size_t lds, hipStream_t s) {
    if ((int64_t)f.T * f.k <= 1024)
        hipLaunchKernelGGL((k_layout_dispatch_small<1, KIND>), dim3(grid), dim3(1024), lds, s, f);
    else
        hipLaunchKernelGGL((k_layout_dispatch_small<4, KIND>), dim3(grid), dim3(1024), lds, s, f);
}

// The packed arguments; every pointer of the handle lies in one workspace
// (ep_layout's map), so each is a 32-bit offset from its base.
static FusedArgs pack_fused(const LayoutArgs& la, const DispatchArgs& da, char* ws) {
    FusedArgs f = {};
    f.idx = la.idx;
    f.w = la.w;
    f.ws = ws;
    f.x = da.x;
    f.x_scales = da.x_scales;
    f.recv = da.recv;
    f.recv_scales = da.recv_scales;
    auto off = [ws](const void* p) { return (uint32_t)((const char*)p - ws); };
    f.o_cnt = off(la.cnt);
    f.o_pad = off(la.pad);
    f.o_eoff = off(la.expert_off);
    f.o_doff = off(la.dest_off);
    f.o_dtok = off(la.dest_tokens);
    f.o_slot = off(la.slot);
    f.o_rsrc = off(la.row_src);
    f.o_rw = off(la.row_w);
    f.o_flags = off(la.err_flags);
    f.T = la.T;
    f.H = da.H;
    f.A = la.A;
    f.C = la.C;
    f.pad_pieces_per_expert = da.pad_pieces_per_expert;
    f.npad_blocks = da.npad_blocks;
    f.E = (int16_t)la.E;
    f.k = (int16_t)la.k;
    f.D = (int16_t)la.D;
    f.epd = (int16_t)la.epd;
    f.nbits = (int16_t)la.nbits;
    f.idx_bits = (int16_t)la.idx_bits;
    f.mode = (int16_t)la.mode;
    f.zero_pad = (int16_t)da.zero_pad;
    f.nsplit = (int16_t)da.nsplit;
    f.seg = (int16_t)da.seg;
    f.pad_rows_per_piece = (int16_t)da.pad_rows_per_piece;
    return f;
}

hipError_t fused_layout_dispatch_fits(const LayoutArgs& la, const DispatchArgs& da, bool* fits) {
    *fits = false;
    if ((int64_t)la.T * la.k > kSmallMaxPairs || la.E > kSmallMaxExperts) return hipSuccess;
    // Each zero-fill piece of the single launch takes a block that redoes
    // the small layout; once those blocks and one per token exceed the
    // resident blocks, the grid runs in rounds and the two launches (layout,
    // then the dispatch kernel's capped zero-fill loop) are faster.
    DispatchArgs d = da;
    set_pad_pieces(d, kFusedPadRowsPerPiece);
    if (d.npad_blocks > 0) {
        int cus = 0;
        const hipError_t e = device_cu_count(&cus);
        if (e != hipSuccess) return e;
        if ((int64_t)la.T + d.npad_blocks > (int64_t)kFusedBlocksPerCU * cus) return hipSuccess;
    }
    *fits = true;
    return hipSuccess;
}

hipError_t launch_layout_dispatch_small(int kind, const LayoutArgs& la, const DispatchArgs& args, char* ws,
                                        hipStream_t stream) {
    DispatchArgs da = args;
    set_pad_pieces(da, kFusedPadRowsPerPiece);
    const bool fp8 = kind == kDispatchFp8Quant || kind == kDispatchFp8Copy;
    const int nvec = fp8 ? da.H / 16 : da.H / 8;
    // Pieces per row: as many as keep the grid within kFusedBlocksPerCU
    // blocks per CU (padding blocks included), at least 64 vectors per
    // piece, at most 1024 (one vector per thread).
    int cus = 0;
    hipError_t err = device_cu_count(&cus);
    if (err != hipSuccess) return err;
    const int resident = kFusedBlocksPerCU * cus;
    // rows that follow from counts: one more block publishes the counts
    const int by_rank = la.mode == EP_MODE_FIXED || la.A == 1;
    int nsplit = da.T > 0 ? max(1, (resident - da.npad_blocks - by_rank) / da.T) : 1;
    nsplit = min(nsplit, (nvec + 63) / 64);
    nsplit = max(nsplit, (nvec + 1023) / 1024);
    nsplit = max(nsplit, 1);
    int seg = (nvec + nsplit - 1) / nsplit;
    seg = (seg + 7) & ~7;
    da.seg = seg;
    da.nsplit = (nvec + seg - 1) / seg;
    int grid = da.T * da.nsplit + da.npad_blocks + by_rank;
    if (grid == 0) grid = 1;  // the handle of an empty batch is still written
    const size_t lds = small_layout_lds_bytes(la.E, la.D);
    if (launch_debug())
        launch_debug_print("k_layout_dispatch_small", dim3(grid), dim3(1024),
                           "kind %d tokens %d pieces/row %d vectors/piece %d zero-fill blocks %d", kind, da.T,
                           da.nsplit, da.seg, da.npad_blocks);
    const FusedArgs f = pack_fused(la, da, ws);
    switch (kind) {
        case kDispatchBf16: launch_fused_kind<kDispatchBf16>(f, grid, lds, stream); break;
        case kDispatchFp8Quant: launch_fused_kind<kDispatchFp8Quant>(f, grid, lds, stream); break;
        case kDispatchFp8Copy: launch_fused_kind<kDispatchFp8Copy>(f, grid, lds, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ep
