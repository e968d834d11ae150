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
// in LDS. The first blocks copy one piece (seg vectors) of one token's row
// each; the last ones zero-fill padding rows; block 0 also writes the
// handle's arrays (where rows follow from counts, each token writes its own
// pairs' slots and rows and block 0 the counts and offsets). A token
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
// needs only these 2k counts, not the whole layout. Each wave counts, for
// every j, the matching pairs among its loaded ids with one ballot per group
// of 64 and count; the per-wave counts are summed in wave order. Part 0 of
// the token also writes the pairs' slot, row_src and row_w. The k rows land
// in s_slot. Every thread of the block must call it (`tok` is block-uniform).
template <int IT>
__device__ __forceinline__ void rank_layout_token_slots(const LayoutArgs& a, const int ids[IT], const bool val[IT],
                                                        int64_t base, bool tok, int t, int part, int32_t* s_slot) {
    __shared__ int32_t s_e[kMaxTopk];
    __shared__ int32_t s_wc[kLayoutWaves][kMaxTopk];
    __shared__ int32_t s_wb[kLayoutWaves][kMaxTopk];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool fixed = a.mode == EP_MODE_FIXED;
    const int64_t p0 = (int64_t)t * a.k;
    if (tok) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int64_t p = base + it * kWave + lane;
            if (p >= p0 && p < p0 + a.k) s_e[p - p0] = val[it] ? ids[it] : -1;
        }
    }
    __syncthreads();
    if (tok) {
        for (int j = 0; j < a.k; ++j) {
            const int e = s_e[j];  // the same in every lane: a uniform branch
            int n = 0, nb = 0;
            if (e >= 0) {
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int64_t p = base + it * kWave + lane;
                    n += __popcll(ballot64(val[it] && ids[it] == e && p < p0 + j));
                    if (!fixed) nb += __popcll(ballot64(val[it] && ids[it] < e));
                }
            }
            if (lane == 0) {
                s_wc[w][j] = n;
                if (!fixed) s_wb[w][j] = nb;
            }
        }
    }
    __syncthreads();
    if (tok && tid < a.k) {
        const int e = s_e[tid];
        int r = 0, b = 0;
        for (int ww = 0; ww < kLayoutWaves; ++ww) r += s_wc[ww][tid];
        if (!fixed)
            for (int ww = 0; ww < kLayoutWaves; ++ww) b += s_wb[ww][tid];
        int32_t s = -1;
        if (e >= 0) s = fixed ? (r < a.C ? e * a.C + r : -1) : b + r;
        s_slot[tid] = s;
        if (part == 0) {
            a.slot[p0 + tid] = s;
            if (s >= 0) {
                a.row_src[s] = (int32_t)(p0 + tid);
                if (a.w) a.row_w[s] = a.w[p0 + tid];
            }
        }
    }
}

template <int IT, int KIND>
__global__ __launch_bounds__(1024) void k_layout_dispatch_small(LayoutArgs la, DispatchArgs da) {
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_slot[kMaxTopk];
    const int ntok = da.T * da.nsplit;                  // token-piece blocks come first
    const bool tok = (int)blockIdx.x < ntok;
    const int t = tok ? (int)blockIdx.x / da.nsplit : 0;
    const int part = tok ? (int)blockIdx.x % da.nsplit : 0;
    const int c = part * da.seg + (int)threadIdx.x;
    const int c_end = min((part + 1) * da.seg, dispatch_nvec<KIND>(da));
    const bool act = tok && (int)threadIdx.x < da.seg && c < c_end;
    const DispatchRaw raw = dispatch_load<KIND>(da, t, c, act);

    if (la.mode == EP_MODE_FIXED || la.A == 1) {  // rows follow from counts; uniform across the grid
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
        rank_layout_token_slots<IT>(la, ids, val, base, tok, t, part, s_slot);
        if (blockIdx.x == 0) rank_layout_publish_counts<IT>(la, ids, val, bad, base, lds);
        __syncthreads();
        if (!tok || (int)threadIdx.x >= ((da.seg + 63) & ~63)) return;
        const int my_s = lane < la.k ? s_slot[lane] : -1;
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
        const int pb = (int)blockIdx.x - ntok;
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
static void launch_fused_kind(const LayoutArgs& la, const DispatchArgs& da, int grid, size_t lds, hipStream_t s) {
    if ((int64_t)la.T * la.k <= 1024)
        hipLaunchKernelGGL((k_layout_dispatch_small<1, KIND>), dim3(grid), dim3(1024), lds, s, la, da);
    else
        hipLaunchKernelGGL((k_layout_dispatch_small<4, KIND>), dim3(grid), dim3(1024), lds, s, la, da);
}

bool fused_layout_dispatch_fits(int64_t pairs, int E) { return pairs <= kSmallMaxPairs && E <= kSmallMaxExperts; }

hipError_t launch_layout_dispatch_small(int kind, const LayoutArgs& la, const DispatchArgs& args,
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
    int nsplit = da.T > 0 ? max(1, (resident - da.npad_blocks) / da.T) : 1;
    nsplit = min(nsplit, (nvec + 63) / 64);
    nsplit = max(nsplit, (nvec + 1023) / 1024);
    nsplit = max(nsplit, 1);
    int seg = (nvec + nsplit - 1) / nsplit;
    seg = (seg + 7) & ~7;
    da.seg = seg;
    da.nsplit = (nvec + seg - 1) / seg;
    int grid = da.T * da.nsplit + da.npad_blocks;
    if (grid == 0) grid = 1;  // the handle of an empty batch is still written
    const size_t lds = small_layout_lds_bytes(la.E, la.D);
    if (launch_debug())
        launch_debug_print("k_layout_dispatch_small", dim3(grid), dim3(1024),
                           "kind %d tokens %d pieces/row %d vectors/piece %d zero-fill blocks %d", kind, da.T,
                           da.nsplit, da.seg, da.npad_blocks);
    switch (kind) {
        case kDispatchBf16: launch_fused_kind<kDispatchBf16>(la, da, grid, lds, stream); break;
        case kDispatchFp8Quant: launch_fused_kind<kDispatchFp8Quant>(la, da, grid, lds, stream); break;
        case kDispatchFp8Copy: launch_fused_kind<kDispatchFp8Copy>(la, da, grid, lds, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ep
