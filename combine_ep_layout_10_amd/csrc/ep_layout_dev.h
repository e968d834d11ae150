// Device code of the layout shared by the layout kernels and the fused
// single-launch layout + dispatch (internal).
//
// Pair p = t*k + j holds expert id topk_idx[p]. A wave ranks 64 consecutive
// pairs at once: lanes holding the same expert form a peer mask (ballots
// over the id bits), and a pair's rank among them is the number of peers in
// lower lanes. Counts carried from group to group and from wave to wave in
// LDS extend the rank to any chunk of consecutive pairs, which gives every
// pair its stable position inside its expert (ascending p).
#pragma once

#include "ep_internal.h"

namespace ep {

__device__ __forceinline__ int load_id(const LayoutArgs& a, int64_t p, bool& valid, bool& bad) {
    long long v = a.idx_bits == 64 ? ((const long long*)a.idx)[p] : (long long)((const int*)a.idx)[p];
    valid = v >= 0 && v < a.E;
    bad = !valid && v != -1;
    return valid ? (int)v : 0;
}

// Loads the id of this lane's pair in the group at `base`.
__device__ __forceinline__ int load_group(const LayoutArgs& a, int64_t base, bool& v, bool& bad) {
    const int64_t p = base + lane_id();
    v = false;
    bad = false;
    return p < (int64_t)a.T * a.k ? load_id(a, p, v, bad) : 0;
}

// Pair (t, j) is counted for destination dd when no earlier pair of token t
// goes to dd. Earlier pairs in this group of 64 are the lanes below this one
// that hold the same token: a peer mask over the bits of dd (ballots, as for
// the expert ids) restricted to them; pairs in an earlier group are loaded.
__device__ __forceinline__ bool first_in_dest(const LayoutArgs& a, int64_t base, int dd, bool v) {
    const int lane = lane_id();
    const int64_t p = base + lane;
    const int j = (int)(p % a.k);
    const int dbits = a.D > 1 ? 32 - __clz(a.D - 1) : 0;
    const uint64_t same = match_peers(dd, v, dbits);
    const int below = j < lane ? j : lane;  // same-token lanes below this one in the group
    const uint64_t tok_below = lanes_below(lane) & ~lanes_below(lane - below);
    bool first = v && (same & tok_below) == 0;
    if (v && j > lane) {
        for (int jj = 0; jj < j - lane; ++jj) {
            bool v2, b2;
            const int e2 = load_id(a, p - j + jj, v2, b2);
            if (v2 && e2 / a.epd == dd) first = false;
        }
    }
    return first;
}

// One wave ranks its chunk [base, base + IT*64) in order. On return:
//   ids/val hold each lane's expert per group; rank[it] = rank of the pair
//   inside this wave's chunk among pairs of the same expert;
//   wcnt[e] (this wave's LDS row) = pairs of expert e in the chunk.
// Also counts first-in-destination pairs into dh (LDS) and reports bad ids.
template <int IT, bool DEST>
__device__ __forceinline__ bool wave_rank(const LayoutArgs& a, int64_t base, int ids[IT], bool val[IT],
                                          int rank[IT], int32_t* wcnt, int32_t* dh) {
    const int lane = lane_id();
    const int64_t P = (int64_t)a.T * a.k;
    bool bad_any = false;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t p = base + it * kWave + lane;
        bool v = false, b = false;
        ids[it] = p < P ? load_id(a, p, v, b) : 0;
        val[it] = v;
        bad_any |= b;
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int e = ids[it];
        const bool v = val[it];
        const uint64_t peers = match_peers(e, v, a.nbits);
        int pre = 0;
        if (v) pre = wcnt[e];
        rank[it] = pre + __popcll(peers & lanes_below(lane));
        if (v && (int)(__ffsll((long long)peers) - 1) == lane) wcnt[e] = pre + __popcll(peers);
        if (DEST) {
            const int dd = v ? e / a.epd : -1;
            if (first_in_dest(a, base + it * kWave, dd, v)) atomicAdd(&dh[dd], 1);
        }
    }
    return bad_any;
}

// Padding rows of the experts e = first, first + step, ...: row_src = -1,
// row_w = 0 (COMPACT only).
__device__ __forceinline__ void emit_padding_meta(const LayoutArgs& a, const int32_t* off, const int32_t* cnt,
                                                  int first, int step) {
    if (a.mode != EP_MODE_COMPACT) return;
    for (int e = first; e < a.E; e += step) {
        const int r0 = off[e] + cnt[e], r1 = off[e + 1];
        for (int r = r0 + threadIdx.x; r < r1; r += blockDim.x) {
            a.row_src[r] = -1;
            if (a.w) a.row_w[r] = 0.0f;
        }
    }
}

// Result of small_layout: per-lane ids and ranks of the block's pairs plus
// the LDS arrays of the layout (valid after small_layout returns).
//   wcnt[16][E]  base of each wave inside each expert (prefix over waves)
//   dh[D]        distinct tokens per destination (only when asked for)
//   s_off[E+1]   expert offsets (COMPACT: scan of padded counts; FIXED: e*C)
//   s_cnt[E]     pairs per expert
// padv is the padded count of expert tid (threads tid < E), bad / over the
// error conditions of the whole layout (block-uniform).
template <int IT>
struct SmallLayout {
    int ids[IT], rank[IT];
    bool val[IT];
    int32_t *wcnt, *dh, *s_off, *s_cnt;
    int padv;
    bool bad, over;
    int64_t base;  // first pair of this wave's chunk
};

// LDS bytes small_layout needs.
__host__ __device__ inline size_t small_layout_lds_bytes(int E, int D) {
    return sizeof(int32_t) * (16 * (size_t)E + D + E + 1 + E);
}

// The whole layout of P <= 1024 * IT pairs (E <= 512) inside one block of
// 1024 threads, with no global writes: wave w ranks the chunk of IT groups
// starting at pair w * IT * 64. `dest` asks for the distinct-token counts
// per destination (they need extra loads). Every thread must call it.
template <int IT>
__device__ __forceinline__ void small_layout(const LayoutArgs& a, int32_t* lds, bool dest, SmallLayout<IT>& L) {
    constexpr int NW = 16;
    __shared__ int tmp[17];
    L.wcnt = lds;                       // [NW][E]
    L.dh = L.wcnt + NW * a.E;           // [D]
    L.s_off = L.dh + a.D;               // [E+1]
    L.s_cnt = L.s_off + a.E + 1;        // [E]
    const int tid = threadIdx.x, w = tid >> 6;
    for (int i = tid; i < NW * a.E + a.D; i += 1024) lds[i] = 0;
    __syncthreads();
    L.base = (int64_t)w * (IT * kWave);
    bool bad = dest ? wave_rank<IT, true>(a, L.base, L.ids, L.val, L.rank, L.wcnt + w * a.E, L.dh)
                    : wave_rank<IT, false>(a, L.base, L.ids, L.val, L.rank, L.wcnt + w * a.E, L.dh);
    L.bad = __syncthreads_or(bad);
    int padv = 0;
    bool over = false;
    if (tid < a.E) {
        const int e = tid;
        int run = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const int c = L.wcnt[ww * a.E + e];
            L.wcnt[ww * a.E + e] = run;
            run += c;
        }
        L.s_cnt[e] = run;
        if (a.mode == EP_MODE_COMPACT) {
            padv = (run + a.A - 1) / a.A * a.A;
        } else {
            padv = run < a.C ? run : a.C;
            over = run > a.C;
        }
    }
    L.over = __syncthreads_or(over);
    L.padv = padv;
    if (a.mode == EP_MODE_COMPACT) {  // uniform: the scan's barriers are reached by all or none
        int total;
        const int excl = block_exclusive_scan(padv, tmp, &total);
        if (tid < a.E) L.s_off[tid] = excl;
        if (tid == 0) L.s_off[a.E] = total;
    } else if (tid <= a.E) {
        L.s_off[tid] = tid * a.C;  // FIXED: expert e owns [e*C, e*C + C) whatever the counts
    }
    __syncthreads();
}

// Receive row of this lane's pair in group `it` (-1 when skipped).
template <int IT>
__device__ __forceinline__ int32_t small_layout_slot(const LayoutArgs& a, const SmallLayout<IT>& L, int it) {
    if (!L.val[it]) return -1;
    const int w = threadIdx.x >> 6;
    const int e = L.ids[it];
    const int r = L.wcnt[w * a.E + e] + L.rank[it];
    if (a.mode == EP_MODE_COMPACT) return L.s_off[e] + r;
    return r < a.C ? e * a.C + r : -1;
}

// Writes the handle's arrays from a finished small_layout (one block).
template <int IT>
__device__ __forceinline__ void small_layout_publish(const LayoutArgs& a, const SmallLayout<IT>& L) {
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < a.E) {
        a.cnt[tid] = L.s_cnt[tid];
        a.pad[tid] = L.padv;
    }
    for (int e = tid; e <= a.E; e += 1024) a.expert_off[e] = L.s_off[e];
    for (int d = tid; d <= a.D; d += 1024) a.dest_off[d] = L.s_off[d * a.epd];
    for (int d = tid; d < a.D; d += 1024) a.dest_tokens[d] = L.dh[d];
    if (tid == 0) a.err_flags[0] = (L.bad ? EP_ERRFLAG_BAD_ID : 0u) | (L.over ? EP_ERRFLAG_OVERFLOW : 0u);
    const int64_t P = (int64_t)a.T * a.k;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t p = L.base + it * kWave + lane;
        if (p >= P) continue;
        const int32_t s = small_layout_slot<IT>(a, L, it);
        a.slot[p] = s;
        if (s >= 0) {
            a.row_src[s] = (int32_t)p;
            if (a.w) a.row_w[s] = a.w[p];
        }
    }
    emit_padding_meta(a, L.s_off, L.s_cnt, 0, 1);
}

}  // namespace ep
