// Layout kernels: per-expert counts, padded offsets and the stable slot of
// every (token, k) pair — the routing metadata the DeepEP README's
// dispatch_forward returns in its handle (per-expert received-token counts
// for GEMM, counts padded to expert_alignment; "Example use in model training
// or inference prefilling"), built for the receive rows of one GPU.
//
// Stable order: rows of one expert hold its pairs in ascending pair index
// p = t*k + j. Pairs are split into contiguous chunks: one chunk per wave,
// several waves per block. Inside a wave, 64 consecutive pairs are ranked
// with ballots (lanes holding the same expert id form a peer mask; a lane's
// rank is the number of peers below it) and a per-wave running count in LDS
// carries the order from one group of 64 to the next. Across waves and
// blocks, exclusive prefix sums of the per-chunk counts give the base of each
// chunk inside each expert. No atomics decide any position, so the result is
// deterministic and independent of scheduling.
//
// Large layouts take three kernels (count per block -> one-block scan ->
// assign); small ones (pairs <= 4096, E <= 512) take one single-block kernel.
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
// goes to dd. Earlier pairs in this group of 64 are read from their lanes;
// those in an earlier group are loaded.
__device__ __forceinline__ bool first_in_dest(const LayoutArgs& a, int64_t base, int dd, bool v) {
    const int lane = lane_id();
    const int64_t p = base + lane;
    const int j = (int)(p % a.k);
    bool first = v;
    for (int m = 1; m < a.k; ++m) {
        const int other = __shfl(dd, (lane - m) & (kWave - 1), kWave);
        if (m <= j && lane >= m && other == dd) first = false;
    }
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

// ---------------------------------------------------------------- multi-block
// A block is kLayoutWaves waves; each wave owns one group of 64 consecutive
// pairs, so a block covers kLayoutPairsPerBlock consecutive pairs.

// Per-block expert counts, distinct-token counts per destination, bad ids.
__global__ __launch_bounds__(kLayoutWaves * 64) void k_layout_count(LayoutArgs a) {
    extern __shared__ int32_t lds[];
    int32_t* hist = lds;          // [E]
    int32_t* dh = lds + a.E;      // [D]
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    for (int i = tid; i < a.E + a.D; i += blockDim.x) lds[i] = 0;
    const int64_t base = ((int64_t)blockIdx.x * kLayoutWaves + w) * kWave;
    bool v, bad;
    const int e = load_group(a, base, v, bad);
    const uint64_t peers = match_peers(e, v, a.nbits);
    const int dd = v ? e / a.epd : -1;
    const bool first = first_in_dest(a, base, dd, v);
    __syncthreads();
    if (v && (int)(__ffsll((long long)peers) - 1) == lane) atomicAdd(&hist[e], __popcll(peers));
    if (first) atomicAdd(&dh[dd], 1);
    bad = __syncthreads_or(bad);
    for (int i = tid; i < a.E; i += blockDim.x) a.bpart[(int64_t)blockIdx.x * a.E + i] = hist[i];
    for (int d = tid; d < a.D; d += blockDim.x) a.dpart[(int64_t)blockIdx.x * a.D + d] = dh[d];
    if (tid == 0) a.fpart[blockIdx.x] = bad ? EP_ERRFLAG_BAD_ID : 0u;
}

// Counts, pads, offsets and the base of every block inside every expert.
// One block of 1024 threads; E <= 1024. Each expert's prefix over the count
// blocks is split between tpe threads (contiguous block ranges), so the
// loads of one expert column are issued in parallel.
__global__ __launch_bounds__(1024) void k_layout_scan(LayoutArgs a, int tpe) {
    __shared__ int32_t s_off[1025];
    __shared__ int32_t s_part[1024];
    __shared__ int32_t s_dest[1024];
    __shared__ int tmp[17];
    const int tid = threadIdx.x;
    const int e = tid / tpe, q = tid % tpe;
    const bool col = e < a.E;
    const int per = (a.nblk + tpe - 1) / tpe;
    const int b0 = q * per, b1 = min(a.nblk, b0 + per);
    // Every global load is issued before the first barrier: one round trip.
    int cache[16];
    if (col) {
#pragma unroll
        for (int u = 0; u < 16; ++u) cache[u] = (b0 + u < b1) ? a.bpart[(int64_t)(b0 + u) * a.E + e] : 0;
    }
    uint32_t f = 0;
    for (int b = tid; b < a.nblk; b += 1024) f |= a.fpart[b];
    const int ndp = a.nblk * a.D;
    const int dval = tid < ndp ? a.dpart[tid] : 0;
    for (int d = tid; d < a.D; d += 1024) s_dest[d] = 0;
    __syncthreads();
    if (tid < ndp) atomicAdd(&s_dest[tid % a.D], dval);
    for (int i = tid + 1024; i < ndp; i += 1024) atomicAdd(&s_dest[i % a.D], a.dpart[i]);

    int sum = 0;
    if (col) {
#pragma unroll
        for (int u = 0; u < 16; ++u) sum += cache[u];
        for (int b = b0 + 16; b < b1; ++b) sum += a.bpart[(int64_t)b * a.E + e];
    }
    s_part[tid] = sum;
    __syncthreads();
    int pre = 0, total = 0;
    if (col) {
        for (int qq = 0; qq < tpe; ++qq) {
            const int v = s_part[e * tpe + qq];
            if (qq < q) pre += v;
            total += v;
        }
        int run = pre;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (b0 + u < b1) a.bpart[(int64_t)(b0 + u) * a.E + e] = run;
            run += cache[u];
        }
        for (int b = b0 + 16; b < b1; ++b) {
            const int v = a.bpart[(int64_t)b * a.E + e];
            a.bpart[(int64_t)b * a.E + e] = run;
            run += v;
        }
    }
    int padv = 0;
    if (col && q == 0) {
        a.cnt[e] = total;
        if (a.mode == EP_MODE_COMPACT) {
            padv = (total + a.A - 1) / a.A * a.A;
        } else {
            padv = total < a.C ? total : a.C;
            if (total > a.C) f |= EP_ERRFLAG_OVERFLOW;
        }
        a.pad[e] = padv;
    }
    int sum_pad;
    const int excl = block_exclusive_scan(padv, tmp, &sum_pad);  // q != 0 threads add 0
    if (col && q == 0) s_off[e] = a.mode == EP_MODE_COMPACT ? excl : e * a.C;
    if (tid == 0) s_off[a.E] = a.mode == EP_MODE_COMPACT ? sum_pad : a.E * a.C;
    __syncthreads();
    for (int i = tid; i <= a.E; i += 1024) a.expert_off[i] = s_off[i];
    for (int d = tid; d <= a.D; d += 1024) a.dest_off[d] = s_off[d * a.epd];
    for (int d = tid; d < a.D; d += 1024) a.dest_tokens[d] = s_dest[d];
    const uint32_t fo = (uint32_t)__syncthreads_or(f & EP_ERRFLAG_BAD_ID);
    const uint32_t fv = (uint32_t)__syncthreads_or(f & EP_ERRFLAG_OVERFLOW);
    if (tid == 0) a.err_flags[0] = (fo ? EP_ERRFLAG_BAD_ID : 0u) | (fv ? EP_ERRFLAG_OVERFLOW : 0u);
}

// Writes the slot of a pair whose rank inside its expert is r.
__device__ __forceinline__ void emit_slot(const LayoutArgs& a, int64_t p, int e, int r, int32_t off_e) {
    int32_t s;
    if (a.mode == EP_MODE_COMPACT) {
        s = off_e + r;
    } else {
        s = r < a.C ? e * a.C + r : -1;
    }
    a.slot[p] = s;
    if (s >= 0) {
        a.row_src[s] = (int32_t)p;
        if (a.w) a.row_w[s] = a.w[p];
    }
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

// Stable slots: rank inside the wave's group (ballots), plus the counts of
// the earlier waves of the block, plus the block's base inside the expert.
__global__ __launch_bounds__(kLayoutWaves * 64) void k_layout_assign(LayoutArgs a) {
    extern __shared__ int32_t lds[];
    int32_t* bbase = lds;                              // [E] block base (+ expert offset)
    int32_t* s_off = bbase + a.E;                      // [E+1] expert offsets
    int32_t* s_cnt = s_off + a.E + 1;                  // [E] counts
    uint16_t* wc = (uint16_t*)(s_cnt + a.E);           // [kLayoutWaves][E] per-wave counts
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    // Every global load is issued before the first barrier: one round trip.
    const int64_t base = ((int64_t)blockIdx.x * kLayoutWaves + w) * kWave;
    const int64_t p = base + lane;
    const bool live = p < (int64_t)a.T * a.k;
    bool v, bad;
    const int e = load_group(a, base, v, bad);
    const float wp = (a.w != nullptr && live) ? a.w[p] : 0.0f;
    for (int i = tid; i < a.E; i += blockDim.x) {
        const int off = a.expert_off[i];
        bbase[i] = a.bpart[(int64_t)blockIdx.x * a.E + i] + (a.mode == EP_MODE_COMPACT ? off : 0);
        s_off[i] = off;
        s_cnt[i] = a.cnt[i];
    }
    if (tid == 0) s_off[a.E] = a.expert_off[a.E];
    for (int i = tid; i < kLayoutWaves * a.E; i += blockDim.x) wc[i] = 0;
    const uint64_t peers = match_peers(e, v, a.nbits);
    const int rank = __popcll(peers & lanes_below(lane));
    __syncthreads();
    if (v && (int)(__ffsll((long long)peers) - 1) == lane) wc[w * a.E + e] = (uint16_t)__popcll(peers);
    __syncthreads();
    for (int i = tid; i < a.E; i += blockDim.x) {
        int run = 0;
#pragma unroll
        for (int ww = 0; ww < kLayoutWaves; ++ww) {
            const int c = wc[ww * a.E + i];
            wc[ww * a.E + i] = (uint16_t)run;
            run += c;
        }
    }
    __syncthreads();
    if (live) {
        if (!v) {
            a.slot[p] = -1;
        } else {
            const int r = bbase[e] + wc[w * a.E + e] + rank;   // COMPACT: row; FIXED: rank in expert
            int32_t s;
            if (a.mode == EP_MODE_COMPACT)
                s = r;
            else
                s = r < a.C ? e * a.C + r : -1;
            a.slot[p] = s;
            if (s >= 0) {
                a.row_src[s] = (int32_t)p;
                if (a.w) a.row_w[s] = wp;
            }
        }
    }
    emit_padding_meta(a, s_off, s_cnt, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------- one block

template <int IT>
__global__ __launch_bounds__(1024) void k_layout_small(LayoutArgs a) {
    constexpr int NW = 16;
    extern __shared__ int32_t lds[];
    int32_t* wcnt = lds;                      // [NW][E]
    int32_t* dh = wcnt + NW * a.E;            // [D]
    int32_t* s_off = dh + a.D;                // [E+1]
    int32_t* s_cnt = s_off + a.E + 1;         // [E]
    __shared__ int tmp[17];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    for (int i = tid; i < NW * a.E + a.D; i += 1024) lds[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)w * (IT * kWave);
    int ids[IT], rank[IT];
    bool val[IT];
    bool bad = wave_rank<IT, true>(a, base, ids, val, rank, wcnt + w * a.E, dh);
    bad = __syncthreads_or(bad);
    int padv = 0;
    bool over = false;
    if (tid < a.E) {
        const int e = tid;
        int run = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const int c = wcnt[ww * a.E + e];
            wcnt[ww * a.E + e] = run;
            run += c;
        }
        s_cnt[e] = run;
        a.cnt[e] = run;
        if (a.mode == EP_MODE_COMPACT) {
            padv = (run + a.A - 1) / a.A * a.A;
        } else {
            padv = run < a.C ? run : a.C;
            over = run > a.C;
        }
        a.pad[e] = padv;
    }
    over = __syncthreads_or(over);
    int total;
    const int excl = block_exclusive_scan(padv, tmp, &total);
    if (tid < a.E) s_off[tid] = a.mode == EP_MODE_COMPACT ? excl : tid * a.C;
    if (tid == 0) s_off[a.E] = a.mode == EP_MODE_COMPACT ? total : a.E * a.C;
    __syncthreads();
    for (int e = tid; e <= a.E; e += 1024) a.expert_off[e] = s_off[e];
    for (int d = tid; d <= a.D; d += 1024) a.dest_off[d] = s_off[d * a.epd];
    for (int d = tid; d < a.D; d += 1024) a.dest_tokens[d] = dh[d];
    if (tid == 0) a.err_flags[0] = (bad ? EP_ERRFLAG_BAD_ID : 0u) | (over ? EP_ERRFLAG_OVERFLOW : 0u);
    const int64_t P = (int64_t)a.T * a.k;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t p = base + it * kWave + lane;
        if (p >= P) continue;
        if (!val[it]) {
            a.slot[p] = -1;
            continue;
        }
        const int e = ids[it];
        emit_slot(a, p, e, wcnt[w * a.E + e] + rank[it], s_off[e]);
    }
    emit_padding_meta(a, s_off, s_cnt, 0, 1);
}

// ---------------------------------------------------------------- launch

hipError_t launch_layout(const LayoutArgs& a, bool small, hipStream_t stream) {
    if (small) {
        const int P = a.T * a.k;
        const size_t lds = sizeof(int32_t) * (16 * a.E + a.D + a.E + 1 + a.E);
        if (P <= 1024)
            hipLaunchKernelGGL(k_layout_small<1>, dim3(1), dim3(1024), lds, stream, a);
        else
            hipLaunchKernelGGL(k_layout_small<4>, dim3(1), dim3(1024), lds, stream, a);
        return hipGetLastError();
    }
    const size_t lds_count = sizeof(int32_t) * (a.E + a.D);
    const size_t lds_assign = sizeof(int32_t) * (3 * a.E + 1) + sizeof(uint16_t) * kLayoutWaves * a.E;
    hipLaunchKernelGGL(k_layout_count, dim3(a.nblk), dim3(kLayoutWaves * 64), lds_count, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    int tpe = 1;
    while (tpe < 16 && (tpe * 2) * a.E <= 1024) tpe *= 2;
    hipLaunchKernelGGL(k_layout_scan, dim3(1), dim3(1024), 0, stream, a, tpe);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_layout_assign, dim3(a.nblk), dim3(kLayoutWaves * 64), lds_assign, stream, a);
    return hipGetLastError();
}

}  // namespace ep
