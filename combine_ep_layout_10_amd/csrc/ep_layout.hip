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
// Large layouts take two kernels (count per block -> assign, which reduces
// the per-block counts itself), or three (count -> one-block scan -> assign)
// when the matrix of per-block counts is too large to be re-read by every
// block; small ones (pairs <= 4096, E <= 512) take one single-block kernel.
#include "ep_internal.h"
#include "ep_layout_dev.h"

namespace ep {

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

// Column sums of the per-block counts, done inside every assign block when
// the partial matrix is small (nblk * E <= kInlineScanMaxCells): the count
// of expert e before this block (pre) and over all blocks (tot). tpe threads
// share one expert column (blocks q, q + tpe, ...); consecutive lanes hold
// consecutive experts, so each load instruction reads one contiguous row
// piece. Results land in s_pre[E] / s_tot[E] after the final barrier.
__device__ __forceinline__ void inline_column_sums(const LayoutArgs& a, int32_t* s_q, int32_t* s_pre,
                                                   int32_t* s_tot) {
    const int tid = threadIdx.x;
    const int me = (int)blockIdx.x;
    int pre = 0, tot = 0;
    if (tid < a.tpe * a.E) {
        const int e = tid % a.E, q = tid / a.E;
        int b = q;
        for (; b + 7 * a.tpe < a.nblk; b += 8 * a.tpe) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = a.bpart[(int64_t)(b + u * a.tpe) * a.E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                tot += v[u];
                pre += (b + u * a.tpe < me) ? v[u] : 0;
            }
        }
        for (; b < a.nblk; b += a.tpe) {
            const int v = a.bpart[(int64_t)b * a.E + e];
            tot += v;
            pre += b < me ? v : 0;
        }
        s_q[tid] = pre;
        s_q[1024 + tid] = tot;
    }
    __syncthreads();
    for (int e = tid; e < a.E; e += blockDim.x) {
        int p = 0, t = 0;
        for (int q = 0; q < a.tpe; ++q) {
            p += s_q[q * a.E + e];
            t += s_q[1024 + q * a.E + e];
        }
        s_pre[e] = p;
        s_tot[e] = t;
    }
    __syncthreads();
}

// Stable slots: rank inside the wave's group (ballots), plus the counts of
// the earlier waves of the block, plus the block's base inside the expert.
// INLINE: the block also derives counts, padded sizes and expert offsets
// from the per-block counts itself (block 0 publishes them, with the
// destination sums and the error word), so the layout needs no separate scan
// launch. Otherwise k_layout_scan has already turned the per-block counts
// into per-block bases and written the offsets.
template <bool INLINE>
__global__ __launch_bounds__(kLayoutWaves * 64) void k_layout_assign(LayoutArgs a) {
    extern __shared__ int32_t lds[];
    int32_t* bbase = lds;                              // [E] block base (+ expert offset)
    int32_t* s_off = bbase + a.E;                      // [E+1] expert offsets
    int32_t* s_cnt = s_off + a.E + 1;                  // [E] counts
    uint16_t* wc = (uint16_t*)(s_cnt + a.E);           // [kLayoutWaves][E] per-wave counts
    int32_t* s_q = (int32_t*)(wc + kLayoutWaves * a.E);  // INLINE: [2][1024] partial sums
    __shared__ int tmp[17];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    // The ids (and weights) of this block are loaded before anything waits.
    const int64_t base = ((int64_t)blockIdx.x * kLayoutWaves + w) * kWave;
    const int64_t p = base + lane;
    const bool live = p < (int64_t)a.T * a.k;
    bool v, bad;
    const int e = load_group(a, base, v, bad);
    const float wp = (a.w != nullptr && live) ? a.w[p] : 0.0f;
    if (INLINE) {
        // block 0 also sums the destination counts and error bits
        const bool lead = blockIdx.x == 0;
        const int ndp = a.nblk * a.D;
        const int dval = (lead && tid < ndp) ? a.dpart[tid] : 0;
        uint32_t f = (lead && tid < a.nblk) ? a.fpart[tid] : 0u;
        inline_column_sums(a, s_q, bbase, s_cnt);      // bbase = count before this block, s_cnt = totals
        int padv = 0;
        bool over = false;
        if (tid < a.E) {
            const int tot = s_cnt[tid];
            if (a.mode == EP_MODE_COMPACT) {
                padv = (tot + a.A - 1) / a.A * a.A;
            } else {
                padv = tot < a.C ? tot : a.C;
                over = tot > a.C;
            }
        }
        int sum_pad;
        const int excl = block_exclusive_scan(padv, tmp, &sum_pad);
        if (tid < a.E) {
            s_off[tid] = a.mode == EP_MODE_COMPACT ? excl : tid * a.C;
            if (a.mode == EP_MODE_COMPACT) bbase[tid] += excl;
        }
        if (tid == 0) s_off[a.E] = a.mode == EP_MODE_COMPACT ? sum_pad : a.E * a.C;
        if (lead) {
            if (tid < a.E) {
                a.cnt[tid] = s_cnt[tid];
                a.pad[tid] = padv;
            }
            for (int b = tid + blockDim.x; b < a.nblk; b += blockDim.x) f |= a.fpart[b];
            int32_t* s_dest = s_q;                     // the partial sums are consumed
            for (int d = tid; d < a.D; d += blockDim.x) s_dest[d] = 0;
            __syncthreads();
            if (tid < ndp) atomicAdd(&s_dest[tid % a.D], dval);
            for (int i = tid + blockDim.x; i < ndp; i += blockDim.x) atomicAdd(&s_dest[i % a.D], a.dpart[i]);
            __syncthreads();
            for (int d = tid; d < a.D; d += blockDim.x) a.dest_tokens[d] = s_dest[d];
            const uint32_t fo = (uint32_t)__syncthreads_or(f & EP_ERRFLAG_BAD_ID);
            const uint32_t fv = (uint32_t)__syncthreads_or(over);
            if (tid == 0) a.err_flags[0] = (fo ? EP_ERRFLAG_BAD_ID : 0u) | (fv ? EP_ERRFLAG_OVERFLOW : 0u);
            for (int i = tid; i <= a.E; i += blockDim.x) a.expert_off[i] = s_off[i];
            for (int d = tid; d <= a.D; d += blockDim.x) a.dest_off[d] = s_off[d * a.epd];
        }
    } else {
        for (int i = tid; i < a.E; i += blockDim.x) {
            const int off = a.expert_off[i];
            bbase[i] = a.bpart[(int64_t)blockIdx.x * a.E + i] + (a.mode == EP_MODE_COMPACT ? off : 0);
            s_off[i] = off;
            s_cnt[i] = a.cnt[i];
        }
        if (tid == 0) s_off[a.E] = a.expert_off[a.E];
    }
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

// The whole layout in one block (pairs <= 1024 * IT, E <= 512).
template <int IT>
__global__ __launch_bounds__(1024) void k_layout_small(LayoutArgs a) {
    extern __shared__ int32_t lds[];
    SmallLayout<IT> L;
    small_layout<IT>(a, lds, true, L);
    small_layout_publish<IT>(a, L);
}

// ---------------------------------------------------------------- launch

hipError_t launch_layout(const LayoutArgs& args, bool small, hipStream_t stream) {
    LayoutArgs a = args;
    if (small) {
        const int P = a.T * a.k;
        const size_t lds = small_layout_lds_bytes(a.E, a.D);
        if (launch_debug()) launch_debug_print("k_layout_small", dim3(1), dim3(1024), "pairs %d", P);
        if (P <= 1024)
            hipLaunchKernelGGL(k_layout_small<1>, dim3(1), dim3(1024), lds, stream, a);
        else
            hipLaunchKernelGGL(k_layout_small<4>, dim3(1), dim3(1024), lds, stream, a);
        return hipGetLastError();
    }
    const size_t lds_count = sizeof(int32_t) * (a.E + a.D);
    size_t lds_assign = sizeof(int32_t) * (3 * a.E + 1) + sizeof(uint16_t) * kLayoutWaves * a.E;
    const bool inline_scan = (int64_t)a.nblk * a.E <= kInlineScanMaxCells;
    if (inline_scan) lds_assign += sizeof(int32_t) * 2 * 1024;
    // threads per expert column: a power of two with tpe * E <= 1024 (the
    // one-block scan caches at most 16 partials per thread, so it stops there)
    a.tpe = 1;
    while ((inline_scan || a.tpe < 16) && (a.tpe * 2) * a.E <= 1024) a.tpe *= 2;
    if (launch_debug())
        launch_debug_print("k_layout_count+assign", dim3(a.nblk), dim3(kLayoutWaves * 64),
                           "pairs %lld scan %s threads/expert %d", (long long)a.T * a.k,
                           inline_scan ? "inline" : "one-block", a.tpe);
    hipLaunchKernelGGL(k_layout_count, dim3(a.nblk), dim3(kLayoutWaves * 64), lds_count, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (inline_scan) {
        hipLaunchKernelGGL(k_layout_assign<true>, dim3(a.nblk), dim3(kLayoutWaves * 64), lds_assign, stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_layout_scan, dim3(1), dim3(1024), 0, stream, a, a.tpe);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_layout_assign<false>, dim3(a.nblk), dim3(kLayoutWaves * 64), lds_assign, stream, a);
    return hipGetLastError();
}

}  // namespace ep
