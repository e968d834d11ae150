/*
 * CPU oracle for MoE dispatch / combine on one GPU's share of the work.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, single-threaded
 * definition that the GPU library is checked against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never does. It shares no source, header, table or helper with
 * the GPU library.
 *
 * What is computed, and where the pages say so:
 *   - The problem: DeepEP README (community translation), opening paragraph
 *     and section "Interfaces and examples": dispatch routes each token to the
 *     experts of its top-k choice, combine reduces the expert outputs back.
 *   - Per-expert counts meant for the expert GEMM and the expert_alignment argument:
 *     same README, "Example use in model training or inference prefilling"
 *     (dispatch_forward: handle.num_recv_tokens_per_expert_list,
 *     expert_alignment). The README's "New features" list names the new GEMM
 *     layout of EPv2.
 *   - FP8 dispatch with x given as (data, scale_factors): same section,
 *     dispatch_forward docstring; the "Performance" section fixes FP8 dispatch
 *     and BF16 combine for the 8K x 7168 x top-8 setting.
 *   - Backward duals: dispatch_backward is a combine that also returns the
 *     combined weight gradients, combine_backward is a dispatch on the handle
 *     (same section, dispatch_backward / combine_backward); the weighted
 *     combine's gradient with respect to its weights is one dot product per
 *     (token, k) pair.
 *   - A fixed per-expert receive capacity for decode: "Example use in
 *     inference decoding" (num_max_tokens_per_rank, cached handle).
 * The pages give no kernel internals, rounding rules or FP8 recipe. Where
 * they are silent this file takes one plain reading, stated at each function:
 * stable slot order by (token, k) index, padding rows zero-filled,
 * scale = amax / 448 with both divisions IEEE binary32 round-to-nearest-even,
 * OCP E4M3FN with saturation to +-448, combine accumulating in binary32 with
 * fused multiply-add in k order from +0, then bfloat16 round-to-nearest-even.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC -lm
 * (no -march flags: no vector or fused code that would alter rounding).
 * The per-token loops carry OpenMP work-sharing pragmas, used only by a
 * second build of this same file (-fopenmp) that times the oracle on several
 * host cores. Tokens are independent, every (token, k) pair writes its own
 * receive row, and nothing inside a token's computation changes order, so
 * both builds give the same bits; the plain build ignores the pragmas.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_MODE_COMPACT 0
#define ORA_MODE_FIXED 1

#define ORA_FLAG_BAD_ID 1u
#define ORA_FLAG_OVERFLOW 2u

/* ---------------------------------------------------------------------- */
/* Number formats                                                          */
/* ---------------------------------------------------------------------- */

/* bfloat16 -> binary32 is exact: the 16 bits are the upper half of a float. */
static float ora_bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even mantissa.
 * bfloat16 keeps the upper 16 bits of the binary32 pattern. For finite
 * inputs the magnitude is monotone in the low 31 bits, so the nearest
 * bfloat16 is the truncation or the next pattern up; the discarded half
 * decides, and an exact half goes to the pattern with an even last bit.
 * A carry out of the mantissa steps the exponent, which is the correct
 * next value (up to infinity for the largest finite inputs). */
uint16_t ora_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t hi = (uint16_t)(u >> 16);
    uint32_t lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi = (uint16_t)(hi + 1u);
    return hi;
}

/* Value of a non-negative OCP E4M3FN code 0x00..0x7E (bias 7, three
 * mantissa bits; exponent field 0 holds the subnormals m * 2^-9; 0x7F is NaN
 * and there is no infinity, so 0x7E = 1.75 * 2^8 = 448 is the largest). */
double ora_e4m3_code_value(int code) {
    int e = (code >> 3) & 0xF, m = code & 7;
    if (e == 0)
        return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, e - 7);
}

/* binary32 -> OCP E4M3FN, round to nearest with ties to the even mantissa,
 * saturating: magnitudes at or beyond 448 give 448. The sign is kept, so
 * -0 and negative values that round to zero give 0x80.
 * Written from the format's definition: find the two neighbouring codes
 * around |v| by bisection over the ordered code values, then choose the
 * nearer one, the even one on a tie. Inputs are finite (NaN is rejected by
 * the callers' input checks). */
uint8_t ora_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    /* largest code c with value(c) <= a; codes are increasing in value */
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (ora_e4m3_code_value(mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo;
    double below = ora_e4m3_code_value(c);
    if (below == a)
        return (uint8_t)(sign | c);
    double above = ora_e4m3_code_value(c + 1);
    double dlo = a - below, dhi = above - a; /* exact: few significant bits */
    int q;
    if (dlo < dhi)
        q = c;
    else if (dhi < dlo)
        q = c + 1;
    else
        q = (c & 1) ? c + 1 : c; /* tie: even mantissa (code LSB = mantissa LSB) */
    return (uint8_t)(sign | q);
}

/* ---------------------------------------------------------------------- */
/* Layout: counts, alignment, offsets, stable slots                         */
/* ---------------------------------------------------------------------- */

static int64_t ora_read_idx(const void* idx, int idx_bits, int64_t p) {
    if (idx_bits == 32)
        return ((const int32_t*)idx)[p];
    return ((const int64_t*)idx)[p];
}

/* Layout of the receive side of one GPU.
 *
 * Follows the README's dispatch_forward example: per-expert received-token
 * counts for the GEMM, counts padded to expert_alignment, expert-contiguous
 * receive rows (EPv2's GEMM layout), with experts grouped into D destination
 * buffers. Readings where the page is silent:
 *   - id == -1 is a masked pair; any other id outside [0, E) is masked and
 *     raises ORA_FLAG_BAD_ID.
 *   - cnt[e] = number of unmasked pairs routed to e.
 *   - COMPACT: pad[e] = ceil(cnt[e] / A) * A (0 for an empty expert);
 *     expert_off = exclusive scan of pad in expert-id order;
 *     rows of expert e: [expert_off[e], expert_off[e] + pad[e]); the last
 *     pad[e] - cnt[e] of them are padding (row_src = -1, row_w = 0).
 *   - FIXED (decode): expert e owns rows [e*C, e*C + C); the first C pairs
 *     of e in (t, j) order get rows, later ones are masked and raise
 *     ORA_FLAG_OVERFLOW; pad[e] = min(cnt[e], C); expert_off[e] = e*C.
 *   - Experts map to destinations in contiguous ranges: d = e / (E / D);
 *     dest_off[d] = expert_off[d * E / D]; dest_tokens[d] = number of
 *     distinct tokens with at least one unmasked pair routed into d.
 *   - Slot order inside an expert is ascending (t, j): the stable order.
 *   - row_src[s] = t*k + j of the pair in row s; row_w[s] = topk_w[t, j]
 *     (written only when topk_w is given).
 * Returns the flags. Output arrays: cnt, pad [E]; expert_off [E+1];
 * dest_off [D+1]; dest_tokens [D]; slot [T*k]; row_src, row_w [rows bound].
 */
uint32_t ora_layout(int mode, int T, int E, int k, int A, int D, int C, int idx_bits,
                    const void* topk_idx, const float* topk_w,
                    int32_t* cnt, int32_t* pad, int32_t* expert_off,
                    int32_t* dest_off, int32_t* dest_tokens,
                    int32_t* slot, int32_t* row_src, float* row_w) {
    uint32_t flags = 0;
    int64_t P = (int64_t)T * k;
    int epd = E / D; /* experts per destination */

    /* 1. validate and count */
    for (int e = 0; e < E; ++e)
        cnt[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        int64_t id = ora_read_idx(topk_idx, idx_bits, p);
        if (id == -1)
            continue;
        if (id < 0 || id >= E) {
            flags |= ORA_FLAG_BAD_ID;
            continue;
        }
        cnt[id] += 1;
    }

    /* 2. distinct tokens per destination */
    for (int d = 0; d < D; ++d)
        dest_tokens[d] = 0;
    for (int t = 0; t < T; ++t) {
        for (int d = 0; d < D; ++d) {
            int hit = 0;
            for (int j = 0; j < k; ++j) {
                int64_t id = ora_read_idx(topk_idx, idx_bits, (int64_t)t * k + j);
                if (id >= 0 && id < E && id / epd == d)
                    hit = 1;
            }
            dest_tokens[d] += hit;
        }
    }

    /* 3. alignment and offsets */
    if (mode == ORA_MODE_COMPACT) {
        expert_off[0] = 0;
        for (int e = 0; e < E; ++e) {
            pad[e] = (cnt[e] + A - 1) / A * A;
            expert_off[e + 1] = expert_off[e] + pad[e];
        }
    } else {
        for (int e = 0; e < E; ++e) {
            pad[e] = cnt[e] < C ? cnt[e] : C;
            expert_off[e] = e * C;
            if (cnt[e] > C)
                flags |= ORA_FLAG_OVERFLOW;
        }
        expert_off[E] = E * C;
    }
    for (int d = 0; d <= D; ++d)
        dest_off[d] = expert_off[d * epd];

    /* 4. stable slots: walk pairs in (t, j) order with one cursor per expert */
    int32_t cursor[4096];
    for (int e = 0; e < E; ++e)
        cursor[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        int64_t id = ora_read_idx(topk_idx, idx_bits, p);
        if (id < 0 || id >= E) {
            slot[p] = -1;
            continue;
        }
        if (mode == ORA_MODE_FIXED && cursor[id] >= C) {
            slot[p] = -1; /* beyond capacity */
            continue;
        }
        int32_t s = expert_off[id] + cursor[id];
        cursor[id] += 1;
        slot[p] = s;
        row_src[s] = (int32_t)p;
        if (topk_w)
            row_w[s] = topk_w[p];
    }
    /* 5. padding rows (COMPACT only) */
    if (mode == ORA_MODE_COMPACT) {
        for (int e = 0; e < E; ++e) {
            for (int32_t r = expert_off[e] + cnt[e]; r < expert_off[e] + pad[e]; ++r) {
                row_src[r] = -1;
                if (topk_w)
                    row_w[r] = 0.0f;
            }
        }
    }
    return flags;
}

/* Padding rows of expert e: [expert_off[e] + cnt[e], expert_off[e] + pad[e]).
 * Empty in FIXED mode, where pad[e] <= cnt[e]. */
static int32_t ora_pad_begin(const int32_t* cnt, const int32_t* expert_off, int e) {
    return expert_off[e] + cnt[e];
}

/* ---------------------------------------------------------------------- */
/* Dispatch                                                                */
/* ---------------------------------------------------------------------- */

/* BF16 dispatch (README dispatch_forward, BF16 x): each unmasked pair's row
 * is a bitwise copy of its token's hidden row. With pair weights given
 * (combine_backward of a weighted combine), the copy for pair (t, j) is
 * bf16_rne(w[t, j] * float(x[t, h])), one binary32 multiply.
 * Padding rows are zero when zero_pad is set. */
void ora_dispatch_bf16(int T, int H, int k, int E, const uint16_t* x,
                       const int32_t* slot, const float* pair_w,
                       const int32_t* cnt, const int32_t* pad, const int32_t* expert_off,
                       int zero_pad, uint16_t* recv) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t s = slot[(int64_t)t * k + j];
            if (s < 0)
                continue;
            for (int h = 0; h < H; ++h) {
                uint16_t v = x[(int64_t)t * H + h];
                if (pair_w)
                    v = ora_bf16_rne(pair_w[(int64_t)t * k + j] * ora_bf16_value(v));
                recv[(int64_t)s * H + h] = v;
            }
        }
    }
    if (zero_pad) {
#pragma omp parallel for schedule(static)
        for (int e = 0; e < E; ++e)
            for (int32_t r = ora_pad_begin(cnt, expert_off, e); r < expert_off[e] + pad[e]; ++r)
                for (int h = 0; h < H; ++h)
                    recv[(int64_t)r * H + h] = 0;
    }
}

/* 1x128 FP8 quantisation of one token block (README: FP8 dispatch with
 * per-token scale factors; the 1x128 block size and the 448 divisor are the
 * E4M3FN range). amax = max |x| over the block (exact in binary32);
 * amax == 0 gives scale 0 and all-zero codes; otherwise
 * scale = amax / 448 and q[h] = E4M3(x[h] / scale), both divisions IEEE
 * binary32 round-to-nearest-even. */
float ora_quantize_block(const uint16_t* xb, int n, uint8_t* q) {
    float amax = 0.0f;
    for (int h = 0; h < n; ++h) {
        float a = fabsf(ora_bf16_value(xb[h]));
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0f) {
        for (int h = 0; h < n; ++h)
            q[h] = 0x00;
        return 0.0f;
    }
    float scale = amax / 448.0f;
    for (int h = 0; h < n; ++h) {
        float v = ora_bf16_value(xb[h]) / scale;
        q[h] = ora_e4m3_encode(v);
    }
    return scale;
}

/* FP8 dispatch with quantisation: every slot of token t receives the same
 * codes and the same H/128 scales (row-major [rows, H/128] binary32).
 * Padding rows get code 0x00 and scale 0 when zero_pad is set. */
void ora_dispatch_fp8(int T, int H, int k, int E, const uint16_t* x, const int32_t* slot,
                      const int32_t* cnt, const int32_t* pad, const int32_t* expert_off,
                      int zero_pad, uint8_t* recv, float* recv_scales) {
    int nb = H / 128;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        uint8_t q[128];
        for (int b = 0; b < nb; ++b) {
            float s = ora_quantize_block(x + (int64_t)t * H + (int64_t)b * 128, 128, q);
            for (int j = 0; j < k; ++j) {
                int32_t r = slot[(int64_t)t * k + j];
                if (r < 0)
                    continue;
                memcpy(recv + (int64_t)r * H + (int64_t)b * 128, q, 128);
                recv_scales[(int64_t)r * nb + b] = s;
            }
        }
    }
    if (zero_pad) {
#pragma omp parallel for schedule(static)
        for (int e = 0; e < E; ++e)
            for (int32_t r = ora_pad_begin(cnt, expert_off, e); r < expert_off[e] + pad[e]; ++r) {
                memset(recv + (int64_t)r * H, 0, (size_t)H);
                for (int b = 0; b < nb; ++b)
                    recv_scales[(int64_t)r * nb + b] = 0.0f;
            }
    }
}

/* combine_backward of a weighted combine with FP8 output (README
 * combine_backward: a dispatch of the output gradient on the handle; the
 * gradient may travel as FP8). Reading taken here: the copy for pair (t, j)
 * is the BF16 weighted copy, bf16_rne(w[t, j] * float(g[t, h])), quantised
 * per 1x128 block exactly as the FP8 dispatch quantises x; each pair has its
 * own scales since each has its own weight. Padding rows get code 0x00 and
 * scale 0 when zero_pad is set. */
void ora_combine_backward_fp8(int T, int H, int k, int E, const uint16_t* g, const float* pair_w,
                              const int32_t* slot, const int32_t* cnt, const int32_t* pad,
                              const int32_t* expert_off, int zero_pad, uint8_t* recv, float* recv_scales) {
    int nb = H / 128;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        uint16_t row[128];
        uint8_t q[128];
        for (int j = 0; j < k; ++j) {
            int32_t r = slot[(int64_t)t * k + j];
            if (r < 0)
                continue;
            float w = pair_w[(int64_t)t * k + j];
            for (int b = 0; b < nb; ++b) {
                for (int i = 0; i < 128; ++i)
                    row[i] = ora_bf16_rne(w * ora_bf16_value(g[(int64_t)t * H + (int64_t)b * 128 + i]));
                recv_scales[(int64_t)r * nb + b] = ora_quantize_block(row, 128, q);
                memcpy(recv + (int64_t)r * H + (int64_t)b * 128, q, 128);
            }
        }
    }
    if (zero_pad) {
#pragma omp parallel for schedule(static)
        for (int e = 0; e < E; ++e)
            for (int32_t r = ora_pad_begin(cnt, expert_off, e); r < expert_off[e] + pad[e]; ++r) {
                memset(recv + (int64_t)r * H, 0, (size_t)H);
                for (int b = 0; b < nb; ++b)
                    recv_scales[(int64_t)r * nb + b] = 0.0f;
            }
    }
}

/* FP8 dispatch of an already quantised input (README: x given as the tuple
 * (data, scale_factors)): codes and scales copied bitwise to every slot. */
void ora_dispatch_fp8_prequant(int T, int H, int k, int E, const uint8_t* xq, const float* xs,
                               const int32_t* slot, const int32_t* cnt, const int32_t* pad,
                               const int32_t* expert_off, int zero_pad,
                               uint8_t* recv, float* recv_scales) {
    int nb = H / 128;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t r = slot[(int64_t)t * k + j];
            if (r < 0)
                continue;
            memcpy(recv + (int64_t)r * H, xq + (int64_t)t * H, (size_t)H);
            memcpy(recv_scales + (int64_t)r * nb, xs + (int64_t)t * nb, sizeof(float) * (size_t)nb);
        }
    }
    if (zero_pad) {
#pragma omp parallel for schedule(static)
        for (int e = 0; e < E; ++e)
            for (int32_t r = ora_pad_begin(cnt, expert_off, e); r < expert_off[e] + pad[e]; ++r) {
                memset(recv + (int64_t)r * H, 0, (size_t)H);
                for (int b = 0; b < nb; ++b)
                    recv_scales[(int64_t)r * nb + b] = 0.0f;
            }
    }
}

/* ---------------------------------------------------------------------- */
/* Combine                                                                 */
/* ---------------------------------------------------------------------- */

/* Combine (README combine_forward / dispatch_backward): for each token t and
 * channel h, acc starts at +0 and, for j = 0..k-1 over unmasked pairs,
 * acc = fmaf(w[t, j], float(y[slot[t, j], h]), acc) in binary32, or
 * acc = acc + float(y[...]) when no weights are given; out = bf16_rne(acc).
 * With row_vals given, out_vals[t, j] = row_vals[slot[t, j]] (0 when masked):
 * the combined per-pair values that dispatch_backward returns for the
 * received weight gradients. */
void ora_combine(int T, int H, int k, const uint16_t* y, const int32_t* slot,
                 const float* w, uint16_t* out, const float* row_vals, float* out_vals) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int32_t s = slot[(int64_t)t * k + j];
                if (s < 0)
                    continue;
                float v = ora_bf16_value(y[(int64_t)s * H + h]);
                if (w)
                    acc = fmaf(w[(int64_t)t * k + j], v, acc);
                else
                    acc = acc + v;
            }
            out[(int64_t)t * H + h] = ora_bf16_rne(acc);
        }
        if (row_vals && out_vals) {
            for (int j = 0; j < k; ++j) {
                int32_t s = slot[(int64_t)t * k + j];
                out_vals[(int64_t)t * k + j] = s < 0 ? 0.0f : row_vals[s];
            }
        }
    }
}

/* Gradient of the weighted combine with respect to its weights. The
 * combine above computes out[t] = sum_j w[t, j] * y[slot[t, j]] (README
 * combine_forward, weighted; its backward, README combine_backward, is a
 * dispatch of grad_out for the expert outputs). For a loss whose gradient
 * with respect to out[t] is g[t], the gradient with respect to w[t, j] is
 * therefore sum_h g[t, h] * y[slot[t, j], h]: the dot product of the token's
 * output gradient with the expert-output row of pair (t, j). Masked and
 * overflowed pairs (slot -1) take no part in the combine and get 0.
 * Computed in binary64: every product of two bfloat16 values is exact in
 * binary64 (8 + 8 significand bits), and the H products are added in order
 * h = 0..H-1. */
void ora_combine_weight_grad(int T, int H, int k, const uint16_t* grad_out, const uint16_t* y,
                             const int32_t* slot, double* grad_w) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t s = slot[(int64_t)t * k + j];
            double acc = 0.0;
            if (s >= 0) {
                for (int h = 0; h < H; ++h) {
                    double g = (double)ora_bf16_value(grad_out[(int64_t)t * H + h]);
                    double v = (double)ora_bf16_value(y[(int64_t)s * H + h]);
                    acc += g * v;
                }
            }
            grad_w[(int64_t)t * k + j] = acc;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Consumer: FP8 grouped GEMM over the aligned expert-major layout          */
/* ---------------------------------------------------------------------- */

/* binary64 -> bfloat16, round to nearest even, directly from the double (no
 * intermediate binary32 rounding). Finite inputs within the bf16 range. */
static uint16_t ora_bf16_rne_f64(double v) {
    if (v == 0.0)
        return signbit(v) ? 0x8000 : 0x0000;
    uint16_t sign = v < 0 ? 0x8000 : 0x0000;
    double a = fabs(v);
    int e;
    frexp(a, &e);                      /* a = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                     /* bf16 keeps 8 significant bits */
    if (q < -133)
        q = -133;                      /* subnormal bf16 spacing 2^-133 */
    double m = ldexp(a, -q);           /* exact */
    double r = floor(m);
    double frac = m - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0))
        r += 1.0;
    double val = ldexp(r, q);
    float f = (float)val;              /* exact: val has <= 9 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* The grouped GEMM the layout exists for (README: per-expert received-token
 * counts meant for the expert GEMM, rows padded to expert_alignment; "New features": the
 * new GEMM layout): rows of expert e, [row_begin[e], row_end[e]), times that
 * expert's weight matrix. A is the dispatched E4M3 codes [rows, K] with
 * 1x128 scales sa [rows, K/128]; expert e's weights are E4M3 codes
 * B[e] [N, K] (one row per output channel) with 128x128 block scales
 * sb[e] [N/128, K/128]. For row r of expert e and channel n:
 *   C[r, n] = bf16( sum_kb sa[r, kb] * sb[e, n/128, kb]
 *                          * sum_{k in block kb} A[r, k] * B[e, n, k] )
 * with decoded code values, in binary64 (each block sum of 128 products of
 * E4M3 values is exact in binary64), rounded once to bf16. */
static double ora_gemm_one(int K, int N, int e, int64_t r, int64_t n, const uint8_t* A, const float* sa,
                           const uint8_t* B, const float* sb) {
    int kb_n = K / 128, nb_n = N / 128;
    const uint8_t* a = A + r * (int64_t)K;
    const uint8_t* b = B + ((int64_t)e * N + n) * (int64_t)K;
    double acc = 0.0;
    for (int kb = 0; kb < kb_n; ++kb) {
        double blk = 0.0;
        for (int k = kb * 128; k < kb * 128 + 128; ++k)
            blk += ora_e4m3_code_value(a[k] & 0x7F) * ((a[k] & 0x80) ? -1.0 : 1.0)
                   * ora_e4m3_code_value(b[k] & 0x7F) * ((b[k] & 0x80) ? -1.0 : 1.0);
        acc += (double)sa[r * kb_n + kb] * (double)sb[((int64_t)e * nb_n + n / 128) * kb_n + kb] * blk;
    }
    return acc;
}

/* Every row of every expert range: C [rows, N] bf16. */
void ora_grouped_gemm_fp8(int E, int K, int N, const int32_t* row_begin, const int32_t* row_end,
                          const uint8_t* A, const float* sa, const uint8_t* B, const float* sb, uint16_t* C) {
    for (int e = 0; e < E; ++e)
        for (int64_t r = row_begin[e]; r < row_end[e]; ++r)
            for (int64_t n = 0; n < N; ++n)
                C[r * N + n] = ora_bf16_rne_f64(ora_gemm_one(K, N, e, r, n, A, sa, B, sb));
}

/* Selected outputs only: pairs[2i] = r, pairs[2i+1] = n; out[i] = C[r, n]
 * (0 when r lies in no expert range). For checking full-size results. */
void ora_grouped_gemm_fp8_at(int E, int K, int N, const int32_t* row_begin, const int32_t* row_end,
                             const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                             const int64_t* pairs, int64_t n_pairs, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_pairs; ++i) {
        int64_t r = pairs[2 * i], n = pairs[2 * i + 1];
        int e = 0;
        while (e < E && !(r >= row_begin[e] && r < row_end[e]))
            ++e;
        out[i] = e < E ? ora_bf16_rne_f64(ora_gemm_one(K, N, e, r, n, A, sa, B, sb)) : 0;
    }
}

/* Batch form of the codec for tests: encode n binary32 values. */
void ora_e4m3_encode_many(const float* v, int64_t n, uint8_t* q) {
    for (int64_t i = 0; i < n; ++i)
        q[i] = ora_e4m3_encode(v[i]);
}

void ora_bf16_rne_many(const float* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = ora_bf16_rne(v[i]);
}

/* Threads the OpenMP build's loops use (n > 0 sets them); 1 in the plain
 * build, whose loops run on the calling thread. */
int ora_threads(int n) {
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
