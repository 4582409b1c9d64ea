/*
 * moe_oracle.c -- plain, slow, obviously correct CPU oracle for the MoE
 * layout / dispatch / combine path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library calls, links or
 * includes this file. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it. It shares no code, header, table
 * or helper with the GPU library.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math), so
 * that every fp32 operation is the one written here, rounded once.
 *
 * What it computes, and where each step comes from:
 *
 *   layout   -- DeepEP (deepseek-ai/DeepEP repository dump), deep_ep.cpp,
 *               Buffer::get_dispatch_layout: per-expert token counts of the
 *               top-k ids; Buffer::intranode_dispatch: the receive buffer is
 *               expert-contiguous and sized for the worst case when
 *               num_worst_tokens is given (no host wait), with recv_src_idx
 *               naming each received row's source. The order of rows inside
 *               one expert's segment is not fixed by the pages; the oracle
 *               takes ascending (token, k) -- a stable counting sort.
 *               Masked ids: the vLLM branch compare ds-exp-2...ds-exp-ag,
 *               mask_topk_ids writes -1 for padded tokens; any id < 0 is
 *               skipped. ids >= E are counted in *status and skipped.
 *   dispatch -- deep_ep.cpp intranode dispatch outputs recv_x, recv_x_scales,
 *               recv_topk_idx, recv_topk_weights: every received row carries
 *               the token's whole payload. Byte copies, no conversion.
 *   combine  -- the same compare page, moe_reduce_scatter.cu, POLL + REDUCE
 *               phase: bf16 inputs summed into fp32 accumulators in a fixed
 *               order, one conversion to bf16 at the end; DeepEP
 *               low_latency_combine takes topk_weights fp32 to weight the
 *               expert outputs. Here: acc = +0; for k ascending with a valid
 *               row, acc = fmaf(w[t,k], y[row,h], acc); out = bf16_rne(acc).
 *
 * Parity unpinned: these readings rest on this oracle's own definition,
 * because no page fixes them. The tests pin that the oracle computes exactly
 * these readings (a stable counting sort, brute force, hand-worked cases,
 * exact rationals), not that the pages require them.
 *  - layout: the order of rows inside one expert's segment (ascending
 *    (token, k)) and what expert_alignment does (each segment padded to a
 *    multiple of align with unused rows);
 *  - combine epilogue: where the two biases enter (after the top-k sum, in
 *    fp32, bias_0 then bias_1, then the residual); DeepEP's combine kernel
 *    body is not on the pages;
 *  - FP8 cast: the floor 2^-126 under the block scale (it decides the scale
 *    stored for an all-zero or nearly-zero block; the codes of an all-zero
 *    block are 0 under any positive floor, and that is pinned) and the
 *    element step as one fp32 division x / s rather than a product with a
 *    reciprocal;
 *  - padded receive metadata: each expert's row range from the single
 *    source packed as (begin << 32) | count in the int64 the pages name;
 *  - backward: the sums over k as fp32 additions in ascending k (the
 *    combine's order) and the weight-gradient dot products formed in double
 *    and rounded once. The pages give the backward's dataflow only; the
 *    double results are pinned against float64 autograd within their
 *    rounding bound, the fp32 bit patterns are this reading's.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_ALIGN (-2)
#define ORC_ERR_LIMIT (-3)
#define ORC_ERR_CAPACITY (-4)
#define ORC_ERR_NOMEM (-5) /* a host buffer of the oracle itself could not be allocated */

#define ORC_MAX_K 32
#define ORC_MAX_E 1024

int oracle_version(void) { return 1; }

/* Rows the receive buffer must hold so that no routing can overflow it:
 * every (token, k) pair, plus the padding each expert segment can need when
 * it is rounded up to a multiple of `align`. */
int64_t oracle_required_cap(int32_t N, int32_t K, int32_t E, int32_t align) {
    int64_t c = (int64_t)N * K;
    if (align > 1) c += (int64_t)E * (align - 1);
    return c;
}

/* Layout: counts[e], offsets[0..E], pos[t*K+k], row_pair[0..cap), *status. */
int oracle_layout(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K, int32_t E,
                  int32_t align, int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* row_pair,
                  int64_t cap, int32_t* status) {
    if (N < 0 || K < 1 || E < 1 || align < 1) return ORC_ERR_ARG;
    if (K > ORC_MAX_K || E > ORC_MAX_E) return ORC_ERR_LIMIT;
    if ((int64_t)N * K >= ((int64_t)1 << 31)) return ORC_ERR_LIMIT;
    if (N > 0 && ids_row_stride < K) return ORC_ERR_ARG;
    if (cap < oracle_required_cap(N, K, E, align)) return ORC_ERR_CAPACITY;
    if (cap >= ((int64_t)1 << 31)) return ORC_ERR_LIMIT;

    int32_t bad = 0;

    /* counts: one increment per valid (t, k), in (t, k) order. */
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int32_t t = 0; t < N; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = ids[(int64_t)t * ids_row_stride + k];
            if (e < 0) continue;
            if (e >= E) { ++bad; continue; }
            counts[e] += 1;
        }
    }

    /* offsets: exclusive running sum of counts rounded up to `align`. */
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) {
        int32_t padded = (counts[e] + align - 1) / align * align;
        offsets[e + 1] = offsets[e] + padded;
    }

    /* pos / row_pair: walk the pairs in (t, k) order; each valid pair takes
     * the next free row of its expert's segment. */
    for (int64_t r = 0; r < cap; ++r) row_pair[r] = -1;
    int32_t cursor[ORC_MAX_E];
    for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int32_t t = 0; t < N; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = ids[(int64_t)t * ids_row_stride + k];
            int32_t p = -1;
            if (e >= 0 && e < E) {
                p = cursor[e];
                cursor[e] += 1;
                row_pair[p] = t * K + k;
            }
            pos[(int64_t)t * K + k] = p;
        }
    }
    if (status) *status = bad;
    return ORC_OK;
}

/* One payload field: byte rows of `row_bytes`, read from src with
 * src_row_stride bytes between tokens, written to dst with dst_row_stride
 * bytes between receive rows. */
typedef struct {
    const void* src;
    int64_t src_row_stride;
    void* dst;
    int64_t dst_row_stride;
    int64_t row_bytes;
} oracle_field;

/* Dispatch: dst_f[pos[t,k]] <- src_f[t] for every valid (t, k) and field f.
 * pos == NULL means the identity map pos[t] = t with K == 1 (pack/unpack). */
int oracle_dispatch(const oracle_field* fields, int32_t nfields, int32_t N, int32_t K,
                    const int32_t* pos) {
    if (nfields < 1 || nfields > 4 || N < 0 || K < 1 || K > ORC_MAX_K) return ORC_ERR_ARG;
    if (pos == NULL && K != 1) return ORC_ERR_ARG;
    for (int f = 0; f < nfields; ++f)
        if (fields[f].row_bytes < 0) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < N; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t p = pos ? pos[(int64_t)t * K + k] : t;
            if (p < 0) continue;
            for (int f = 0; f < nfields; ++f) {
                const oracle_field* d = &fields[f];
                memcpy((char*)d->dst + (int64_t)p * d->dst_row_stride,
                       (const char*)d->src + (int64_t)t * d->src_row_stride, (size_t)d->row_bytes);
            }
        }
    }
    return ORC_OK;
}

/* bf16 -> fp32: the bf16 pattern is the top half of the fp32 pattern. */
float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even (NaN -> 0x7FC0).
 * Adding 0x7FFF plus the lowest kept bit carries into the kept half exactly
 * when the dropped half is above one half, or equal to it with the kept
 * half odd. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* double -> bf16, round to nearest, ties to even, in one step: scale the
 * magnitude so the 8 kept significand bits are the integer part, round that
 * with rint (nearest-even in the default rounding mode), and rebuild. */
uint16_t oracle_bf16_from_f64(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double m = fabs(v);
    if (m == 0.0) return sign;
    int e;
    frexp(m, &e);                    /* m = f * 2^e, 0.5 <= f < 1 */
    if (e < -125) e = -125;          /* bf16 subnormal range shares one quantum */
    double q = ldexp(1.0, e - 8);    /* spacing of bf16 values near m */
    double r = rint(m / q) * q;      /* exact: m / q < 2^9 */
    if (r >= 0x1.0p128) return sign | 0x7F80;
    float f = (float)r;              /* exactly representable */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* The fp32 accumulator of one output element: acc = +0, then for k
 * ascending with a valid row, acc = fmaf(w[t,k], y[row, h], acc). */
static float combine_acc(const uint16_t* y, int64_t y_row_stride, const float* w,
                         int64_t w_row_stride, const int32_t* pos, int32_t K, int32_t t, int32_t h) {
    float acc = 0.0f;
    for (int32_t k = 0; k < K; ++k) {
        int32_t p = pos[(int64_t)t * K + k];
        if (p < 0) continue;
        float yv = oracle_bf16_to_f32(y[(int64_t)p * y_row_stride + h]);
        acc = fmaf(w[(int64_t)t * w_row_stride + k], yv, acc);
    }
    return acc;
}

/* Combine: out[t,h] = bf16_rne(fp32 accumulator of (t, h)). */
int oracle_combine(const uint16_t* y, int64_t y_row_stride, const float* w, int64_t w_row_stride,
                   const int32_t* pos, int32_t N, int32_t K, int32_t Hc, uint16_t* out,
                   int64_t out_row_stride) {
    if (N < 0 || K < 1 || K > ORC_MAX_K || Hc < 0) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < N; ++t)
        for (int32_t h = 0; h < Hc; ++h)
            out[(int64_t)t * out_row_stride + h] =
                oracle_f32_to_bf16(combine_acc(y, y_row_stride, w, w_row_stride, pos, K, t, h));
    return ORC_OK;
}

/* The same reduction with the fp32 accumulators written out unrounded, so
 * the order and fusion of the chain can be checked on their own. */
int oracle_combine_acc(const uint16_t* y, int64_t y_row_stride, const float* w,
                       int64_t w_row_stride, const int32_t* pos, int32_t N, int32_t K, int32_t Hc,
                       float* acc_out) {
    if (N < 0 || K < 1 || K > ORC_MAX_K || Hc < 0) return ORC_ERR_ARG;
    for (int32_t t = 0; t < N; ++t)
        for (int32_t h = 0; h < Hc; ++h)
            acc_out[(int64_t)t * Hc + h] = combine_acc(y, y_row_stride, w, w_row_stride, pos, K, t, h);
    return ORC_OK;
}

/* Combine epilogue: the combine accumulator of every element of a token,
 * then (each only if given, all in fp32):
 *   acc += bias0[t,h]; acc += bias1[t,h]
 *     -- DeepEP (repository dump, deep_ep.cpp, Buffer::intranode_combine):
 *        optional bias_0 / bias_1 [num_recv_tokens, hidden], dtype of x;
 *        where they are added is not shown, taken here after the top-k sum.
 *   with a residual:
 *     acc += residual[t,h];  residual_out[t,h] = bf16(acc)
 *     scale = 1 / sqrt(sum_h acc^2 / Hc + eps)
 *     out[t,h] = bf16(acc * scale * gamma[h])
 *     -- vLLM branch compare ds-exp-2...ds-exp-ag, moe_rs_fused.cu, fused
 *        POLL + REDUCE + RESIDUAL + RMSNORM phase: fp32 sum plus residual,
 *        that value stored as the new residual, RMSNorm of the same fp32
 *        values with gamma.
 *   without a residual: out[t,h] = bf16(acc).
 * The pages fix fp32 for the sums but not the order of the sum of squares
 * (a block tree there), so the oracle forms it and the scale in double and
 * rounds each normed element once from double. */
int oracle_combine_epilogue(const uint16_t* y, int64_t y_row_stride, const float* w,
                            int64_t w_row_stride, const int32_t* pos, int32_t N, int32_t K,
                            int32_t Hc, const uint16_t* bias0, const uint16_t* bias1,
                            const uint16_t* residual, const uint16_t* gamma, float eps,
                            uint16_t* residual_out, uint16_t* out) {
    if (N < 0 || K < 1 || K > ORC_MAX_K || Hc < 0) return ORC_ERR_ARG;
    if (residual && (!gamma || !residual_out)) return ORC_ERR_ARG;
    /* One Hc-float row per thread, taken from the heap once per parallel
     * region: a row per token on the stack would grow every thread's stack
     * by 4*Hc bytes per token until the loop ends. */
    int oom = 0;
#pragma omp parallel reduction(|| : oom)
    {
        float* acc = (float*)malloc((size_t)(Hc > 0 ? Hc : 1) * sizeof(float));
        if (!acc) oom = 1;
#pragma omp for schedule(static)
        for (int32_t t = 0; t < N; ++t) {
            if (!acc) continue;
            for (int32_t h = 0; h < Hc; ++h) {
                float a = combine_acc(y, y_row_stride, w, w_row_stride, pos, K, t, h);
                int64_t i = (int64_t)t * Hc + h;
                if (bias0) a = a + oracle_bf16_to_f32(bias0[i]);
                if (bias1) a = a + oracle_bf16_to_f32(bias1[i]);
                if (residual) a = a + oracle_bf16_to_f32(residual[i]);
                acc[h] = a;
            }
            if (!residual) {
                for (int32_t h = 0; h < Hc; ++h)
                    out[(int64_t)t * Hc + h] = oracle_f32_to_bf16(acc[h]);
                continue;
            }
            double ss = 0.0;
            for (int32_t h = 0; h < Hc; ++h) ss += (double)acc[h] * (double)acc[h];
            double scale = 1.0 / sqrt(ss / (double)Hc + (double)eps);
            for (int32_t h = 0; h < Hc; ++h) {
                int64_t i = (int64_t)t * Hc + h;
                residual_out[i] = oracle_f32_to_bf16(acc[h]);
                double v = (double)acc[h] * scale * (double)oracle_bf16_to_f32(gamma[h]);
                out[i] = oracle_bf16_from_f64(v);
            }
        }
        free(acc);
    }
    return oom ? ORC_ERR_NOMEM : ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Low-latency dispatch forms (DeepEP repository dump, deep_ep.cpp,
 * Buffer::low_latency_dispatch; config.hpp, LowLatencyLayout):
 *  - a padded per-expert receive buffer packed_recv_x [E, M, H] with
 *    packed_recv_count [E] and the source of every row;
 *  - FP8 cast on dispatch: bf16 x, e4m3 payload, fp32 scales per token and
 *    per 128 channels stored column-major [E, H/128, M], or (use_ue8m0, which
 *    needs round_scale) power-of-two scales as 8-bit exponents packed four to
 *    an int32 [E, H/512, M].
 * The cast itself is not on the pages; this oracle takes, per 128-channel
 * block of a token: amax = max |x| (fp32), s = amax / 448 but at least
 * 2^-126, with round_scale s = the smallest power of two >= s, and
 * q = e4m3(x / s) (fp32 division, round to nearest even, saturating to
 * +-448; e4m3fn: 4 exponent bits, bias 7, no infinities).
 * ------------------------------------------------------------------------- */

/* Padded layout: expert e's segment starts at row e*M; the first M pairs of
 * expert e in (t, k) order take rows e*M .. e*M+M-1, later ones are dropped.
 * counts[e] = rows filled; status[0] = ids >= E, status[1] = pairs dropped
 * for capacity. row_pair[E*M] as in oracle_layout. */
int oracle_layout_padded(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                         int32_t E, int32_t M, int32_t* counts, int32_t* pos, int32_t* row_pair,
                         int32_t* status) {
    if (N < 0 || K < 1 || E < 1 || M < 0) return ORC_ERR_ARG;
    if (K > ORC_MAX_K || E > ORC_MAX_E) return ORC_ERR_LIMIT;
    if ((int64_t)N * K >= ((int64_t)1 << 31) || (int64_t)E * M >= ((int64_t)1 << 31))
        return ORC_ERR_LIMIT;
    if (N > 0 && ids_row_stride < K) return ORC_ERR_ARG;
    int32_t bad = 0, dropped = 0;
    for (int64_t r = 0; r < (int64_t)E * M; ++r) row_pair[r] = -1;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int32_t t = 0; t < N; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = ids[(int64_t)t * ids_row_stride + k];
            int32_t p = -1;
            if (e >= E) {
                ++bad;
            } else if (e >= 0) {
                if (counts[e] < M) {
                    p = e * M + counts[e];
                    counts[e] += 1;
                    row_pair[p] = t * K + k;
                } else {
                    ++dropped;
                }
            }
            pos[(int64_t)t * K + k] = p;
        }
    }
    if (status) {
        status[0] = bad;
        status[1] = dropped;
    }
    return ORC_OK;
}

/* Receive metadata of the padded layout for one source (DeepEP repository
 * dump, deep_ep.cpp, Buffer::low_latency_dispatch, which returns
 * packed_recv_layout_range int64 [num_local_experts, num_ranks] and updates
 * the int32 diagnosis tensor cumulative_local_expert_recv_stats
 * [num_local_experts]; the kernel that fills them is not on the pages).
 * With one source, expert e's rows from it are all its rows: begin 0 and
 * count counts[e], packed as (begin << 32) | count -- the packing is this
 * oracle's reading (parity unpinned); the stats gain each expert's rows. */
void oracle_padded_recv_meta(const int32_t* counts, int32_t E, int64_t* layout_range,
                             int32_t* recv_stats) {
    for (int32_t e = 0; e < E; ++e) {
        const int64_t begin = 0, count = counts[e];
        if (layout_range) layout_range[e] = (begin << 32) | count;
        if (recv_stats) recv_stats[e] += counts[e];
    }
}

/* fp32 -> e4m3fn, round to nearest even, finite overflow saturates to
 * +-448, NaN -> 0x7F. e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; normals 2^-6 .. 448, subnormals multiples of 2^-9. Done on the value:
 * find its spacing, round the scaled value with rint, rebuild the code. */
uint8_t oracle_f32_to_e4m3(float f) {
    if (isnan(f)) return 0x7F;
    uint8_t sign = signbit(f) ? 0x80 : 0;
    double m = fabs((double)f);
    if (m >= 448.0) return sign | 0x7E;
    int e;
    frexp(m, &e);                       /* m = g * 2^e, 0.5 <= g < 1 */
    if (e < -5) e = -5;                 /* subnormal range: spacing 2^-9 */
    double q = ldexp(1.0, e - 4);       /* spacing of e4m3 values near m */
    double r = rint(m / q) * q;         /* exact */
    if (r >= 448.0) return sign | 0x7E;
    if (r == 0.0) return sign;
    int re;
    double g = frexp(r, &re);           /* r = g * 2^re */
    int biased = re - 1 + 7;            /* exponent of 1.xxx * 2^(re-1) */
    uint8_t code;
    if (biased <= 0) {                  /* subnormal: r = mant * 2^-9 */
        code = (uint8_t)(r / ldexp(1.0, -9));
    } else {
        int mant = (int)((g * 2.0 - 1.0) * 8.0 + 0.5);
        code = (uint8_t)((biased << 3) | mant);
    }
    return sign | code;
}

float oracle_e4m3_to_f32(uint8_t c) {
    int s = c >> 7, ex = (c >> 3) & 15, mn = c & 7;
    if (ex == 15 && mn == 7) return NAN;
    double v = ex == 0 ? ldexp((double)mn, -9) : ldexp(1.0 + mn / 8.0, ex - 7);
    return (float)(s ? -v : v);
}

/* The scale of one 128-channel block of bf16 values. */
float oracle_fp8_block_scale(const uint16_t* x, int round_scale) {
    float amax = 0.0f;
    for (int i = 0; i < 128; ++i) {
        float a = fabsf(oracle_bf16_to_f32(x[i]));
        if (a > amax) amax = a;
    }
    float s = amax / 448.0f;
    if (s < 0x1.0p-126f) s = 0x1.0p-126f;
    /* An infinite s (the block holds an infinity) has no power of two above
     * it and stays infinite; frexpf leaves an infinity's exponent unset. */
    if (round_scale && isfinite(s)) {
        int e;
        float g = frexpf(s, &e);       /* s = g * 2^e, 0.5 <= g < 1 */
        s = (g == 0.5f) ? s : ldexpf(1.0f, e);
    }
    return s;
}

/* Quantising dispatch: for every valid (t, k), row p = pos[t*K+k] gets the
 * e4m3 codes of x[t] (H bytes at dst + p*dst_row_stride) and, per block b,
 * its scale. scale_mode 0: fp32 rows, scales[p*scale_row_stride + b];
 * 1: fp32 column-major per expert, scales[((p/M)*(H/128) + b)*M + p%M];
 * 2: ue8m0 column-major per expert, int32 words [((p/M)*(H/512) + b/4)*M + p%M],
 *    byte b%4 = biased exponent of the (power-of-two) scale;
 * 3: fp32 per token, scales[t*scale_row_stride + b], for every token. */
int oracle_dispatch_fp8(const uint16_t* x, int64_t x_row_stride, int32_t N, int32_t K, int32_t H,
                        const int32_t* pos, uint8_t* dst, int64_t dst_row_stride, void* scales,
                        int32_t scale_mode, int64_t scale_row_stride, int32_t M,
                        int32_t round_scale) {
    if (N < 0 || K < 1 || K > ORC_MAX_K || H < 0 || H % 128 != 0) return ORC_ERR_ARG;
    if (scale_mode < 0 || scale_mode > 3) return ORC_ERR_ARG;
    if (scale_mode == 2 && (!round_scale || H % 512 != 0)) return ORC_ERR_ARG;
    if ((scale_mode == 1 || scale_mode == 2) && M < 1) return ORC_ERR_ARG;
    const int32_t nb = H / 128;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < N; ++t) {
        const uint16_t* xr = x + (int64_t)t * x_row_stride;
        if (scale_mode == 3)
            for (int32_t b = 0; b < nb; ++b)
                ((float*)scales)[(int64_t)t * scale_row_stride + b] =
                    oracle_fp8_block_scale(xr + 128 * b, round_scale);
        for (int32_t k = 0; k < K; ++k) {
            int32_t p = pos[(int64_t)t * K + k];
            if (p < 0) continue;
            for (int32_t b = 0; b < nb; ++b) {
                float s = oracle_fp8_block_scale(xr + 128 * b, round_scale);
                for (int i = 0; i < 128; ++i)
                    dst[(int64_t)p * dst_row_stride + 128 * b + i] =
                        oracle_f32_to_e4m3(oracle_bf16_to_f32(xr[128 * b + i]) / s);
                if (scale_mode == 3) {
                    /* written once per token above */
                } else if (scale_mode == 0) {
                    ((float*)scales)[(int64_t)p * scale_row_stride + b] = s;
                } else if (scale_mode == 1) {
                    ((float*)scales)[((int64_t)(p / M) * nb + b) * M + p % M] = s;
                } else {
                    uint32_t bits;
                    memcpy(&bits, &s, 4);
                    uint8_t* word = (uint8_t*)((uint32_t*)scales +
                                               ((int64_t)(p / M) * (nb / 4) + b / 4) * M + p % M);
                    word[b % 4] = (uint8_t)(bits >> 23);
                }
            }
        }
    }
    return ORC_OK;
}

/* Scales placed by expert row (the receive-side scale layouts of the
 * low-latency dispatch, deep_ep.cpp, Buffer::low_latency_dispatch): row
 * p = e*M + m of the padded layout holds pair r = row_pair[p], a pair of
 * token r / K, so it takes that token's scales. scale_mode 1: fp32
 * scales[(e*(H/128) + b)*M + m]; 2: int32 word (e*(H/512) + b/4)*M + m whose
 * byte b%4 is the biased exponent of the token's scale of block b. Rows with
 * row_pair < 0 (or >= N*K) are left untouched. */
int oracle_scatter_scales(const float* token_scales, int64_t token_scale_row_stride, int32_t N,
                          int32_t K, int32_t H, const int32_t* row_pair, int32_t E, int32_t M,
                          void* scales, int32_t scale_mode) {
    if (N < 0 || K < 1 || H < 0 || H % 128 != 0 || E < 0 || M < 1) return ORC_ERR_ARG;
    if (scale_mode != 1 && scale_mode != 2) return ORC_ERR_ARG;
    if (scale_mode == 2 && H % 512 != 0) return ORC_ERR_ARG;
    const int32_t nb = H / 128;
    for (int32_t e = 0; e < E; ++e) {
        for (int32_t m = 0; m < M; ++m) {
            int32_t r = row_pair[(int64_t)e * M + m];
            if (r < 0 || (int64_t)r >= (int64_t)N * K) continue;
            const float* ts = token_scales + (int64_t)(r / K) * token_scale_row_stride;
            for (int32_t b = 0; b < nb; ++b) {
                if (scale_mode == 1) {
                    ((float*)scales)[((int64_t)e * nb + b) * M + m] = ts[b];
                } else {
                    uint32_t bits;
                    memcpy(&bits, &ts[b], 4);
                    uint8_t* word =
                        (uint8_t*)((uint32_t*)scales + ((int64_t)e * (nb / 4) + b / 4) * M + m);
                    word[b % 4] = (uint8_t)((bits >> 23) & 0xFF);
                }
            }
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Backward (DeepEP repository dump, README, "Example use in model training":
 * the backward of a dispatch is a combine of the received rows' gradients,
 * with the gradients of the received top-k weights combined alongside; the
 * backward of a combine is a dispatch of the output gradient).
 * With the forward  recv[pos[t,k]] = x[t]  and
 * out[t] = sum_k w[t,k] * y[pos[t,k]], the chain rule gives:
 *   dispatch backward: grad_x[t,h] = sum over valid k of grad_recv[pos[t,k],h]
 *                      grad_w_in[t,j] = sum over valid k of grad_recv_w[pos[t,k],j]
 *   combine backward:  grad_y[pos[t,k],h] = w[t,k] * grad_out[t,h]
 *                      grad_w[t,k] = sum_h grad_out[t,h] * y[pos[t,k],h]
 * Precision (readings): the sums over k are fp32 additions with k ascending
 * starting at +0 (the combine's order), rounded once to bf16; grad_y is one
 * fp32 product rounded to bf16; the dot products grad_w are formed in double
 * and rounded once to fp32 (their order is not fixed anywhere). Masked pairs
 * (pos < 0) contribute nothing and get grad_w = 0; rows of grad_y that no
 * pair lands on are not written.
 * ------------------------------------------------------------------------- */
int oracle_dispatch_backward(const uint16_t* grad_recv, int64_t grad_recv_row_stride,
                             const float* grad_recv_w, int64_t grad_recv_w_row_stride,
                             const int32_t* pos, int32_t N, int32_t K, int32_t H,
                             uint16_t* grad_x, int64_t grad_x_row_stride, float* grad_w,
                             int64_t grad_w_row_stride) {
    if (N < 0 || K < 1 || K > ORC_MAX_K || H < 0) return ORC_ERR_ARG;
    if ((grad_recv_w == NULL) != (grad_w == NULL)) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < N; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int32_t p = pos[(int64_t)t * K + k];
                if (p < 0) continue;
                acc = acc + oracle_bf16_to_f32(grad_recv[(int64_t)p * grad_recv_row_stride + h]);
            }
            grad_x[(int64_t)t * grad_x_row_stride + h] = oracle_f32_to_bf16(acc);
        }
        if (grad_w) {
            for (int32_t j = 0; j < K; ++j) {
                float acc = 0.0f;
                for (int32_t k = 0; k < K; ++k) {
                    int32_t p = pos[(int64_t)t * K + k];
                    if (p < 0) continue;
                    acc = acc + grad_recv_w[(int64_t)p * grad_recv_w_row_stride + j];
                }
                grad_w[(int64_t)t * grad_w_row_stride + j] = acc;
            }
        }
    }
    return ORC_OK;
}

int oracle_combine_backward(const uint16_t* grad_out, int64_t grad_out_row_stride, const float* w,
                            int64_t w_row_stride, const uint16_t* y, int64_t y_row_stride,
                            const int32_t* pos, int32_t N, int32_t K, int32_t Hc,
                            uint16_t* grad_y, int64_t grad_y_row_stride, float* grad_w,
                            int64_t grad_w_row_stride) {
    if (N < 0 || K < 1 || K > ORC_MAX_K || Hc < 0) return ORC_ERR_ARG;
    if (grad_w != NULL && y == NULL) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < N; ++t) {
        const uint16_t* g = grad_out + (int64_t)t * grad_out_row_stride;
        for (int32_t k = 0; k < K; ++k) {
            int32_t p = pos[(int64_t)t * K + k];
            if (p < 0) {
                if (grad_w) grad_w[(int64_t)t * grad_w_row_stride + k] = 0.0f;
                continue;
            }
            float wk = w[(int64_t)t * w_row_stride + k];
            for (int32_t h = 0; h < Hc; ++h)
                grad_y[(int64_t)p * grad_y_row_stride + h] =
                    oracle_f32_to_bf16(wk * oracle_bf16_to_f32(g[h]));
            if (grad_w) {
                double dot = 0.0;
                const uint16_t* yr = y + (int64_t)p * y_row_stride;
                for (int32_t h = 0; h < Hc; ++h)
                    dot += (double)oracle_bf16_to_f32(g[h]) * (double)oracle_bf16_to_f32(yr[h]);
                grad_w[(int64_t)t * grad_w_row_stride + k] = (float)dot;
            }
        }
    }
    return ORC_OK;
}
