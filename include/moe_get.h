/*
 * moe_get.h -- C ABI of the MI355X (gfx950) MoE routing layout, dispatch and
 * combine library (libmoe_get.so).
 *
 * The three calls are one GPU's share of an expert-parallel MoE layer:
 *
 *   moe_get_layout  per-expert histogram of the top-k ids, its exclusive
 *                   prefix scan, and a stable row for every (token, k) pair
 *                   in an expert-contiguous receive buffer.
 *   moe_dispatch    copies each token's payload (hidden bytes, scales, top-k
 *                   ids and weights, or one packed record) into the rows the
 *                   layout gave it.
 *   moe_combine     gathers the expert outputs back to token order as a
 *                   top-k weighted bf16 sum, accumulated in fp32.
 *
 * Conventions shared by every call:
 *   - Pointers named as device pointers must be device memory (or memory the
 *     device can access); the `fields` array itself is host memory.
 *   - Every call only enqueues work on `stream` (0 = the null stream) and
 *     returns; it never synchronizes and never waits on the host. A call
 *     may enqueue several kernels in order (the layout takes one or two;
 *     a job past 2^31 work-items runs in pieces of at most that size).
 *   - The library never allocates, frees or keeps state between calls; all
 *     buffers belong to the caller. Inputs are read-only and must not
 *     overlap outputs. (One exception: moe_get_layout_noalloc keeps its
 *     workspace in a static device array of the library, described there.
 *     The combine calls also remember, per device, its compute-unit count
 *     and whether a kernel fits in registers: facts of the device and of the
 *     build, not of any call.)
 *   - Return value: MOE_OK (0) or a negative MOE_ERR_* code; argument
 *     problems are found before anything is enqueued. moe_last_error()
 *     describes the last failure of the calling thread.
 *   - Data-dependent problems (an id >= E) never fail a call: they are
 *     counted into the optional device status word and the entry is skipped.
 *   - Rows named by pos (as written by the layout calls) are trusted: the
 *     copy and reduction kernels do not check them against the size of the
 *     buffers they index, which the caller allocates with the layout's
 *     capacity. A row outside its buffer is an out-of-bounds access, as an
 *     invalid pointer would be. (moe_scatter_scales alone reads row_pair
 *     defensively: entries outside [0, N*K) leave their row untouched.)
 *   - N = 0 is allowed and enqueues only the writes of empty results.
 */
#ifndef MOE_GET_H
#define MOE_GET_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_ARG (-1)        /* null pointer, negative size, bad count */
#define MOE_ERR_ALIGN (-2)      /* pointer, stride or row size not aligned */
#define MOE_ERR_LIMIT (-3)      /* K, E or a size beyond the supported range */
#define MOE_ERR_CAPACITY (-4)   /* receive capacity below the worst case */
#define MOE_ERR_WORKSPACE (-5)  /* workspace missing or too small */
#define MOE_ERR_HIP (-6)        /* the HIP runtime refused a launch */

#define MOE_MAX_TOPK 32
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_FIELDS 4

/* Library version (major * 10000 + minor * 100 + patch). */
int moe_version(void);

/* Text for the last non-zero return on this thread ("" if none). The string
 * stays valid until the next call on the same thread. */
const char* moe_last_error(void);

/*
 * Rows a receive buffer needs so that no routing of N tokens over E experts
 * with top-K can overflow it: N*K, plus E*(align-1) when each expert segment
 * is padded to a multiple of `align`. Returns -1 for invalid arguments.
 * (DeepEP repository dump, deep_ep.cpp, intranode dispatch: num_worst_tokens
 * sizes the receive buffer for the worst case so no host wait is needed.)
 */
int64_t moe_required_capacity(int32_t N, int32_t K, int32_t E, int32_t align);

/* Bytes of device workspace moe_get_layout needs for these sizes (a multiple
 * of 256; 0 only if the arguments are invalid). The contents need no
 * initialization and are scratch between calls. */
size_t moe_layout_workspace_bytes(int32_t N, int32_t K, int32_t E);

/*
 * Routing layout. Defined by DeepEP (repository dump, deep_ep.cpp,
 * Buffer::get_dispatch_layout: num_tokens_per_expert counts the top-k ids per
 * expert) and the expert-contiguous receive buffer of its dispatch, whose
 * recv_src_idx names the source of each received row. Masked ids follow the
 * vLLM branch compare ds-exp-2...ds-exp-ag (mask_topk_ids writes -1).
 *
 *   ids[t*ids_row_stride + k]  (device, int32)  expert of pair (t, k), for
 *        t < N, k < K. Any id < 0 is masked (skipped); an id >= E is
 *        skipped and counted in *status. ids_row_stride >= K, in int32
 *        elements, so the ids may sit inside larger per-token records.
 *   counts[E]       (device, out) valid pairs per expert.
 *   offsets[E+1]    (device, out) offsets[0] = 0, offsets[e+1] = offsets[e]
 *        + counts[e] rounded up to a multiple of `align` (align >= 1);
 *        offsets[E] = rows used.
 *   pos[N*K]        (device, out, row-major [N, K]) the receive row of pair
 *        (t, k), or -1 if masked. Within an expert's segment the rows follow
 *        ascending (t, k): the order is deterministic and independent of
 *        the launch shape.
 *   row_pair[cap]   (device, out) t*K + k of the pair in each row; -1 for
 *        padding rows and rows >= offsets[E].
 *   cap             rows of the receive buffer; must be at least
 *        moe_required_capacity(N, K, E, align) and below 2^31.
 *   order[N*K]      (device, out, may be NULL) the dispatch plan: the order
 *        in which moe_dispatch should visit the pairs. It is not part of the
 *        layout's definition, and any permutation gives the same dispatch:
 *        every valid pair (pos >= 0) appears once, and the remaining entries
 *        are -1. Its arrangement is this library's choice for the memory:
 *        the pairs are taken in tiles of C consecutive pairs, C = N*K / B
 *        rounded up to a multiple of 256 (B = 64 tiles for E <= 256, 32 for
 *        E <= 512, 16 beyond), and a tile lists its valid pairs by
 *        ascending receive row, then -1 for its masked and out-of-range
 *        pairs. The dispatch then writes each tile's rows as one sorted
 *        sweep over the receive buffer, while the tile's source rows stay
 *        in one XCD's L2 (at the prefill shape a tile is 512 pairs, 64
 *        tokens). Batches of at most 2048 pairs, and batches whose tiles
 *        would exceed 4096 pairs, take the index order (-1 for the masked
 *        pairs).
 *   workspace       (device) at least moe_layout_workspace_bytes(N, K, E)
 *        bytes, 4-byte aligned; not shared with a concurrent call.
 *   status          (device, out, may be NULL) number of ids >= E.
 *
 * Launches (the outputs are the same in every form): one for batches of at
 * most 2048 pairs, and one for 2049 .. 32768 pairs whose ids are contiguous
 * (ids_row_stride == K) and start on a 16-byte boundary; two otherwise. The
 * one-launch forms do not touch the workspace, which is still checked.
 *
 * Limits: 1 <= K <= 32, 1 <= E <= 1024, N >= 0, N*K < 2^31. Pointers must be
 * 4-byte aligned. Errors: MOE_ERR_ARG, MOE_ERR_LIMIT, MOE_ERR_CAPACITY,
 * MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_get_layout(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K, int32_t E,
                   int32_t align, int32_t* counts, int32_t* offsets, int32_t* pos,
                   int32_t* row_pair, int64_t cap, int32_t* order, void* workspace,
                   size_t workspace_bytes, int32_t* status, hipStream_t stream);

/*
 * moe_get_layout without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, outputs, limits and
 * errors as moe_get_layout, minus the workspace. Its workspace is a static
 * device array inside the library (65 792 bytes, the most any accepted size
 * needs, one copy per GPU, held until the process ends); the call allocates
 * nothing. Every call on one GPU shares that GPU's copy: calls ordered on
 * one stream are fine, calls that overlap on one GPU (different streams)
 * race. The first call on a device looks up the array's device address
 * (hipGetSymbolAddress) with that device current; a failure there returns
 * MOE_ERR_HIP. Errors: those of moe_get_layout except MOE_ERR_WORKSPACE.
 */
int moe_get_layout_noalloc(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                           int32_t E, int32_t align, int32_t* counts, int32_t* offsets,
                           int32_t* pos, int32_t* row_pair, int64_t cap, int32_t* order,
                           int32_t* status, hipStream_t stream);

/*
 * One payload field of a dispatch: `row_bytes` bytes per token, read from
 * src + t*src_row_stride and written to dst + row*dst_row_stride (device
 * pointers, strides in bytes). The field is copied byte for byte, whatever
 * it holds (fp8/bf16 hidden states, fp32 or byte scales, ids, weights).
 */
typedef struct moe_field {
    const void* src;
    int64_t src_row_stride;
    void* dst;
    int64_t dst_row_stride;
    int64_t row_bytes;
} moe_field;

/*
 * Dispatch. For every token t < N, every k < K with pos[t*K+k] >= 0 and
 * every field f: dst_f row pos[t*K+k] <- src_f row t. Each received row thus
 * carries the token's whole payload, as DeepEP's dispatch returns recv_x,
 * recv_x_scales, recv_topk_idx and recv_topk_weights per received token
 * (repository dump, deep_ep.cpp, Buffer::intranode_dispatch).
 *
 *   fields[nfields]  (host array) 1..4 fields. Separate-tensor mode passes
 *        hidden, scales, ids and weights; packed-record mode passes one
 *        field whose rows are whole per-token records (ids, weights, hidden,
 *        scales at 16-byte aligned offsets, as the per-token tensors are
 *        packed in the vLLM branch compare ds-exp-2...ds-exp-ag,
 *        moe_allgather.cu make_desc).
 *   pos  (device, [N, K] row-major) rows from moe_get_layout. pos == NULL
 *        means the identity pos[t] = t and requires K == 1: that call packs
 *        separate tensors into records or unpacks records into tensors.
 *   order  (device, [N*K], may be NULL) the dispatch plan moe_get_layout
 *        wrote for the same pos: the pairs are copied in the plan's order
 *        (entries -1 are skipped) instead of in index order. The result is
 *        the same byte for byte; only the order of the writes changes, which
 *        the receive buffer's memory prefers (see moe_get_layout). It is a
 *        hint: payloads above 8 KiB per token are copied in index order
 *        whatever order holds, because a tile's source rows would no longer
 *        stay in L2, and so are batches of at most 2048 pairs (for which
 *        moe_get_layout's plan is the index order anyway), sparing each wave
 *        the dependent read of its plan entry. Entries must be -1 or pair
 *        indices below N*K, each valid pair exactly once; they are trusted,
 *        as pos is.
 *
 * Rows no pair maps to are left untouched. Two pairs must not share a row
 * (moe_get_layout guarantees it). Alignment: row_bytes, both strides and
 * both pointers must be multiples of 4; when all of them are multiples of
 * 16 (every field), the copy runs in 16-byte vectors. Limits: 1 <= K <= 32,
 * N*K < 2^31, and one wave per (pair, 64 vectors of the payload) gives
 * N*K*ceil(V/64) < 2^31 with V the payload's vectors per token (its bytes
 * over 16, or over 4 when the 4-byte form runs): a 7456-byte payload
 * (466 vectors) allows N*K < 2^28. Errors: MOE_ERR_ARG, MOE_ERR_LIMIT,
 * MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_dispatch(const moe_field* fields, int32_t nfields, int32_t N, int32_t K,
                 const int32_t* pos, const int32_t* order, hipStream_t stream);

/*
 * Combine. For every token t < N and h < Hc:
 *     acc = +0.0f
 *     for k = 0 .. K-1 with p = pos[t*K+k] >= 0:
 *         acc = fmaf(w[t*w_row_stride + k], float(y[p*y_row_stride + h]), acc)
 *     out[t*out_row_stride + h] = bf16(acc), rounded to nearest even.
 * fp32 accumulation in a fixed order with one rounding to bf16 at the end,
 * as the reduction of the vLLM branch compare ds-exp-2...ds-exp-ag
 * (moe_reduce_scatter.cu, POLL + REDUCE phase); fp32 top-k weights scale the
 * expert outputs as in DeepEP's low_latency_combine (deep_ep.cpp). The
 * result goes straight into the caller's buffer with no staging copy (vLLM
 * PR 49194, "Eliminate staging from NCCL symmetric reduce-scatter"). A token
 * whose pairs are all masked gets +0.
 *
 *   y    (device, bf16 bits) expert outputs, rows as given by pos,
 *        y_row_stride in elements.
 *   w    (device, fp32) top-k weights [N, K], w_row_stride in elements
 *        (>= K; the weights may sit inside per-token records).
 *   pos  (device, int32 [N, K] row-major) rows from moe_get_layout.
 *   out  (device, bf16 bits) [N, Hc], out_row_stride in elements.
 *
 * Alignment: y, out and their strides (in bytes) multiples of 4 and Hc even;
 * when they are multiples of 16 and Hc of 8, the kernel moves 16-byte
 * vectors. w and pos 4-byte aligned. Limits: 1 <= K <= 32, Hc >= 0.
 * Errors: MOE_ERR_ARG, MOE_ERR_LIMIT, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_combine(const void* y, int64_t y_row_stride, const float* w, int64_t w_row_stride,
                const int32_t* pos, int32_t N, int32_t K, int32_t Hc, void* out,
                int64_t out_row_stride, hipStream_t stream);

/*
 * Padded per-expert layout, the receive form of DeepEP's low-latency dispatch
 * (repository dump, deep_ep.cpp, Buffer::low_latency_dispatch: packed_recv_x
 * [num_local_experts, max_tokens, hidden] with packed_recv_count and the
 * source of each row). Expert e owns rows e*M .. e*M+M-1; its pairs take them
 * in ascending (t, k) order, and pairs beyond M are dropped (pos = -1).
 *
 *   counts[E]      (device, out) rows filled per expert, min(pairs, M).
 *   pos[N*K]       (device, out) row of pair (t, k), -1 if masked, out of
 *                  range or dropped.
 *   row_pair[E*M]  (device, out) t*K + k of each row, -1 for unfilled rows.
 *   layout_range[E]  (device, out, int64, may be NULL, 8-byte aligned) the
 *                  single-source form of packed_recv_layout_range
 *                  [num_local_experts, num_ranks]: for expert e, the rows
 *                  that came from this (the only) source, as
 *                  (begin << 32) | count with begin = 0 and count =
 *                  counts[e]. The pages give the tensor's shape and type,
 *                  not the packing of the two numbers into 64 bits; this
 *                  packing is this library's reading.
 *   recv_stats[E]  (device, in/out, int32, may be NULL) the diagnosis
 *                  tensor cumulative_local_expert_recv_stats: counts[e] is
 *                  added to recv_stats[e], so that over calls it holds the
 *                  rows each expert has received.
 *   status         (device, out, may be NULL) two int32: [0] ids >= E,
 *                  [1] pairs dropped for capacity.
 *   workspace      as for moe_get_layout (moe_layout_workspace_bytes).
 * With M >= N and distinct ids per token nothing is dropped. Limits as
 * moe_get_layout, plus M >= 1 and E*M < 2^31. Errors: MOE_ERR_ARG,
 * MOE_ERR_LIMIT, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_get_layout_padded(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                          int32_t E, int32_t M, int32_t* counts, int32_t* pos, int32_t* row_pair,
                          int64_t* layout_range, int32_t* recv_stats, void* workspace,
                          size_t workspace_bytes, int32_t* status, hipStream_t stream);

/* Scale layouts of moe_dispatch_fp8. */
#define MOE_SCALE_ROWS 0   /* fp32 [rows, H/128]: scales[row*scale_row_stride + b] */
#define MOE_SCALE_COLS 1   /* fp32 column-major per expert, [E, H/128, M] */
#define MOE_SCALE_UE8M0 2  /* int32 [E, H/512, M], byte j of a word = exponent of block 4i+j */
#define MOE_SCALE_TOKENS 3 /* fp32 [N, H/128] per token: scales[t*scale_row_stride + b] */

/*
 * Dispatch with an FP8 cast, as DeepEP's low-latency dispatch does with
 * use_fp8 (repository dump, deep_ep.cpp, Buffer::low_latency_dispatch:
 * bf16 x, e4m3 payload, fp32 scales per token and 128 channels stored
 * column-major, or with use_ue8m0 -- which needs round_scale -- power-of-two
 * scales as 8-bit exponents, four per int32). The cast itself is not on the
 * pages; this library takes, per token and 128-channel block b:
 *     amax = max |x|,  s = max(amax / 448, 2^-126)            (fp32)
 *     round_scale: s = the smallest power of two >= s
 *     q[h] = e4m3(x[h] / s)   (fp32 division; e4m3fn, round to nearest
 *                              even, finite overflow saturates to +-448)
 * For every valid pair, row p = pos[t*K+k] gets the H code bytes at
 * dst + p*dst_row_stride and the H/128 scales in scale_format:
 *   MOE_SCALE_ROWS   fp32 scales[p*scale_row_stride + b]
 *   MOE_SCALE_COLS   fp32 scales[((p/M)*(H/128) + b)*M + p%M]   (M = rows_per_expert)
 *   MOE_SCALE_UE8M0  int32 word ((p/M)*(H/512) + b/4)*M + p%M, byte b%4 = biased
 *                    exponent of s (needs round_scale and H % 512 == 0)
 *   MOE_SCALE_TOKENS fp32 scales[t*scale_row_stride + b], once per token and
 *                    for every token (whether or not a pair of it is valid);
 *                    moe_scatter_scales then places them by expert row
 * x: bf16 bits, 16-byte aligned, row stride a multiple of 8 elements;
 * dst: 16-byte aligned, row stride a multiple of 16 bytes; scales 4-byte aligned.
 * H % 128 == 0. Rows no pair maps to are left untouched. Errors:
 * MOE_ERR_ARG, MOE_ERR_ALIGN, MOE_ERR_LIMIT, MOE_ERR_HIP.
 */
int moe_dispatch_fp8(const void* x, int64_t x_row_stride, int32_t N, int32_t K, int32_t H,
                     const int32_t* pos, void* dst, int64_t dst_row_stride, void* scales,
                     int32_t scale_format, int64_t scale_row_stride, int32_t rows_per_expert,
                     int32_t round_scale, hipStream_t stream);

/*
 * Column-major or UE8M0 scales of the padded layout from token-major ones:
 * moe_dispatch_fp8(..., MOE_SCALE_TOKENS into token_scales, ...) followed by
 * this call leaves in `scales` exactly what moe_dispatch_fp8 with
 * MOE_SCALE_COLS / MOE_SCALE_UE8M0 and rows_per_expert = M writes there, when
 * row_pair is the padded layout's (moe_get_layout_padded) for the same pos.
 * The layouts are those of DeepEP's low-latency receive scales (repository
 * dump, deep_ep.cpp, Buffer::low_latency_dispatch: per expert, column-major
 * over the expert's rows; with use_ue8m0, four exponents per int32).
 * It also places per-token scales a caller already holds (its own
 * quantiser's) into the receive layout. For fp32 column-major scales the two
 * calls are faster than the one-call form: written by destination row, each
 * 128-byte line of a column is stored whole, where the one-call form stores
 * each scale on its own beside other tokens' rows.
 *
 * For every row p = e*M + m (e < E, m < M) with 0 <= row_pair[p] < N*K, i.e.
 * pair r = row_pair[p] of token t = r / K:
 *   MOE_SCALE_COLS   scales[(e*(H/128) + b)*M + m] = token_scales[t*tss + b]
 *   MOE_SCALE_UE8M0  int32 word (e*(H/512) + b/4)*M + m, byte b%4 = bits 23..30
 *                    (the exponent field) of token_scales[t*tss + b]; the
 *                    scales must be powers of two (dispatch with round_scale)
 * Other rows (row_pair[p] < 0 or >= N*K) are left untouched.
 * token_scales: fp32 [N, tss], tss = token_scale_row_stride >= H/128;
 * row_pair: int32 [E*M]; scales as above. All device pointers, 4-byte aligned.
 * H % 128 == 0 (UE8M0: H % 512 == 0); N*K and E*M below 2^31. N = 0, E = 0
 * or H = 0 enqueue nothing. Errors: MOE_ERR_ARG, MOE_ERR_ALIGN,
 * MOE_ERR_LIMIT, MOE_ERR_HIP.
 */
int moe_scatter_scales(const float* token_scales, int64_t token_scale_row_stride, int32_t N,
                       int32_t K, int32_t H, const int32_t* row_pair, int32_t E, int32_t M,
                       void* scales, int32_t scale_format, hipStream_t stream);

/*
 * Optional terms applied after the top-k sum by moe_combine_epilogue. All
 * pointers are device pointers to bf16 bits; row strides are in elements. A
 * NULL pointer leaves its term out.
 *   bias0, bias1  [N, Hc] per-token biases added to the fp32 sum (DeepEP
 *                 repository dump, deep_ep.cpp, Buffer::intranode_combine
 *                 takes bias_0 / bias_1 [num_recv_tokens, hidden]; added here
 *                 after the top-k sum, bias0 first).
 *   residual      [N, Hc] skip connection. When given, the sum plus residual
 *                 is written to residual_out and RMS-normalised into out with
 *                 gamma [Hc] and eps, as the fused reduce-scatter + residual +
 *                 RMSNorm kernel of the vLLM branch compare
 *                 ds-exp-2...ds-exp-ag (moe_rs_fused.cu) does.
 */
typedef struct moe_epilogue {
    const void* bias0;
    int64_t bias0_row_stride;
    const void* bias1;
    int64_t bias1_row_stride;
    const void* residual;
    int64_t residual_row_stride;
    const void* gamma;
    float eps;
    void* residual_out;
    int64_t residual_out_row_stride;
} moe_epilogue;

/*
 * Combine with an epilogue. For every token t, with acc[h] the fp32 value
 * moe_combine computes before its final rounding:
 *     acc[h] += bias0[t,h]; acc[h] += bias1[t,h]           (fp32, if given)
 *     without residual:  out[t,h] = bf16(acc[h])
 *     with residual:     acc[h] += residual[t,h];  residual_out[t,h] = bf16(acc[h])
 *                        s = 1 / sqrt(sum_h acc[h]^2 / Hc + eps)
 *                        out[t,h] = bf16(acc[h] * s * gamma[h])
 * residual_out is bit-exact with that definition; out of the RMSNorm is within
 * one bf16 ulp of it (the sum of squares is an fp32 tree sum, s a hardware
 * reciprocal square root). ep == NULL is moe_combine.
 *
 * Alignment: y, out and every given row pointer 16-byte aligned with strides
 * multiples of 8 elements, Hc a multiple of 8. Limits: Hc <= 65536 when any
 * term is given, 1 <= K <= 32, eps >= 0. Errors: MOE_ERR_ARG (residual
 * without gamma or residual_out, negative eps), MOE_ERR_ALIGN, MOE_ERR_LIMIT,
 * MOE_ERR_HIP.
 */
int moe_combine_epilogue(const void* y, int64_t y_row_stride, const float* w,
                         int64_t w_row_stride, const int32_t* pos, int32_t N, int32_t K,
                         int32_t Hc, const moe_epilogue* ep, void* out, int64_t out_row_stride,
                         hipStream_t stream);

/*
 * Per-token records: up to 4 fields (e.g. ids, weights, hidden, scales) at
 * 16-byte aligned offsets inside one record per token, the packing of the
 * vLLM branch compare ds-exp-2...ds-exp-ag (moe_allgather.cu, make_desc),
 * here one record per token as the packed-record workload has it.
 *
 * moe_record_offsets (host only, no GPU): offsets[f] = the offset of field f
 * (the running end rounded up to 16); returns the record size (the end
 * rounded up to 16), or a negative MOE_ERR_ARG when nfields is outside 1..4
 * or a row_bytes is negative or not a multiple of 4. offsets may be NULL.
 *
 * moe_pack_records: for every token t and field f, copies fields[f].row_bytes
 * bytes from fields[f].src + t*fields[f].src_row_stride to records +
 * t*record_row_stride + offsets[f] (the fields' dst members are ignored).
 * moe_unpack_records: the reverse, into fields[f].dst + t*dst_row_stride
 * (src members ignored). Both are moe_dispatch with K = 1 and pos = NULL on
 * redirected fields, with its alignment rules (16-byte alignment of the
 * records, their stride and the fields gives the 16-byte path) and errors;
 * record_row_stride must be at least the record size (MOE_ERR_ARG).
 */
int64_t moe_record_offsets(const int64_t* row_bytes, int32_t nfields, int64_t* offsets);
int moe_pack_records(const moe_field* fields, int32_t nfields, int32_t N, void* records,
                     int64_t record_row_stride, hipStream_t stream);
int moe_unpack_records(const void* records, int64_t record_row_stride, int32_t N,
                       const moe_field* fields, int32_t nfields, hipStream_t stream);

/*
 * Layout and dispatch in one launch, for small (decode-sized) batches: the
 * same results as moe_get_layout(ids, ..., E, align, counts, offsets, pos,
 * row_pair, cap, ..., status) followed by moe_dispatch(fields, nfields, N, K,
 * pos), bit for bit, without the layout's workspace. Every workgroup derives
 * the offsets and its token's rows from one pass over the batch's ids, so the
 * three launches of the two calls become one. Cited passages: those of
 * moe_get_layout and moe_dispatch (DeepEP repository dump, deep_ep.cpp,
 * Buffer::get_dispatch_layout, Buffer::intranode_dispatch).
 *
 * Arguments, layouts and alignment are those of the two calls (status may be
 * NULL). counts, offsets and row_pair are written even when N = 0. Limits:
 * N*K <= 8192 (larger batches: the two calls), 1 <= K <= 32,
 * 1 <= E <= 1024, cap >= moe_required_capacity(N, K, E, align), cap < 2^31,
 * and at most 2^23 workgroups in the one launch: N * ceil(V / 256) with V
 * the payload's vectors per token (16 or 4 bytes). Errors: MOE_ERR_ARG,
 * MOE_ERR_ALIGN, MOE_ERR_LIMIT, MOE_ERR_CAPACITY, MOE_ERR_HIP.
 */
int moe_layout_dispatch(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                        int32_t E, int32_t align, int32_t* counts, int32_t* offsets, int32_t* pos,
                        int32_t* row_pair, int64_t cap, int32_t* status, const moe_field* fields,
                        int32_t nfields, hipStream_t stream);

/*
 * Padded layout and FP8 dispatch in one launch, for small (decode-sized)
 * batches: the same results as moe_get_layout_padded(ids, ..., E, M, counts,
 * pos, row_pair, ..., status) followed by moe_dispatch_fp8(x, ..., pos, dst,
 * ..., scales, scale_format, ..., M, round_scale), bit for bit, without the
 * layout's workspace. In the padded layout the row of a pair needs no global
 * offsets (expert e starts at e*M), so every workgroup finds its token's rows
 * from one pass over the batch's ids; the launch count at decode drops from
 * three to one. Cited passages: those of moe_get_layout_padded and
 * moe_dispatch_fp8 (DeepEP repository dump, deep_ep.cpp,
 * Buffer::low_latency_dispatch).
 *
 * Arguments, layouts and alignment are those of the two calls it replaces
 * (ids with a row stride in elements; x bf16; dst, scales as in
 * moe_dispatch_fp8 with rows_per_expert = M; status[2]; layout_range and
 * recv_stats optional, as in moe_get_layout_padded). counts, row_pair,
 * status, layout_range and recv_stats are written even when N = 0. Limits: N*K <= 8192 (larger batches:
 * the two calls), 1 <= K <= 32, 1 <= E <= 1024, M >= 1, E*M < 2^31,
 * H % 128 == 0, and at most 2^23 workgroups in the one launch:
 * N * ceil(H / 4096). Errors: MOE_ERR_ARG, MOE_ERR_ALIGN, MOE_ERR_LIMIT,
 * MOE_ERR_HIP.
 */
int moe_dispatch_fp8_padded(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                            int32_t E, int32_t M, const void* x, int64_t x_row_stride, int32_t H,
                            int32_t* counts, int32_t* pos, int32_t* row_pair,
                            int64_t* layout_range, int32_t* recv_stats, int32_t* status,
                            void* dst, int64_t dst_row_stride, void* scales, int32_t scale_format,
                            int64_t scale_row_stride, int32_t round_scale, hipStream_t stream);

/*
 * Backward of the dispatch (DeepEP repository dump, README, "Example use in
 * model training": the backward of a dispatch is a combine of the received
 * rows' gradients, with the received top-k weights' gradients combined
 * alongside). For the forward recv[pos[t,k]] = x[t]:
 *     grad_x[t,h] = bf16(fp32 sum over valid k, ascending, from +0, of
 *                        grad_recv[pos[t,k], h])
 *     grad_w[t,j] = fp32 sum over valid k, ascending, of grad_recv_w[pos[t,k], j]
 * (j < K: the weights row every received row carried). Masked pairs
 * (pos < 0) add nothing; an all-masked token gets +0. grad_recv_w and
 * grad_w are both NULL (no weight gradients) or both given. Results are
 * bit-exact with that definition.
 *
 * grad_recv [rows, H] and grad_x [N, H] are bf16 with row strides in
 * elements (>= H, even; 16-byte vectors when both are 16-byte aligned with
 * strides and H multiples of 8), grad_recv_w [rows, >= K] and grad_w
 * [N, >= K] fp32 with row strides in floats. pos is moe_get_layout's (or
 * moe_get_layout_padded's). Limits: 1 <= K <= 32, N*K < 2^31. Errors:
 * MOE_ERR_ARG (NULL pointer, only one of grad_recv_w / grad_w, stride below
 * its row), MOE_ERR_ALIGN (odd H or stride, pointer not 4-byte aligned),
 * MOE_ERR_LIMIT, MOE_ERR_HIP.
 */
int moe_dispatch_backward(const void* grad_recv, int64_t grad_recv_row_stride,
                          const float* grad_recv_w, int64_t grad_recv_w_row_stride,
                          const int32_t* pos, int32_t N, int32_t K, int32_t H, void* grad_x,
                          int64_t grad_x_row_stride, float* grad_w, int64_t grad_w_row_stride,
                          hipStream_t stream);

/*
 * Backward of the combine (same README passage: the backward of a combine
 * is a dispatch). For the forward out[t] = sum_k w[t,k] * y[pos[t,k]]:
 *     grad_y[pos[t,k], h] = bf16(w[t,k] * grad_out[t,h])   (one fp32 product)
 *     grad_w[t,k] = sum_h grad_out[t,h] * y[pos[t,k], h]   (fp32)
 * grad_y is bit-exact with that definition; rows of grad_y that no pair
 * lands on are not written. grad_w is 0 for masked pairs; otherwise each
 * lane of a 1024-thread workgroup keeps an fp32 FMA chain over its channels
 * (8 per 16-byte vector), then a fixed butterfly over the 64 lanes of a wave
 * and the 16 waves in order: within (8*ceil(Hc/8192) + 22) * 2^-24 *
 * sum_h |grad_out[t,h] * y[pos[t,k],h]| of the exact value, and the same on
 * every run. grad_w == NULL skips the weight gradients (y may then be NULL
 * and is not read).
 *
 * grad_out [N, Hc], y [rows, Hc] and grad_y [rows, Hc] are bf16, 16-byte
 * aligned with row strides multiples of 8 elements and >= Hc; Hc a multiple
 * of 8. w [N, >= K] and grad_w [N, >= K] fp32. Limits: Hc <= 32768,
 * 1 <= K <= 32. Errors: MOE_ERR_ARG (NULL pointer, grad_w without y, stride
 * below its row), MOE_ERR_ALIGN, MOE_ERR_LIMIT, MOE_ERR_HIP.
 */
int moe_combine_backward(const void* grad_out, int64_t grad_out_row_stride, const float* w,
                         int64_t w_row_stride, const void* y, int64_t y_row_stride,
                         const int32_t* pos, int32_t N, int32_t K, int32_t Hc, void* grad_y,
                         int64_t grad_y_row_stride, float* grad_w, int64_t grad_w_row_stride,
                         hipStream_t stream);

/*
 * Device check of a layout's index arrays. moe_dispatch, moe_combine and the
 * other calls that take pos do not bound-check it (a row outside the receive
 * buffer is an out-of-bounds access); a caller whose pos comes from
 * elsewhere can check it with this call first. What it checks restates the
 * layout's definition (DeepEP, repository dump, deep_ep.cpp,
 * Buffer::get_dispatch_layout, and the receive buffer whose recv_src_idx
 * names each row's source): each pair has one row or none, each used row
 * names its pair, and the dispatch plan lists pairs that have rows.
 *
 *   pos[N*K]       (device) rows of the pairs, as moe_get_layout writes them.
 *   row_pair[cap]  (device, may be NULL) the pair of each row, -1 if none.
 *   cap            rows of the receive buffer (E*M for a padded layout).
 *   order[N*K]     (device, may be NULL) a dispatch plan.
 *   status[4]      (device, in/out) counts added to it (it is not cleared):
 *     [0] pairs whose pos is neither -1 nor a row < cap;
 *     [1] pairs with a row whose row_pair entry does not name them (two pairs
 *         in one row, or a row_pair that disagrees; row_pair given);
 *     [2] rows whose row_pair entry is neither -1 nor a pair whose pos is
 *         that row (row_pair given);
 *     [3] plan entries that are neither -1 nor a pair with a row (order
 *         given).
 * All four zero: pos and row_pair are inverse maps between the valid pairs
 * and the used rows, and every row moe_dispatch would write lies in the
 * receive buffer. A plan that repeats or omits a pair is not detected (the
 * dispatch then writes a row twice or not at all, within the buffer). Every
 * read the check makes is guarded by the ranges it checks, so any input is
 * safe. Limits: N*K and cap below 2^31. Errors: MOE_ERR_ARG, MOE_ERR_LIMIT,
 * MOE_ERR_ALIGN (int32 pointers 4-byte aligned), MOE_ERR_HIP.
 */
int moe_check_layout(const int32_t* pos, int32_t N, int32_t K, const int32_t* row_pair,
                     int64_t cap, const int32_t* order, int32_t* status, hipStream_t stream);

/*
 * The debug build's status (the library built with MOE_DEBUG,
 * libmoe_get_debug.so). There, every call that writes a layout
 * (moe_get_layout, moe_get_layout_noalloc, moe_get_layout_padded,
 * moe_layout_dispatch, moe_dispatch_fp8_padded) also runs moe_check_layout
 * on its own outputs, on its stream, adding to counters per GPU that start
 * at zero when the library loads: out[0..3] as moe_check_layout's status,
 * out[4] the number of layout calls checked. moe_debug_status copies the
 * five to out[5] (host memory) after the stream's earlier work, and with
 * reset != 0 then sets them to zero on the stream. out[0..3] all zero: every
 * layout since the last reset was consistent. Errors: MOE_ERR_LIMIT in the
 * release build; MOE_ERR_ARG (out NULL), MOE_ERR_HIP.
 */
int moe_debug_status(int32_t* out, int32_t reset, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GET_H */
