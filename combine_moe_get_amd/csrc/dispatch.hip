// dispatch.hip -- byte scatter of each token's payload fields into the
// receive rows the layout assigned to its (token, k) pairs.
//
// Definition: every received row carries its token's whole payload, as
// DeepEP's dispatch returns recv_x, recv_x_scales, recv_topk_idx and
// recv_topk_weights per received token (repository dump, deep_ep.cpp,
// Buffer::intranode_dispatch); fields are opaque bytes at 16-byte
// granularity, as the tensors packed by make_desc in the vLLM branch
// compare ds-exp-2...ds-exp-ag (moe_allgather.cu).
//
// Launch shape: one wave per (token, k, 64-vector segment of the
// concatenated fields), segments of one receive row on consecutive waves.
// Each lane loads one vector of the token's source row and stores it to the
// pair's receive row; the K waves of a token re-read the same source bytes.
// Workgroups are handed to the 8 XCDs round-robin, each XCD with its own L2,
// so the kernel renumbers them: XCD x runs the x-th contiguous eighth of the
// work, which keeps all waves of a token on one XCD and its re-reads in that
// L2 (without this, measured source reads were 4x the source bytes). Every
// load and store instruction of a wave covers 64 consecutive vectors of one
// row (1 KiB with 16-byte vectors). Measured
// on MI355X at the prefill shape, this many-short-waves form writes faster
// than one wave storing each loaded vector K times, and only with
// non-temporal stores.
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kXcds = 8;   // MI355X: 8 XCDs, workgroup i runs on XCD i % 8
// The layout's plan visits a tile of ~4096 pairs (512 tokens of top-8) in
// receive-row order, which re-reads each source row from L2 only while the
// tile's source rows fit in an XCD's 4 MB L2: payloads of at most this many
// bytes per token. Larger payloads take the pairs in index order, where the
// K pairs of a token are copied together.
constexpr int64_t kPlanMaxPayloadBytes = 8192;

// Receive bytes up to which the rows take ordinary stores (and stay in the
// caches) rather than non-temporal ones. Measured with prefill-shaped rows
// (7456 bytes per token): the one-launch layout+dispatch at 128 tokens
// (7.6 MB) 9.70 -> 9.45 us per decode step with ordinary stores, while at
// 1024 tokens (61 MB) the dispatch took 32.6 against 35.1 us and at 4096
// tokens 67 against 98 us with non-temporal ones.
constexpr int64_t kPlainStoreMaxBytes = (int64_t)16 << 20;

// Whether a dispatch of N*K rows of `payload` bytes takes ordinary stores.
inline bool plain_stores(int64_t N, int64_t K, int64_t payload) {
    return N * K * payload <= kPlainStoreMaxBytes;
}

struct DispatchArgs {
    const char* src[MOE_MAX_FIELDS];
    char* dst[MOE_MAX_FIELDS];
    int64_t sstride[MOE_MAX_FIELDS];
    int64_t dstride[MOE_MAX_FIELDS];
    int32_t vend[MOE_MAX_FIELDS];  // running end of each field, in vectors
    const int32_t* pos;            // NULL: identity, K == 1
    const int32_t* order;          // NULL: pairs in index order; else the plan's order (-1: skip)
    int32_t N;
    int32_t K;
    int32_t V;                     // vectors per token over all fields
    int32_t segs;                  // 64-vector segments per token
};

// Stores one vector of a receive row: non-temporal (streamed out) or
// ordinary (kept in the caches), chosen per launch by plain_stores.
template <bool PLAIN, typename VecT>
__device__ __forceinline__ void store_row(VecT val, VecT* q) {
    if constexpr (PLAIN)
        *q = val;
    else
        __builtin_nontemporal_store(val, q);
}

template <typename VecT, bool PLAIN>
__global__ __launch_bounds__(kThreads) void dispatch_kernel(const DispatchArgs a,
                                                            uint32_t first_block) {
    const int lane = threadIdx.x & (kWave - 1);
    // Logical workgroup: XCD (blockIdx % 8) takes a contiguous eighth of this
    // launch's range. The grid is a multiple of 8, so this is a bijection
    // onto [first_block, first_block + gridDim.x).
    const uint32_t per_xcd = gridDim.x / kXcds;
    const uint32_t lb = first_block + (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const uint32_t gw = lb * kWavesPerBlock + threadIdx.x / kWave;
    const uint32_t item = __builtin_amdgcn_readfirstlane(gw / (uint32_t)a.segs);
    if (item >= (uint32_t)a.N * (uint32_t)a.K) return;
    const int32_t seg = (int32_t)(gw - item * (uint32_t)a.segs);
    const int32_t v = seg * kWave + lane;
    if (v >= a.V) return;
    // The pair this wave copies (t*K + k): the item-th of the layout's plan,
    // or the item-th pair itself.
    const int32_t planned = a.order ? a.order[item] : (int32_t)item;
    if (planned < 0) return;
    const uint32_t pair = (uint32_t)planned;
    // The row is fetched before the token is derived, so that the two
    // dependent fetches (plan entry, then row) are not held apart by the
    // division. pos == NULL is the identity, with K == 1.
    const int32_t p = a.pos ? a.pos[pair] : (int32_t)pair;
    if (p < 0) return;
    const int32_t t = __builtin_amdgcn_readfirstlane(pair / (uint32_t)a.K);

    // Which field this lane's vector belongs to, and its offset inside it.
    const int f1 = v >= a.vend[0], f2 = v >= a.vend[1], f3 = v >= a.vend[2];
    const char* src = f3 ? a.src[3] : f2 ? a.src[2] : f1 ? a.src[1] : a.src[0];
    char* dst = f3 ? a.dst[3] : f2 ? a.dst[2] : f1 ? a.dst[1] : a.dst[0];
    const int64_t ss = f3 ? a.sstride[3] : f2 ? a.sstride[2] : f1 ? a.sstride[1] : a.sstride[0];
    const int64_t ds = f3 ? a.dstride[3] : f2 ? a.dstride[2] : f1 ? a.dstride[1] : a.dstride[0];
    const int32_t v0 = f3 ? a.vend[2] : f2 ? a.vend[1] : f1 ? a.vend[0] : 0;
    const int64_t inner = (int64_t)(v - v0) * sizeof(VecT);

    // Receive rows are written once and not read back by this pass: past
    // kPlainStoreMaxBytes, non-temporal stores stream them out instead of
    // parking them as dirty lines in the caches, where the combine that
    // follows would pay for the write-back.
    const VecT val = *reinterpret_cast<const VecT*>(src + (int64_t)t * ss + inner);
    store_row<PLAIN>(val, reinterpret_cast<VecT*>(dst + (int64_t)p * ds + inner));
}

// ---------------------------------------------------------------------------
// Layout and dispatch in one launch, for small batches (N*K <= 8192). The
// row of pair (t, k) with expert e is offsets[e] + r, r the number of
// earlier pairs in (t, k) order with expert e; offsets is the exclusive scan
// of the aligned per-expert totals. Both come from one pass over the batch's
// ids, cheap enough at this size for every workgroup to make it itself.
// Workgroup (t, g) takes token t and the 64-vector segments 4g .. 4g+3 of its
// concatenated fields (one per wave):
//   1. its segment loads are issued first; then one pass over all ids gives
//      the per-expert totals (LDS integer atomics: order-independent), the
//      out-of-range count and, per expert, the pairs of earlier tokens;
//   2. the offsets: an exclusive scan of the aligned totals over E <= 1024;
//   3. the token's rows; workgroup (t, 0) writes pos and row_pair, workgroup
//      0 counts, offsets and status, and the unused rows (alignment padding
//      of expert e by workgroup e mod grid, rows past the used ones by all)
//      are marked -1 -- used and unused rows are disjoint sets derived from
//      the same totals;
//   4. each wave stores its vectors to the K rows (store_row).
// ---------------------------------------------------------------------------

constexpr int kFusedMaxPairs = 8192;

struct FusedLayout {
    const int32_t* ids;
    int64_t ids_stride;
    int32_t E, align, groups;
    int64_t cap;
    int32_t* counts;
    int32_t* offsets;
    int32_t* pos;
    int32_t* row_pair;
    int32_t* order;    // the dispatch plan of a layout-only call (may be NULL)
    int32_t* status;
};

template <typename VecT, bool PLAIN>
__global__ __launch_bounds__(kThreads) void layout_dispatch_kernel(const DispatchArgs a,
                                                                   const FusedLayout f) {
    __shared__ int32_t tot[MOE_MAX_EXPERTS];
    __shared__ int32_t off[MOE_MAX_EXPERTS + 1];
    __shared__ int32_t bef[MOE_MAX_EXPERTS];
    __shared__ int32_t rows[MOE_MAX_TOPK];
    __shared__ int32_t tok_e[MOE_MAX_TOPK];
    __shared__ int32_t wave_sums[kWavesPerBlock];
    __shared__ int32_t nbad_s;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t t = blockIdx.x / (uint32_t)f.groups;
    const int32_t g = (int32_t)(blockIdx.x - t * (uint32_t)f.groups);
    const int32_t K = a.K, E = f.E;
    const int32_t nk = a.N * K;
    const bool has_token = t < (uint32_t)a.N;   // N = 0: one workgroup, layout outputs only

    // 1. this wave's vector of the token's payload, loaded before the count
    const int32_t seg = g * kWavesPerBlock + wave;
    const int32_t v = seg * kWave + lane;
    const bool moves = has_token && v < a.V;
    const int f1 = v >= a.vend[0], f2 = v >= a.vend[1], f3 = v >= a.vend[2];
    const char* src = f3 ? a.src[3] : f2 ? a.src[2] : f1 ? a.src[1] : a.src[0];
    char* dst = f3 ? a.dst[3] : f2 ? a.dst[2] : f1 ? a.dst[1] : a.dst[0];
    const int64_t ss = f3 ? a.sstride[3] : f2 ? a.sstride[2] : f1 ? a.sstride[1] : a.sstride[0];
    const int64_t ds = f3 ? a.dstride[3] : f2 ? a.dstride[2] : f1 ? a.dstride[1] : a.dstride[0];
    const int32_t v0 = f3 ? a.vend[2] : f2 ? a.vend[1] : f1 ? a.vend[0] : 0;
    const int64_t inner = (int64_t)(v - v0) * sizeof(VecT);
    VecT val{};
    if (moves) val = *reinterpret_cast<const VecT*>(src + (int64_t)t * ss + inner);

    for (int e = threadIdx.x; e < E; e += kThreads) {
        tot[e] = 0;
        bef[e] = 0;
    }
    if ((int32_t)threadIdx.x < K)
        tok_e[threadIdx.x] = has_token ? f.ids[(int64_t)t * f.ids_stride + threadIdx.x] : -1;
    if (threadIdx.x == 0) nbad_s = 0;
    __syncthreads();

    count_batch_ids(f.ids, f.ids_stride, nk, K, E, (int32_t)t * K, tot, bef, &nbad_s);
    __syncthreads();

    // 2. offsets: thread i scans experts 4i .. 4i+3 (E <= 1024)
    int32_t mine[4], sum4 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = threadIdx.x * 4 + j;
        mine[j] = e < E ? tot[e] : 0;
    }
    if (f.align > 1) {
        // cap >= N*K + E*(align - 1) and cap < 2^31 (host checks): 32 bits
        const uint32_t al = (uint32_t)f.align;
#pragma unroll
        for (int j = 0; j < 4; ++j) mine[j] = (int32_t)(((uint32_t)mine[j] + al - 1u) / al * al);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) sum4 += mine[j];
    const int32_t x = wave_inclusive_scan(sum4);
    if (lane == kWave - 1) wave_sums[wave] = x;
    __syncthreads();
    int32_t run = x - sum4, used = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        run += w < wave ? wave_sums[w] : 0;
        used += wave_sums[w];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = threadIdx.x * 4 + j;
        if (e < E) off[e] = run;
        run += mine[j];
    }
    if (threadIdx.x == 0) off[E] = used;
    __syncthreads();

    // 3. rows of the token's pairs; layout outputs
    if (has_token && (int32_t)threadIdx.x < K) {
        const int32_t k = threadIdx.x;
        const int32_t e = tok_e[k];
        int32_t p = -1;
        if (e >= 0 && e < E) p = off[e] + rank_in_expert(tok_e, bef, k);
        rows[k] = p;
        if (g == 0) {
            f.pos[(int64_t)t * K + k] = p;
            if (p >= 0) f.row_pair[p] = (int32_t)t * K + k;
            // small batches: the plan is the pairs in index order, -1 for
            // the masked and out-of-range ones
            if (f.order != nullptr) f.order[(int64_t)t * K + k] = p >= 0 ? (int32_t)t * K + k : -1;
        }
    }
    if (blockIdx.x == 0) {
        for (int e = threadIdx.x; e < E; e += kThreads) {
            f.counts[e] = tot[e];
            f.offsets[e] = off[e];
        }
        if (threadIdx.x == 0) {
            f.offsets[E] = used;
            if (f.status != nullptr) f.status[0] = nbad_s;
        }
    }
    const uint32_t B = gridDim.x;
    if (f.align > 1)
        for (int32_t e = blockIdx.x; e < E; e += (int32_t)B)
            for (int32_t r = off[e] + tot[e] + threadIdx.x; r < off[e + 1]; r += kThreads)
                f.row_pair[r] = -1;
    for (int64_t r = used + (int64_t)blockIdx.x * kThreads + threadIdx.x; r < f.cap;
         r += (int64_t)B * kThreads)
        f.row_pair[r] = -1;
    __syncthreads();

    // 4. the token's vectors to its K rows
    if (!moves) return;
    for (int32_t k = 0; k < K; ++k) {
        const int32_t p = rows[k];
        if (p >= 0) store_row<PLAIN>(val, reinterpret_cast<VecT*>(dst + (int64_t)p * ds + inner));
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

// Validates the payload fields and fills a's field tables (vector ends in
// units of 16 or 4 bytes, *all16 says which). Returns MOE_OK or an error set
// through fail() with `who` as its prefix.
static int prepare_fields(const moe_field* fields, int32_t nfields, int32_t N, DispatchArgs& a,
                          bool* all16_out, int64_t* total_out, const char* who) {
    if (fields == nullptr || nfields < 1 || nfields > MOE_MAX_FIELDS)
        return fail(MOE_ERR_ARG, "%s: need 1..%d fields (got %d%s)", who, MOE_MAX_FIELDS,
                    nfields, fields ? "" : ", NULL array");
    bool all16 = true;
    int64_t total_bytes = 0;
    for (int f = 0; f < nfields; ++f) {
        const moe_field& d = fields[f];
        if (d.row_bytes < 0) return fail(MOE_ERR_ARG, "%s: field %d row_bytes < 0", who, f);
        if (d.row_bytes > 0 && N > 0 && (d.src == nullptr || d.dst == nullptr))
            return fail(MOE_ERR_ARG, "%s: field %d has a NULL pointer", who, f);
        if (!aligned(d.src, 4) || !aligned(d.dst, 4) || !aligned(d.src_row_stride, 4) ||
            !aligned(d.dst_row_stride, 4) || !aligned(d.row_bytes, 4))
            return fail(MOE_ERR_ALIGN, "%s: field %d pointers, strides and row_bytes must be "
                        "multiples of 4 bytes", who, f);
        if (N > 1 && d.src_row_stride < d.row_bytes)
            return fail(MOE_ERR_ARG, "%s: field %d src_row_stride < row_bytes", who, f);
        if (d.dst_row_stride < d.row_bytes)
            return fail(MOE_ERR_ARG, "%s: field %d dst_row_stride < row_bytes", who, f);
        all16 = all16 && aligned(d.src, 16) && aligned(d.dst, 16) &&
                aligned(d.src_row_stride, 16) && aligned(d.dst_row_stride, 16) &&
                aligned(d.row_bytes, 16);
        total_bytes += d.row_bytes;
    }
    const int vb = all16 ? 16 : 4;
    if (total_bytes / vb >= ((int64_t)1 << 30))
        return fail(MOE_ERR_LIMIT, "%s: %lld payload bytes per token is too large", who,
                    (long long)total_bytes);
    int32_t vend = 0;
    for (int f = 0; f < MOE_MAX_FIELDS; ++f) {
        if (f < nfields) {
            a.src[f] = static_cast<const char*>(fields[f].src);
            a.dst[f] = static_cast<char*>(fields[f].dst);
            a.sstride[f] = fields[f].src_row_stride;
            a.dstride[f] = fields[f].dst_row_stride;
            vend += (int32_t)(fields[f].row_bytes / vb);
        }
        a.vend[f] = vend;
    }
    a.V = vend;
    a.segs = ceil_div<int32_t>(vend, kWave);
    *all16_out = all16;
    *total_out = total_bytes;
    return MOE_OK;
}

extern "C" int moe_dispatch(const moe_field* fields, int32_t nfields, int32_t N, int32_t K,
                            const int32_t* pos, const int32_t* order, hipStream_t stream) {
    if (N < 0 || K < 1) return fail(MOE_ERR_ARG, "moe_dispatch: need N >= 0, K >= 1");
    if (K > MOE_MAX_TOPK) return fail(MOE_ERR_LIMIT, "moe_dispatch: K=%d > %d", K, MOE_MAX_TOPK);
    if ((int64_t)N * K >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_dispatch: N*K must be below 2^31");
    if (pos == nullptr && K != 1 && N > 0)
        return fail(MOE_ERR_ARG, "moe_dispatch: pos == NULL (identity) requires K == 1");
    if (!aligned(pos, 4) || !aligned(order, 4))
        return fail(MOE_ERR_ALIGN, "moe_dispatch: pos and order must be 4-byte aligned");
    DispatchArgs a{};
    bool all16 = true;
    int64_t total_bytes = 0;
    const int rc = prepare_fields(fields, nfields, N, a, &all16, &total_bytes, "moe_dispatch");
    if (rc != MOE_OK) return rc;
    if (N == 0 || total_bytes == 0) return ok();
    a.pos = pos;
    // The plan is followed only where it can pay: payloads whose tile of
    // source rows stays in L2, and batches past kOneLaunchPairs pairs (for
    // which the layout's plan is not the index order; below, reading a plan
    // entry would only add a dependent load before each wave's row).
    a.order = total_bytes <= kPlanMaxPayloadBytes && (int64_t)N * K > kOneLaunchPairs ? order
                                                                                       : nullptr;
    a.N = N;
    a.K = K;
    const int64_t waves = (int64_t)N * K * a.segs;
    if (waves >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_dispatch: N*K*segments=%lld waves must be below 2^31",
                    (long long)waves);
    const int64_t blocks = ceil_div<int64_t>(ceil_div<int64_t>(waves, kWavesPerBlock), kXcds) * kXcds;
    constexpr int64_t kPiece = kMaxLaunchItems / kThreads;
    static_assert(kPiece % kXcds == 0, "every piece must keep the XCD renumbering a bijection");
    clear_launch_error();
    const bool plain = plain_stores(N, K, total_bytes);
    in_pieces(blocks, kPiece, [&](int64_t first, int64_t count) {
        if (all16 && plain)
            dispatch_kernel<u32x4, true><<<(uint32_t)count, kThreads, 0, stream>>>(a, (uint32_t)first);
        else if (all16)
            dispatch_kernel<u32x4, false><<<(uint32_t)count, kThreads, 0, stream>>>(a, (uint32_t)first);
        else if (plain)
            dispatch_kernel<uint32_t, true><<<(uint32_t)count, kThreads, 0, stream>>>(a, (uint32_t)first);
        else
            dispatch_kernel<uint32_t, false><<<(uint32_t)count, kThreads, 0, stream>>>(a, (uint32_t)first);
    });
    return check_launch("moe_dispatch");
}

// Launches the one-launch layout+dispatch kernel for the payload in `a`
// (a.V = 0: the layout part only): one workgroup per (token, group of
// kWavesPerBlock segments); N = 0 still runs one workgroup, since counts,
// offsets, status and row_pair are outputs.
static int launch_layout_dispatch(const DispatchArgs& a, bool all16, const int32_t* ids,
                                  int64_t ids_row_stride, int32_t E, int32_t align,
                                  int32_t* counts, int32_t* offsets, int32_t* pos,
                                  int32_t* row_pair, int64_t cap, int32_t* order,
                                  int32_t* status, hipStream_t stream, const char* who) {
    FusedLayout f;
    f.ids = ids;
    f.ids_stride = ids_row_stride;
    f.E = E;
    f.align = align;
    f.groups = a.segs > 0 ? ceil_div<int32_t>(a.segs, kWavesPerBlock) : 1;
    f.cap = cap;
    f.counts = counts;
    f.offsets = offsets;
    f.pos = pos;
    f.row_pair = row_pair;
    f.order = order;
    f.status = status;
    const int64_t blocks = a.N > 0 ? (int64_t)a.N * f.groups : 1;
    if (blocks > kMaxLaunchItems / kThreads)
        return fail(MOE_ERR_LIMIT, "%s: %lld workgroups (tokens x payload segments / %d) exceed "
                    "one launch", who, (long long)blocks, kWavesPerBlock);
    const bool plain = plain_stores(a.N, a.K, (int64_t)a.V * (all16 ? 16 : 4));
    clear_launch_error();
    if (all16 && plain)
        layout_dispatch_kernel<u32x4, true><<<(uint32_t)blocks, kThreads, 0, stream>>>(a, f);
    else if (all16)
        layout_dispatch_kernel<u32x4, false><<<(uint32_t)blocks, kThreads, 0, stream>>>(a, f);
    else if (plain)
        layout_dispatch_kernel<uint32_t, true><<<(uint32_t)blocks, kThreads, 0, stream>>>(a, f);
    else
        layout_dispatch_kernel<uint32_t, false><<<(uint32_t)blocks, kThreads, 0, stream>>>(a, f);
    const int rc = check_launch(who);
    if (rc != MOE_OK) return rc;
    return debug_check_layout(who, pos, (int64_t)a.N * a.K, row_pair, cap, order, stream);
}

extern "C" int moe_layout_dispatch(const int32_t* ids, int64_t ids_row_stride, int32_t N,
                                   int32_t K, int32_t E, int32_t align, int32_t* counts,
                                   int32_t* offsets, int32_t* pos, int32_t* row_pair, int64_t cap,
                                   int32_t* status, const moe_field* fields, int32_t nfields,
                                   hipStream_t stream) {
    if (N < 0 || K < 1 || E < 1 || align < 1)
        return fail(MOE_ERR_ARG, "moe_layout_dispatch: need N >= 0, K >= 1, E >= 1, align >= 1");
    if (K > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_LIMIT, "moe_layout_dispatch: K=%d E=%d beyond K <= %d, E <= %d", K, E,
                    MOE_MAX_TOPK, MOE_MAX_EXPERTS);
    if ((int64_t)N * K > kFusedMaxPairs)
        return fail(MOE_ERR_LIMIT, "moe_layout_dispatch: N*K=%lld above %d (use moe_get_layout + "
                    "moe_dispatch)", (long long)N * K, kFusedMaxPairs);
    const int64_t need = moe_required_capacity(N, K, E, align);
    if (cap < need)
        return fail(MOE_ERR_CAPACITY, "moe_layout_dispatch: cap=%lld below the worst case %lld",
                    (long long)cap, (long long)need);
    if (cap >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_layout_dispatch: cap must be below 2^31");
    if (counts == nullptr || offsets == nullptr || (cap > 0 && row_pair == nullptr))
        return fail(MOE_ERR_ARG, "moe_layout_dispatch: counts, offsets and row_pair must not be "
                    "NULL");
    if (N > 0 && (ids == nullptr || pos == nullptr || ids_row_stride < K))
        return fail(MOE_ERR_ARG, "moe_layout_dispatch: NULL ids/pos or ids_row_stride < K");
    if (!aligned(ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(pos, 4) ||
        !aligned(row_pair, 4) || !aligned(status, 4))
        return fail(MOE_ERR_ALIGN, "moe_layout_dispatch: int32 pointers must be 4-byte aligned");
    DispatchArgs a{};
    bool all16 = true;
    int64_t total_bytes = 0;
    const int rc = prepare_fields(fields, nfields, N, a, &all16, &total_bytes,
                                  "moe_layout_dispatch");
    if (rc != MOE_OK) return rc;
    a.pos = nullptr;
    a.N = N;
    a.K = K;
    return launch_layout_dispatch(a, all16, ids, ids_row_stride, E, align, counts, offsets, pos,
                                  row_pair, cap, nullptr, status, stream, "moe_layout_dispatch");
}

int moe::layout_one_launch(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                           int32_t E, int32_t align, int32_t* counts, int32_t* offsets,
                           int32_t* pos, int32_t* row_pair, int64_t cap, int32_t* order,
                           int32_t* status, hipStream_t stream) {
    DispatchArgs a{};   // no payload: no vectors per token, no segments
    a.pos = nullptr;
    a.N = N;
    a.K = K;
    return launch_layout_dispatch(a, false, ids, ids_row_stride, E, align, counts, offsets, pos,
                                  row_pair, cap, order, status, stream, "moe_get_layout");
}

extern "C" int64_t moe_record_offsets(const int64_t* row_bytes, int32_t nfields,
                                      int64_t* offsets) {
    if (row_bytes == nullptr || nfields < 1 || nfields > MOE_MAX_FIELDS)
        return fail(MOE_ERR_ARG, "moe_record_offsets: need 1..%d fields", MOE_MAX_FIELDS);
    int64_t cur = 0;
    for (int f = 0; f < nfields; ++f) {
        if (row_bytes[f] < 0 || row_bytes[f] % 4 != 0)
            return fail(MOE_ERR_ARG, "moe_record_offsets: field %d row_bytes must be a "
                        "non-negative multiple of 4", f);
        cur = (cur + 15) / 16 * 16;
        if (offsets != nullptr) offsets[f] = cur;
        cur += row_bytes[f];
    }
    ok();
    return (cur + 15) / 16 * 16;
}

// Pack and unpack are the identity dispatch (K = 1, pos = NULL) with one
// side of every field redirected into the record buffer.
static int record_fields(const moe_field* fields, int32_t nfields, const void* records,
                         int64_t record_row_stride, bool pack, moe_field* out, const char* who) {
    if (fields == nullptr || nfields < 1 || nfields > MOE_MAX_FIELDS)
        return fail(MOE_ERR_ARG, "%s: need 1..%d fields", who, MOE_MAX_FIELDS);
    int64_t rb[MOE_MAX_FIELDS], off[MOE_MAX_FIELDS];
    for (int f = 0; f < nfields; ++f) rb[f] = fields[f].row_bytes;
    const int64_t rec = moe_record_offsets(rb, nfields, off);
    if (rec < 0) return (int)rec;
    if (record_row_stride < rec)
        return fail(MOE_ERR_ARG, "%s: record_row_stride=%lld below the record size %lld", who,
                    (long long)record_row_stride, (long long)rec);
    for (int f = 0; f < nfields; ++f) {
        char* slot = static_cast<char*>(const_cast<void*>(records)) + off[f];
        out[f] = fields[f];
        if (pack) {
            out[f].dst = slot;
            out[f].dst_row_stride = record_row_stride;
        } else {
            out[f].src = slot;
            out[f].src_row_stride = record_row_stride;
        }
    }
    return MOE_OK;
}

extern "C" int moe_pack_records(const moe_field* fields, int32_t nfields, int32_t N,
                                void* records, int64_t record_row_stride, hipStream_t stream) {
    if (N > 0 && records == nullptr) return fail(MOE_ERR_ARG, "moe_pack_records: NULL records");
    moe_field f[MOE_MAX_FIELDS];
    const int rc = record_fields(fields, nfields, records, record_row_stride, true, f,
                                 "moe_pack_records");
    if (rc != MOE_OK) return rc;
    return moe_dispatch(f, nfields, N, 1, nullptr, nullptr, stream);
}

extern "C" int moe_unpack_records(const void* records, int64_t record_row_stride, int32_t N,
                                  const moe_field* fields, int32_t nfields, hipStream_t stream) {
    if (N > 0 && records == nullptr) return fail(MOE_ERR_ARG, "moe_unpack_records: NULL records");
    moe_field f[MOE_MAX_FIELDS];
    const int rc = record_fields(fields, nfields, records, record_row_stride, false, f,
                                 "moe_unpack_records");
    if (rc != MOE_OK) return rc;
    return moe_dispatch(f, nfields, N, 1, nullptr, nullptr, stream);
}
