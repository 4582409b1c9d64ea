// layout.hip -- routing layout: per-expert histogram, exclusive prefix scan
// and stable row assignment for every (token, k) pair.
//
// Definition: DeepEP (repository dump, deep_ep.cpp, get_dispatch_layout)
// counts the top-k ids per expert; the dispatch fills an expert-contiguous
// receive buffer whose recv_src_idx names each row's source. Masked ids (-1)
// as written by mask_topk_ids (vLLM branch compare ds-exp-2...ds-exp-ag).
// Rows inside one expert's segment follow ascending (t, k).
//
// Three launches on the caller's stream, no atomics deciding any order:
//   1. hist   -- each workgroup takes a contiguous chunk of pairs; each of
//                its 4 waves a contiguous quarter. A wave finds the lanes that
//                share an expert with one ballot per id bit, and the lowest
//                such lane adds the group size to the wave's own LDS row.
//                The workgroup writes its per-expert totals H[b][e].
//   2. scan   -- one workgroup: per expert, the exclusive prefix of H over
//                the chunks (in place), the totals (counts), and the
//                exclusive scan of the aligned totals (offsets).
//   3. assign -- each workgroup recounts its waves, turns the counts into
//                per-wave bases (offsets[e] + chunk prefix + earlier waves),
//                and walks its pairs again in order: the row of a pair is its
//                wave's base for the expert plus the number of lower lanes in
//                the same 64-pair step with that expert. Then all workgroups
//                mark unused rows with -1.
// Kernel boundaries are the only grid-wide ordering used, so the result does
// not depend on scheduling.
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;              // hist / assign workgroup
constexpr int kWaves = kThreads / kWave;   // 4
constexpr int kScanThreads = 1024;
constexpr int kScanRows = 16;              // chunk rows one scan thread holds
constexpr int kPrefetch = 16;              // 64-pair steps of ids held in registers

struct Plan {
    int32_t chunk;    // pairs per workgroup (multiple of kThreads)
    int32_t blocks;   // number of chunks
    int32_t ecols;    // E padded to a power of two >= 64
    int32_t lanes;    // scan threads per expert column
    int32_t rows;     // chunk rows per scan thread
    int32_t nbits;    // ceil(log2(E))
};

int32_t next_pow2(int32_t x) {
    int32_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

Plan make_plan(int32_t N, int32_t K, int32_t E) {
    Plan p;
    const int64_t nk = (int64_t)N * K;
    p.ecols = next_pow2(E) < kWave ? kWave : next_pow2(E);
    p.lanes = kScanThreads / p.ecols;
    const int64_t max_blocks = (int64_t)kScanRows * p.lanes;
    int64_t chunk = ceil_div<int64_t>(ceil_div<int64_t>(nk, max_blocks), kThreads) * kThreads;
    if (chunk < kThreads) chunk = kThreads;
    p.chunk = (int32_t)chunk;
    p.blocks = (int32_t)ceil_div<int64_t>(nk, chunk);
    p.rows = (int32_t)ceil_div<int64_t>(p.blocks, p.lanes);
    p.nbits = 0;
    while ((1 << p.nbits) < E) ++p.nbits;
    return p;
}

size_t workspace_for(const Plan& p, int32_t E) {
    // H[blocks][E] then bad[blocks]
    size_t bytes = ((size_t)p.blocks * E + p.blocks) * sizeof(int32_t);
    bytes = (bytes + 255) / 256 * 256;
    return bytes < 256 ? 256 : bytes;
}

// Expert id of flat pair i = t*K + k.
__device__ __forceinline__ int32_t load_id(const int32_t* __restrict__ ids, int64_t stride,
                                           uint32_t i, uint32_t K) {
    const uint32_t t = i / K;
    const uint32_t k = i - t * K;
    return ids[(int64_t)t * stride + k];
}

// Lanes of this wave holding the same valid expert as the calling lane
// (valid for valid lanes only): one ballot per bit of the id.
__device__ __forceinline__ uint64_t same_expert_lanes(int32_t e, bool valid, int nbits) {
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// Adds this wave's per-expert counts over its quarter of the chunk into
// cnt[wave*E + e]; returns the number of ids >= E it saw.
__device__ __forceinline__ int32_t count_wave(const int32_t* __restrict__ ids, int64_t stride,
                                              uint32_t nk, uint32_t K, int32_t E, int nbits,
                                              uint32_t first, int steps, int32_t* cnt_row,
                                              int lane) {
    int32_t bad = 0;
    for (int s0 = 0; s0 < steps; s0 += kPrefetch) {
        int32_t e_reg[kPrefetch];
#pragma unroll
        for (int j = 0; j < kPrefetch; ++j) {
            const uint32_t i = first + (uint32_t)(s0 + j) * kWave + lane;
            e_reg[j] = (s0 + j < steps && i < nk) ? load_id(ids, stride, i, K) : -1;
        }
#pragma unroll
        for (int j = 0; j < kPrefetch; ++j) {
            if (s0 + j < steps) {   // wave-uniform
                const int32_t e = e_reg[j];
                const bool valid = e >= 0 && e < E;
                bad += __popcll(__ballot(e >= E));
                const uint64_t peers = same_expert_lanes(e, valid, nbits);
                if (valid && lane == __ffsll((long long)peers) - 1) cnt_row[e] += __popcll(peers);
                __builtin_amdgcn_wave_barrier();
            }
        }
    }
    return bad;
}

__global__ __launch_bounds__(kThreads) void layout_hist(const int32_t* __restrict__ ids,
                                                        int64_t stride, uint32_t nk, uint32_t K,
                                                        int32_t E, int32_t chunk, int nbits,
                                                        int32_t* __restrict__ H,
                                                        int32_t* __restrict__ bad_out) {
    __shared__ int32_t cnt[kWaves * MOE_MAX_EXPERTS];
    __shared__ int32_t wbad[kWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    for (int x = threadIdx.x; x < kWaves * E; x += kThreads) cnt[x] = 0;
    __syncthreads();

    const int quarter = chunk / kWaves;
    const uint32_t first = (uint32_t)blockIdx.x * chunk + wave * quarter;
    const int32_t bad = count_wave(ids, stride, nk, K, E, nbits, first, quarter / kWave,
                                   cnt + wave * E, lane);
    if (lane == 0) wbad[wave] = bad;
    __syncthreads();

    int32_t* row = H + (int64_t)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += kThreads)
        row[e] = cnt[e] + cnt[E + e] + cnt[2 * E + e] + cnt[3 * E + e];
    if (threadIdx.x == 0) bad_out[blockIdx.x] = wbad[0] + wbad[1] + wbad[2] + wbad[3];
}

__global__ __launch_bounds__(kScanThreads) void layout_scan(int32_t* __restrict__ H,
                                                            const int32_t* __restrict__ bad,
                                                            int32_t blocks, int32_t E,
                                                            int32_t ecols, int32_t lanes,
                                                            int32_t rows, int32_t align,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ status) {
    __shared__ int32_t part[kScanThreads];
    __shared__ int32_t scan[kScanThreads];
    __shared__ int32_t sbad;
    const int j = threadIdx.x;
    const int e = j & (ecols - 1);
    const int q = j / ecols;          // which slice of chunk rows
    const int g0 = q * rows;

    int32_t r[kScanRows];
    int32_t sum = 0;
#pragma unroll
    for (int x = 0; x < kScanRows; ++x) {
        const int g = g0 + x;
        r[x] = (x < rows && g < blocks && e < E) ? H[(int64_t)g * E + e] : 0;
        sum += r[x];
    }
    part[j] = sum;
    if (j == 0) sbad = 0;
    __syncthreads();

    int32_t before = 0, total = 0;
    for (int x = 0; x < lanes; ++x) {
        const int32_t v = part[x * ecols + e];
        before += (x < q) ? v : 0;
        total += v;
    }
    if (e < E) {
        int32_t run = before;
#pragma unroll
        for (int x = 0; x < kScanRows; ++x) {
            const int g = g0 + x;
            if (x < rows && g < blocks) {
                H[(int64_t)g * E + e] = run;
                run += r[x];
            }
        }
        if (q == 0) counts[e] = total;
    }

    // Inclusive scan of the aligned totals over the expert columns.
    const int64_t padded = (q == 0 && e < E) ? ((int64_t)total + align - 1) / align * align : 0;
    if (j < ecols) scan[j] = (int32_t)padded;
    __syncthreads();
    for (int off = 1; off < ecols; off <<= 1) {
        const int32_t v = (j < ecols && j >= off) ? scan[j - off] : 0;
        __syncthreads();
        if (j < ecols) scan[j] += v;
        __syncthreads();
    }
    if (j < E) offsets[j + 1] = scan[j];
    if (j == 0) offsets[0] = 0;

    int32_t b = 0;
    for (int g = j; g < blocks; g += kScanThreads) b += bad[g];
    if (b) atomicAdd(&sbad, b);
    __syncthreads();
    if (j == 0 && status) *status = sbad;
}

__global__ __launch_bounds__(kThreads) void layout_assign(
    const int32_t* __restrict__ ids, int64_t stride, uint32_t nk, uint32_t K, int32_t E,
    int32_t chunk, int nbits, int32_t blocks, int32_t align, const int32_t* __restrict__ H,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ row_pair, int64_t cap) {
    __shared__ int32_t cnt[kWaves * MOE_MAX_EXPERTS];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int b = blockIdx.x;

    if (b < blocks) {
        for (int x = threadIdx.x; x < kWaves * E; x += kThreads) cnt[x] = 0;
        __syncthreads();
        const int quarter = chunk / kWaves;
        const int steps = quarter / kWave;
        const uint32_t first = (uint32_t)b * chunk + wave * quarter;
        int32_t* mine = cnt + wave * E;
        count_wave(ids, stride, nk, K, E, nbits, first, steps, mine, lane);
        __syncthreads();

        // Per-wave bases: expert offset + earlier chunks + earlier waves.
        const int32_t* hrow = H + (int64_t)b * E;
        for (int e = threadIdx.x; e < E; e += kThreads) {
            int32_t run = offsets[e] + hrow[e];
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const int32_t c = cnt[w * E + e];
                cnt[w * E + e] = run;
                run += c;
            }
        }
        __syncthreads();

        for (int s0 = 0; s0 < steps; s0 += kPrefetch) {
            int32_t e_reg[kPrefetch];
#pragma unroll
            for (int j = 0; j < kPrefetch; ++j) {
                const uint32_t i = first + (uint32_t)(s0 + j) * kWave + lane;
                e_reg[j] = (s0 + j < steps && i < nk) ? load_id(ids, stride, i, K) : -1;
            }
#pragma unroll
            for (int j = 0; j < kPrefetch; ++j) {
                if (s0 + j < steps) {   // wave-uniform
                    const uint32_t i = first + (uint32_t)(s0 + j) * kWave + lane;
                    const int32_t e = e_reg[j];
                    const bool valid = e >= 0 && e < E;
                    const uint64_t peers = same_expert_lanes(e, valid, nbits);
                    int32_t p = -1;
                    if (valid) p = mine[e] + __popcll(peers & lanes_below(lane));
                    __builtin_amdgcn_wave_barrier();
                    if (valid && lane == __ffsll((long long)peers) - 1) mine[e] += __popcll(peers);
                    __builtin_amdgcn_wave_barrier();
                    if (i < nk) pos[i] = p;
                    if (valid && p < cap) row_pair[p] = (int32_t)i;
                }
            }
        }
    }

    // Rows no pair landed in: past the used rows, and alignment padding.
    const int64_t used = offsets[E];
    for (int64_t r = used + (int64_t)b * kThreads + threadIdx.x; r < cap;
         r += (int64_t)gridDim.x * kThreads)
        row_pair[r] = -1;
    if (align > 1) {
        for (int e = b; e < E; e += gridDim.x) {
            const int32_t hi = offsets[e + 1];
            for (int32_t r = offsets[e] + counts[e] + threadIdx.x; r < hi; r += kThreads)
                row_pair[r] = -1;
        }
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int64_t moe_required_capacity(int32_t N, int32_t K, int32_t E, int32_t align) {
    if (N < 0 || K < 1 || E < 1 || align < 1) return -1;
    int64_t c = (int64_t)N * K;
    if (align > 1) c += (int64_t)E * (align - 1);
    return c;
}

extern "C" size_t moe_layout_workspace_bytes(int32_t N, int32_t K, int32_t E) {
    if (N < 0 || K < 1 || K > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return 0;
    if ((int64_t)N * K >= ((int64_t)1 << 31)) return 0;
    return workspace_for(make_plan(N, K, E), E);
}

extern "C" int moe_get_layout(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                              int32_t E, int32_t align, int32_t* counts, int32_t* offsets,
                              int32_t* pos, int32_t* row_pair, int64_t cap, void* workspace,
                              size_t workspace_bytes, int32_t* status, hipStream_t stream) {
    if (N < 0 || K < 1 || E < 1 || align < 1)
        return fail(MOE_ERR_ARG, "moe_get_layout: need N >= 0, K >= 1, E >= 1, align >= 1 "
                    "(got N=%d K=%d E=%d align=%d)", N, K, E, align);
    if (K > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_LIMIT, "moe_get_layout: K=%d E=%d beyond K <= %d, E <= %d", K, E,
                    MOE_MAX_TOPK, MOE_MAX_EXPERTS);
    const int64_t nk = (int64_t)N * K;
    if (nk >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_get_layout: N*K=%lld must be below 2^31", (long long)nk);
    if (N > 0 && (ids == nullptr || pos == nullptr))
        return fail(MOE_ERR_ARG, "moe_get_layout: ids and pos must not be NULL");
    if (N > 0 && ids_row_stride < K)
        return fail(MOE_ERR_ARG, "moe_get_layout: ids_row_stride=%lld < K=%d",
                    (long long)ids_row_stride, K);
    if (counts == nullptr || offsets == nullptr)
        return fail(MOE_ERR_ARG, "moe_get_layout: counts and offsets must not be NULL");
    const int64_t need = moe_required_capacity(N, K, E, align);
    if (cap < need)
        return fail(MOE_ERR_CAPACITY, "moe_get_layout: cap=%lld below the worst case %lld",
                    (long long)cap, (long long)need);
    if (cap >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_get_layout: cap=%lld must be below 2^31", (long long)cap);
    if (cap > 0 && row_pair == nullptr)
        return fail(MOE_ERR_ARG, "moe_get_layout: row_pair must not be NULL");
    if (!aligned(ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(pos, 4) ||
        !aligned(row_pair, 4) || !aligned(status, 4))
        return fail(MOE_ERR_ALIGN, "moe_get_layout: int32 pointers must be 4-byte aligned");
    const Plan p = make_plan(N, K, E);
    const size_t ws = workspace_for(p, E);
    if (workspace == nullptr || workspace_bytes < ws)
        return fail(MOE_ERR_WORKSPACE, "moe_get_layout: workspace of %zu bytes needed, got %zu%s",
                    ws, workspace_bytes, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 4))
        return fail(MOE_ERR_ALIGN, "moe_get_layout: workspace must be 4-byte aligned");

    clear_launch_error();
    int32_t* H = static_cast<int32_t*>(workspace);
    int32_t* bad = H + (int64_t)p.blocks * E;
    if (p.blocks > 0)
        layout_hist<<<p.blocks, kThreads, 0, stream>>>(ids, ids_row_stride, (uint32_t)nk,
                                                       (uint32_t)K, E, p.chunk, p.nbits, H, bad);
    layout_scan<<<1, kScanThreads, 0, stream>>>(H, bad, p.blocks, E, p.ecols, p.lanes, p.rows,
                                                align, counts, offsets, status);
    layout_assign<<<p.blocks > 0 ? p.blocks : 1, kThreads, 0, stream>>>(
        ids, ids_row_stride, (uint32_t)nk, (uint32_t)K, E, p.chunk, p.nbits, p.blocks, align, H,
        counts, offsets, pos, row_pair, cap);
    return check_launch("moe_get_layout");
}
