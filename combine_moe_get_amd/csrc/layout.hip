// layout.hip -- routing layout: per-expert histogram, exclusive prefix scan
// and stable row assignment for every (token, k) pair.
//
// Definition: DeepEP (repository dump, deep_ep.cpp, get_dispatch_layout)
// counts the top-k ids per expert; the dispatch fills an expert-contiguous
// receive buffer whose recv_src_idx names each row's source. Masked ids (-1)
// as written by mask_topk_ids (vLLM branch compare ds-exp-2...ds-exp-ag).
// Rows inside one expert's segment follow ascending (t, k).
//
// Three forms, all on the caller's stream, none with an atomic that decides
// any order (LDS atomics only add counts, and sums do not depend on order):
//   - two launches, for any batch:
//     1. hist   -- each workgroup takes a contiguous chunk of pairs; each of
//                  its 4 waves a contiguous quarter. A wave finds the lanes
//                  that share an expert with one ballot per id bit, and the
//                  lowest such lane adds the group size to the wave's own LDS
//                  row. The workgroup writes its per-expert totals H[b][e].
//     2. assign -- every workgroup reduces the whole (small) H matrix itself:
//                  per expert, the sum over earlier chunks and the total; an
//                  exclusive scan of the aligned totals gives the offsets
//                  (workgroup 0 also writes counts, offsets and status). It
//                  then recounts its waves, turns the counts into per-wave
//                  bases (offset + earlier chunks + earlier waves), and walks
//                  its pairs again in order: the row of a pair is its wave's
//                  base for the expert plus the number of lower lanes in the
//                  same 64-pair step with that expert. Finally all workgroups
//                  mark unused rows with -1. H has at most 16384 entries, so
//                  the redundant reduction costs each workgroup at most 64
//                  loads per thread.
//   - one launch for mid-size batches of contiguous ids (layout_onepass):
//     every workgroup counts the whole batch itself with LDS atomics instead
//     of reading H, then assigns its chunk as `assign` does;
//   - one launch for batches of at most kOneLaunchPairs pairs: the layout
//     part of the one-launch dispatch kernels (dispatch.hip, quant.hip).
// The kernel boundary is the only grid-wide ordering used, so the result
// does not depend on scheduling, and every form gives the same outputs.
#include <mutex>

#include "internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;              // hist / assign workgroup
constexpr int kWaves = kThreads / kWave;   // 4
constexpr int kHEntries = 16384;           // bound on chunks * padded experts
constexpr int kMaxChunks = 64;
// 64-pair steps of ids held in registers per batch: 4 for small chunks
// (short straight-line code, see reduce_chunks), 16 for large ones (one
// load round instead of four per pass).
constexpr int kBatchSmall = 4;
constexpr int kBatchLarge = 16;

struct Plan {
    int32_t chunk;    // pairs per workgroup (multiple of kThreads)
    int32_t blocks;   // number of chunks
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
    const int32_t ecols = next_pow2(E) < kThreads ? kThreads : next_pow2(E);
    const int64_t max_blocks = kHEntries / ecols < kMaxChunks ? kHEntries / ecols : kMaxChunks;
    int64_t chunk = ceil_div<int64_t>(ceil_div<int64_t>(nk, max_blocks), kThreads) * kThreads;
    if (chunk < kThreads) chunk = kThreads;
    p.chunk = (int32_t)chunk;
    p.blocks = (int32_t)ceil_div<int64_t>(nk, chunk);
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
// (valid for valid lanes only). Per id bit b, a ballot m of the lanes with
// bit b set; the lanes that differ from this lane in bit b are m, or ~m
// when this lane has the bit: m ^ s with s = bit b spread over all 32 bits
// (0 or -1). The lanes that differ in no bit and are valid are the peers.
// All kMaxIdBits bits, without a branch: past the id's top bit (E <= 2^bits)
// every valid lane has 0, so only invalid lanes differ there.
constexpr int kMaxIdBits = 10;
static_assert((1 << kMaxIdBits) >= MOE_MAX_EXPERTS, "expert ids fit kMaxIdBits bits");

__device__ __forceinline__ uint64_t same_expert_lanes(int32_t e, bool valid, int /*nbits*/) {
    uint32_t dlo = 0, dhi = 0;   // lanes that differ in some bit
#pragma unroll
    for (int b = 0; b < kMaxIdBits; ++b) {
        const int32_t sb = (int32_t)((uint32_t)e << (31 - b)) >> 31;   // bit b: 0 or -1
        const uint64_t m = __ballot(sb != 0);
        dlo |= (uint32_t)sb ^ (uint32_t)m;
        dhi |= (uint32_t)sb ^ (uint32_t)(m >> 32);
    }
    return ~(((uint64_t)dhi << 32) | dlo) & __ballot(valid);
}

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// Loads the expert ids of 64-pair steps s0 .. s0+B-1 of a wave's
// quarter (-1 past the quarter or past the last pair). All loads are issued
// before any is used. Contiguous ids (stride == K) need no division by K.
template <int B>
__device__ __forceinline__ void load_ids(int32_t (&e_reg)[B],
                                         const int32_t* __restrict__ ids, int64_t stride,
                                         uint32_t nk, uint32_t K, uint32_t first, int s0,
                                         int steps, int lane) {
    if (stride == (int64_t)K) {
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const uint32_t i = first + (uint32_t)(s0 + j) * kWave + lane;
            e_reg[j] = (s0 + j < steps && i < nk) ? ids[i] : -1;
        }
    } else {
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const uint32_t i = first + (uint32_t)(s0 + j) * kWave + lane;
            e_reg[j] = (s0 + j < steps && i < nk) ? load_id(ids, stride, i, K) : -1;
        }
    }
}

// Adds one batch of steps to the wave's counts cnt_row[e]; returns the number
// of ids >= E in the batch. With peers_out, also keeps each step's
// same-expert lanes for rank_batch.
template <int B>
__device__ __forceinline__ int32_t count_batch(const int32_t (&e_reg)[B], int s0,
                                               int steps, int32_t E, int nbits, int32_t* cnt_row,
                                               int lane, uint64_t* peers_out = nullptr) {
    int32_t bad = 0;
#pragma unroll
    for (int j = 0; j < B; ++j) {
        if (s0 + j < steps) {   // wave-uniform
            const int32_t e = e_reg[j];
            const bool valid = e >= 0 && e < E;
            bad += __popcll(__ballot(e >= E));
            const uint64_t peers = same_expert_lanes(e, valid, nbits);
            if (peers_out != nullptr) peers_out[j] = peers;
            if (valid && lane == __ffsll((long long)peers) - 1) cnt_row[e] += __popcll(peers);
            __builtin_amdgcn_wave_barrier();
        }
    }
    return bad;
}

// Gives every pair of one batch its row: the wave's running base for the
// expert plus the number of lower lanes in the same step with that expert
// (peers_in: the steps' same-expert lanes kept by count_batch).
// In the padded form (M > 0) expert e's segment is rows e*M .. e*M+M-1 and
// a pair ranked past it is dropped (pos = -1).
// With a plan (order != nullptr), a valid pair also takes its slot in the
// plan: the tile's start, plus the tile's pairs of lower experts
// (tile_scan[e]), plus its rank among the tile's pairs of expert e (its row
// minus tile_row[e], the row of the first of them). With tile_row ==
// nullptr the plan is the index order: every pair in its own slot, -1 for
// the masked ones.
template <int B>
__device__ __forceinline__ void rank_batch(const int32_t (&e_reg)[B], int s0, int steps,
                                           int32_t E, int nbits, int32_t* base_row,
                                           uint32_t first, uint32_t nk, int lane,
                                           int32_t* __restrict__ pos,
                                           int32_t* __restrict__ row_pair, int64_t cap,
                                           int32_t M, int32_t* __restrict__ order = nullptr,
                                           const int32_t* tile_scan = nullptr,
                                           const int32_t* tile_row = nullptr,
                                           int32_t tile_start = 0,
                                           const uint64_t* peers_in = nullptr) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
        if (s0 + j < steps) {   // wave-uniform
            const uint32_t i = first + (uint32_t)(s0 + j) * kWave + lane;
            const int32_t e = e_reg[j];
            const bool valid = e >= 0 && e < E;
            const uint64_t peers =
                peers_in != nullptr ? peers_in[j] : same_expert_lanes(e, valid, nbits);
            int32_t p = -1;
            if (valid) p = base_row[e] + __popcll(peers & lanes_below(lane));
            __builtin_amdgcn_wave_barrier();
            if (valid && lane == __ffsll((long long)peers) - 1) base_row[e] += __popcll(peers);
            __builtin_amdgcn_wave_barrier();
            if (M > 0 && p >= (e + 1) * M) p = -1;   // past the expert's padded segment
            if (i < nk) pos[i] = p;
            if (p >= 0 && p < cap) row_pair[p] = (int32_t)i;
            if (order != nullptr) {
                if (tile_row == nullptr) {   // a plan in index order
                    if (i < nk) order[i] = p >= 0 ? (int32_t)i : -1;
                } else if (p >= 0) {
                    order[tile_start + tile_scan[e] + (p - tile_row[e])] = (int32_t)i;
                }
            }
        }
    }
}

template <int B>
__global__ __launch_bounds__(kThreads) void layout_hist(const int32_t* __restrict__ ids,
                                                        int64_t stride, uint32_t nk, uint32_t K,
                                                        int32_t E, int32_t chunk, int nbits,
                                                        int32_t* __restrict__ H,
                                                        int32_t* __restrict__ bad_out) {
    __shared__ int32_t cnt[kWaves * MOE_MAX_EXPERTS];
    __shared__ int32_t wbad[kWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int quarter = chunk / kWaves;
    const int steps = quarter / kWave;
    const uint32_t first = (uint32_t)blockIdx.x * chunk + wave * quarter;

    int32_t e_reg[B];
    load_ids(e_reg, ids, stride, nk, K, first, 0, steps, lane);
    for (int x = threadIdx.x; x < kWaves * E; x += kThreads) cnt[x] = 0;
    __syncthreads();

    int32_t* row = cnt + wave * E;
    int32_t bad = count_batch(e_reg, 0, steps, E, nbits, row, lane);
    for (int s0 = B; s0 < steps; s0 += B) {
        load_ids(e_reg, ids, stride, nk, K, first, s0, steps, lane);
        bad += count_batch(e_reg, s0, steps, E, nbits, row, lane);
    }
    if (lane == 0) wbad[wave] = bad;
    __syncthreads();

    int32_t* out = H + (int64_t)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += kThreads)
        out[e] = cnt[e] + cnt[E + e] + cnt[2 * E + e] + cnt[3 * E + e];
    if (threadIdx.x == 0) bad_out[blockIdx.x] = wbad[0] + wbad[1] + wbad[2] + wbad[3];
}

// Exclusive scan over the W*64 threads of a workgroup of one value per
// thread; returns the sum of the values of lower threads and leaves the
// workgroup total in *total. Contains one __syncthreads.
template <int W>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* wave_sums,
                                                        int32_t* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int32_t x = wave_inclusive_scan(v);
    if (lane == kWave - 1) wave_sums[wave] = x;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        before += (w < wave) ? wave_sums[w] : 0;
        all += wave_sums[w];
    }
    *total = all;
    return before + x - v;
}

// Per expert e (columns tid, tid+256, ... of H): pairs in chunks before b
// (before_s) and in all chunks (total_s). C columns per thread and at most
// R chunks, so every load is issued before the first sum. The loads go
// through a buffer descriptor over H[blocks][E]: past its end they return 0,
// so rows g >= blocks need no guard, and without guards each load is one
// instruction rather than a branch around it (this straight-line code is
// fetched cold by every workgroup, so its length is time). Columns e >= E
// load whatever lies there and are not stored.
template <int C, int R>
__device__ __forceinline__ void reduce_chunks(const int32_t* __restrict__ H, int32_t blocks,
                                              int32_t E, int b, int32_t* total_s,
                                              int32_t* before_s) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(H), 0, blocks * E * (int32_t)sizeof(int32_t), kBufferWord3);
    int32_t v[C][R];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int e = threadIdx.x + c * kThreads;
#pragma unroll
        for (int g = 0; g < R; ++g)
            v[c][g] = __builtin_amdgcn_raw_buffer_load_b32(rs, (g * E + e) * 4, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int e = threadIdx.x + c * kThreads;
        int32_t before = 0, total = 0;
#pragma unroll
        for (int g = 0; g < R; ++g) {
            before += (g < b) ? v[c][g] : 0;
            total += v[c][g];
        }
        if (e < E) {
            total_s[e] = total;
            before_s[e] = before;
        }
    }
}

// PLAN: also write the dispatch plan `order` (see moe_get_layout). Its tiles
// are the chunks: chunk b's slots list its valid pairs by ascending row
// (the pairs of lower experts first, then each expert's in (t, k) order),
// then -1 for its masked and out-of-range pairs. Chunks of more than
// kPlanMaxTile pairs write the index order instead.
constexpr int32_t kPlanMaxTile = 4096;

// LDS of the assign step, shared by both layout forms.
template <bool PLAN>
struct AssignLds {
    int32_t cnt[kWaves * MOE_MAX_EXPERTS];   // per-wave counts, then bases
    int32_t total_s[MOE_MAX_EXPERTS];       // valid pairs per expert
    int32_t start_s[MOE_MAX_EXPERTS];       // segment start (offsets[e])
    int32_t base[MOE_MAX_EXPERTS];          // pairs in earlier chunks, then chunk base
    int32_t tile_scan[PLAN ? MOE_MAX_EXPERTS : 1];   // chunk's pairs of lower experts
    int32_t wave_sums[kWaves];
    int32_t used_s;
    int32_t tile_valid_s;
};

// Segment starts from the per-expert totals (total_s) and the pairs in
// earlier chunks (base): an exclusive scan of the aligned totals, or e*M in
// the padded form; base[e] becomes the chunk's first row of expert e. Thread
// i owns experts 4i .. 4i+3 (E <= 1024); their total_s and base entries must
// have been written by this thread or before a barrier. Workgroup 0 writes
// counts, offsets, the padded form's drop count (status[1]) and receive
// metadata; status[0] is left to the caller. Contains barriers: every thread
// of the workgroup calls it.
template <bool PLAN>
__device__ __forceinline__ void segment_starts(AssignLds<PLAN>& s, int b, int32_t E,
                                               int32_t align, int32_t M,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ status,
                                               int64_t* __restrict__ layout_range,
                                               int32_t* __restrict__ recv_stats) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int32_t mine4[4];
    int32_t sum4 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = threadIdx.x * 4 + j;
        mine4[j] = e < E ? s.total_s[e] : 0;
    }
    if (align > 1) {
        // The host checks cap >= N*K + E*(align - 1) and cap < 2^31, so
        // c + align - 1 fits in 32 bits (a 64-bit division is ~100
        // instructions per use).
        const uint32_t a = (uint32_t)align;
#pragma unroll
        for (int j = 0; j < 4; ++j) mine4[j] = (int32_t)(((uint32_t)mine4[j] + a - 1u) / a * a);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) sum4 += mine4[j];
    int32_t used = 0;
    int32_t run = block_exclusive_scan<kWaves>(sum4, s.wave_sums, &used);
    int32_t dropped4 = 0;   // padded form: pairs beyond their expert's M rows
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = threadIdx.x * 4 + j;
        if (e < E) {
            const int32_t start = M > 0 ? e * M : run;
            if (b == 0) {
                const int32_t kept = M > 0 ? min(s.total_s[e], M) : s.total_s[e];
                counts[e] = kept;
                if (offsets != nullptr) offsets[e] = start;
                // Padded form, one source: the range of expert e's rows that
                // came from it (begin 0 in the high half, count in the low),
                // and the running count of rows received.
                if (layout_range != nullptr) layout_range[e] = (int64_t)kept;
                if (recv_stats != nullptr) recv_stats[e] += kept;
            }
            if (M > 0) dropped4 += max(s.total_s[e] - M, 0);
            s.start_s[e] = start;
            s.base[e] += start;
        }
        run += mine4[j];
    }
    if (threadIdx.x == 0) {
        s.used_s = M > 0 ? E * M : used;
        if (b == 0 && offsets != nullptr) offsets[E] = M > 0 ? E * M : used;
    }
    if (M > 0) {
        // status[1]: one sum per wave, then thread 0 adds them
        const int32_t d = wave_sum(dropped4);
        __syncthreads();   // wave_sums is free again after the scan
        if (lane == 0) s.wave_sums[wave] = d;
        __syncthreads();
        if (b == 0 && status != nullptr && threadIdx.x == 0)
            status[1] = s.wave_sums[0] + s.wave_sums[1] + s.wave_sums[2] + s.wave_sums[3];
    }
}

// A chunk's assignment, first half (it needs only the chunk's own ids):
// per-wave counts of chunk b into s.cnt, which must be zero behind a
// barrier, and with a plan the chunk's tile_scan. e_first holds the first
// batch of the wave's ids (later batches are loaded again); peers receives
// the first batch's same-expert lanes for assign_rank. Contains barriers.
template <int B, bool PLAN>
__device__ __forceinline__ void assign_count(AssignLds<PLAN>& s, const int32_t (&e_first)[B],
                                             uint64_t (&peers)[B],
                                             const int32_t* __restrict__ ids, int64_t stride,
                                             uint32_t nk, uint32_t K, int32_t E, int nbits,
                                             int32_t chunk, int b, bool active) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int quarter = chunk / kWaves;
    const int steps = active ? quarter / kWave : 0;
    const uint32_t first = (uint32_t)b * chunk + wave * quarter;

    int32_t* mine = s.cnt + wave * E;
    count_batch(e_first, 0, steps, E, nbits, mine, lane, peers);
    for (int s0 = B; s0 < steps; s0 += B) {
        int32_t e_reg[B];
        load_ids(e_reg, ids, stride, nk, K, first, s0, steps, lane);
        count_batch(e_reg, s0, steps, E, nbits, mine, lane);
    }
    __syncthreads();

    if (PLAN && chunk <= kPlanMaxTile) {
        // The chunk's plan slots: an exclusive scan over the experts of the
        // chunk's pairs per expert (its four waves' counts) places each
        // expert's run; the run's first row will be the chunk base base[e].
        int32_t t4[4], tsum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = threadIdx.x * 4 + j;
            t4[j] = e < E ? s.cnt[e] + s.cnt[E + e] + s.cnt[2 * E + e] + s.cnt[3 * E + e] : 0;
            tsum += t4[j];
        }
        int32_t tvalid = 0;
        int32_t trun = block_exclusive_scan<kWaves>(tsum, s.wave_sums, &tvalid);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = threadIdx.x * 4 + j;
            if (e < E) s.tile_scan[e] = trun;
            trun += t4[j];
        }
        if (threadIdx.x == 0) s.tile_valid_s = tvalid;
        // (the scan's barrier already orders the t4 reads of cnt before
        // assign_rank rewrites it)
    }
}

// Second half: the per-wave bases (chunk base + earlier waves) from s.cnt
// and the final chunk bases s.base, both behind a barrier; then the rows
// of the chunk's pairs in order, and the chunk's plan tile. Contains
// barriers.
template <int B, bool PLAN>
__device__ __forceinline__ void assign_rank(AssignLds<PLAN>& s, const int32_t (&e_first)[B],
                                            const uint64_t (&peers)[B],
                                            const int32_t* __restrict__ ids, int64_t stride,
                                            uint32_t nk, uint32_t K, int32_t E, int nbits,
                                            int32_t chunk, int b, bool active,
                                            int32_t* __restrict__ pos,
                                            int32_t* __restrict__ row_pair, int64_t cap,
                                            int32_t M, int32_t* __restrict__ order) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int quarter = chunk / kWaves;
    const int steps = active ? quarter / kWave : 0;
    const uint32_t first = (uint32_t)b * chunk + wave * quarter;
    const bool sorted = PLAN && chunk <= kPlanMaxTile;   // wave-uniform

    for (int e = threadIdx.x; e < E; e += kThreads) {
        int32_t r = s.base[e];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int32_t c = s.cnt[w * E + e];
            s.cnt[w * E + e] = r;
            r += c;
        }
    }
    __syncthreads();

    int32_t* mine = s.cnt + wave * E;
    const int32_t tile_start = b * chunk;
    const int32_t* const run_row = sorted ? s.base : nullptr;
    rank_batch(e_first, 0, steps, E, nbits, mine, first, nk, lane, pos, row_pair, cap, M, order,
               s.tile_scan, run_row, tile_start, peers);
    for (int s0 = B; s0 < steps; s0 += B) {
        int32_t e_reg[B];
        load_ids(e_reg, ids, stride, nk, K, first, s0, steps, lane);
        rank_batch(e_reg, s0, steps, E, nbits, mine, first, nk, lane, pos, row_pair, cap, M, order,
                   s.tile_scan, run_row, tile_start);
    }
    if (sorted && active) {
        // The chunk's slots past its valid pairs (its masked and out-of-range
        // pairs) hold -1.
        const int32_t len = (int32_t)min((int64_t)(b + 1) * chunk, (int64_t)nk) - tile_start;
        for (int32_t j = s.tile_valid_s + (int32_t)threadIdx.x; j < len; j += kThreads)
            order[tile_start + j] = -1;
    }
}

// Rows no pair landed in get -1: past the used rows and alignment padding,
// or in the padded form the rows of each segment past its kept pairs. Every
// workgroup of the grid (which may exceed the chunks) takes a strided share.
template <bool PLAN>
__device__ __forceinline__ void mark_unused_rows(const AssignLds<PLAN>& s, int b, int32_t E,
                                                 int32_t align, int32_t M, int64_t cap,
                                                 int32_t* __restrict__ row_pair) {
    if (M > 0) {
        for (int64_t r = (int64_t)b * kThreads + threadIdx.x; r < cap;
             r += (int64_t)gridDim.x * kThreads) {
            const int32_t e = (int32_t)((uint32_t)r / (uint32_t)M);
            if ((int32_t)r - e * M >= min(s.total_s[e], M)) row_pair[r] = -1;
        }
        return;
    }
    for (int64_t r = s.used_s + (int64_t)b * kThreads + threadIdx.x; r < cap;
         r += (int64_t)gridDim.x * kThreads)
        row_pair[r] = -1;
    if (align > 1) {
        for (int e = b; e < E; e += gridDim.x) {
            const int32_t hi = e + 1 < E ? s.start_s[e + 1] : s.used_s;
            for (int32_t r = s.start_s[e] + s.total_s[e] + threadIdx.x; r < hi; r += kThreads)
                row_pair[r] = -1;
        }
    }
}

template <int B, bool PLAN>
__global__ __launch_bounds__(kThreads) void layout_assign(
    const int32_t* __restrict__ ids, int64_t stride, uint32_t nk, uint32_t K, int32_t E,
    int32_t chunk, int nbits, int32_t blocks, int32_t align, const int32_t* __restrict__ H,
    const int32_t* __restrict__ bad, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ status, int32_t* __restrict__ pos, int32_t* __restrict__ row_pair,
    int64_t cap, int32_t M, int32_t* __restrict__ order, int64_t* __restrict__ layout_range,
    int32_t* __restrict__ recv_stats) {
    __shared__ AssignLds<PLAN> s;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int b = blockIdx.x;
    const bool active = b < blocks;
    const int quarter = chunk / kWaves;
    const int steps = active ? quarter / kWave : 0;
    const uint32_t first = (uint32_t)b * chunk + wave * quarter;

    // The ids of the first batch and the chunk histograms are fetched
    // together; the ids stay in registers for both passes.
    int32_t e_first[B];
    load_ids(e_first, ids, stride, nk, K, first, 0, steps, lane);
    // Few chunks (small batches) take a short form of the reduction: the
    // straight-line code a workgroup runs once is fetched into a cold
    // instruction cache, so its length shows in small-batch latency.
    if (blocks <= 16) {
        if (E <= kThreads)
            reduce_chunks<1, 16>(H, blocks, E, b, s.total_s, s.base);
        else
            reduce_chunks<4, 16>(H, blocks, E, b, s.total_s, s.base);
    } else if (E <= kThreads) {
        reduce_chunks<1, kMaxChunks>(H, blocks, E, b, s.total_s, s.base);
    } else if (E <= 2 * kThreads) {
        reduce_chunks<2, kMaxChunks / 2>(H, blocks, E, b, s.total_s, s.base);
    } else {
        reduce_chunks<4, kMaxChunks / 4>(H, blocks, E, b, s.total_s, s.base);
    }
    for (int x = threadIdx.x; x < kWaves * E; x += kThreads) s.cnt[x] = 0;
    __syncthreads();

    segment_starts(s, b, E, align, M, counts, offsets, status, layout_range, recv_stats);
    if (b == 0 && status != nullptr && wave == 0) {
        int32_t nb = 0;
        for (int g = lane; g < blocks; g += kWave) nb += bad[g];
        nb = wave_sum(nb);
        if (lane == 0) status[0] = nb;
    }
    uint64_t peers[B];
    // (assign_count's first barrier also orders segment_starts' base writes
    // before assign_rank reads them)
    assign_count<B, PLAN>(s, e_first, peers, ids, stride, nk, K, E, nbits, chunk, b, active);
    assign_rank<B, PLAN>(s, e_first, peers, ids, stride, nk, K, E, nbits, chunk, b, active, pos,
                         row_pair, cap, M, PLAN ? order : nullptr);
    mark_unused_rows(s, b, E, align, M, cap, row_pair);
}

// ---------------------------------------------------------------------------
// One launch for mid-size batches (kOneLaunchPairs < N*K <= kOnePassMaxPairs,
// contiguous 16-byte-aligned ids): no histogram kernel and no workspace.
// Every workgroup counts the whole batch itself. Its threads issue all their
// 16-byte id loads at once (kOnePassLoads per thread, one round), and while
// they are in flight count the workgroup's own chunk per wave (the first
// half of layout_assign's assignment, which needs no other chunk). Then each
// valid pair adds to a counter of its expert with one LDS atomic: 1 in the
// low half and, for a pair before the workgroup's chunk, also 1 in the high
// half. Additions commute, so the totals and the earlier-chunk counts are
// the same for any order of the atomics, and N*K < 2^16 keeps the halves
// apart. The offsets and the rows of the chunk then follow as in
// layout_assign. At the prefill size this replaces two launches (and a
// second pass over the ids) with one; each workgroup reads the whole 128 KB
// of ids, from L2 after the first workgroup of its XCD.
// ---------------------------------------------------------------------------
constexpr int kOnePassLoads = 32;   // 16-byte loads per thread
constexpr uint32_t kOnePassRound = (uint32_t)kThreads * 4 * kOnePassLoads;   // pairs
constexpr int kOnePassWords = 6144;  // LDS words of the counters

// The counters: E + 2 slots of R = 2^RL copies each. Slot 0 takes masked
// ids (< 0, never read), slot e + 1 expert e, slot E + 1 ids >= E; copy
// (lane mod R) of slot q is word q*R + (lane mod R), so lanes of one wave
// that count the same expert spread over R words instead of serialising on
// one. R = 16 up to E = 382, 8 up to 766, else 4 (within kOnePassWords). A
// slot's count is the sum of its copies; the low halves sum to at most
// N*K < 2^16, so the words are summed whole.
inline int onepass_copies_log2(int32_t E) {
    return (E + 2) * 16 <= kOnePassWords ? 4 : (E + 2) * 8 <= kOnePassWords ? 3 : 2;
}

// The ids of pairs 0 .. kOnePassRound - 1, 16 bytes per load; reads past
// the last id return 0 (and are skipped by count_ids).
__device__ __forceinline__ void load_all_ids(u32x4 (&x)[kOnePassLoads],
                                             const int32_t* __restrict__ ids, uint32_t nk) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(ids), 0, (int32_t)(nk * 4u), kBufferWord3);
#pragma unroll
    for (int j = 0; j < kOnePassLoads; ++j) {
        const uint32_t i0 = ((uint32_t)j * kThreads + threadIdx.x) * 4u;
        x[j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int32_t)(i0 * 4u), 0, 0));
    }
}

// Counts the loaded ids (CHECK: some of them past nk). The slot of an id is
// a clamp to [-1, E] plus one: no branch around the atomic. `before` is a
// multiple of 4 or at least nk, so the four ids of one 16-byte load lie on
// the same side of it. `mine` is this lane's copy of slot 0.
template <bool CHECK, int RL>
__device__ __forceinline__ void count_ids(const u32x4 (&x)[kOnePassLoads], uint32_t nk,
                                          int32_t E, uint32_t before,
                                          uint32_t* __restrict__ mine) {
#pragma unroll
    for (int j = 0; j < kOnePassLoads; ++j) {
        const uint32_t i0 = ((uint32_t)j * kThreads + threadIdx.x) * 4u;
        const uint32_t add = i0 < before ? 0x10001u : 1u;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int32_t q = min(max((int32_t)x[j][c], -1), E) + 1;
            if (!CHECK || i0 + c < nk) atomicAdd(&mine[q << RL], add);
        }
    }
}

// Sum of the R copies of slot q (16-byte LDS reads; q*R*4 is a multiple of 16).
template <int RL>
__device__ __forceinline__ uint32_t slot_sum(const uint32_t* counters, int q) {
    const u32x4* v = reinterpret_cast<const u32x4*>(counters + (q << RL));
    u32x4 a = v[0];
#pragma unroll
    for (int r = 1; r < (1 << RL) / 4; ++r) a += v[r];
    return a[0] + a[1] + a[2] + a[3];
}

template <int B, int RL, bool PLAN>
__global__ __launch_bounds__(kThreads) void layout_onepass(
    const int32_t* __restrict__ ids, uint32_t nk, uint32_t K, int32_t E, int32_t chunk,
    int nbits, int32_t blocks, int32_t align, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ status, int32_t* __restrict__ pos,
    int32_t* __restrict__ row_pair, int64_t cap, int32_t M, int32_t* __restrict__ order,
    int64_t* __restrict__ layout_range, int32_t* __restrict__ recv_stats) {
    constexpr int R = 1 << RL;
    __shared__ AssignLds<PLAN> s;
    __shared__ __attribute__((aligned(16))) uint32_t counters[kOnePassWords];   // slot q, copy r at q*R + r
    const int lane = threadIdx.x & (kWave - 1);
    const int b = blockIdx.x;
    const bool active = b < blocks;
    const int quarter = chunk / kWaves;
    const int steps = active ? quarter / kWave : 0;
    const uint32_t first = (uint32_t)b * chunk + (threadIdx.x / kWave) * quarter;

    int32_t e_first[B];
    load_ids(e_first, ids, (int64_t)K, nk, K, first, 0, steps, lane);
    u32x4 x[kOnePassLoads];
    load_all_ids(x, ids, nk);
    u32x4* const c4 = reinterpret_cast<u32x4*>(counters);
    for (int i = threadIdx.x; i < (E + 2) * (R / 4); i += kThreads) c4[i] = u32x4{0, 0, 0, 0};
    for (int i = threadIdx.x; i < kWaves * E; i += kThreads) s.cnt[i] = 0;
    __syncthreads();

    // The own chunk, while the loads of all ids are in flight.
    uint64_t peers[B];
    assign_count<B, PLAN>(s, e_first, peers, ids, (int64_t)K, nk, K, E, nbits, chunk, b, active);

    const uint32_t before = active ? (uint32_t)b * chunk : nk;
    uint32_t* const mine = counters + (lane & (R - 1));
    if (nk == kOnePassRound)
        count_ids<false, RL>(x, nk, E, before, mine);
    else
        count_ids<true, RL>(x, nk, E, before, mine);
    __syncthreads();
    // Experts tid, tid + 256, ...: totals (low halves) and pairs before the
    // chunk (high halves); thread 0 also takes the ids >= E.
    for (int e = threadIdx.x; e < E; e += kThreads) {
        const uint32_t w = slot_sum<RL>(counters, e + 1);
        s.total_s[e] = (int32_t)(w & 0xffffu);
        s.base[e] = (int32_t)(w >> 16);
    }
    const int32_t nbad = threadIdx.x == 0 ? (int32_t)(slot_sum<RL>(counters, E + 1) & 0xffffu) : 0;
    __syncthreads();

    segment_starts(s, b, E, align, M, counts, offsets, status, layout_range, recv_stats);
    if (b == 0 && status != nullptr && threadIdx.x == 0) status[0] = nbad;
    __syncthreads();   // segment_starts' base writes before assign_rank reads them
    assign_rank<B, PLAN>(s, e_first, peers, ids, (int64_t)K, nk, K, E, nbits, chunk, b, active,
                         pos, row_pair, cap, M, PLAN ? order : nullptr);
    mark_unused_rows(s, b, E, align, M, cap, row_pair);
}

}  // namespace
}  // namespace moe

using namespace moe;

// Both launches of a layout. B, the 64-pair steps of ids a wave holds per
// batch, follows the chunk size: 4 steps when a wave's quarter has at most
// 4 (short code for small batches), else 16 (fewer dependent load rounds).
template <int B>
static void launch_layout_b(const Plan& p, uint32_t assign_grid, const int32_t* ids,
                            int64_t stride, int64_t nk, int32_t K, int32_t E, int32_t align,
                            int32_t* H, int32_t* bad, int32_t* counts, int32_t* offsets,
                            int32_t* status, int32_t* pos, int32_t* row_pair, int64_t cap,
                            int32_t M, int32_t* order, int64_t* layout_range, int32_t* recv_stats,
                            hipStream_t stream) {
    if (p.blocks > 0)
        layout_hist<B><<<p.blocks, kThreads, 0, stream>>>(ids, stride, (uint32_t)nk, (uint32_t)K,
                                                          E, p.chunk, p.nbits, H, bad);
    if (order != nullptr)
        layout_assign<B, true><<<assign_grid, kThreads, 0, stream>>>(
            ids, stride, (uint32_t)nk, (uint32_t)K, E, p.chunk, p.nbits, p.blocks, align, H, bad,
            counts, offsets, status, pos, row_pair, cap, M, order, layout_range, recv_stats);
    else
        layout_assign<B, false><<<assign_grid, kThreads, 0, stream>>>(
            ids, stride, (uint32_t)nk, (uint32_t)K, E, p.chunk, p.nbits, p.blocks, align, H, bad,
            counts, offsets, status, pos, row_pair, cap, M, nullptr, layout_range, recv_stats);
}

static void launch_layout(const Plan& p, uint32_t assign_grid, const int32_t* ids,
                          int64_t stride, int64_t nk, int32_t K, int32_t E, int32_t align,
                          int32_t* H, int32_t* bad, int32_t* counts, int32_t* offsets,
                          int32_t* status, int32_t* pos, int32_t* row_pair, int64_t cap,
                          int32_t M, int32_t* order, int64_t* layout_range, int32_t* recv_stats,
                          hipStream_t stream) {
    if (p.chunk / kThreads > kBatchSmall)
        launch_layout_b<kBatchLarge>(p, assign_grid, ids, stride, nk, K, E, align, H, bad, counts,
                                     offsets, status, pos, row_pair, cap, M, order, layout_range,
                                     recv_stats, stream);
    else
        launch_layout_b<kBatchSmall>(p, assign_grid, ids, stride, nk, K, E, align, H, bad, counts,
                                     offsets, status, pos, row_pair, cap, M, order, layout_range,
                                     recv_stats, stream);
}

// Mid-size batches of contiguous, 16-byte-aligned ids take layout_onepass:
// one launch, no workspace reads or writes. The limit keeps N*K below 2^16
// (the packed counters) and one round of id loads per thread.
constexpr int64_t kOnePassMaxPairs = (int64_t)kThreads * 4 * kOnePassLoads;
static_assert(kOnePassMaxPairs < (1 << 16), "packed counters hold N*K < 2^16");

static bool use_onepass(const int32_t* ids, int64_t stride, int32_t K, int64_t nk) {
    return nk > kOneLaunchPairs && nk <= kOnePassMaxPairs && stride == (int64_t)K &&
           aligned(ids, 16);
}

template <int B, int RL>
static void launch_onepass_br(const Plan& p, uint32_t grid, const int32_t* ids, int64_t nk,
                              int32_t K, int32_t E, int32_t align, int32_t* counts,
                              int32_t* offsets, int32_t* status, int32_t* pos, int32_t* row_pair,
                              int64_t cap, int32_t M, int32_t* order, int64_t* layout_range,
                              int32_t* recv_stats, hipStream_t stream) {
    if (order != nullptr)
        layout_onepass<B, RL, true><<<grid, kThreads, 0, stream>>>(
            ids, (uint32_t)nk, (uint32_t)K, E, p.chunk, p.nbits, p.blocks, align, counts, offsets,
            status, pos, row_pair, cap, M, order, layout_range, recv_stats);
    else
        layout_onepass<B, RL, false><<<grid, kThreads, 0, stream>>>(
            ids, (uint32_t)nk, (uint32_t)K, E, p.chunk, p.nbits, p.blocks, align, counts, offsets,
            status, pos, row_pair, cap, M, nullptr, layout_range, recv_stats);
}

template <int B>
static void launch_onepass_b(const Plan& p, uint32_t grid, const int32_t* ids, int64_t nk,
                             int32_t K, int32_t E, int32_t align, int32_t* counts,
                             int32_t* offsets, int32_t* status, int32_t* pos, int32_t* row_pair,
                             int64_t cap, int32_t M, int32_t* order, int64_t* layout_range,
                             int32_t* recv_stats, hipStream_t stream) {
    switch (onepass_copies_log2(E)) {
    case 4:
        launch_onepass_br<B, 4>(p, grid, ids, nk, K, E, align, counts, offsets, status, pos,
                                row_pair, cap, M, order, layout_range, recv_stats, stream);
        break;
    case 3:
        launch_onepass_br<B, 3>(p, grid, ids, nk, K, E, align, counts, offsets, status, pos,
                                row_pair, cap, M, order, layout_range, recv_stats, stream);
        break;
    default:
        launch_onepass_br<B, 2>(p, grid, ids, nk, K, E, align, counts, offsets, status, pos,
                                row_pair, cap, M, order, layout_range, recv_stats, stream);
    }
}

static void launch_onepass(const Plan& p, uint32_t grid, const int32_t* ids, int64_t nk,
                           int32_t K, int32_t E, int32_t align, int32_t* counts, int32_t* offsets,
                           int32_t* status, int32_t* pos, int32_t* row_pair, int64_t cap,
                           int32_t M, int32_t* order, int64_t* layout_range, int32_t* recv_stats,
                           hipStream_t stream) {
    if (p.chunk / kThreads > kBatchSmall)
        launch_onepass_b<kBatchLarge>(p, grid, ids, nk, K, E, align, counts, offsets, status, pos,
                                      row_pair, cap, M, order, layout_range, recv_stats, stream);
    else
        launch_onepass_b<kBatchSmall>(p, grid, ids, nk, K, E, align, counts, offsets, status, pos,
                                      row_pair, cap, M, order, layout_range, recv_stats, stream);
}

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

// Checks of moe_get_layout's arguments other than the workspace (shared with
// moe_get_layout_noalloc; `fn` names the entry point in the message).
static int check_layout_args(const char* fn, const int32_t* ids, int64_t ids_row_stride,
                             int32_t N, int32_t K, int32_t E, int32_t align,
                             const int32_t* counts, const int32_t* offsets, const int32_t* pos,
                             const int32_t* row_pair, int64_t cap, const int32_t* order,
                             const int32_t* status) {
    if (N < 0 || K < 1 || E < 1 || align < 1)
        return fail(MOE_ERR_ARG, "%s: need N >= 0, K >= 1, E >= 1, align >= 1 "
                    "(got N=%d K=%d E=%d align=%d)", fn, N, K, E, align);
    if (K > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_LIMIT, "%s: K=%d E=%d beyond K <= %d, E <= %d", fn, K, E,
                    MOE_MAX_TOPK, MOE_MAX_EXPERTS);
    const int64_t nk = (int64_t)N * K;
    if (nk >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "%s: N*K=%lld must be below 2^31", fn, (long long)nk);
    if (N > 0 && (ids == nullptr || pos == nullptr))
        return fail(MOE_ERR_ARG, "%s: ids and pos must not be NULL", fn);
    if (N > 0 && ids_row_stride < K)
        return fail(MOE_ERR_ARG, "%s: ids_row_stride=%lld < K=%d", fn,
                    (long long)ids_row_stride, K);
    if (counts == nullptr || offsets == nullptr)
        return fail(MOE_ERR_ARG, "%s: counts and offsets must not be NULL", fn);
    const int64_t need = moe_required_capacity(N, K, E, align);
    if (cap < need)
        return fail(MOE_ERR_CAPACITY, "%s: cap=%lld below the worst case %lld", fn,
                    (long long)cap, (long long)need);
    if (cap >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "%s: cap=%lld must be below 2^31", fn, (long long)cap);
    if (cap > 0 && row_pair == nullptr)
        return fail(MOE_ERR_ARG, "%s: row_pair must not be NULL", fn);
    if (!aligned(ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(pos, 4) ||
        !aligned(row_pair, 4) || !aligned(order, 4) || !aligned(status, 4))
        return fail(MOE_ERR_ALIGN, "%s: int32 pointers must be 4-byte aligned", fn);
    return MOE_OK;
}

// The layout proper, on validated arguments, with its workspace at H (at
// least workspace_for(make_plan(N, K, E), E) bytes).
static int run_layout(const char* fn, const int32_t* ids, int64_t ids_row_stride, int32_t N,
                      int32_t K, int32_t E, int32_t align, int32_t* counts, int32_t* offsets,
                      int32_t* pos, int32_t* row_pair, int64_t cap, int32_t* order, int32_t* H,
                      int32_t* status, hipStream_t stream) {
    const int64_t nk = (int64_t)N * K;
    if (N > 0 && nk <= kOneLaunchPairs)
        return layout_one_launch(ids, ids_row_stride, N, K, E, align, counts, offsets, pos,
                                 row_pair, cap, order, status, stream);
    const Plan p = make_plan(N, K, E);
    clear_launch_error();
    if (use_onepass(ids, ids_row_stride, K, nk)) {
        launch_onepass(p, p.blocks, ids, nk, K, E, align, counts, offsets, status, pos, row_pair,
                       cap, 0, order, nullptr, nullptr, stream);
    } else {
        int32_t* bad = H + (int64_t)p.blocks * E;
        launch_layout(p, p.blocks > 0 ? p.blocks : 1, ids, ids_row_stride, nk, K, E, align, H,
                      bad, counts, offsets, status, pos, row_pair, cap, 0, order, nullptr, nullptr,
                      stream);
    }
    const int rc = check_launch(fn);
    if (rc != MOE_OK) return rc;
    return debug_check_layout(fn, pos, nk, row_pair, cap, order, stream);
}

extern "C" int moe_get_layout(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                              int32_t E, int32_t align, int32_t* counts, int32_t* offsets,
                              int32_t* pos, int32_t* row_pair, int64_t cap, int32_t* order,
                              void* workspace, size_t workspace_bytes, int32_t* status,
                              hipStream_t stream) {
    const int rc = check_layout_args("moe_get_layout", ids, ids_row_stride, N, K, E, align,
                                     counts, offsets, pos, row_pair, cap, order, status);
    if (rc != MOE_OK) return rc;
    const size_t ws = workspace_for(make_plan(N, K, E), E);
    if (workspace == nullptr || workspace_bytes < ws)
        return fail(MOE_ERR_WORKSPACE, "moe_get_layout: workspace of %zu bytes needed, got %zu%s",
                    ws, workspace_bytes, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 4))
        return fail(MOE_ERR_ALIGN, "moe_get_layout: workspace must be 4-byte aligned");
    return run_layout("moe_get_layout", ids, ids_row_stride, N, K, E, align, counts, offsets, pos,
                      row_pair, cap, order, static_cast<int32_t*>(workspace), status, stream);
}

// ---------------------------------------------------------------------------
// moe_get_layout_noalloc: moe_get_layout for callers that cannot allocate
// device memory. Its workspace is `scratch`, a file-scope device array that
// holds the largest workspace any accepted size needs (kHEntries histogram
// entries plus kMaxChunks out-of-range counts: 65 792 bytes), one copy per
// GPU, kept until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: the kernels get the array's device address,
// looked up once per device with hipGetSymbolAddress. Every call on a GPU
// shares that GPU's copy, so calls that overlap on one GPU (on different
// streams) race; calls in one stream's order do not. Nothing in the array
// has to start at zero: the histogram kernel writes every entry the assign
// kernel reads.
// ---------------------------------------------------------------------------
constexpr size_t kScratchWords = (size_t)kHEntries + kMaxChunks;
static __device__ __align__(256) int32_t scratch[kScratchWords];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device
}  // namespace

// The device address of `scratch` on the device that runs `stream`, looked
// up on the first call for that device (with that device current).
static int scratch_on(hipStream_t stream, int32_t** out) {
    int dev = -1;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "moe_get_layout_noalloc: no device for the stream: %s",
                    hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_LIMIT, "moe_get_layout_noalloc: device %d beyond %d devices", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* ptr = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || ptr == nullptr)
            return fail(MOE_ERR_HIP, "moe_get_layout_noalloc: scratch address on device %d: %s",
                        dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<int32_t*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

extern "C" int moe_get_layout_noalloc(const int32_t* ids, int64_t ids_row_stride, int32_t N,
                                      int32_t K, int32_t E, int32_t align, int32_t* counts,
                                      int32_t* offsets, int32_t* pos, int32_t* row_pair,
                                      int64_t cap, int32_t* order, int32_t* status,
                                      hipStream_t stream) {
    const char* fn = "moe_get_layout_noalloc";
    int rc = check_layout_args(fn, ids, ids_row_stride, N, K, E, align, counts, offsets, pos,
                               row_pair, cap, order, status);
    if (rc != MOE_OK) return rc;
    const size_t ws = workspace_for(make_plan(N, K, E), E);
    if (ws > sizeof(scratch))
        return fail(MOE_ERR_LIMIT, "%s: these sizes need %zu bytes of workspace, beyond the "
                    "%zu-byte static scratch", fn, ws, sizeof(scratch));
    int32_t* H = nullptr;
    rc = scratch_on(stream, &H);
    if (rc != MOE_OK) return rc;
    return run_layout(fn, ids, ids_row_stride, N, K, E, align, counts, offsets, pos, row_pair,
                      cap, order, H, status, stream);
}

extern "C" int moe_get_layout_padded(const int32_t* ids, int64_t ids_row_stride, int32_t N,
                                     int32_t K, int32_t E, int32_t M, int32_t* counts,
                                     int32_t* pos, int32_t* row_pair, int64_t* layout_range,
                                     int32_t* recv_stats, void* workspace, size_t workspace_bytes,
                                     int32_t* status, hipStream_t stream) {
    if (N < 0 || K < 1 || E < 1 || M < 1)
        return fail(MOE_ERR_ARG, "moe_get_layout_padded: need N >= 0, K >= 1, E >= 1, M >= 1 "
                    "(got N=%d K=%d E=%d M=%d)", N, K, E, M);
    if (K > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_LIMIT, "moe_get_layout_padded: K=%d E=%d beyond K <= %d, E <= %d", K,
                    E, MOE_MAX_TOPK, MOE_MAX_EXPERTS);
    const int64_t nk = (int64_t)N * K;
    const int64_t cap = (int64_t)E * M;
    if (nk >= ((int64_t)1 << 31) || cap >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_get_layout_padded: N*K and E*M must be below 2^31");
    if (N > 0 && (ids == nullptr || pos == nullptr))
        return fail(MOE_ERR_ARG, "moe_get_layout_padded: ids and pos must not be NULL");
    if (N > 0 && ids_row_stride < K)
        return fail(MOE_ERR_ARG, "moe_get_layout_padded: ids_row_stride < K");
    if (counts == nullptr || row_pair == nullptr)
        return fail(MOE_ERR_ARG, "moe_get_layout_padded: counts and row_pair must not be NULL");
    if (!aligned(ids, 4) || !aligned(counts, 4) || !aligned(pos, 4) || !aligned(row_pair, 4) ||
        !aligned(recv_stats, 4) || !aligned(status, 4) || !aligned(layout_range, 8))
        return fail(MOE_ERR_ALIGN, "moe_get_layout_padded: int32 pointers must be 4-byte aligned "
                    "and layout_range 8-byte aligned");
    const Plan p = make_plan(N, K, E);
    const size_t ws = workspace_for(p, E);
    if (workspace == nullptr || workspace_bytes < ws)
        return fail(MOE_ERR_WORKSPACE, "moe_get_layout_padded: workspace of %zu bytes needed, "
                    "got %zu", ws, workspace_bytes);
    if (!aligned(workspace, 4))
        return fail(MOE_ERR_ALIGN, "moe_get_layout_padded: workspace must be 4-byte aligned");
    // The one-launch form marks unused rows from N workgroups: used for small
    // batches with at most 2^18 padded rows (and a status word to write).
    if (N > 0 && nk <= kOneLaunchPairs && cap <= (1 << 18) && status != nullptr)
        return layout_padded_one_launch(ids, ids_row_stride, N, K, E, M, counts, pos, row_pair,
                                        layout_range, recv_stats, status, stream);
    clear_launch_error();
    int32_t* H = static_cast<int32_t*>(workspace);
    int32_t* bad = H + (int64_t)p.blocks * E;
    // Workgroups past the chunks only mark unused rows: one per 2048 rows,
    // at most 256.
    int64_t grid = ceil_div<int64_t>(cap, 8 * kThreads);
    if (grid > 256) grid = 256;
    if (grid < p.blocks) grid = p.blocks;
    if (grid < 1) grid = 1;
    if (use_onepass(ids, ids_row_stride, K, nk))
        launch_onepass(p, (uint32_t)grid, ids, nk, K, E, 1, counts, nullptr, status, pos,
                       row_pair, cap, M, nullptr, layout_range, recv_stats, stream);
    else
        launch_layout(p, (uint32_t)grid, ids, ids_row_stride, nk, K, E, 1, H, bad, counts,
                      nullptr, status, pos, row_pair, cap, M, nullptr, layout_range, recv_stats,
                      stream);
    const int rc = check_launch("moe_get_layout_padded");
    if (rc != MOE_OK) return rc;
    return debug_check_layout("moe_get_layout_padded", pos, nk, row_pair, cap, nullptr, stream);
}
