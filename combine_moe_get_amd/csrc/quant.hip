// quant.hip -- dispatch with an FP8 (e4m3fn) cast and per-128-channel scales,
// the payload form of DeepEP's low-latency dispatch with use_fp8 (repository
// dump, deep_ep.cpp, Buffer::low_latency_dispatch: bf16 x, e4m3 payload,
// fp32 scales per token and 128 channels stored column-major, or 8-bit
// exponents of power-of-two scales with use_ue8m0 and round_scale).
//
// The cast is not on the pages; this library takes, per token and block:
// s = max(amax / 448, 2^-126), rounded up to a power of two with round_scale,
// q = e4m3(x / s) with round to nearest even and saturation at +-448.
//
// The cast depends on the token only, so one wave quantises a (token, 1024
// channels) slice once and writes it to the rows of all K pairs. Lane i
// holds 16 channels (two 16-byte loads); the 8 lanes of a 128-channel block
// exchange their partial amax with three DPP lane swaps, so every lane of
// the block derives the same scale. Each destination row then takes one
// 16-byte non-temporal store per lane: 1 KiB contiguous per wave and row.
#include "fp8.hpp"
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kChanPerLane = 16;
constexpr int kChanPerWave = kWave * kChanPerLane;   // 1024
constexpr int kBlock = 128;
constexpr int kLanesPerBlock = kBlock / kChanPerLane;  // 8

struct Fp8Args {
    const uint16_t* x;
    int64_t xs;          // elements
    int32_t N, K, H, segs;
    const int32_t* pos;  // NULL: identity (K == 1)
    uint8_t* dst;
    int64_t ds;          // bytes
    void* scales;
    int32_t mode;
    int64_t srs;         // MOE_SCALE_ROWS, MOE_SCALE_TOKENS: floats between rows
    int32_t M;           // rows per expert for the column-major forms
    int32_t round_scale;
};

// max of v over the 8 lanes of an aligned lane group (DPP within a row of
// 16 lanes: swap neighbours, swap pairs, then mirror the two quads).
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    return v;
}

// Loads this lane's 16 channels of segment seg (1024 channels) of token t;
// lanes past H get zeros. The 8 lanes of a 128-channel block are either all
// inside H or all past it (H % 128 == 0).
__device__ __forceinline__ bool load_segment(const Fp8Args& a, uint32_t t, int32_t seg, int lane,
                                             float (&f)[16]) {
    const int32_t c0 = seg * kChanPerWave + lane * kChanPerLane;
    const bool active = c0 < a.H;
    if (active) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.x + (int64_t)t * a.xs + c0);
        const u32x4 v0 = __builtin_nontemporal_load(src);
        const u32x4 v1 = __builtin_nontemporal_load(src + 1);
        const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = 0.0f;
    }
    return active;
}

// Quantises a loaded segment of token t once and stores it, with its scales,
// to the rows of the token's K pairs: lane k < K holds the row of pair k in
// pk (-1: not dispatched). Token-major scales are stored once, for the token.
// Every lane takes part in the lane swaps.
__device__ __forceinline__ void cast_and_store(const Fp8Args& a, uint32_t t, int32_t seg,
                                               int lane, int32_t pk, const float (&f)[16],
                                               bool active) {
    const int32_t c0 = seg * kChanPerWave + lane * kChanPerLane;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = group8_max(amax);

    float s = amax / 448.0f;
    s = fmaxf(s, __uint_as_float(0x00800000u));      // at least 2^-126
    if (a.round_scale) {
        const uint32_t sb = __float_as_uint(s);
        if (sb & 0x007FFFFFu) s = __uint_as_float((sb & 0x7F800000u) + 0x00800000u);
    }
    const u32x4 codes = {pack4(f, s), pack4(f + 4, s), pack4(f + 8, s), pack4(f + 12, s)};

    const int32_t b = c0 / kBlock;                   // this lane's block
    const int32_t nb = a.H / kBlock;
    // UE8M0: each 512 channels (32 lanes) form one word of four exponents,
    // assembled in lanes 0 and 32 from the first lane of each block.
    const uint32_t ex = __float_as_uint(s) >> 23;
    const uint32_t up8 = __shfl_down(ex, 8, kWave), up16 = __shfl_down(ex, 16, kWave),
                   up24 = __shfl_down(ex, 24, kWave);
    const uint32_t word = ex | (up8 << 8) | (up16 << 16) | (up24 << 24);

    if (a.mode == MOE_SCALE_TOKENS && (lane & (kLanesPerBlock - 1)) == 0 && active)
        static_cast<float*>(a.scales)[(int64_t)t * a.srs + b] = s;
    for (int32_t k = 0; k < a.K; ++k) {
        const int32_t p = __builtin_amdgcn_readlane(pk, k);
        if (p < 0) continue;
        if (active)
            __builtin_nontemporal_store(codes, reinterpret_cast<u32x4*>(a.dst + (int64_t)p * a.ds + c0));
        if (a.mode == MOE_SCALE_TOKENS) continue;   // stored once above
        if (a.mode == MOE_SCALE_UE8M0) {
            if ((lane & 31) == 0 && active) {
                const int64_t i = ((int64_t)(p / a.M) * (nb / 4) + b / 4) * a.M + p % a.M;
                static_cast<uint32_t*>(a.scales)[i] = word;
            }
        } else if ((lane & (kLanesPerBlock - 1)) == 0 && active) {
            const int64_t i = a.mode == MOE_SCALE_ROWS
                                  ? (int64_t)p * a.srs + b
                                  : ((int64_t)(p / a.M) * nb + b) * a.M + p % a.M;
            static_cast<float*>(a.scales)[i] = s;
        }
    }
}

__global__ __launch_bounds__(256) void dispatch_fp8_kernel(const Fp8Args a, uint32_t first_block) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t gw = (first_block + blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
    const uint32_t t = __builtin_amdgcn_readfirstlane(gw / (uint32_t)a.segs);
    if (t >= (uint32_t)a.N) return;
    const int32_t seg = (int32_t)(gw - t * (uint32_t)a.segs);

    // Rows of the token's K pairs: lane k < K fetches pos[t*K + k].
    int32_t pk = (int32_t)t;
    if (a.pos != nullptr) pk = lane < a.K ? a.pos[(int64_t)t * a.K + lane] : -1;
    float f[16];
    const bool active = load_segment(a, t, seg, lane, f);
    cast_and_store(a, t, seg, lane, pk, f, active);
}

// ---------------------------------------------------------------------------
// Padded layout and FP8 dispatch in one launch, for small batches. In the
// padded layout pair (t, k) with expert e lands on row e*M + r, where r is the
// number of earlier pairs in (t, k) order with the same expert (r >= M:
// dropped): no global offsets are needed, so every workgroup can find its
// token's rows from one pass over the batch's ids. Workgroup (t, g) takes
// token t and the 1024-channel segments 4g .. 4g+3 (one per wave):
//   1. one pass over all N*K ids: per-expert totals in LDS (integer atomics,
//      so the totals do not depend on their order) and, per expert, the
//      pairs of earlier tokens, bef(e);
//   2. r(t, k) = bef(e_k) + (earlier k' < k of the token with e_k' = e_k);
//      workgroup (t, 0) writes pos and row_pair of the token's pairs;
//   3. workgroup 0 writes counts and status from the totals; every expert's
//      unused rows are marked -1 by workgroup e mod (number of workgroups);
//   4. each wave casts and stores its segment (cast_and_store), whose
//      channels it loaded before step 1.
// Used and unused rows are disjoint sets derived from the same totals, so
// no two workgroups write the same row_pair entry.
// ---------------------------------------------------------------------------

constexpr int kFusedThreads = 256;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedMaxPairs = 8192;

struct FusedArgs {
    const int32_t* ids;
    int64_t ids_stride;
    int32_t E, groups;   // groups: workgroups per token
    int32_t* counts;
    int32_t* pos;
    int32_t* row_pair;
    int64_t* layout_range;   // may be NULL
    int32_t* recv_stats;     // may be NULL
    int32_t* status;
};

__global__ __launch_bounds__(kFusedThreads) void dispatch_fp8_padded_kernel(const Fp8Args a,
                                                                            const FusedArgs f) {
    __shared__ int32_t tot[MOE_MAX_EXPERTS];
    __shared__ int32_t bef[MOE_MAX_EXPERTS];
    __shared__ int32_t rows[MOE_MAX_TOPK];
    __shared__ int32_t tok_e[MOE_MAX_TOPK];
    __shared__ int32_t nbad_s, drop_s;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t t = blockIdx.x / (uint32_t)f.groups;
    const int32_t g = (int32_t)(blockIdx.x - t * (uint32_t)f.groups);
    const int32_t K = a.K, E = f.E, M = a.M;
    const int32_t nk = a.N * K;
    // N = 0 launches one workgroup for counts, status and row_pair only
    const bool has_token = t < (uint32_t)a.N;
    const int32_t* idrow = f.ids + (int64_t)t * f.ids_stride;

    // The token's channels do not depend on the layout: their loads are
    // issued first and complete during the count pass.
    const int32_t seg = g * kFusedWaves + wave;
    const bool casts = has_token && seg < a.segs;
    float xv[16];
    bool active = false;
    if (casts) active = load_segment(a, t, seg, lane, xv);

    for (int e = threadIdx.x; e < E; e += kFusedThreads) {
        tot[e] = 0;
        bef[e] = 0;
    }
    if ((int32_t)threadIdx.x < K) tok_e[threadIdx.x] = has_token ? idrow[threadIdx.x] : -1;
    if (threadIdx.x == 0) nbad_s = drop_s = 0;
    __syncthreads();

    // 1. totals, bad ids, and per expert the pairs of tokens before t
    count_batch_ids(f.ids, f.ids_stride, nk, K, E, (int32_t)t * K, tot, bef, &nbad_s);
    __syncthreads();

    // 2. the token's rows
    if (has_token && (int32_t)threadIdx.x < K) {
        const int32_t k = threadIdx.x;
        const int32_t e = tok_e[k];
        int32_t p = -1;
        if (e >= 0 && e < E) {
            const int32_t r = rank_in_expert(tok_e, bef, k);
            if (r < M) p = e * M + r;
        }
        rows[k] = p;
        if (g == 0) {
            f.pos[(int64_t)t * K + k] = p;
            if (p >= 0) f.row_pair[p] = (int32_t)t * K + k;
        }
    }

    // 3. counts and status (workgroup 0), unused rows (spread by expert)
    const uint32_t B = gridDim.x;
    if (blockIdx.x == 0) {
        int32_t d = 0;
        for (int e = threadIdx.x; e < E; e += kFusedThreads) {
            const int32_t kept = min(tot[e], M);
            f.counts[e] = kept;
            // one source: its range of expert e's rows (begin 0 in the high
            // half, count in the low) and the running count received
            if (f.layout_range != nullptr) f.layout_range[e] = (int64_t)kept;
            if (f.recv_stats != nullptr) f.recv_stats[e] += kept;
            d += max(tot[e] - M, 0);
        }
        if (d) atomicAdd(&drop_s, d);
    }
    for (int32_t e = blockIdx.x; e < E; e += (int32_t)B)
        for (int32_t r = min(tot[e], M) + threadIdx.x; r < M; r += kFusedThreads)
            f.row_pair[(int64_t)e * M + r] = -1;
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        f.status[0] = nbad_s;
        f.status[1] = drop_s;
    }

    // 4. cast and store this workgroup's segments
    if (!casts) return;
    const int32_t pk = lane < K ? rows[lane] : -1;
    cast_and_store(a, t, seg, lane, pk, xv, active);
}

// ---------------------------------------------------------------------------
// Column-major scales from token-major ones. Row p = e*M + m of the padded
// layout holds pair r = row_pair[p] (-1: unused), i.e. token r / K, so its
// scale of block b is token_scales[(r / K)*tss + b]. Written by destination
// row, every store is a run along m: one wave takes 64 consecutive rows of
// one expert, loads their row_pair entries once, gathers each lane's token
// scales and stores one 256-byte run per block (fp32) or per 4-block word
// (UE8M0). Entries outside [0, N*K) count as unused, so the gathers stay
// inside the token scales whatever row_pair holds.
//
// The gathers are unconditional, so that all of them are in flight at once:
// a lane without a row reads token 0's scales and stores nothing, and block
// indices past the last block are clamped to it. (Loads under a per-lane
// condition each wait for the one before: a wave's kGather gathers would
// take kGather round trips.) With 16-byte aligned token rows and H % 512 ==
// 0 a lane fetches four blocks per load.
// ---------------------------------------------------------------------------

constexpr int kScatterThreads = 256;
constexpr int kGather = 64;   // floats gathered per lane and pass

struct ScatterArgs {
    const float* ts;
    int64_t tss;          // floats between token rows
    const int32_t* row_pair;
    int32_t NK, K, E, M, chunks, nb;
    void* out;
    int32_t mode;
};

// Units u0 .. u0 + J - 1 of one token's scales, each index clamped to the
// last unit (nu - 1). A unit is 4 blocks (QUAD: one 16-byte load when VEC) or
// one block.
template <bool VEC, bool QUAD, int J>
__device__ __forceinline__ void gather_units(const float* src, int32_t u0, int32_t nu,
                                             float (&v)[kGather]) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int32_t u = min(u0 + j, nu - 1);
        if constexpr (QUAD && VEC) {
            const u32x4 q = reinterpret_cast<const u32x4*>(src)[u];
            v[4 * j] = __uint_as_float(q.x);
            v[4 * j + 1] = __uint_as_float(q.y);
            v[4 * j + 2] = __uint_as_float(q.z);
            v[4 * j + 3] = __uint_as_float(q.w);
        } else if constexpr (QUAD) {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[4 * j + c] = src[4 * u + c];
        } else {
            v[j] = src[u];
        }
    }
    // Keep the loads here: the stores that use them sit under a per-lane
    // condition, into which the compiler would otherwise sink them.
#pragma unroll
    for (int j = 0; j < (QUAD ? 4 * J : J); ++j) asm volatile("" : "+v"(v[j]));
}

template <bool VEC>
__global__ __launch_bounds__(kScatterThreads) void scatter_scales_kernel(const ScatterArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(
        blockIdx.x * (kScatterThreads / kWave) + threadIdx.x / kWave);
    // Chunk-major numbering: waves 0 .. E-1 take chunk 0 of every expert,
    // the next E chunk 1, and so on. The used rows of an expert are its first
    // ones, so the waves with work come first and their workgroups spread
    // over all XCDs (workgroup i runs on XCD i mod 8). Expert-major numbering
    // put them on the workgroups 16e at M = 4096, all on one XCD (28 us
    // against 10 us at M = 4128 for the same bytes).
    const uint32_t c = wave / (uint32_t)a.E;
    if (c >= (uint32_t)a.chunks) return;
    const uint32_t e = wave - c * (uint32_t)a.E;
    const int32_t m = (int32_t)c * kWave + lane;
    const int32_t r = m < a.M ? a.row_pair[(int64_t)e * a.M + m] : -1;
    const bool valid = r >= 0 && r < a.NK;
    if (__ballot(valid) == 0) return;
    const float* src = a.ts + (valid ? (int64_t)(r / a.K) * a.tss : 0);   // N >= 1

    if (a.mode == MOE_SCALE_COLS && !VEC) {   // any nb: one block per unit
        float* dst = static_cast<float*>(a.out) + (int64_t)e * a.nb * a.M + m;
        for (int32_t u0 = 0; u0 < a.nb; u0 += kGather) {
            float v[kGather];
            gather_units<false, false, kGather>(src, u0, a.nb, v);
            if (!valid) continue;
#pragma unroll
            for (int j = 0; j < kGather; ++j)
                if (u0 + j < a.nb) dst[(int64_t)(u0 + j) * a.M] = v[j];
        }
        return;
    }
    constexpr int J = kGather / 4;   // quads per pass
    const int32_t nq = a.nb / 4;
    if (a.mode == MOE_SCALE_COLS) {
        float* dst = static_cast<float*>(a.out) + (int64_t)e * a.nb * a.M + m;
        for (int32_t u0 = 0; u0 < nq; u0 += J) {
            float v[kGather];
            gather_units<VEC, true, J>(src, u0, nq, v);
            if (!valid) continue;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int32_t q = u0 + j;
                if (q >= nq) break;
#pragma unroll
                for (int c = 0; c < 4; ++c) dst[(int64_t)(4 * q + c) * a.M] = v[4 * j + c];
            }
        }
    } else {
        // UE8M0: byte c of word q is the exponent field of block 4q + c
        // (the scales are powers of two, so the field is the whole value).
        uint32_t* dst = static_cast<uint32_t*>(a.out) + (int64_t)e * nq * a.M + m;
        for (int32_t u0 = 0; u0 < nq; u0 += J) {
            float v[kGather];
            gather_units<VEC, true, J>(src, u0, nq, v);
            if (!valid) continue;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int32_t q = u0 + j;
                if (q >= nq) break;
                const uint32_t w = ((__float_as_uint(v[4 * j]) >> 23) & 0xFFu) |
                                   (((__float_as_uint(v[4 * j + 1]) >> 23) & 0xFFu) << 8) |
                                   (((__float_as_uint(v[4 * j + 2]) >> 23) & 0xFFu) << 16) |
                                   (((__float_as_uint(v[4 * j + 3]) >> 23) & 0xFFu) << 24);
                dst[(int64_t)q * a.M] = w;
            }
        }
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

// Launches the padded one-launch kernel on the cast arguments `a` (a.segs =
// 0: the layout part only): one workgroup per (token, group of kFusedWaves
// segments); N = 0 still runs one workgroup, since counts, status and every
// row_pair entry are outputs.
static int launch_padded_one_launch(const Fp8Args& a, const int32_t* ids, int64_t ids_row_stride,
                                    int32_t E, int32_t* counts, int32_t* pos, int32_t* row_pair,
                                    int64_t* layout_range, int32_t* recv_stats, int32_t* status,
                                    hipStream_t stream, const char* who) {
    FusedArgs f;
    f.ids = ids;
    f.ids_stride = ids_row_stride;
    f.E = E;
    f.groups = a.segs > 0 ? ceil_div<int32_t>(a.segs, kFusedWaves) : 1;
    f.counts = counts;
    f.pos = pos;
    f.row_pair = row_pair;
    f.layout_range = layout_range;
    f.recv_stats = recv_stats;
    f.status = status;
    const int64_t blocks = a.N > 0 ? (int64_t)a.N * f.groups : 1;
    if (blocks > kMaxLaunchItems / kFusedThreads)
        return fail(MOE_ERR_LIMIT, "%s: %lld workgroups (tokens x ceil(H/%d)) exceed one launch",
                    who, (long long)blocks, kFusedWaves * kChanPerWave);
    clear_launch_error();
    dispatch_fp8_padded_kernel<<<(uint32_t)blocks, kFusedThreads, 0, stream>>>(a, f);
    const int rc = check_launch(who);
    if (rc != MOE_OK) return rc;
    return debug_check_layout(who, pos, (int64_t)a.N * a.K, row_pair, (int64_t)E * a.M, nullptr,
                              stream);
}

extern "C" int moe_dispatch_fp8_padded(const int32_t* ids, int64_t ids_row_stride, int32_t N,
                                       int32_t K, int32_t E, int32_t M, const void* x,
                                       int64_t x_row_stride, int32_t H, int32_t* counts,
                                       int32_t* pos, int32_t* row_pair, int64_t* layout_range,
                                       int32_t* recv_stats, int32_t* status, void* dst,
                                       int64_t dst_row_stride, void* scales, int32_t scale_format,
                                       int64_t scale_row_stride, int32_t round_scale,
                                       hipStream_t stream) {
    if (N < 0 || K < 1 || E < 1 || M < 1 || H < 0)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8_padded: need N >= 0, K >= 1, E >= 1, M >= 1, "
                    "H >= 0");
    if (K > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_LIMIT, "moe_dispatch_fp8_padded: K=%d E=%d beyond K <= %d, E <= %d",
                    K, E, MOE_MAX_TOPK, MOE_MAX_EXPERTS);
    if ((int64_t)N * K > kFusedMaxPairs)
        return fail(MOE_ERR_LIMIT, "moe_dispatch_fp8_padded: N*K=%lld above %d (use "
                    "moe_get_layout_padded + moe_dispatch_fp8)", (long long)N * K, kFusedMaxPairs);
    if ((int64_t)E * M >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_dispatch_fp8_padded: E*M must be below 2^31");
    if (scale_format < MOE_SCALE_ROWS || scale_format > MOE_SCALE_TOKENS)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8_padded: unknown scale_format %d", scale_format);
    if (H % kBlock != 0)
        return fail(MOE_ERR_ALIGN, "moe_dispatch_fp8_padded: H=%d must be a multiple of 128", H);
    if (scale_format == MOE_SCALE_UE8M0 && (!round_scale || H % (4 * kBlock) != 0))
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8_padded: ue8m0 scales need round_scale and "
                    "H %% 512 == 0");
    if ((scale_format == MOE_SCALE_ROWS || scale_format == MOE_SCALE_TOKENS) &&
        scale_row_stride < H / kBlock)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8_padded: scale_row_stride < H/128");
    if (counts == nullptr || row_pair == nullptr || status == nullptr)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8_padded: counts, row_pair and status must not "
                    "be NULL");
    if (N > 0 && (ids == nullptr || pos == nullptr || ids_row_stride < K))
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8_padded: NULL ids/pos or ids_row_stride < K");
    if (N > 0 && H > 0 && (x == nullptr || dst == nullptr || scales == nullptr))
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8_padded: NULL pointer");
    if (!aligned(x, 16) || x_row_stride % 8 != 0 || (N > 0 && H > 0 && x_row_stride < H))
        return fail(MOE_ERR_ALIGN, "moe_dispatch_fp8_padded: x must be 16-byte aligned with a row "
                    "stride that is a multiple of 8 elements and >= H");
    if (!aligned(dst, 16) || dst_row_stride % 16 != 0 || (N > 0 && H > 0 && dst_row_stride < H))
        return fail(MOE_ERR_ALIGN, "moe_dispatch_fp8_padded: dst must be 16-byte aligned with a "
                    "row stride that is a multiple of 16 bytes and >= H");
    if (!aligned(scales, 4) || !aligned(ids, 4) || !aligned(counts, 4) || !aligned(pos, 4) ||
        !aligned(row_pair, 4) || !aligned(recv_stats, 4) || !aligned(status, 4) ||
        !aligned(layout_range, 8))
        return fail(MOE_ERR_ALIGN, "moe_dispatch_fp8_padded: int32 and scale pointers must be "
                    "4-byte aligned and layout_range 8-byte aligned");

    Fp8Args a;
    a.x = static_cast<const uint16_t*>(x);
    a.xs = x_row_stride;
    a.N = N;
    a.K = K;
    a.H = H;
    a.segs = ceil_div<int32_t>(H, kChanPerWave);
    a.pos = nullptr;
    a.dst = static_cast<uint8_t*>(dst);
    a.ds = dst_row_stride;
    a.scales = scales;
    a.mode = scale_format;
    a.srs = scale_row_stride;
    a.M = M;
    a.round_scale = round_scale ? 1 : 0;
    return launch_padded_one_launch(a, ids, ids_row_stride, E, counts, pos, row_pair, layout_range,
                                    recv_stats, status, stream, "moe_dispatch_fp8_padded");
}

int moe::layout_padded_one_launch(const int32_t* ids, int64_t ids_row_stride, int32_t N,
                                  int32_t K, int32_t E, int32_t M, int32_t* counts, int32_t* pos,
                                  int32_t* row_pair, int64_t* layout_range, int32_t* recv_stats,
                                  int32_t* status, hipStream_t stream) {
    Fp8Args a{};        // no channels: the kernel's layout part only
    a.N = N;
    a.K = K;
    a.M = M;
    return launch_padded_one_launch(a, ids, ids_row_stride, E, counts, pos, row_pair, layout_range,
                                    recv_stats, status, stream, "moe_get_layout_padded");
}

extern "C" int moe_dispatch_fp8(const void* x, int64_t x_row_stride, int32_t N, int32_t K,
                                int32_t H, const int32_t* pos, void* dst, int64_t dst_row_stride,
                                void* scales, int32_t scale_format, int64_t scale_row_stride,
                                int32_t rows_per_expert, int32_t round_scale, hipStream_t stream) {
    if (N < 0 || K < 1 || H < 0)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8: need N >= 0, K >= 1, H >= 0");
    if (K > MOE_MAX_TOPK) return fail(MOE_ERR_LIMIT, "moe_dispatch_fp8: K=%d > %d", K, MOE_MAX_TOPK);
    if (scale_format < MOE_SCALE_ROWS || scale_format > MOE_SCALE_TOKENS)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8: unknown scale_format %d", scale_format);
    if (H % kBlock != 0)
        return fail(MOE_ERR_ALIGN, "moe_dispatch_fp8: H=%d must be a multiple of 128", H);
    if (scale_format == MOE_SCALE_UE8M0 && (!round_scale || H % (4 * kBlock) != 0))
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8: ue8m0 scales need round_scale and H %% 512 == 0");
    if ((scale_format == MOE_SCALE_COLS || scale_format == MOE_SCALE_UE8M0) && rows_per_expert < 1)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8: column-major scales need rows_per_expert >= 1");
    if ((scale_format == MOE_SCALE_ROWS || scale_format == MOE_SCALE_TOKENS) &&
        scale_row_stride < H / kBlock)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8: scale_row_stride < H/128");
    if (pos == nullptr && K != 1 && N > 0)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8: pos == NULL (identity) requires K == 1");
    const int32_t segs = ceil_div<int32_t>(H, kChanPerWave);
    const int64_t waves = (int64_t)N * segs;
    if ((int64_t)N * K >= ((int64_t)1 << 31) || waves >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_dispatch_fp8: N*K and N*ceil(H/1024) must be below 2^31");
    if (N == 0 || H == 0) return ok();
    if (x == nullptr || dst == nullptr || scales == nullptr)
        return fail(MOE_ERR_ARG, "moe_dispatch_fp8: NULL pointer");
    if (!aligned(x, 16) || x_row_stride % 8 != 0 || x_row_stride < H)
        return fail(MOE_ERR_ALIGN, "moe_dispatch_fp8: x must be 16-byte aligned with a row stride "
                    "that is a multiple of 8 elements and >= H");
    if (!aligned(dst, 16) || dst_row_stride % 16 != 0 || dst_row_stride < H)
        return fail(MOE_ERR_ALIGN, "moe_dispatch_fp8: dst must be 16-byte aligned with a row stride "
                    "that is a multiple of 16 bytes and >= H");
    if (!aligned(scales, 4) || !aligned(pos, 4))
        return fail(MOE_ERR_ALIGN, "moe_dispatch_fp8: scales and pos must be 4-byte aligned");

    Fp8Args a;
    a.x = static_cast<const uint16_t*>(x);
    a.xs = x_row_stride;
    a.N = N;
    a.K = K;
    a.H = H;
    a.segs = segs;
    a.pos = pos;
    a.dst = static_cast<uint8_t*>(dst);
    a.ds = dst_row_stride;
    a.scales = scales;
    a.mode = scale_format;
    a.srs = scale_row_stride;
    a.M = rows_per_expert;
    a.round_scale = round_scale ? 1 : 0;
    // Small batches (decode) launch one-wave workgroups to spread over more
    // CUs; large ones four-wave workgroups.
    const int threads = waves < 4096 ? kWave : 4 * kWave;
    const int64_t blocks = ceil_div<int64_t>(waves, threads / kWave);
    clear_launch_error();
    in_pieces(blocks, kMaxLaunchItems / threads, [&](int64_t first, int64_t count) {
        dispatch_fp8_kernel<<<(uint32_t)count, threads, 0, stream>>>(a, (uint32_t)first);
    });
    return check_launch("moe_dispatch_fp8");
}

extern "C" int moe_scatter_scales(const float* token_scales, int64_t token_scale_row_stride,
                                  int32_t N, int32_t K, int32_t H, const int32_t* row_pair,
                                  int32_t E, int32_t M, void* scales, int32_t scale_format,
                                  hipStream_t stream) {
    if (N < 0 || K < 1 || H < 0 || E < 0 || M < 1)
        return fail(MOE_ERR_ARG, "moe_scatter_scales: need N >= 0, K >= 1, H >= 0, E >= 0, M >= 1");
    if (scale_format != MOE_SCALE_COLS && scale_format != MOE_SCALE_UE8M0)
        return fail(MOE_ERR_ARG, "moe_scatter_scales: scale_format must be MOE_SCALE_COLS or "
                    "MOE_SCALE_UE8M0, not %d", scale_format);
    if (H % kBlock != 0)
        return fail(MOE_ERR_ALIGN, "moe_scatter_scales: H=%d must be a multiple of 128", H);
    if (scale_format == MOE_SCALE_UE8M0 && H % (4 * kBlock) != 0)
        return fail(MOE_ERR_ARG, "moe_scatter_scales: ue8m0 scales need H %% 512 == 0");
    if (token_scale_row_stride < H / kBlock)
        return fail(MOE_ERR_ARG, "moe_scatter_scales: token_scale_row_stride < H/128");
    if ((int64_t)N * K >= ((int64_t)1 << 31) || (int64_t)E * M >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_scatter_scales: N*K and E*M must be below 2^31");
    if (N == 0 || E == 0 || H == 0) return ok();   // N = 0: no row_pair entry is valid
    if (token_scales == nullptr || row_pair == nullptr || scales == nullptr)
        return fail(MOE_ERR_ARG, "moe_scatter_scales: NULL pointer");
    if (!aligned(token_scales, 4) || !aligned(row_pair, 4) || !aligned(scales, 4))
        return fail(MOE_ERR_ALIGN, "moe_scatter_scales: pointers must be 4-byte aligned");

    ScatterArgs a;
    a.ts = token_scales;
    a.tss = token_scale_row_stride;
    a.row_pair = row_pair;
    a.NK = N * K;
    a.K = K;
    a.E = E;
    a.M = M;
    a.chunks = ceil_div<int32_t>(M, kWave);
    a.nb = H / kBlock;
    a.out = scales;
    a.mode = scale_format;
    const int64_t waves = (int64_t)E * a.chunks;
    const int64_t blocks = ceil_div<int64_t>(waves, kScatterThreads / kWave);
    const bool vec = aligned(token_scales, 16) && token_scale_row_stride % 4 == 0 && a.nb % 4 == 0;
    clear_launch_error();
    if (vec)
        scatter_scales_kernel<true><<<(uint32_t)blocks, kScatterThreads, 0, stream>>>(a);
    else
        scatter_scales_kernel<false><<<(uint32_t)blocks, kScatterThreads, 0, stream>>>(a);
    return check_launch("moe_scatter_scales");
}
