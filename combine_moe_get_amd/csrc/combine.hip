// combine.hip -- top-k weighted gather-reduce of the expert outputs back to
// token order.
//
// Definition: out[t,h] = bf16_rne( fp32 chain over k ascending of
// fmaf(w[t,k], y[pos[t,k], h], acc) ), starting at +0 and skipping masked
// pairs. fp32 accumulation in a fixed order with one bf16 rounding at the end
// follows the reduction of the vLLM branch compare ds-exp-2...ds-exp-ag
// (moe_reduce_scatter.cu, POLL + REDUCE phase); fp32 top-k weights scale the
// expert outputs as in DeepEP's low_latency_combine (repository dump,
// deep_ep.cpp). The sum is written straight into the caller's output (vLLM PR
// 49194, "Eliminate staging from NCCL symmetric reduce-scatter").
//
// Launch shape: one wave per (token, 64-vector segment of the output row).
// The token's K rows and weights are wave-uniform scalar loads. Each lane
// loads up to 8 expert rows before the first FMA; each load instruction of a
// wave reads 1 KiB contiguous of one expert row. Small batches issue the 8
// loads together, large ones one at a time (combine_kernel's PIPE). Large
// batches of 16-byte rows with K <= 8 take the held form instead
// (combine_held_kernel): one workgroup per compute unit at a time keeps its
// tokens' sums in registers and stores them after its last row load. No
// MFMA: nothing here is a contraction.
// The final rounding uses gfx950's v_cvt_pk_bf16_f32 (round to nearest
// even).
#include <algorithm>
#include <mutex>

#include "internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kXcds = 8;   // MI355X: 8 XCDs, workgroup i runs on XCD i % 8
constexpr int kBatch = 8;   // expert rows loaded before the FMAs that use them

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
    const f32x2 f = {lo, hi};
    const bf16x2 b = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// W words (2 bf16 each) per lane: W = 4 moves 16-byte vectors, W = 1 4-byte words.
template <int W>
struct Words {
    uint32_t w[W];
};

// One pair's expert row as a buffer descriptor: the row's bytes from its
// start, or an empty range for a masked pair (p < 0), whose loads then
// return 0 without touching memory. Every lane can thus load every pair of
// a batch unconditionally. That matters: with a load under a branch the
// compiler cannot count the loads in flight and waits for all of them
// before issuing the next, one memory round trip per pair.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint16_t* y, int64_t ys,
                                                          int32_t p, uint32_t row_bytes) {
    const uint16_t* row = y + (p < 0 ? 0 : (int64_t)p * ys);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(row), 0,
                                             __builtin_bit_cast(int32_t, p < 0 ? 0u : row_bytes),
                                             kBufferWord3);
}

// W words of a row at byte offset `off` (non-temporal: each expert-output
// element is read exactly once).
template <int W>
__device__ __forceinline__ Words<W> load_row_words(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Words<W> v;
    if constexpr (W == 4) {
        const u32x4 q = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int32_t)off, 0, kBufferNT));
        v.w[0] = q.x; v.w[1] = q.y; v.w[2] = q.z; v.w[3] = q.w;
    } else {
        v.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int32_t)off, 0, kBufferNT);
    }
    return v;
}

template <int W>
__device__ __forceinline__ Words<W> load_words(const uint16_t* p) {
    Words<W> r;
    // Each expert-output element is read exactly once: non-temporal loads
    // keep the stream from displacing other data in L2 and the last-level
    // cache.
    if constexpr (W == 4) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    return r;
}

// The combined rows are written once and not read back by this call:
// non-temporal stores (measured: the prefill combine 95 -> 88 us in the
// layout -> dispatch -> combine sequence, because ordinary stores leave dirty
// lines that the next kernels pay to write back).
template <int W>
__device__ __forceinline__ void store_words(uint16_t* p, const Words<W>& r) {
    if constexpr (W == 4) {
        const u32x4 v = {r.w[0], r.w[1], r.w[2], r.w[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    } else {
        __builtin_nontemporal_store(r.w[0], reinterpret_cast<uint32_t*>(p));
    }
}

// Sums of K-wide fp32 rows over a token's pairs (the dispatch backward's
// weight gradients): gin[pos[t,k], j] summed over valid k ascending into
// gout[t, j], one lane per j.
struct RowSums {
    const float* gin;
    int64_t gins;
    float* gout;
    int64_t gouts;
};

// UNIT: every weight is 1 (the dispatch backward): acc + y, which is what
// fmaf(1, y, acc) computes, without loading weights.
// PIPE: how a lane's K row loads are issued. With PIPE every pair of a batch
// is loaded unconditionally through row_rsrc, so all of them are in flight
// together; without it each load sits under a branch on its pair's mask,
// and the compiler issues the 16-byte ones one after another (each waits
// for the ones before). Small batches are latency-bound and take the first form (the
// decode combine: 7.4 -> 5.8 us); at large ones the second measured faster
// (the prefill combine: 88.2-88.6 us, against 90.1-91.0 us with 2, 4 or 8
// loads in flight per lane).
template <int W, bool UNIT, bool PIPE>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const uint16_t* __restrict__ y, int64_t ys, const float* __restrict__ w, int64_t wst,
    const int32_t* __restrict__ pos, int32_t N, int32_t K, int32_t V, int32_t segs,
    uint16_t* __restrict__ out, int64_t os, const RowSums rs, int64_t first_block) {
    constexpr int E = 2 * W;   // bf16 elements per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (first_block + blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave;
    const int32_t t = __builtin_amdgcn_readfirstlane((int32_t)(gw / segs));
    if (t >= N) return;
    const int32_t seg = (int32_t)(gw - (int64_t)t * segs);
    const int32_t* prow = pos + (int64_t)t * K;
    if (UNIT && rs.gout != nullptr && seg == 0 && lane < K) {
        float a = 0.0f;
        for (int32_t k = 0; k < K; ++k) {
            const int32_t p = prow[k];
            if (p >= 0) a = a + rs.gin[(int64_t)p * rs.gins + lane];
        }
        rs.gout[(int64_t)t * rs.gouts + lane] = a;
    }
    const int32_t v = seg * kWave + lane;
    if (v >= V) return;

    const float* wrow = UNIT ? nullptr : w + (int64_t)t * wst;
    const int64_t col = (int64_t)v * E;

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;

    const uint32_t row_bytes = 4u * W * (uint32_t)V;
    const uint32_t off = (uint32_t)col * 2;
    for (int k0 = 0; k0 < K; k0 += kBatch) {
        int32_t p[kBatch];
        float wk[kBatch];
        Words<W> val[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int k = k0 + j;
            p[j] = k < K ? prow[k] : -1;
            wk[j] = UNIT ? 1.0f : (k < K ? wrow[k] : 0.0f);
            if constexpr (PIPE)
                val[j] = load_row_words<W>(row_rsrc(y, ys, p[j], row_bytes), off);
            else if (p[j] >= 0)
                val[j] = load_words<W>(y + (int64_t)p[j] * ys + col);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (p[j] < 0) continue;
#pragma unroll
            for (int q = 0; q < W; ++q) {
                if (UNIT) {
                    acc[2 * q] = acc[2 * q] + lo_bf16(val[j].w[q]);
                    acc[2 * q + 1] = acc[2 * q + 1] + hi_bf16(val[j].w[q]);
                } else {
                    acc[2 * q] = __builtin_fmaf(wk[j], lo_bf16(val[j].w[q]), acc[2 * q]);
                    acc[2 * q + 1] = __builtin_fmaf(wk[j], hi_bf16(val[j].w[q]), acc[2 * q + 1]);
                }
            }
        }
    }

    Words<W> r;
#pragma unroll
    for (int q = 0; q < W; ++q) r.w[q] = pack_bf16_rne(acc[2 * q], acc[2 * q + 1]);
    store_words<W>(out + (int64_t)t * os + col, r);
}


// ---------------------------------------------------------------------------
// The held form of the combine (and, with UNIT, of the dispatch backward),
// for large batches of 16-byte rows with K <= 8 and 8 to 224 segments per
// row.
//
// combine_kernel stores each output vector as soon as it is summed, so its
// writes stream out interleaved with the expert-row reads all through the
// launch. Here each workgroup takes T consecutive tokens (one workgroup per
// compute unit at a time: its registers allow no second one) and keeps all
// of their summed vectors in registers until its last row load has been
// issued and used, then stores them together. The reads of a round of
// workgroups then run without writes between them. The sums are the same
// fp32 chains in k order with one rounding, so the output is bit-identical
// to combine_kernel's. Measured at 4096 tokens of 7168 channels: 85.3-86.5
// us against 88.7-89.0 us.
//
// Each wave holds up to kHeldUnits vectors (4 registers each); units are
// (token, 64-vector segment) pairs, numbered token-major over the
// workgroup's tokens, unit u on wave u % 8. Two units' 16 row loads are in
// flight together. The token's pairs are staged in LDS, padded to 8 (row
// -1, weight 0 past K), so no load waits behind a scalar fetch. With UNIT
// (every weight 1: adds, as combine_kernel's unit form) the wave of each
// token's first segment also sums the token's K weight-gradient rows, lane
// j taking entry j.
// ---------------------------------------------------------------------------
constexpr int kHeldThreads = 512;
constexpr int kHeldWaves = kHeldThreads / kWave;
constexpr int kHeldUnits = 28;        // output vectors held per lane
constexpr int kHeldGroup = 2;         // units whose row loads are in flight together
constexpr int kHeldMaxTokens = 64;    // tokens a workgroup stages (8 pairs each)

template <bool UNIT>
__global__ __launch_bounds__(kHeldThreads) void combine_held_kernel(
    const uint16_t* __restrict__ y, int64_t ys, const float* __restrict__ w, int64_t wst,
    const int32_t* __restrict__ pos, int32_t N, int32_t K, int32_t V, int32_t segs, int32_t T,
    uint16_t* __restrict__ out, int64_t os, const RowSums rs) {
    __shared__ int32_t srow[kHeldMaxTokens * kBatch];
    __shared__ float sw[kHeldMaxTokens * kBatch];
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x / kWave));
    const int64_t t0 = (int64_t)blockIdx.x * T;
    const int32_t nt = (int32_t)min((int64_t)T, (int64_t)N - t0);
    for (int32_t j = threadIdx.x; j < nt * kBatch; j += kHeldThreads) {
        const int32_t tl = j / kBatch, k = j % kBatch;
        srow[j] = k < K ? pos[(t0 + tl) * K + k] : -1;
        sw[j] = UNIT ? 1.0f : (k < K ? w[(t0 + tl) * wst + k] : 0.0f);
    }
    __syncthreads();
    const int32_t units = nt * segs;
    const uint32_t row_bytes = 16u * (uint32_t)V;
    const bool sums = UNIT && rs.gout != nullptr;

    Words<4> held[kHeldUnits];
#pragma unroll
    for (int i0 = 0; i0 < kHeldUnits; i0 += kHeldGroup) {
        // wave-uniform; units past the last one (g > 0) repeat its loads and
        // are never stored
        if (wave + kHeldWaves * i0 < units) {
            Words<4> val[kHeldGroup][kBatch];
            float wk[kHeldGroup][kBatch];
            int32_t p[kHeldGroup][kBatch];
            float gsum[kHeldGroup][kBatch];   // the weight-gradient rows (UNIT, segment 0)
            int32_t seg0[kHeldGroup];
#pragma unroll
            for (int g = 0; g < kHeldGroup; ++g) {
                const int32_t u = min(wave + kHeldWaves * (i0 + g), units - 1);
                const int32_t tl = u / segs;
                const int32_t v = (u - tl * segs) * kWave + lane;
                seg0[g] = u == wave + kHeldWaves * (i0 + g) && u - tl * segs == 0 ? tl : -1;
                int32_t pr[kBatch];
                float wr[kBatch];
#pragma unroll
                for (int k = 0; k < kBatch; ++k) {
                    pr[k] = srow[tl * kBatch + k];
                    wr[k] = sw[tl * kBatch + k];
                }
#pragma unroll
                for (int k = 0; k < kBatch; ++k) {
                    p[g][k] = __builtin_amdgcn_readfirstlane(pr[k]);
                    wk[g][k] = __builtin_bit_cast(
                        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int32_t, wr[k])));
                    // lanes past the row (v >= V) read beyond the range: 0
                    val[g][k] = load_row_words<4>(row_rsrc(y, ys, p[g][k], row_bytes),
                                                  (uint32_t)v * 16u);
                }
                if (sums && seg0[g] >= 0) {
                    // lane j < K: entry j of each pair's weight-gradient row
                    // (lanes past K and masked pairs read 0 and touch nothing)
#pragma unroll
                    for (int k = 0; k < kBatch; ++k) {
                        const float* row = rs.gin + (p[g][k] < 0 ? 0 : (int64_t)p[g][k] * rs.gins);
                        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                            const_cast<float*>(row), 0,
                            __builtin_bit_cast(int32_t, p[g][k] < 0 ? 0u : 4u * (uint32_t)K),
                            kBufferWord3);
                        gsum[g][k] = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(r, lane * 4, 0, 0));
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < kHeldGroup; ++g) {
                float acc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
                for (int k = 0; k < kBatch; ++k) {
                    if (p[g][k] < 0) continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (UNIT) {
                            acc[2 * q] = acc[2 * q] + lo_bf16(val[g][k].w[q]);
                            acc[2 * q + 1] = acc[2 * q + 1] + hi_bf16(val[g][k].w[q]);
                        } else {
                            acc[2 * q] =
                                __builtin_fmaf(wk[g][k], lo_bf16(val[g][k].w[q]), acc[2 * q]);
                            acc[2 * q + 1] =
                                __builtin_fmaf(wk[g][k], hi_bf16(val[g][k].w[q]), acc[2 * q + 1]);
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    held[i0 + g].w[q] = pack_bf16_rne(acc[2 * q], acc[2 * q + 1]);
                if (sums && seg0[g] >= 0) {
                    // k ascending from +0, masked pairs skipped: combine_kernel's order
                    float a = 0.0f;
#pragma unroll
                    for (int k = 0; k < kBatch; ++k)
                        if (p[g][k] >= 0) a = a + gsum[g][k];
                    if (lane < K) rs.gout[(t0 + seg0[g]) * rs.gouts + lane] = a;
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kHeldUnits; ++i) {
        const int32_t u = wave + kHeldWaves * i;
        if (u < units) {
            const int32_t tl = u / segs;
            const int32_t v = (u - tl * segs) * kWave + lane;
            if (v < V) store_words<4>(out + (t0 + tl) * os + (int64_t)v * 8, held[i]);
        }
    }
}

// Whether combine_held_kernel keeps everything in registers (no scratch
// memory) on this build; checked once. If it ever spilled, the plain form is
// used throughout.
template <bool UNIT>
bool held_kernel_ok() {
    static std::once_flag once;
    static bool ok = false;
    std::call_once(once, [] {
        hipFuncAttributes attr{};
        ok = hipFuncGetAttributes(&attr,
                                  reinterpret_cast<const void*>(&combine_held_kernel<UNIT>)) ==
                 hipSuccess &&
             attr.localSizeBytes == 0 && attr.maxThreadsPerBlock >= kHeldThreads;
        (void)hipGetLastError();
    });
    return ok;
}

// Compute units of the device that runs `stream` (0 if unknown), looked up
// once per device.
int stream_cus(hipStream_t stream) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int cus[kMaxDevices];
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 0;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 0;
        (void)hipGetLastError();
        cus[dev] = n > 0 ? n : -1;
    }
    return cus[dev] > 0 ? cus[dev] : 0;
}

// Tokens per workgroup of the held form for N tokens of `segs` segments on
// `cus` compute units, or 0 where the form does not apply. A workgroup holds
// at most 8 * kHeldUnits units; T is the smallest count that covers the
// batch in the fewest rounds of `cus` workgroups, so the last round is
// nearly full.
int32_t held_tokens(int64_t N, int32_t segs, int cus) {
    if (cus <= 0 || segs < 8 || segs > kHeldWaves * kHeldUnits) return 0;
    const int64_t tmax = std::min<int64_t>(kHeldWaves * kHeldUnits / segs, kHeldMaxTokens);
    const int64_t rounds = ceil_div<int64_t>(N, (int64_t)cus * tmax);
    const int64_t T = ceil_div<int64_t>(N, (int64_t)cus * rounds);
    if (ceil_div<int64_t>(N, T) > kMaxLaunchItems / kHeldThreads) return 0;   // one launch
    return (int32_t)T;
}

// A token's K pairs (K <= MOE_MAX_TOPK) for the one-workgroup-per-token
// kernels, staged in LDS: threads k < K load pair k's row and weight, and
// after one barrier every wave reads them from LDS. Loading them per wave as
// scalars waits once per pair before the pair's row can be fetched. Must be
// called by every thread of the workgroup (it holds a barrier).
struct TokenPairs {
    int32_t row[MOE_MAX_TOPK];
    float w[MOE_MAX_TOPK];
};

__device__ __forceinline__ void stage_token_pairs(TokenPairs& tp, const int32_t* prow,
                                                  const float* wrow, int32_t K) {
    if ((int32_t)threadIdx.x < K) {
        tp.row[threadIdx.x] = prow[threadIdx.x];
        tp.w[threadIdx.x] = wrow[threadIdx.x];
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Combine with an epilogue (biases; residual add + RMSNorm).
//
// One workgroup per token: its fp32 values stay in registers (VPT 16-byte
// vectors per lane) from the top-k sum through the workgroup-wide sum of
// squares to the normalised output, so the epilogue costs no extra pass over
// memory: the token's K expert rows, biases and residual are read once and
// residual_out and out written once.
// ---------------------------------------------------------------------------

struct EpilogueArgs {
    const uint16_t* y;
    int64_t ys;
    const float* w;
    int64_t wst;
    const int32_t* pos;
    int32_t N, K, V;   // V = Hc / 8
    float hc;          // Hc as a float (the mean's divisor)
    const uint16_t* b0;
    int64_t b0s;
    const uint16_t* b1;
    int64_t b1s;
    const uint16_t* res;
    int64_t rs;
    const uint16_t* gamma;
    float eps;
    uint16_t* res_out;
    int64_t ros;
    uint16_t* out;
    int64_t os;
};

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const uint16_t* p) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = acc[2 * i] + lo_bf16(q[i]);
        acc[2 * i + 1] = acc[2 * i + 1] + hi_bf16(q[i]);
    }
}

// Output rows are written once per call and not read back by it:
// non-temporal stores keep them from lingering as dirty cache lines that the
// next kernels would have to write back (measured on the prefill step: the
// epilogue step went from 243 to 172 us).
__device__ __forceinline__ void store_bf16x8(uint16_t* p, const float (&v)[8]) {
    const u32x4 r = {pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3]),
                     pack_bf16_rne(v[4], v[5]), pack_bf16_rne(v[6], v[7])};
    __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p));
}

constexpr int kEpiThreads = 1024;
constexpr int kEpiWaves = kEpiThreads / kWave;

template <int VPT>
__global__ __launch_bounds__(kEpiThreads) void combine_epilogue_kernel(const EpilogueArgs a,
                                                                        int32_t first_token) {
    __shared__ float wave_ss[kEpiWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int32_t t = first_token + (int32_t)blockIdx.x;
    __shared__ TokenPairs tp;
    stage_token_pairs(tp, a.pos + (int64_t)t * a.K, a.w + (int64_t)t * a.wst, a.K);

    float acc[VPT][8];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int32_t v = threadIdx.x + j * kEpiThreads;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
        if (v >= a.V) continue;
        const int64_t col = (int64_t)v * 8;
        for (int k0 = 0; k0 < a.K; k0 += kBatch) {
            int32_t p[kBatch];
            float wk[kBatch];
            Words<4> val[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const int k = k0 + i;
                p[i] = k < a.K ? tp.row[k] : -1;
                wk[i] = k < a.K ? tp.w[k] : 0.0f;
                val[i] = load_row_words<4>(row_rsrc(a.y, a.ys, p[i], (uint32_t)a.V * 16),
                                           (uint32_t)col * 2);
            }
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                if (p[i] < 0) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[j][2 * q] = __builtin_fmaf(wk[i], lo_bf16(val[i].w[q]), acc[j][2 * q]);
                    acc[j][2 * q + 1] = __builtin_fmaf(wk[i], hi_bf16(val[i].w[q]), acc[j][2 * q + 1]);
                }
            }
        }
        if (a.b0) add_bf16x8(acc[j], a.b0 + (int64_t)t * a.b0s + col);
        if (a.b1) add_bf16x8(acc[j], a.b1 + (int64_t)t * a.b1s + col);
        if (a.res) add_bf16x8(acc[j], a.res + (int64_t)t * a.rs + col);
    }

    if (a.res == nullptr) {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int32_t v = threadIdx.x + j * kEpiThreads;
            if (v < a.V) store_bf16x8(a.out + (int64_t)t * a.os + (int64_t)v * 8, acc[j]);
        }
        return;
    }

    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int32_t v = threadIdx.x + j * kEpiThreads;
        if (v >= a.V) continue;
        store_bf16x8(a.res_out + (int64_t)t * a.ros + (int64_t)v * 8, acc[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(acc[j][e], acc[j][e], ss);
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if (lane == 0) wave_ss[wave] = ss;
    __syncthreads();
    float total = 0.0f;
#pragma unroll
    for (int i = 0; i < kEpiWaves; ++i) total += wave_ss[i];
    const float s = rsqrtf(total / a.hc + a.eps);

#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int32_t v = threadIdx.x + j * kEpiThreads;
        if (v >= a.V) continue;
        const int64_t col = (int64_t)v * 8;
        const u32x4 g = *reinterpret_cast<const u32x4*>(a.gamma + col);
        const uint32_t gq[4] = {g.x, g.y, g.z, g.w};
        float o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[2 * q] = (acc[j][2 * q] * s) * lo_bf16(gq[q]);
            o[2 * q + 1] = (acc[j][2 * q + 1] * s) * hi_bf16(gq[q]);
        }
        store_bf16x8(a.out + (int64_t)t * a.os + col, o);
    }
}

// ---------------------------------------------------------------------------
// Combine backward: the dual of the combine is a dispatch of the output
// gradient, scaled by each pair's weight, plus the weights' gradients
//   grad_y[pos[t,k], h] = bf16_rne(w[t,k] * grad_out[t,h])       (fp32 product)
//   grad_w[t,k]         = sum_h grad_out[t,h] * y[pos[t,k], h]   (fp32)
// (DeepEP repository dump, README, "Example use in model training": the
// backward of the combine is a dispatch). One workgroup per (token, k) pair:
// each lane loads its channels of the token's gradient row and of the
// pair's expert row, stores the scaled row and keeps one fp32 FMA chain over
// its channels; the 64 lanes of a wave are summed by a fixed butterfly and
// the waves in index order, so the result does not depend on scheduling.
// Workgroups are renumbered so that XCD x (workgroup i runs on XCD i mod 8)
// takes a contiguous eighth of the pairs: a token's K pairs then run on one
// XCD and read its gradient row from that L2. Measured at prefill against
// one workgroup per token looping over the token's pairs (same outputs bit
// for bit): 189.5 against 198.5 us.
// ---------------------------------------------------------------------------

struct BackwardArgs {
    const uint16_t* g;   // grad_out [N, Hc]
    int64_t gs;
    const float* w;
    int64_t wst;
    const uint16_t* y;   // NULL: no weight gradients
    int64_t ys;
    const int32_t* pos;
    int32_t N, K, V;     // V = Hc / 8
    uint32_t first;      // the launch piece's first pair (beside N, K, V: one load fetches all four)
    uint16_t* gy;
    int64_t gys;
    float* gw;
    int64_t gws;
};

// Lane tid of a workgroup of blockDim threads takes vectors tid + j*blockDim
// (j < VPT) of the row. blockDim is 1024 when the row has more than 1024
// vectors, else the row's vectors rounded up to whole waves. WANT_W: the
// weight gradients are wanted (y is read and the dot products formed).
template <int VPT, bool WANT_W>
__global__ __launch_bounds__(kEpiThreads) void combine_backward_kernel(const BackwardArgs a) {
    __shared__ float part[kEpiWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // Logical workgroup: XCD (blockIdx % 8) takes a contiguous eighth of this
    // piece. The grid is a multiple of 8, so this is a bijection. 32-bit
    // index arithmetic (N*K < 2^31): a 64-bit division would be a long
    // software routine in every workgroup.
    const uint32_t per_xcd = gridDim.x / kXcds;
    const uint32_t pair = a.first + (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const bool live = pair < (uint32_t)a.N * (uint32_t)a.K;   // else the grid's padding
    const int32_t p = live ? a.pos[pair] : -1;
    const uint32_t tu = pair / (uint32_t)a.K;
    const int32_t k = (int32_t)(pair - tu * (uint32_t)a.K);
    const int64_t t = tu;
    float d = 0.0f;
    // No early return: one condition around each lane's work keeps the
    // kernel-argument fetches in few rounds (the workgroup's life is a short
    // chain of dependent loads, and every extra round lengthens it). A
    // masked pair stores nothing and gets a zero weight gradient below.
    if constexpr (VPT == 1) {
        const int32_t v = threadIdx.x;
        if (p >= 0 && v < a.V) {
            const float wk = a.w[t * a.wst + k];
            const int64_t col = (int64_t)v * 8;
            // the gradient row with ordinary loads: the token's other K-1
            // pairs read it again from L2
            const u32x4 gq = *reinterpret_cast<const u32x4*>(a.g + t * a.gs + col);
            const uint32_t g[4] = {gq.x, gq.y, gq.z, gq.w};
            Words<4> yv;
            if (WANT_W) yv = load_words<4>(a.y + (int64_t)p * a.ys + col);
            float o[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o[2 * q] = wk * lo_bf16(g[q]);
                o[2 * q + 1] = wk * hi_bf16(g[q]);
            }
            store_bf16x8(a.gy + (int64_t)p * a.gys + col, o);
            if (WANT_W) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    d = __builtin_fmaf(lo_bf16(g[q]), lo_bf16(yv.w[q]), d);
                    d = __builtin_fmaf(hi_bf16(g[q]), hi_bf16(yv.w[q]), d);
                }
            }
        }
    } else if (p >= 0 && a.V > 0) {
        const float wk = a.w[t * a.wst + k];
        // Every lane issues all its loads first (vectors past the row clamped
        // to its last one, then neither stored nor summed): a load under a
        // per-lane branch would wait for the ones before it.
        Words<4> g[VPT], yv[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int64_t col = (int64_t)min((int32_t)threadIdx.x + j * (int32_t)blockDim.x,
                                             a.V - 1) * 8;
            const u32x4 gq = *reinterpret_cast<const u32x4*>(a.g + t * a.gs + col);
            g[j] = Words<4>{{gq.x, gq.y, gq.z, gq.w}};
            if (WANT_W) yv[j] = load_words<4>(a.y + (int64_t)p * a.ys + col);
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int32_t v = threadIdx.x + j * (int32_t)blockDim.x;
            if (v >= a.V) continue;
            float o[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o[2 * q] = wk * lo_bf16(g[j].w[q]);
                o[2 * q + 1] = wk * hi_bf16(g[j].w[q]);
            }
            store_bf16x8(a.gy + (int64_t)p * a.gys + (int64_t)v * 8, o);
            if (WANT_W) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    d = __builtin_fmaf(lo_bf16(g[j].w[q]), lo_bf16(yv[j].w[q]), d);
                    d = __builtin_fmaf(hi_bf16(g[j].w[q]), hi_bf16(yv[j].w[q]), d);
                }
            }
        }
    }
    if (!WANT_W) return;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) d += __shfl_xor(d, off, kWave);
    if (lane == 0) part[wave] = d;
    __syncthreads();
    if (live && threadIdx.x == 0) {
        float sum = 0.0f;
        for (int wv = 0; wv < (int)(blockDim.x / kWave); ++wv) sum += part[wv];
        a.gw[t * a.gws + k] = p >= 0 ? sum : 0.0f;
    }
}

// Pairs per workgroup of the grouped combine backward.
constexpr int kBwdGroup = 4;

// The combine backward for rows of at most 1024 vectors and K a multiple of
// kBwdGroup: workgroup j takes kBwdGroup consecutive pairs of one token.
// Each lane loads its vector of the token's gradient row once and the
// pairs' expert rows together; per pair the lane's FMA chain, the butterfly
// and the wave order of the sum are those of combine_backward_kernel<1>,
// so the results are the same bit for bit. (Measured at the prefill shape:
// 190.0-190.5 against 193.8-194.2 us for one pair per workgroup; eight
// pairs took 192.9 us.)
template <bool WANT_W>
__global__ __launch_bounds__(kEpiThreads) void combine_backward_group_kernel(const BackwardArgs a) {
    __shared__ float part[kBwdGroup][kEpiWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // XCD (blockIdx % 8) takes a contiguous eighth of this piece's groups.
    const uint32_t per_xcd = gridDim.x / kXcds;
    const uint32_t grp = a.first + (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const uint32_t pair0 = grp * kBwdGroup;
    const bool live = pair0 < (uint32_t)a.N * (uint32_t)a.K;   // else the grid's padding
    int32_t p[kBwdGroup];
#pragma unroll
    for (int i = 0; i < kBwdGroup; ++i) p[i] = live ? a.pos[pair0 + i] : -1;
    const uint32_t tu = pair0 / (uint32_t)a.K;
    const int32_t k0 = (int32_t)(pair0 - tu * (uint32_t)a.K);
    const int64_t t = tu;
    float d[kBwdGroup];
#pragma unroll
    for (int i = 0; i < kBwdGroup; ++i) d[i] = 0.0f;
    const int32_t v = threadIdx.x;
    if (live && v < a.V) {
        const int64_t col = (int64_t)v * 8;
        const u32x4 gq = *reinterpret_cast<const u32x4*>(a.g + t * a.gs + col);
        const uint32_t g[4] = {gq.x, gq.y, gq.z, gq.w};
        Words<4> yv[kBwdGroup];
        float wk[kBwdGroup];
        // every pair's loads are issued before the first store; a masked
        // pair reads row 0 and neither stores nor sums it
#pragma unroll
        for (int i = 0; i < kBwdGroup; ++i) {
            wk[i] = a.w[t * a.wst + k0 + i];
            if (WANT_W) yv[i] = load_words<4>(a.y + (int64_t)max(p[i], 0) * a.ys + col);
        }
#pragma unroll
        for (int i = 0; i < kBwdGroup; ++i) {
            if (p[i] < 0) continue;
            float o[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o[2 * q] = wk[i] * lo_bf16(g[q]);
                o[2 * q + 1] = wk[i] * hi_bf16(g[q]);
            }
            store_bf16x8(a.gy + (int64_t)p[i] * a.gys + col, o);
            if (WANT_W) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    d[i] = __builtin_fmaf(lo_bf16(g[q]), lo_bf16(yv[i].w[q]), d[i]);
                    d[i] = __builtin_fmaf(hi_bf16(g[q]), hi_bf16(yv[i].w[q]), d[i]);
                }
            }
        }
    }
    if (!WANT_W) return;
#pragma unroll
    for (int i = 0; i < kBwdGroup; ++i) {
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) d[i] += __shfl_xor(d[i], off, kWave);
        if (lane == 0) part[i][wave] = d[i];
    }
    __syncthreads();
    if (live && threadIdx.x < kBwdGroup) {
        const int i = threadIdx.x;
        float sum = 0.0f;
        for (int wv = 0; wv < (int)(blockDim.x / kWave); ++wv) sum += part[i][wv];
        a.gw[t * a.gws + k0 + i] = p[i] >= 0 ? sum : 0.0f;
    }
}

// Launches one piece of combine_kernel<W, UNIT, PIPE>.
template <int W, bool UNIT>
void launch_combine_piece(bool pipe, int64_t first, int64_t count, hipStream_t stream,
                          const uint16_t* y, int64_t ys, const float* w, int64_t wst,
                          const int32_t* pos, int32_t N, int32_t K, int32_t V, int32_t segs,
                          uint16_t* out, int64_t os, const RowSums& rs) {
    if (pipe)
        combine_kernel<W, UNIT, true><<<(uint32_t)count, kThreads, 0, stream>>>(
            y, ys, w, wst, pos, N, K, V, segs, out, os, rs, first);
    else
        combine_kernel<W, UNIT, false><<<(uint32_t)count, kThreads, 0, stream>>>(
            y, ys, w, wst, pos, N, K, V, segs, out, os, rs, first);
}

// Jobs of at most this many waves (one per token and 64-vector segment)
// issue all K row loads of a lane together (PIPE); larger ones one by one.
// The two measured alike at 1024-2048 tokens of 7168 channels (14336-28672
// waves).
constexpr int64_t kPipeMaxWaves = 32768;

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_combine(const void* y, int64_t y_row_stride, const float* w,
                           int64_t w_row_stride, const int32_t* pos, int32_t N, int32_t K,
                           int32_t Hc, void* out, int64_t out_row_stride, hipStream_t stream) {
    if (N < 0 || K < 1 || Hc < 0)
        return fail(MOE_ERR_ARG, "moe_combine: need N >= 0, K >= 1, Hc >= 0");
    if (K > MOE_MAX_TOPK) return fail(MOE_ERR_LIMIT, "moe_combine: K=%d > %d", K, MOE_MAX_TOPK);
    if ((int64_t)N * K >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_combine: N*K must be below 2^31");
    if (N == 0 || Hc == 0) return ok();
    if (y == nullptr || w == nullptr || pos == nullptr || out == nullptr)
        return fail(MOE_ERR_ARG, "moe_combine: NULL pointer");
    if (w_row_stride < K) return fail(MOE_ERR_ARG, "moe_combine: w_row_stride < K");
    if (out_row_stride < Hc || y_row_stride < Hc)
        return fail(MOE_ERR_ARG, "moe_combine: y and out row strides must be >= Hc");
    if ((Hc & 1) || !aligned(y, 4) || !aligned(out, 4) || (y_row_stride & 1) ||
        (out_row_stride & 1) || !aligned(w, 4) || !aligned(pos, 4))
        return fail(MOE_ERR_ALIGN, "moe_combine: Hc and the bf16 strides must be even; y, out, "
                    "w and pos 4-byte aligned");
    const bool vec16 = (Hc % 8 == 0) && aligned(y, 16) && aligned(out, 16) &&
                       (y_row_stride % 8 == 0) && (out_row_stride % 8 == 0);
    const int32_t per_lane = vec16 ? 8 : 2;
    const int32_t V = Hc / per_lane;
    const int32_t segs = ceil_div<int32_t>(V, kWave);
    const int64_t blocks = ceil_div<int64_t>((int64_t)N * segs, kWavesPerBlock);
    if (blocks >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_combine: launch of %lld workgroups too large",
                    (long long)blocks);
    const auto* yy = static_cast<const uint16_t*>(y);
    auto* oo = static_cast<uint16_t*>(out);
    const RowSums none = {nullptr, 0, nullptr, 0};
    clear_launch_error();
    const bool pipe = (int64_t)N * segs <= kPipeMaxWaves;
    // Large batches of 16-byte rows with K <= 8 take the held form.
    const int32_t T = !pipe && vec16 && K <= kBatch && held_kernel_ok<false>()
                          ? held_tokens(N, segs, stream_cus(stream))
                          : 0;
    if (T > 0) {
        combine_held_kernel<false><<<(uint32_t)ceil_div<int64_t>(N, T), kHeldThreads, 0, stream>>>(
            yy, y_row_stride, w, w_row_stride, pos, N, K, V, segs, T, oo, out_row_stride, none);
        return check_launch("moe_combine");
    }
    in_pieces(blocks, kMaxLaunchItems / kThreads, [&](int64_t first, int64_t count) {
        if (vec16)
            launch_combine_piece<4, false>(pipe, first, count, stream, yy, y_row_stride, w,
                                           w_row_stride, pos, N, K, V, segs, oo, out_row_stride,
                                           none);
        else
            launch_combine_piece<1, false>(pipe, first, count, stream, yy, y_row_stride, w,
                                           w_row_stride, pos, N, K, V, segs, oo, out_row_stride,
                                           none);
    });
    return check_launch("moe_combine");
}

extern "C" int moe_dispatch_backward(const void* grad_recv, int64_t grad_recv_row_stride,
                                     const float* grad_recv_w, int64_t grad_recv_w_row_stride,
                                     const int32_t* pos, int32_t N, int32_t K, int32_t H,
                                     void* grad_x, int64_t grad_x_row_stride, float* grad_w,
                                     int64_t grad_w_row_stride, hipStream_t stream) {
    if (N < 0 || K < 1 || H < 0)
        return fail(MOE_ERR_ARG, "moe_dispatch_backward: need N >= 0, K >= 1, H >= 0");
    if (K > MOE_MAX_TOPK)
        return fail(MOE_ERR_LIMIT, "moe_dispatch_backward: K=%d > %d", K, MOE_MAX_TOPK);
    if ((int64_t)N * K >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_dispatch_backward: N*K must be below 2^31");
    if ((grad_recv_w == nullptr) != (grad_w == nullptr))
        return fail(MOE_ERR_ARG, "moe_dispatch_backward: grad_recv_w and grad_w go together");
    if (N == 0 || (H == 0 && grad_w == nullptr)) return ok();
    if (pos == nullptr || (H > 0 && (grad_recv == nullptr || grad_x == nullptr)))
        return fail(MOE_ERR_ARG, "moe_dispatch_backward: NULL pointer");
    if (grad_w != nullptr && (grad_recv_w_row_stride < K || grad_w_row_stride < K))
        return fail(MOE_ERR_ARG, "moe_dispatch_backward: weight-gradient row strides must be >= K");
    if (H > 0 && (grad_recv_row_stride < H || grad_x_row_stride < H))
        return fail(MOE_ERR_ARG, "moe_dispatch_backward: row strides must be >= H");
    if ((H & 1) || (H > 0 && (!aligned(grad_recv, 4) || !aligned(grad_x, 4))) ||
        (grad_recv_row_stride & 1) || (grad_x_row_stride & 1) || !aligned(pos, 4) ||
        !aligned(grad_recv_w, 4) || !aligned(grad_w, 4))
        return fail(MOE_ERR_ALIGN, "moe_dispatch_backward: H and the bf16 strides must be even; "
                    "all pointers 4-byte aligned");
    const bool vec16 = (H % 8 == 0) && aligned(grad_recv, 16) && aligned(grad_x, 16) &&
                       (grad_recv_row_stride % 8 == 0) && (grad_x_row_stride % 8 == 0);
    const int32_t V = H / (vec16 ? 8 : 2);
    const int32_t segs = V > 0 ? ceil_div<int32_t>(V, kWave) : 1;   // H = 0: weights only
    const int64_t blocks = ceil_div<int64_t>((int64_t)N * segs, kWavesPerBlock);
    if (blocks >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_dispatch_backward: launch of %lld workgroups too large",
                    (long long)blocks);
    const auto* gr = static_cast<const uint16_t*>(grad_recv);
    auto* gx = static_cast<uint16_t*>(grad_x);
    const RowSums rs = {grad_recv_w, grad_recv_w_row_stride, grad_w, grad_w_row_stride};
    clear_launch_error();
    const bool pipe = (int64_t)N * segs <= kPipeMaxWaves;
    // Large batches of 16-byte rows with K <= 8 take the held form, with the
    // weight-gradient sums in the waves of each token's first segment.
    const int32_t T = H > 0 && !pipe && vec16 && K <= kBatch && held_kernel_ok<true>()
                          ? held_tokens(N, segs, stream_cus(stream))
                          : 0;
    if (T > 0) {
        combine_held_kernel<true><<<(uint32_t)ceil_div<int64_t>(N, T), kHeldThreads, 0, stream>>>(
            gr, grad_recv_row_stride, nullptr, 0, pos, N, K, V, segs, T, gx, grad_x_row_stride,
            rs);
        return check_launch("moe_dispatch_backward");
    }
    in_pieces(blocks, kMaxLaunchItems / kThreads, [&](int64_t first, int64_t count) {
        if (vec16)
            launch_combine_piece<4, true>(pipe, first, count, stream, gr, grad_recv_row_stride,
                                          nullptr, 0, pos, N, K, V, segs, gx, grad_x_row_stride,
                                          rs);
        else
            launch_combine_piece<1, true>(pipe, first, count, stream, gr, grad_recv_row_stride,
                                          nullptr, 0, pos, N, K, V, segs, gx, grad_x_row_stride,
                                          rs);
    });
    return check_launch("moe_dispatch_backward");
}


extern "C" int moe_combine_epilogue(const void* y, int64_t y_row_stride, const float* w,
                                    int64_t w_row_stride, const int32_t* pos, int32_t N, int32_t K,
                                    int32_t Hc, const moe_epilogue* ep, void* out,
                                    int64_t out_row_stride, hipStream_t stream) {
    if (ep == nullptr || (ep->bias0 == nullptr && ep->bias1 == nullptr && ep->residual == nullptr))
        return moe_combine(y, y_row_stride, w, w_row_stride, pos, N, K, Hc, out, out_row_stride,
                           stream);
    if (N < 0 || K < 1 || Hc < 0)
        return fail(MOE_ERR_ARG, "moe_combine_epilogue: need N >= 0, K >= 1, Hc >= 0");
    if (K > MOE_MAX_TOPK)
        return fail(MOE_ERR_LIMIT, "moe_combine_epilogue: K=%d > %d", K, MOE_MAX_TOPK);
    if ((int64_t)N * K >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_combine_epilogue: N*K must be below 2^31");
    if (ep->residual != nullptr && (ep->gamma == nullptr || ep->residual_out == nullptr))
        return fail(MOE_ERR_ARG, "moe_combine_epilogue: a residual needs gamma and residual_out");
    if (ep->residual != nullptr && !(ep->eps >= 0.0f && ep->eps < INFINITY))
        return fail(MOE_ERR_ARG, "moe_combine_epilogue: eps must be finite and >= 0");
    if (Hc > kEpiThreads * 8 * 8)
        return fail(MOE_ERR_LIMIT, "moe_combine_epilogue: Hc=%d > %d", Hc, kEpiThreads * 8 * 8);
    if (N == 0 || Hc == 0) return ok();
    if (y == nullptr || w == nullptr || pos == nullptr || out == nullptr)
        return fail(MOE_ERR_ARG, "moe_combine_epilogue: NULL pointer");
    if (w_row_stride < K) return fail(MOE_ERR_ARG, "moe_combine_epilogue: w_row_stride < K");
    struct Row { const void* p; int64_t stride; const char* name; };
    const Row rows[] = {{y, y_row_stride, "y"}, {out, out_row_stride, "out"},
                        {ep->bias0, ep->bias0_row_stride, "bias0"},
                        {ep->bias1, ep->bias1_row_stride, "bias1"},
                        {ep->residual, ep->residual_row_stride, "residual"},
                        {ep->residual ? ep->residual_out : nullptr, ep->residual_out_row_stride,
                         "residual_out"}};
    if (Hc % 8 != 0 || !aligned(w, 4) || !aligned(pos, 4) ||
        (ep->residual && !aligned(ep->gamma, 16)))
        return fail(MOE_ERR_ALIGN, "moe_combine_epilogue: Hc must be a multiple of 8, gamma "
                    "16-byte aligned, w and pos 4-byte aligned");
    for (const Row& r : rows) {
        if (r.p == nullptr) continue;
        if (!aligned(r.p, 16) || r.stride % 8 != 0)
            return fail(MOE_ERR_ALIGN, "moe_combine_epilogue: %s must be 16-byte aligned with a "
                        "row stride that is a multiple of 8 elements", r.name);
        if (r.stride < Hc)
            return fail(MOE_ERR_ARG, "moe_combine_epilogue: %s row stride < Hc", r.name);
    }

    EpilogueArgs a;
    a.y = static_cast<const uint16_t*>(y);
    a.ys = y_row_stride;
    a.w = w;
    a.wst = w_row_stride;
    a.pos = pos;
    a.N = N;
    a.K = K;
    a.V = Hc / 8;
    a.hc = (float)Hc;
    a.b0 = static_cast<const uint16_t*>(ep->bias0);
    a.b0s = ep->bias0_row_stride;
    a.b1 = static_cast<const uint16_t*>(ep->bias1);
    a.b1s = ep->bias1_row_stride;
    a.res = static_cast<const uint16_t*>(ep->residual);
    a.rs = ep->residual_row_stride;
    a.gamma = static_cast<const uint16_t*>(ep->gamma);
    a.eps = ep->eps;
    a.res_out = static_cast<uint16_t*>(ep->residual ? ep->residual_out : nullptr);
    a.ros = ep->residual_out_row_stride;
    a.out = static_cast<uint16_t*>(out);
    a.os = out_row_stride;
    const int vpt = ceil_div<int32_t>(a.V, kEpiThreads);
    clear_launch_error();
    in_pieces(N, kMaxLaunchItems / kEpiThreads, [&](int64_t first, int64_t count) {
        const int32_t t0 = (int32_t)first;
        if (vpt <= 1)
            combine_epilogue_kernel<1><<<(uint32_t)count, kEpiThreads, 0, stream>>>(a, t0);
        else if (vpt <= 2)
            combine_epilogue_kernel<2><<<(uint32_t)count, kEpiThreads, 0, stream>>>(a, t0);
        else if (vpt <= 4)
            combine_epilogue_kernel<4><<<(uint32_t)count, kEpiThreads, 0, stream>>>(a, t0);
        else
            combine_epilogue_kernel<8><<<(uint32_t)count, kEpiThreads, 0, stream>>>(a, t0);
    });
    return check_launch("moe_combine_epilogue");
}

extern "C" int moe_combine_backward(const void* grad_out, int64_t grad_out_row_stride,
                                    const float* w, int64_t w_row_stride, const void* y,
                                    int64_t y_row_stride, const int32_t* pos, int32_t N,
                                    int32_t K, int32_t Hc, void* grad_y, int64_t grad_y_row_stride,
                                    float* grad_w, int64_t grad_w_row_stride,
                                    hipStream_t stream) {
    if (N < 0 || K < 1 || Hc < 0)
        return fail(MOE_ERR_ARG, "moe_combine_backward: need N >= 0, K >= 1, Hc >= 0");
    if (K > MOE_MAX_TOPK)
        return fail(MOE_ERR_LIMIT, "moe_combine_backward: K=%d > %d", K, MOE_MAX_TOPK);
    if ((int64_t)N * K >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_combine_backward: N*K must be below 2^31");
    // At most 4 vectors per lane: with 8 (Hc above 32768) the 1024-thread
    // workgroup's 128-register limit would spill.
    if (Hc > kEpiThreads * 8 * 4)
        return fail(MOE_ERR_LIMIT, "moe_combine_backward: Hc=%d > %d", Hc, kEpiThreads * 8 * 4);
    if (grad_w != nullptr && y == nullptr && Hc > 0)
        return fail(MOE_ERR_ARG, "moe_combine_backward: weight gradients need y");
    if (N == 0 || (Hc == 0 && grad_w == nullptr)) return ok();
    if (w == nullptr || pos == nullptr ||
        (Hc > 0 && (grad_out == nullptr || grad_y == nullptr || (grad_w && y == nullptr))))
        return fail(MOE_ERR_ARG, "moe_combine_backward: NULL pointer");
    if (w_row_stride < K || (grad_w != nullptr && grad_w_row_stride < K))
        return fail(MOE_ERR_ARG, "moe_combine_backward: w and grad_w row strides must be >= K");
    if (Hc % 8 != 0 || !aligned(w, 4) || !aligned(pos, 4) || !aligned(grad_w, 4))
        return fail(MOE_ERR_ALIGN, "moe_combine_backward: Hc must be a multiple of 8; w, pos and "
                    "grad_w 4-byte aligned");
    struct Row { const void* p; int64_t stride; const char* name; };
    const Row rows[] = {{grad_out, grad_out_row_stride, "grad_out"},
                        {grad_y, grad_y_row_stride, "grad_y"},
                        {grad_w ? y : nullptr, y_row_stride, "y"}};
    for (const Row& r : rows) {
        if (r.p == nullptr) continue;
        if (!aligned(r.p, 16) || r.stride % 8 != 0)
            return fail(MOE_ERR_ALIGN, "moe_combine_backward: %s must be 16-byte aligned with a "
                        "row stride that is a multiple of 8 elements", r.name);
        if (r.stride < Hc)
            return fail(MOE_ERR_ARG, "moe_combine_backward: %s row stride < Hc", r.name);
    }

    BackwardArgs a;
    a.g = static_cast<const uint16_t*>(grad_out);
    a.gs = grad_out_row_stride;
    a.w = w;
    a.wst = w_row_stride;
    a.y = grad_w ? static_cast<const uint16_t*>(y) : nullptr;
    a.ys = y_row_stride;
    a.pos = pos;
    a.N = N;
    a.K = K;
    a.V = Hc / 8;
    a.gy = static_cast<uint16_t*>(grad_y);
    a.gys = grad_y_row_stride;
    a.gw = grad_w;
    a.gws = grad_w_row_stride;
    const int vpt = ceil_div<int32_t>(a.V, kEpiThreads);
    const int threads = vpt > 1 ? kEpiThreads
                                : (int)std::max<int64_t>(kWave, ceil_div<int64_t>(a.V, kWave) * kWave);
    const int64_t pairs = (int64_t)N * K;
    const int64_t piece = kMaxLaunchItems / kEpiThreads / kXcds * kXcds;
    clear_launch_error();
    if (vpt <= 1 && K % kBwdGroup == 0) {
        const int64_t groups = ceil_div<int64_t>(pairs / kBwdGroup, kXcds) * kXcds;
        in_pieces(groups, piece, [&](int64_t first, int64_t count) {
            BackwardArgs b = a;
            b.first = (uint32_t)first;
            if (grad_w != nullptr)
                combine_backward_group_kernel<true><<<(uint32_t)count, threads, 0, stream>>>(b);
            else
                combine_backward_group_kernel<false><<<(uint32_t)count, threads, 0, stream>>>(b);
        });
        return check_launch("moe_combine_backward");
    }
    const int64_t blocks = ceil_div<int64_t>(pairs, kXcds) * kXcds;
    in_pieces(blocks, piece, [&](int64_t first, int64_t count) {
        BackwardArgs b = a;
        b.first = (uint32_t)first;
        const bool ww = grad_w != nullptr;
        if (vpt <= 1 && ww)
            combine_backward_kernel<1, true><<<(uint32_t)count, threads, 0, stream>>>(b);
        else if (vpt <= 1)
            combine_backward_kernel<1, false><<<(uint32_t)count, threads, 0, stream>>>(b);
        else if (vpt <= 2 && ww)
            combine_backward_kernel<2, true><<<(uint32_t)count, threads, 0, stream>>>(b);
        else if (vpt <= 2)
            combine_backward_kernel<2, false><<<(uint32_t)count, threads, 0, stream>>>(b);
        else if (ww)
            combine_backward_kernel<4, true><<<(uint32_t)count, threads, 0, stream>>>(b);
        else
            combine_backward_kernel<4, false><<<(uint32_t)count, threads, 0, stream>>>(b);
    });
    return check_launch("moe_combine_backward");
}
