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
// issues the loads of up to 8 expert rows before the first FMA, so every
// lane keeps 8 x 16 bytes in flight; each load instruction of a wave reads 1
// KiB contiguous of one expert row. No MFMA: nothing here is a contraction.
// The final rounding uses gfx950's v_cvt_pk_bf16_f32 (round to nearest
// even).
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
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

template <int W>
__device__ __forceinline__ void store_words(uint16_t* p, const Words<W>& r) {
    if constexpr (W == 4) {
        const u32x4 v = {r.w[0], r.w[1], r.w[2], r.w[3]};
        *reinterpret_cast<u32x4*>(p) = v;
    } else {
        *reinterpret_cast<uint32_t*>(p) = r.w[0];
    }
}

template <int W>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const uint16_t* __restrict__ y, int64_t ys, const float* __restrict__ w, int64_t wst,
    const int32_t* __restrict__ pos, int32_t N, int32_t K, int32_t V, int32_t segs,
    uint16_t* __restrict__ out, int64_t os) {
    constexpr int E = 2 * W;   // bf16 elements per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int32_t t = __builtin_amdgcn_readfirstlane((int32_t)(gw / segs));
    if (t >= N) return;
    const int32_t seg = (int32_t)(gw - (int64_t)t * segs);
    const int32_t v = seg * kWave + lane;
    if (v >= V) return;

    const int32_t* prow = pos + (int64_t)t * K;
    const float* wrow = w + (int64_t)t * wst;
    const int64_t col = (int64_t)v * E;

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += kBatch) {
        int32_t p[kBatch];
        float wk[kBatch];
        Words<W> val[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int k = k0 + j;
            p[j] = k < K ? prow[k] : -1;
            wk[j] = k < K ? wrow[k] : 0.0f;
            if (p[j] >= 0) val[j] = load_words<W>(y + (int64_t)p[j] * ys + col);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (p[j] < 0) continue;
#pragma unroll
            for (int q = 0; q < W; ++q) {
                acc[2 * q] = __builtin_fmaf(wk[j], lo_bf16(val[j].w[q]), acc[2 * q]);
                acc[2 * q + 1] = __builtin_fmaf(wk[j], hi_bf16(val[j].w[q]), acc[2 * q + 1]);
            }
        }
    }

    Words<W> r;
#pragma unroll
    for (int q = 0; q < W; ++q) r.w[q] = pack_bf16_rne(acc[2 * q], acc[2 * q + 1]);
    store_words<W>(out + (int64_t)t * os + col, r);
}

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
    clear_launch_error();
    if (vec16)
        combine_kernel<4><<<(uint32_t)blocks, kThreads, 0, stream>>>(
            yy, y_row_stride, w, w_row_stride, pos, N, K, V, segs, oo, out_row_stride);
    else
        combine_kernel<1><<<(uint32_t)blocks, kThreads, 0, stream>>>(
            yy, y_row_stride, w, w_row_stride, pos, N, K, V, segs, oo, out_row_stride);
    return check_launch("moe_combine");
}
