// internal.hpp -- helpers shared by the libmoe_get.so translation units.
// Not installed; the public interface is include/moe_get.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "moe_get.h"

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// The debug build (compiled with -DMOE_DEBUG, libmoe_get_debug.so): every
// layout call also checks its own outputs on the device and adds what it
// finds to a per-device status (moe_debug_status).
#ifdef MOE_DEBUG
constexpr bool kDebug = true;
#else
constexpr bool kDebug = false;
#endif

// Records `fmt` as this thread's last error and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears this thread's last error and returns MOE_OK.
int ok();
// Drops an error a previous, unrelated HIP call may have left behind, so
// that check_launch reports only the launches that follow.
inline void clear_launch_error() { (void)hipGetLastError(); }
// Maps a launch error (hipGetLastError after a launch) to MOE_ERR_HIP.
int check_launch(const char* what);

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline bool aligned(int64_t v, int64_t a) { return (v & (a - 1)) == 0; }

template <typename T>
__host__ __device__ constexpr T ceil_div(T a, T b) { return (a + b - 1) / b; }

// A launch holds fewer than 2^32 work-items along x (HIP refuses a larger
// grid as an invalid configuration). Kernels whose grid grows with the batch
// are launched in pieces of at most this many work-items, one after another
// on the same stream, each told the index of its first workgroup; the
// one-launch kernels, which need their whole grid at once, refuse larger jobs.
constexpr int64_t kMaxLaunchItems = (int64_t)1 << 31;

// Calls launch(first, count) for consecutive pieces of [0, total), each of
// at most `piece` workgroups, and stops after a launch that failed, so that
// check_launch reports that failure rather than a later launch's status.
template <typename F>
inline void in_pieces(int64_t total, int64_t piece, F&& launch) {
    for (int64_t first = 0; first < total; first += piece) {
        launch(first, total - first < piece ? total - first : piece);
        if (hipPeekAtLastError() != hipSuccess) return;
    }
}

// 16-byte and 4-byte lane payloads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Inclusive prefix sum over the 64 lanes of a wave (lane i gets the sum of
// lanes 0 .. i), in six DPP steps instead of a chain of LDS-routed shuffles:
// shifts by 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from
// outside the row add 0), then lane 15 of rows 0 and 2 added to rows 1 and 3
// (row_bcast:15), then lane 31 added to rows 2 and 3 (row_bcast:31). Every
// lane of the wave must be active.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);    // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);    // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);    // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);    // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// Sum over the 64 lanes of a wave, in every lane (all lanes active).
__device__ __forceinline__ int32_t wave_sum(int32_t x) {
    return __builtin_amdgcn_readlane(wave_inclusive_scan(x), kWave - 1);
}

// Third word of a gfx9 buffer descriptor for raw (untyped) loads, which are
// range-checked against num_records: loads past it return 0 and touch no
// memory.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer load: non-temporal (the nt bit on gfx950).
constexpr int kBufferNT = 2;

// Layouts of small batches in one launch: the layout part of the one-launch
// dispatch kernels, run without a payload. Every workgroup counts the whole
// batch itself, which beats the two-kernel layout (histogram, then
// assignment) up to about kOneLaunchPairs pairs. Same outputs as the
// two-kernel layout; arguments are validated by the caller.
constexpr int64_t kOneLaunchPairs = 2048;
int layout_one_launch(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                      int32_t E, int32_t align, int32_t* counts, int32_t* offsets, int32_t* pos,
                      int32_t* row_pair, int64_t cap, int32_t* order, int32_t* status,
                      hipStream_t stream);
int layout_padded_one_launch(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K,
                             int32_t E, int32_t M, int32_t* counts, int32_t* pos,
                             int32_t* row_pair, int64_t* layout_range, int32_t* recv_stats,
                             int32_t* status, hipStream_t stream);

// In the debug build, launches the check of moe_check_layout on a layout's
// outputs (pos for nk pairs, row_pair for cap rows, the plan if given),
// adding to the device's debug status; returns MOE_OK at once otherwise.
int debug_check_layout(const char* fn, const int32_t* pos, int64_t nk, const int32_t* row_pair,
                       int64_t cap, const int32_t* order, hipStream_t stream);

// The one-pass layout of the one-launch forms (small batches): every
// workgroup counts the whole batch itself. tot[E], bef[E] and *nbad live in
// LDS and start at 0. Adds, over all pairs i < nk (ids read with a row
// stride; contiguous ids, stride == K, without a division by K): each valid
// id to tot[id] and, for pairs of earlier tokens (i < before), to bef[id];
// ids >= E to *nbad. LDS integer atomics: the sums do not depend on their
// order. Each thread loads kIdBatch ids, from clamped indices so that no
// load sits under a branch, before it counts any: up to kIdBatch * blockDim.x
// pairs cost one dependent memory round trip rather than one per
// blockDim.x pairs. The caller synchronizes before and after.
constexpr int kIdBatch = 8;

__device__ __forceinline__ void count_batch_ids(const int32_t* __restrict__ ids, int64_t stride,
                                                int32_t nk, int32_t K, int32_t E, int32_t before,
                                                int32_t* tot, int32_t* bef, int32_t* nbad) {
    const bool contiguous = stride == (int64_t)K;
    const int32_t step = (int32_t)blockDim.x;
    int32_t bad = 0;
    for (int32_t i0 = threadIdx.x; i0 < nk; i0 += kIdBatch * step) {
        int32_t e[kIdBatch];
#pragma unroll
        for (int j = 0; j < kIdBatch; ++j) {
            const int32_t i = min(i0 + j * step, nk - 1);
            if (contiguous) {
                e[j] = ids[i];
            } else {
                const int32_t ti = i / K;
                e[j] = ids[(int64_t)ti * stride + (i - ti * K)];
            }
        }
#pragma unroll
        for (int j = 0; j < kIdBatch; ++j) {
            const int32_t i = i0 + j * step;
            const int32_t ej = i < nk ? e[j] : -1;
            if (ej >= E) {
                ++bad;
            } else if (ej >= 0) {
                atomicAdd(&tot[ej], 1);
                if (i < before) atomicAdd(&bef[ej], 1);
            }
        }
    }
    if (bad) atomicAdd(nbad, bad);
}

// Rank of the token's pair k among the pairs with its (valid) expert, in
// (t, k) order: the pairs of earlier tokens with that expert (bef) plus the
// earlier k' of the token itself with the same expert.
__device__ __forceinline__ int32_t rank_in_expert(const int32_t* tok_e, const int32_t* bef,
                                                  int32_t k) {
    const int32_t e = tok_e[k];
    int32_t r = bef[e];
    for (int32_t j = 0; j < k; ++j) r += tok_e[j] == e;
    return r;
}

}  // namespace moe
