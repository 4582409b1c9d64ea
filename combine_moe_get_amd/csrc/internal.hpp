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

// 16-byte and 4-byte lane payloads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

}  // namespace moe
