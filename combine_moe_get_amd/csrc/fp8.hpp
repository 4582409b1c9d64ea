// fp8.hpp -- the e4m3fn encoder of the FP8 dispatch (quant.hip), in a header
// of its own so that a test program can check it on every fp32 input. Not
// installed; the public interface is include/moe_get.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// e4m3fn codes of f[0..3] / s, byte j from f[j]. The quotient is the
// correctly rounded fp32 division; gfx950's v_cvt_pk_fp8_f32 then rounds to
// nearest even into OCP e4m3fn (subnormals included). It does not saturate,
// so finite quotients are clamped to +-448 first, and NaN (which the clamp
// would turn into a number) maps to 0x7F. This matches the bit-level
// definition (round the 20 dropped mantissa bits to nearest even, rebias,
// saturate at 448, multiples of 2^-9 below 2^-6) on every fp32 input.
__device__ __forceinline__ uint32_t pack4(const float* f, float s) {
    float c[4];
    uint32_t nan = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float q = f[j] / s;
        nan |= (q != q) ? (0xFFu << (8 * j)) : 0u;
        c[j] = fminf(fmaxf(q, -448.0f), 448.0f);
    }
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
    return ((uint32_t)w & ~nan) | (0x7F7F7F7Fu & nan);
}

}  // namespace moe
