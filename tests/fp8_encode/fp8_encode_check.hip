// fp8_encode_check -- the FP8 dispatch's e4m3fn encoder (moe::pack4 in
// combine_moe_get_amd/csrc/fp8.hpp) against the bit-level definition of the
// cast, on every one of the 2^32 fp32 inputs and in each of the encoder's four
// byte positions (test infrastructure, built by __graft_entry__.build()).
//
// The definition (OCP e4m3fn, round to nearest even, finite overflow
// saturating to +-448, NaN -> 0x7F): for |f| >= 2^-6 round away the 20 low
// mantissa bits to nearest even and rebias the exponent from 127 to 7; below
// 2^-6 the codes are the multiples of 2^-9, i.e. rint(|f| * 512).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "fp8.hpp"

__device__ uint32_t reference_code(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7Fu;                       // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;               // >= 448 and infinity
    if (a < 0x3C800000u)                                     // below 2^-6: subnormal codes
        return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    const uint32_t c = (r >> 20) - (120u << 3);
    return sign | (c > 0x7Eu ? 0x7Eu : c);
}

constexpr int kMaxExamples = 16;

// Thread i encodes inputs (b, b+1, b+2, b+3), b = base + i, with a scale of
// 1 (an exact division), so over consecutive i every input passes through
// every byte position.
__global__ void check(uint64_t base, uint64_t count, unsigned long long* mismatches,
                      uint32_t* examples) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint32_t b = (uint32_t)(base + i);
        float f[4];
        for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(b + (uint32_t)j);
        const uint32_t w = moe::pack4(f, 1.0f);
        for (int j = 0; j < 4; ++j) {
            const uint32_t got = (w >> (8 * j)) & 0xFFu;
            const uint32_t want = reference_code(f[j]);
            if (got != want) {
                const unsigned long long k = atomicAdd(mismatches, 1ull);
                if (k < kMaxExamples) {
                    examples[3 * k] = b + (uint32_t)j;
                    examples[3 * k + 1] = want;
                    examples[3 * k + 2] = got;
                }
            }
        }
    }
}

#define CHECK(x)                                                                      \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);    \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

int main() {
    unsigned long long* d_count;
    uint32_t* d_ex;
    CHECK(hipMalloc(&d_count, sizeof(unsigned long long)));
    CHECK(hipMalloc(&d_ex, 3 * kMaxExamples * sizeof(uint32_t)));
    CHECK(hipMemset(d_count, 0, sizeof(unsigned long long)));
    CHECK(hipMemset(d_ex, 0, 3 * kMaxExamples * sizeof(uint32_t)));
    const uint64_t total = 1ull << 32, chunk = 1ull << 30;
    for (uint64_t b = 0; b < total; b += chunk) {
        check<<<8192, 256>>>(b, chunk, d_count, d_ex);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        printf("inputs %llu .. %llu checked\n", (unsigned long long)b,
               (unsigned long long)(b + chunk - 1));
        fflush(stdout);
    }
    unsigned long long n = 0;
    uint32_t ex[3 * kMaxExamples];
    CHECK(hipMemcpy(&n, d_count, sizeof(n), hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(ex, d_ex, sizeof(ex), hipMemcpyDeviceToHost));
    for (unsigned long long i = 0; i < n && i < (unsigned long long)kMaxExamples; ++i)
        printf("  input %08x: want %02x got %02x\n", ex[3 * i], ex[3 * i + 1], ex[3 * i + 2]);
    printf("fp8_encode_check mismatches: %llu\n", n);
    return n == 0 ? 0 : 2;
}
