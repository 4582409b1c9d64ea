// ceilings.hip -- bandwidth ceilings of the memory patterns the layout /
// dispatch / combine kernels use, measured on the same GPU. Built into its
// own library (libmoe_ceilings.so) for `bench.py --ceilings`; the product
// library does not contain or call any of it.
//
// Each kernel moves bytes in one pattern and does nothing else, so its rate
// is what that pattern can reach on this GPU:
//   ceil_read       streaming 16-byte loads (plain or non-temporal); each
//                   wave reads 1 or 8 consecutive KiB (a template argument,
//                   so each form has its own kernel name in a trace)
//   ceil_write      streaming 16-byte stores (plain or non-temporal)
//   ceil_copy       both at once (load, then store the loaded vector)
//   ceil_mix        the combine's ratio as a stream: each wave reads R KiB
//                   and writes 1 KiB
//   ceil_dispatch_stores  the dispatch's stores exactly (one wave per
//                   (pair, 64-vector segment of the concatenated fields),
//                   XCD-contiguous workgroups, rows from pos, non-temporal),
//                   with a constant in place of the loaded source vector
//   ceil_combine_reads    the combine's loads exactly (one wave per (token,
//                   64-vector segment), K expert rows per lane from pos,
//                   non-temporal, one at a time), with no store of the sums
//   ceil_empty      a kernel that does nothing: the fixed cost of a launch
// Loaded values are folded into one word that is stored only if it equals
// a value no input here produces, so no load can be dropped and no store
// adds traffic. Entry points return 0, or -1 when the launch failed.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kXcds = 8;
constexpr uint32_t kNever = 0x7F5A3C1Bu;   // a fold value none of the inputs here give
constexpr int kMaxFields = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4 v, u32x4* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Wave w covers KiB w*PW .. (w+1)*PW - 1 of the buffer; all of a wave's
// loads are issued before the first is used.
template <bool NT, int PW>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src,
                                                        int64_t nvec,
                                                        uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    u32x4 v[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int64_t i = (w * PW + j) * kWave + lane;
        v[j] = i < nvec ? ld<NT>(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int j = 0; j < PW; ++j) acc ^= fold(v[j]);
    if (acc == kNever) sink[0] = acc;
}

template <bool NT, int PW>
__global__ __launch_bounds__(kThreads) void write_kernel(u32x4* __restrict__ dst, int64_t nvec) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const u32x4 val = {(uint32_t)lane, 1u, 2u, 3u};
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int64_t i = (w * PW + j) * kWave + lane;
        if (i < nvec) st<NT>(val, dst + i);
    }
}

template <bool NT, int PW>
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t nvec) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    u32x4 v[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int64_t i = (w * PW + j) * kWave + lane;
        v[j] = i < nvec ? ld<NT>(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int64_t i = (w * PW + j) * kWave + lane;
        if (i < nvec) st<NT>(v[j], dst + i);
    }
}

// Wave w reads KiB w*R .. w*R+R-1 of src (non-temporal) and writes KiB w of
// dst (non-temporal): the combine's R-to-1 mix of reads and writes, streamed.
__global__ __launch_bounds__(kThreads) void mix_kernel(const u32x4* __restrict__ src,
                                                       u32x4* __restrict__ dst, int64_t waves,
                                                       int R) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (w >= waves) return;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int j = 0; j < R; ++j) acc ^= ld<true>(src + (w * R + j) * kWave + lane);
    st<true>(acc, dst + w * kWave + lane);
}

struct StoreArgs {
    char* dst[kMaxFields];
    int64_t dstride[kMaxFields];
    int32_t vend[kMaxFields];   // running end of each field, in 16-byte vectors
    const int32_t* pos;         // NULL: row = pair
    int32_t N, K, V, segs;
};

// The dispatch kernel's grid, renumbering and row addressing, storing a
// constant instead of the token's loaded vector. FROM_POS: rows from pos
// (else row = pair); a template argument, so each form has its own name in a
// kernel trace.
template <bool FROM_POS>
__global__ __launch_bounds__(kThreads) void dispatch_stores_kernel(const StoreArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t per_xcd = gridDim.x / kXcds;
    const uint32_t lb = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const uint32_t gw = lb * kWavesPerBlock + threadIdx.x / kWave;
    const uint32_t pair = __builtin_amdgcn_readfirstlane(gw / (uint32_t)a.segs);
    if (pair >= (uint32_t)a.N * (uint32_t)a.K) return;
    const int32_t seg = (int32_t)(gw - pair * (uint32_t)a.segs);
    const int32_t v = seg * kWave + lane;
    if (v >= a.V) return;
    const int32_t p = FROM_POS ? a.pos[pair] : (int32_t)pair;
    if (p < 0) return;
    const int f1 = v >= a.vend[0], f2 = v >= a.vend[1], f3 = v >= a.vend[2];
    char* dst = f3 ? a.dst[3] : f2 ? a.dst[2] : f1 ? a.dst[1] : a.dst[0];
    const int64_t ds = f3 ? a.dstride[3] : f2 ? a.dstride[2] : f1 ? a.dstride[1] : a.dstride[0];
    const int32_t v0 = f3 ? a.vend[2] : f2 ? a.vend[1] : f1 ? a.vend[0] : 0;
    const u32x4 val = {(uint32_t)v, pair, 7u, 9u};
    __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(dst + (int64_t)p * ds +
                                                              (int64_t)(v - v0) * 16));
}

// The combine kernel's grid and loads (16-byte vectors, one row at a time,
// non-temporal), with the sums folded instead of stored. FROM_POS: rows from
// pos (else row = t*K + k).
template <bool FROM_POS>
__global__ __launch_bounds__(kThreads) void combine_reads_kernel(
    const uint16_t* __restrict__ y, int64_t ys, const int32_t* __restrict__ pos, int32_t N,
    int32_t K, int32_t V, int32_t segs, uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int32_t t = __builtin_amdgcn_readfirstlane((int32_t)(gw / segs));
    if (t >= N) return;
    const int32_t seg = (int32_t)(gw - (int64_t)t * segs);
    const int32_t v = seg * kWave + lane;
    if (v >= V) return;
    uint32_t acc = 0;
    for (int32_t k = 0; k < K; ++k) {
        const int32_t p = FROM_POS ? pos[(int64_t)t * K + k] : t * K + k;
        if (p >= 0)
            acc ^= fold(__builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(y + (int64_t)p * ys) + v));
    }
    if (acc == kNever) sink[0] = acc;
}

// Does nothing (p is always NULL): the cost of a launch and nothing else.
__global__ __launch_bounds__(kThreads) void empty_kernel(uint32_t* p) {
    if (p != nullptr && threadIdx.x == kThreads) p[0] = 0;
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -1; }

int64_t blocks_for(int64_t waves) { return (waves + kWavesPerBlock - 1) / kWavesPerBlock; }

}  // namespace

extern "C" {

// nt: non-temporal loads/stores (1) or plain (0); per_wave: KiB per wave,
// 1 or 8. bytes: a multiple of 16.
#define CEIL_DISPATCH_PW(KERNEL, ...)                                                   \
    do {                                                                                 \
        const int64_t nvec = bytes / 16;                                                 \
        const int64_t pw = per_wave == 8 ? 8 : 1;                                        \
        const uint32_t g = (uint32_t)blocks_for((nvec / kWave + pw - 1) / pw);          \
        if (nt && pw == 8) KERNEL<true, 8><<<g, kThreads, 0, stream>>>(__VA_ARGS__);      \
        else if (nt) KERNEL<true, 1><<<g, kThreads, 0, stream>>>(__VA_ARGS__);            \
        else if (pw == 8) KERNEL<false, 8><<<g, kThreads, 0, stream>>>(__VA_ARGS__);      \
        else KERNEL<false, 1><<<g, kThreads, 0, stream>>>(__VA_ARGS__);                   \
    } while (0)

int ceil_read(const void* src, int64_t bytes, int nt, int per_wave, void* sink,
              hipStream_t stream) {
    if (per_wave != 1 && per_wave != 8) return -1;
    (void)hipGetLastError();
    CEIL_DISPATCH_PW(read_kernel, static_cast<const u32x4*>(src), nvec,
                     static_cast<uint32_t*>(sink));
    return launched();
}

int ceil_write(void* dst, int64_t bytes, int nt, int per_wave, hipStream_t stream) {
    if (per_wave != 1 && per_wave != 8) return -1;
    (void)hipGetLastError();
    CEIL_DISPATCH_PW(write_kernel, static_cast<u32x4*>(dst), nvec);
    return launched();
}

int ceil_copy(const void* src, void* dst, int64_t bytes, int nt, int per_wave,
              hipStream_t stream) {
    if (per_wave != 1 && per_wave != 8) return -1;
    (void)hipGetLastError();
    CEIL_DISPATCH_PW(copy_kernel, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
    return launched();
}

// Reads waves*R KiB of src and writes waves KiB of dst.
int ceil_mix(const void* src, void* dst, int64_t waves, int R, hipStream_t stream) {
    (void)hipGetLastError();
    mix_kernel<<<(uint32_t)blocks_for(waves), kThreads, 0, stream>>>(
        static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), waves, R);
    return launched();
}

// Fields as in moe_dispatch (destination pointer, destination row stride and
// row bytes, all multiples of 16); pos may be NULL (row = pair).
int ceil_dispatch_stores(void* const* dsts, const int64_t* dst_row_strides,
                         const int64_t* row_bytes, int32_t nfields, const int32_t* pos,
                         int32_t N, int32_t K, hipStream_t stream) {
    if (nfields < 1 || nfields > kMaxFields) return -1;
    StoreArgs a{};
    int32_t v = 0;
    for (int f = 0; f < kMaxFields; ++f) {
        if (f < nfields) {
            a.dst[f] = static_cast<char*>(dsts[f]);
            a.dstride[f] = dst_row_strides[f];
            v += (int32_t)(row_bytes[f] / 16);
        }
        a.vend[f] = v;
    }
    a.pos = pos;
    a.N = N;
    a.K = K;
    a.V = v;
    a.segs = (v + kWave - 1) / kWave;
    const int64_t waves = (int64_t)N * K * a.segs;
    const int64_t blocks = (blocks_for(waves) + kXcds - 1) / kXcds * kXcds;
    (void)hipGetLastError();
    if (pos)
        dispatch_stores_kernel<true><<<(uint32_t)blocks, kThreads, 0, stream>>>(a);
    else
        dispatch_stores_kernel<false><<<(uint32_t)blocks, kThreads, 0, stream>>>(a);
    return launched();
}

// y rows of Hc bf16 (Hc a multiple of 8, rows ys elements apart); pos may be
// NULL (row = t*K + k).
int ceil_combine_reads(const void* y, int64_t ys, const int32_t* pos, int32_t N, int32_t K,
                       int32_t Hc, void* sink, hipStream_t stream) {
    const int32_t V = Hc / 8;
    const int32_t segs = (V + kWave - 1) / kWave;
    (void)hipGetLastError();
    const uint32_t g = (uint32_t)blocks_for((int64_t)N * segs);
    if (pos)
        combine_reads_kernel<true><<<g, kThreads, 0, stream>>>(
            static_cast<const uint16_t*>(y), ys, pos, N, K, V, segs, static_cast<uint32_t*>(sink));
    else
        combine_reads_kernel<false><<<g, kThreads, 0, stream>>>(
            static_cast<const uint16_t*>(y), ys, pos, N, K, V, segs, static_cast<uint32_t*>(sink));
    return launched();
}

int ceil_empty(int32_t blocks, hipStream_t stream) {
    (void)hipGetLastError();
    empty_kernel<<<(uint32_t)blocks, kThreads, 0, stream>>>(nullptr);
    return launched();
}

}  // extern "C"
