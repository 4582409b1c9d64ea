// check.hip -- a device check of a layout's index arrays, and the status the
// debug build (MOE_DEBUG) keeps with it.
//
// moe_dispatch, moe_combine and the other calls that take pos trust it: a
// row outside the receive buffer is an out-of-bounds access. Layouts from
// this library are correct by construction (and tested against the oracle);
// a caller who builds pos another way can check it here first. The check
// restates what the layout's definition fixes (DeepEP, repository dump,
// deep_ep.cpp, Buffer::get_dispatch_layout and the receive buffer's
// recv_src_idx): every pair has one row or none, each used row names its
// pair, and the dispatch plan lists pairs that have rows.
//
// DeepEP stops a kernel on a failed device assertion (EP_DEVICE_ASSERT, a
// trap). Here a failed check is a count in a status word, and the kernel
// goes on: every read it makes is guarded by the ranges it checks.
#include <mutex>

#include "internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 1024;

// One pass over pairs and rows, grid-stride. Counts (added to status[0..3]):
//   0: pairs whose pos is neither -1 nor a row < cap;
//   1: pairs with a row whose row_pair does not name them (row_pair given);
//   2: rows whose row_pair is neither -1 nor a pair whose pos is that row
//      (row_pair given);
//   3: plan entries that are neither -1 nor a pair with a row (order given).
// With `checked` (the debug build's status), also adds 1 to *checked.
__global__ __launch_bounds__(kThreads) void check_layout_kernel(
    const int32_t* __restrict__ pos, int64_t nk, const int32_t* __restrict__ row_pair,
    int64_t cap, const int32_t* __restrict__ order, int32_t* __restrict__ status,
    int32_t* __restrict__ checked) {
    if (checked != nullptr && blockIdx.x == 0 && threadIdx.x == 0) atomicAdd(checked, 1);
    int32_t bad[4] = {0, 0, 0, 0};
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t n = nk > cap ? nk : cap;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        if (i < nk) {
            const int32_t p = pos[i];
            if (p != -1 && (p < 0 || p >= cap))
                ++bad[0];
            else if (p >= 0 && row_pair != nullptr && row_pair[p] != (int32_t)i)
                ++bad[1];
            if (order != nullptr) {
                const int32_t o = order[i];
                if (o != -1) {
                    const int32_t q = (o >= 0 && o < nk) ? pos[o] : -1;
                    if (q < 0 || q >= cap) ++bad[3];
                }
            }
        }
        if (i < cap && row_pair != nullptr) {
            const int32_t j = row_pair[i];
            if (j != -1 && (j < 0 || j >= nk || pos[j] != (int32_t)i)) ++bad[2];
        }
    }
    // All lanes are active again here: one sum per wave, one atomic per
    // wave and counter (vector memory atomics).
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int32_t s = wave_sum(bad[c]);
        if ((threadIdx.x & (kWave - 1)) == 0 && s != 0) atomicAdd(&status[c], s);
    }
}

constexpr int kDebugWords = 5;   // the four counts, then the layouts checked

__global__ void zero_debug_kernel(int32_t* __restrict__ s) {
    if (threadIdx.x < kDebugWords) s[threadIdx.x] = 0;
}

void launch_check(const int32_t* pos, int64_t nk, const int32_t* row_pair, int64_t cap,
                  const int32_t* order, int32_t* status, int32_t* checked, hipStream_t stream) {
    const int64_t n = nk > cap ? nk : cap;
    int64_t blocks = ceil_div<int64_t>(n, kThreads);
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    if (blocks < 1) {
        if (checked == nullptr) return;
        blocks = 1;   // an empty layout is still counted
    }
    check_layout_kernel<<<(uint32_t)blocks, kThreads, 0, stream>>>(pos, nk, row_pair, cap, order,
                                                                   status, checked);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_check_layout(const int32_t* pos, int32_t N, int32_t K,
                                const int32_t* row_pair, int64_t cap, const int32_t* order,
                                int32_t* status, hipStream_t stream) {
    if (N < 0 || K < 1 || cap < 0)
        return fail(MOE_ERR_ARG, "moe_check_layout: need N >= 0, K >= 1, cap >= 0 "
                    "(got N=%d K=%d cap=%lld)", N, K, (long long)cap);
    const int64_t nk = (int64_t)N * K;
    if (nk >= ((int64_t)1 << 31) || cap >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_check_layout: N*K and cap must be below 2^31");
    if (status == nullptr || (nk > 0 && pos == nullptr))
        return fail(MOE_ERR_ARG, "moe_check_layout: status and pos must not be NULL");
    if (!aligned(pos, 4) || !aligned(row_pair, 4) || !aligned(order, 4) || !aligned(status, 4))
        return fail(MOE_ERR_ALIGN, "moe_check_layout: int32 pointers must be 4-byte aligned");
    clear_launch_error();
    launch_check(pos, nk, row_pair, cap, order, status, nullptr, stream);
    return check_launch("moe_check_layout");
}

// ---------------------------------------------------------------------------
// The debug build's status: five counters per device, in a file-scope device
// array (`debug_status`, zero when the library loads), to which every layout
// call adds the check of its own outputs (four counts) and 1 (the fifth). In host code `debug_status` names a
// host-side stand-in: the kernels get the array's device address, looked up
// once per device with hipGetSymbolAddress. Layout calls that overlap on one
// GPU add to the same counters, which is what counters are for.
// ---------------------------------------------------------------------------
static __device__ __align__(16) int32_t debug_status[8];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_status_mu;
int32_t* g_status_ptr[kMaxDevices];

int debug_status_on(const char* fn, hipStream_t stream, int32_t** out) {
    int dev = -1;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "%s: no device for the stream: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_LIMIT, "%s: device %d beyond %d devices", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_status_mu);
    if (g_status_ptr[dev] == nullptr) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* ptr = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(debug_status));
        if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || ptr == nullptr)
            return fail(MOE_ERR_HIP, "%s: status address on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        g_status_ptr[dev] = static_cast<int32_t*>(ptr);
    }
    *out = g_status_ptr[dev];
    return MOE_OK;
}
}  // namespace

namespace moe {
int debug_check_layout(const char* fn, const int32_t* pos, int64_t nk, const int32_t* row_pair,
                       int64_t cap, const int32_t* order, hipStream_t stream) {
    if (!kDebug) return MOE_OK;
    int32_t* status = nullptr;
    const int rc = debug_status_on(fn, stream, &status);
    if (rc != MOE_OK) return rc;
    clear_launch_error();
    launch_check(pos, nk, row_pair, cap, order, status, status + 4, stream);
    return check_launch(fn);
}
}  // namespace moe

extern "C" int moe_debug_status(int32_t* out, int32_t reset, hipStream_t stream) {
    const char* fn = "moe_debug_status";
    if (!kDebug)
        return fail(MOE_ERR_LIMIT, "%s: this library is not a debug build (MOE_DEBUG)", fn);
    if (out == nullptr) return fail(MOE_ERR_ARG, "%s: out must not be NULL", fn);
    int32_t* status = nullptr;
    int rc = debug_status_on(fn, stream, &status);
    if (rc != MOE_OK) return rc;
    hipError_t e =
        hipMemcpyAsync(out, status, kDebugWords * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "%s: reading the status: %s", fn, hipGetErrorString(e));
    if (reset) {
        clear_launch_error();
        zero_debug_kernel<<<1, kWave, 0, stream>>>(status);
        return check_launch(fn);
    }
    return ok();
}
