// dispatch.hip -- byte scatter of each token's payload fields into the
// receive rows the layout assigned to its (token, k) pairs.
//
// Definition: every received row carries its token's whole payload, as
// DeepEP's dispatch returns recv_x, recv_x_scales, recv_topk_idx and
// recv_topk_weights per received token (repository dump, deep_ep.cpp,
// Buffer::intranode_dispatch); fields are opaque bytes at 16-byte
// granularity, as the tensors packed by make_desc in the vLLM branch
// compare ds-exp-2...ds-exp-ag (moe_allgather.cu).
//
// Launch shape: one wave per (token, k, 64-vector segment of the
// concatenated fields), segments of one receive row on consecutive waves.
// Each lane loads one vector of the token's source row and stores it to the
// pair's receive row; the K waves of a token re-read the same source bytes.
// Workgroups are handed to the 8 XCDs round-robin, each XCD with its own L2,
// so the kernel renumbers them: XCD x runs the x-th contiguous eighth of the
// work, which keeps all waves of a token on one XCD and its re-reads in that
// L2 (without this, measured source reads were 4x the source bytes). Every load and store instruction of a wave covers
// 64 consecutive vectors of one row (1 KiB with 16-byte vectors). Measured
// on MI355X at the prefill shape, this many-short-waves form writes faster
// than one wave storing each loaded vector K times, and only with
// non-temporal stores.
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kXcds = 8;   // MI355X: 8 XCDs, workgroup i runs on XCD i % 8

struct DispatchArgs {
    const char* src[MOE_MAX_FIELDS];
    char* dst[MOE_MAX_FIELDS];
    int64_t sstride[MOE_MAX_FIELDS];
    int64_t dstride[MOE_MAX_FIELDS];
    int32_t vend[MOE_MAX_FIELDS];  // running end of each field, in vectors
    const int32_t* pos;            // NULL: identity, K == 1
    int32_t N;
    int32_t K;
    int32_t V;                     // vectors per token over all fields
    int32_t segs;                  // 64-vector segments per token
};

template <typename VecT>
__global__ __launch_bounds__(kThreads) void dispatch_kernel(const DispatchArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    // Logical workgroup: XCD (blockIdx % 8) takes a contiguous eighth. The
    // grid is a multiple of 8, so this is a bijection on [0, gridDim.x).
    const uint32_t per_xcd = gridDim.x / kXcds;
    const uint32_t lb = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const uint32_t gw = lb * kWavesPerBlock + threadIdx.x / kWave;
    const uint32_t pair = __builtin_amdgcn_readfirstlane(gw / (uint32_t)a.segs);   // t*K + k
    if (pair >= (uint32_t)a.N * (uint32_t)a.K) return;
    const int32_t seg = (int32_t)(gw - pair * (uint32_t)a.segs);
    const int32_t v = seg * kWave + lane;
    if (v >= a.V) return;
    const int32_t t = __builtin_amdgcn_readfirstlane(pair / (uint32_t)a.K);
    const int32_t p = a.pos ? a.pos[pair] : t;
    if (p < 0) return;

    // Which field this lane's vector belongs to, and its offset inside it.
    const int f1 = v >= a.vend[0], f2 = v >= a.vend[1], f3 = v >= a.vend[2];
    const char* src = f3 ? a.src[3] : f2 ? a.src[2] : f1 ? a.src[1] : a.src[0];
    char* dst = f3 ? a.dst[3] : f2 ? a.dst[2] : f1 ? a.dst[1] : a.dst[0];
    const int64_t ss = f3 ? a.sstride[3] : f2 ? a.sstride[2] : f1 ? a.sstride[1] : a.sstride[0];
    const int64_t ds = f3 ? a.dstride[3] : f2 ? a.dstride[2] : f1 ? a.dstride[1] : a.dstride[0];
    const int32_t v0 = f3 ? a.vend[2] : f2 ? a.vend[1] : f1 ? a.vend[0] : 0;
    const int64_t inner = (int64_t)(v - v0) * sizeof(VecT);

    // Receive rows are written once and not read back by this pass:
    // non-temporal stores stream them out instead of parking them as dirty
    // lines in the caches, where the combine that follows would pay for the
    // write-back.
    const VecT val = *reinterpret_cast<const VecT*>(src + (int64_t)t * ss + inner);
    __builtin_nontemporal_store(val, reinterpret_cast<VecT*>(dst + (int64_t)p * ds + inner));
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_dispatch(const moe_field* fields, int32_t nfields, int32_t N, int32_t K,
                            const int32_t* pos, hipStream_t stream) {
    if (fields == nullptr || nfields < 1 || nfields > MOE_MAX_FIELDS)
        return fail(MOE_ERR_ARG, "moe_dispatch: need 1..%d fields (got %d%s)", MOE_MAX_FIELDS,
                    nfields, fields ? "" : ", NULL array");
    if (N < 0 || K < 1) return fail(MOE_ERR_ARG, "moe_dispatch: need N >= 0, K >= 1");
    if (K > MOE_MAX_TOPK) return fail(MOE_ERR_LIMIT, "moe_dispatch: K=%d > %d", K, MOE_MAX_TOPK);
    if ((int64_t)N * K >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_dispatch: N*K must be below 2^31");
    if (pos == nullptr && K != 1 && N > 0)
        return fail(MOE_ERR_ARG, "moe_dispatch: pos == NULL (identity) requires K == 1");
    if (!aligned(pos, 4)) return fail(MOE_ERR_ALIGN, "moe_dispatch: pos must be 4-byte aligned");

    bool all16 = true;
    int64_t total_bytes = 0;
    for (int f = 0; f < nfields; ++f) {
        const moe_field& d = fields[f];
        if (d.row_bytes < 0) return fail(MOE_ERR_ARG, "moe_dispatch: field %d row_bytes < 0", f);
        if (d.row_bytes > 0 && N > 0 && (d.src == nullptr || d.dst == nullptr))
            return fail(MOE_ERR_ARG, "moe_dispatch: field %d has a NULL pointer", f);
        if (!aligned(d.src, 4) || !aligned(d.dst, 4) || !aligned(d.src_row_stride, 4) ||
            !aligned(d.dst_row_stride, 4) || !aligned(d.row_bytes, 4))
            return fail(MOE_ERR_ALIGN, "moe_dispatch: field %d pointers, strides and row_bytes "
                        "must be multiples of 4 bytes", f);
        if (N > 1 && d.src_row_stride < d.row_bytes)
            return fail(MOE_ERR_ARG, "moe_dispatch: field %d src_row_stride < row_bytes", f);
        if (d.dst_row_stride < d.row_bytes)
            return fail(MOE_ERR_ARG, "moe_dispatch: field %d dst_row_stride < row_bytes", f);
        all16 = all16 && aligned(d.src, 16) && aligned(d.dst, 16) &&
                aligned(d.src_row_stride, 16) && aligned(d.dst_row_stride, 16) &&
                aligned(d.row_bytes, 16);
        total_bytes += d.row_bytes;
    }
    const int vb = all16 ? 16 : 4;
    if (total_bytes / vb >= ((int64_t)1 << 30))
        return fail(MOE_ERR_LIMIT, "moe_dispatch: %lld payload bytes per token is too large",
                    (long long)total_bytes);
    if (N == 0 || total_bytes == 0) return ok();

    DispatchArgs a{};
    int32_t vend = 0;
    for (int f = 0; f < MOE_MAX_FIELDS; ++f) {
        if (f < nfields) {
            a.src[f] = static_cast<const char*>(fields[f].src);
            a.dst[f] = static_cast<char*>(fields[f].dst);
            a.sstride[f] = fields[f].src_row_stride;
            a.dstride[f] = fields[f].dst_row_stride;
            vend += (int32_t)(fields[f].row_bytes / vb);
        }
        a.vend[f] = vend;
    }
    a.pos = pos;
    a.N = N;
    a.K = K;
    a.V = vend;
    a.segs = ceil_div<int32_t>(vend, kWave);
    const int64_t waves = (int64_t)N * K * a.segs;
    if (waves >= ((int64_t)1 << 31))
        return fail(MOE_ERR_LIMIT, "moe_dispatch: N*K*segments=%lld waves must be below 2^31",
                    (long long)waves);
    const int64_t blocks = ceil_div<int64_t>(ceil_div<int64_t>(waves, kWavesPerBlock), kXcds) * kXcds;
    clear_launch_error();
    if (all16)
        dispatch_kernel<u32x4><<<(uint32_t)blocks, kThreads, 0, stream>>>(a);
    else
        dispatch_kernel<uint32_t><<<(uint32_t)blocks, kThreads, 0, stream>>>(a);
    return check_launch("moe_dispatch");
}
