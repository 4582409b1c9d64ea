/*
 * abi_check.c -- the C ABI used from plain C, without Python or torch:
 * moe_get_layout -> moe_dispatch -> moe_combine on a caller-created HIP
 * stream, every result compared with the CPU oracle (test infrastructure,
 * liboracle.so). Layout and dispatch must match bit for bit, the combine
 * within one bf16 ulp. Prints "abi_check ok" and exits 0 on success.
 *
 * Inputs are drawn from a 64-bit LCG: masked (-1) and out-of-range ids,
 * repeated experts within a token, four payload fields, and bf16 values
 * with at most 8 significant bits (exact in bf16).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_get.h"

/* the oracle's entry points (oracle/moe_oracle.c) */
typedef struct {
    const void* src;
    int64_t src_row_stride;
    void* dst;
    int64_t dst_row_stride;
    int64_t row_bytes;
} oracle_field;
int oracle_layout(const int32_t* ids, int64_t ids_row_stride, int32_t N, int32_t K, int32_t E,
                  int32_t align, int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* row_pair,
                  int64_t cap, int32_t* status);
int oracle_dispatch(const oracle_field* fields, int32_t nfields, int32_t N, int32_t K,
                    const int32_t* pos);
int oracle_combine(const uint16_t* y, int64_t y_row_stride, const float* w, int64_t w_row_stride,
                   const int32_t* pos, int32_t N, int32_t K, int32_t Hc, uint16_t* out,
                   int64_t out_row_stride);

#define HIP_OK(x)                                                                       \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            return 1;                                                                   \
        }                                                                               \
    } while (0)
#define MOE_OK_(x)                                                                      \
    do {                                                                                \
        int rc_ = (x);                                                                  \
        if (rc_ != MOE_OK) {                                                            \
            fprintf(stderr, "%s: %d %s\n", #x, rc_, moe_last_error());                 \
            return 1;                                                                   \
        }                                                                               \
    } while (0)

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t draw(void) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(state >> 33);
}

/* a bf16 value with at most 8 significant bits: (-255..255) / 64 */
static uint16_t small_bf16(void) {
    float f = (float)((int)(draw() % 511) - 255) / 64.0f;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static int ordered(uint16_t b) { return (b & 0x8000) ? -(int)(b & 0x7FFF) : (int)(b & 0x7FFF); }

#define NF 4

int main(void) {
    enum { N = 300, K = 8, E = 64, HC = 512 };
    const int64_t row_bytes[NF] = {1024, 32, 32, 32};   /* hidden, scales, ids, weights */
    const int64_t cap = moe_required_capacity(N, K, E, 1);
    const size_t ws_bytes = moe_layout_workspace_bytes(N, K, E);
    if (cap != (int64_t)N * K || ws_bytes == 0) {
        fprintf(stderr, "unexpected sizes cap=%lld ws=%zu\n", (long long)cap, ws_bytes);
        return 1;
    }

    /* host inputs */
    int32_t* ids = malloc(sizeof(int32_t) * N * K);
    float* w = malloc(sizeof(float) * N * K);
    uint8_t* src[NF];
    uint16_t* y = malloc(sizeof(uint16_t) * cap * HC);
    for (int i = 0; i < N * K; ++i) {
        int v = (int)(draw() % (E + 6)) - 1;            /* -1 masked, >= E out of range */
        ids[i] = v;
        w[i] = (float)((int)(draw() % 2001) - 1000) / 128.0f;
    }
    for (int f = 0; f < NF; ++f) {
        src[f] = malloc(row_bytes[f] * N);
        for (int64_t b = 0; b < row_bytes[f] * N; ++b) src[f][b] = (uint8_t)draw();
    }
    for (int64_t i = 0; i < cap * HC; ++i) y[i] = small_bf16();

    /* device buffers and a stream of our own */
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    int32_t *d_ids, *d_counts, *d_offsets, *d_pos, *d_row_pair, *d_order, *d_status;
    float* d_w;
    void* d_ws;
    uint16_t *d_y, *d_out;
    void *d_src[NF], *d_dst[NF];
    HIP_OK(hipMalloc((void**)&d_ids, sizeof(int32_t) * N * K));
    HIP_OK(hipMalloc((void**)&d_counts, sizeof(int32_t) * E));
    HIP_OK(hipMalloc((void**)&d_offsets, sizeof(int32_t) * (E + 1)));
    HIP_OK(hipMalloc((void**)&d_pos, sizeof(int32_t) * N * K));
    HIP_OK(hipMalloc((void**)&d_row_pair, sizeof(int32_t) * cap));
    HIP_OK(hipMalloc((void**)&d_order, sizeof(int32_t) * N * K));
    HIP_OK(hipMalloc((void**)&d_status, sizeof(int32_t)));
    HIP_OK(hipMalloc((void**)&d_w, sizeof(float) * N * K));
    HIP_OK(hipMalloc(&d_ws, ws_bytes));
    HIP_OK(hipMalloc((void**)&d_y, sizeof(uint16_t) * cap * HC));
    HIP_OK(hipMalloc((void**)&d_out, sizeof(uint16_t) * N * HC));
    HIP_OK(hipMemcpy(d_ids, ids, sizeof(int32_t) * N * K, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, w, sizeof(float) * N * K, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_y, y, sizeof(uint16_t) * cap * HC, hipMemcpyHostToDevice));
    moe_field fields[NF];
    for (int f = 0; f < NF; ++f) {
        HIP_OK(hipMalloc(&d_src[f], row_bytes[f] * N));
        HIP_OK(hipMalloc(&d_dst[f], row_bytes[f] * cap));
        HIP_OK(hipMemcpy(d_src[f], src[f], row_bytes[f] * N, hipMemcpyHostToDevice));
        HIP_OK(hipMemset(d_dst[f], 0xA5, row_bytes[f] * cap));
        fields[f].src = d_src[f];
        fields[f].src_row_stride = row_bytes[f];
        fields[f].dst = d_dst[f];
        fields[f].dst_row_stride = row_bytes[f];
        fields[f].row_bytes = row_bytes[f];
    }

    MOE_OK_(moe_get_layout(d_ids, K, N, K, E, 1, d_counts, d_offsets, d_pos, d_row_pair, cap,
                           d_order, d_ws, ws_bytes, d_status, stream));
    MOE_OK_(moe_dispatch(fields, NF, N, K, d_pos, d_order, stream));
    MOE_OK_(moe_combine(d_y, HC, d_w, K, d_pos, N, K, HC, d_out, HC, stream));
    /* the device check of the layout's index arrays: nothing to report */
    int32_t* d_check;
    HIP_OK(hipMalloc((void**)&d_check, 4 * sizeof(int32_t)));
    HIP_OK(hipMemsetAsync(d_check, 0, 4 * sizeof(int32_t), stream));
    MOE_OK_(moe_check_layout(d_pos, N, K, d_row_pair, cap, d_order, d_check, stream));
    HIP_OK(hipStreamSynchronize(stream));
    int32_t g_check[4];
    HIP_OK(hipMemcpy(g_check, d_check, sizeof(g_check), hipMemcpyDeviceToHost));

    /* the oracle on the same inputs */
    int32_t counts[E], offsets[E + 1], status = 0;
    int32_t* pos = malloc(sizeof(int32_t) * N * K);
    int32_t* row_pair = malloc(sizeof(int32_t) * cap);
    if (oracle_layout(ids, K, N, K, E, 1, counts, offsets, pos, row_pair, cap, &status) != 0) {
        fprintf(stderr, "oracle_layout failed\n");
        return 1;
    }
    oracle_field of[NF];
    uint8_t* ref_dst[NF];
    for (int f = 0; f < NF; ++f) {
        ref_dst[f] = malloc(row_bytes[f] * cap);
        memset(ref_dst[f], 0xA5, row_bytes[f] * cap);
        of[f].src = src[f];
        of[f].src_row_stride = row_bytes[f];
        of[f].dst = ref_dst[f];
        of[f].dst_row_stride = row_bytes[f];
        of[f].row_bytes = row_bytes[f];
    }
    uint16_t* ref_out = malloc(sizeof(uint16_t) * N * HC);
    if (oracle_dispatch(of, NF, N, K, pos) != 0 ||
        oracle_combine(y, HC, w, K, pos, N, K, HC, ref_out, HC) != 0) {
        fprintf(stderr, "oracle dispatch/combine failed\n");
        return 1;
    }

    /* compare */
    int32_t g_counts[E], g_offsets[E + 1], g_status;
    int32_t* g_pos = malloc(sizeof(int32_t) * N * K);
    int32_t* g_row_pair = malloc(sizeof(int32_t) * cap);
    uint16_t* g_out = malloc(sizeof(uint16_t) * N * HC);
    HIP_OK(hipMemcpy(g_counts, d_counts, sizeof(g_counts), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_offsets, d_offsets, sizeof(g_offsets), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&g_status, d_status, sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_pos, d_pos, sizeof(int32_t) * N * K, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_row_pair, d_row_pair, sizeof(int32_t) * cap, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_out, d_out, sizeof(uint16_t) * N * HC, hipMemcpyDeviceToHost));
    int bad = 0;
    bad |= memcmp(g_counts, counts, sizeof(counts)) != 0;
    bad |= (memcmp(g_offsets, offsets, sizeof(offsets)) != 0) << 1;
    bad |= (g_status != status) << 2;
    bad |= (memcmp(g_pos, pos, sizeof(int32_t) * N * K) != 0) << 3;
    bad |= (memcmp(g_row_pair, row_pair, sizeof(int32_t) * cap) != 0) << 4;
    for (int f = 0; f < NF; ++f) {
        uint8_t* g = malloc(row_bytes[f] * cap);
        HIP_OK(hipMemcpy(g, d_dst[f], row_bytes[f] * cap, hipMemcpyDeviceToHost));
        bad |= (memcmp(g, ref_dst[f], row_bytes[f] * cap) != 0) << (5 + f);
        free(g);
    }
    int max_ulp = 0;
    for (int i = 0; i < N * HC; ++i) {
        int d = abs(ordered(g_out[i]) - ordered(ref_out[i]));
        if (d > max_ulp) max_ulp = d;
    }
    bad |= (max_ulp > 1) << 9;
    /* the dispatch plan: every valid pair once, -1 in the other entries */
    int32_t* g_order = malloc(sizeof(int32_t) * N * K);
    int32_t* seen = calloc(N * K, sizeof(int32_t));
    HIP_OK(hipMemcpy(g_order, d_order, sizeof(int32_t) * N * K, hipMemcpyDeviceToHost));
    int n_skip = 0, n_valid = 0;
    for (int i = 0; i < N * K; ++i) {
        n_valid += pos[i] >= 0;
        if (g_order[i] < 0) { ++n_skip; continue; }
        if (g_order[i] >= N * K || pos[g_order[i]] < 0 || seen[g_order[i]]++) bad |= 1 << 10;
    }
    bad |= (n_skip != N * K - n_valid) << 10;
    bad |= (g_check[0] | g_check[1] | g_check[2] | g_check[3]) != 0 ? 1 << 11 : 0;
    if (bad) {
        fprintf(stderr, "abi_check: mismatch mask 0x%x (max combine ulp %d)\n", bad, max_ulp);
        return 1;
    }
    printf("abi_check ok: N=%d K=%d E=%d, %d out-of-range ids, %d rows used, combine max ulp %d\n",
           N, K, E, status, offsets[E], max_ulp);
    return 0;
}
