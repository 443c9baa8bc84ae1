/*
 * c_abi_roundtrip.c -- the library used from plain C, with no Python and no
 * torch: device memory comes from the HIP runtime, every stage is called
 * through include/ep.h, and the results are checked on the host against
 * properties that hold for any routing:
 *   - send_slot is a bijection from the routed (token, rank) pairs onto
 *     [0, N), and src_info of every row points back to its token;
 *   - with identity experts (y = recv_x) combine returns x for every routed
 *     token (as values: the fp32 accumulator starts at +0) and +0 elsewhere;
 *   - the grouping holds one entry per valid topk slot, each grouped row is
 *     the receive row it names, and the grouped row total is the sum of the
 *     aligned per-expert counts;
 *   - the fp8 path: the quantiser codes each group's largest magnitude as
 *     +-448; the quantising dispatch assigns the same rows as ep_dispatch and
 *     delivers the quantiser's codes and scales there, as does its cached
 *     mode; the dequantised rows are within half an E4M3 step of x.
 * Built by the package build step (gcc, C11) and run by the GPU tests.
 * Exit status 0 and a final "c abi roundtrip ok" line on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"

#define CHECK_HIP(call)                                                                   \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s:%d %s -> %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
            exit(2);                                                                      \
        }                                                                                 \
    } while (0)
#define CHECK_EP(call)                                                                    \
    do {                                                                                  \
        ep_status_t s_ = (call);                                                          \
        if (s_ != EP_OK) {                                                                \
            fprintf(stderr, "%s:%d %s -> %s\n", __FILE__, __LINE__, #call, ep_status_string(s_)); \
            exit(3);                                                                      \
        }                                                                                 \
    } while (0)
#define FAIL(...)                     \
    do {                              \
        fprintf(stderr, __VA_ARGS__); \
        fputc('\n', stderr);          \
        exit(4);                      \
    } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) { /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545f4914f6cdd1dull) >> 32);
}

static void *dev_alloc(size_t bytes) {
    void *p = NULL;
    CHECK_HIP(hipMalloc(&p, bytes > 0 ? bytes : 16));
    return p;
}

static float bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

int main(void) {
    const int T = 300, H = 256, K = 4, E = 32, R = 8, C = 5, ALIGN = 4;
    const ep_shape_t shape = {T, H, K, E, R, C, 0, ALIGN};
    const int nodes = 1;

    /* inputs: distinct experts per token, some slots masked; bf16 rows of small integers */
    int64_t *idx = malloc(sizeof(int64_t) * T * K);
    float *w = malloc(sizeof(float) * T * K);
    uint16_t *x = malloc(sizeof(uint16_t) * T * H);
    int valid_slots = 0;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < K; ++j) {
            int64_t e;
            int dup;
            do {
                e = next_u32() % E;
                dup = 0;
                for (int q = 0; q < j; ++q) dup |= idx[t * K + q] == e;
            } while (dup);
            idx[t * K + j] = (next_u32() % 10 == 0) ? -1 : e;
            w[t * K + j] = idx[t * K + j] >= 0 ? 0.25f : 0.0f;
            valid_slots += idx[t * K + j] >= 0;
        }
        for (int i = 0; i < H; ++i) {
            const float v = (float)((int)(next_u32() % 64) - 32);
            uint32_t u;
            memcpy(&u, &v, sizeof u);
            x[t * H + i] = (uint16_t)(u >> 16); /* exact: small integers */
        }
    }

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    const size_t ws_bytes = ep_workspace_bytes(&shape);
    if (ws_bytes == 0) FAIL("ep_workspace_bytes returned 0 for a valid shape");
    void *ws = dev_alloc(ws_bytes);
    CHECK_HIP(hipMemset(ws, 0, ws_bytes)); /* once, before first use */
    int64_t *d_idx = dev_alloc(sizeof(int64_t) * T * K);
    float *d_w = dev_alloc(sizeof(float) * T * K);
    void *d_x = dev_alloc(sizeof(uint16_t) * T * H);
    CHECK_HIP(hipMemcpy(d_idx, idx, sizeof(int64_t) * T * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_w, w, sizeof(float) * T * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));
    int32_t *per_rank = dev_alloc(4 * R), *per_node = dev_alloc(4 * nodes), *per_expert = dev_alloc(4 * E);
    uint8_t *in_rank = dev_alloc((size_t)T * R);
    int32_t *gbl = dev_alloc(4 * R * C), *rdma = dev_alloc(4 * nodes * C), *recv_gbl = dev_alloc(4 * R);
    int32_t *recv_rdma = dev_alloc(4 * nodes), *recv_per_expert = dev_alloc(4 * E), *num_recv = dev_alloc(4);
    int32_t *status = dev_alloc(4);
    CHECK_HIP(hipMemset(status, 0, 4));

    CHECK_EP(ep_get_layout(&shape, d_idx, per_rank, per_node, per_expert, in_rank, ws, ws_bytes, status, stream));
    int32_t n = -1;
    CHECK_EP(ep_notify(&shape, in_rank, per_rank, per_node, per_expert, gbl, rdma, recv_gbl, recv_rdma, recv_per_expert,
                       num_recv, &n, ws, ws_bytes, status, stream));
    if (n <= 0 || n > T * R) FAIL("implausible N = %d", n);

    void *recv_x = dev_alloc((size_t)n * H * 2);
    float *recv_w = dev_alloc(sizeof(float) * n * K);
    int64_t *recv_idx = dev_alloc(sizeof(int64_t) * n * K);
    int32_t *src_info = dev_alloc(8 * (size_t)n), *send_slot = dev_alloc(4 * (size_t)T * R);
    void *combined = dev_alloc((size_t)T * H * 2);
    /* dispatch from the routing inputs alone (no workspace): is_token_in_rank and the prefix sums */
    CHECK_EP(ep_dispatch(&shape, d_x, d_idx, d_w, in_rank, gbl, recv_gbl, NULL, 0, n, recv_x, recv_w, recv_idx,
                         src_info, send_slot, EP_FORM_AUTO, status, stream));
    CHECK_EP(ep_combine(&shape, recv_x, recv_w, send_slot, n, combined, NULL, status, stream));

    int32_t *h_aligned = malloc(4 * E);
    CHECK_HIP(hipMemcpyAsync(h_aligned, recv_per_expert, 4 * E, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    int m = 0;
    for (int e = 0; e < E; ++e) m += h_aligned[e];
    void *grouped_x = dev_alloc((size_t)m * H * 2);
    int32_t *grouped_row = dev_alloc(4 * (size_t)m), *num_grouped = dev_alloc(4);
    CHECK_EP(ep_group_by_expert(&shape, recv_x, 2, NULL, 0, recv_idx, recv_w, recv_gbl, recv_per_expert, n, m,
                                grouped_x, NULL, grouped_row, NULL, NULL, num_grouped, status, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    /* read everything back */
    int32_t h_status = -1, h_m = -1;
    int32_t *h_slot = malloc(4 * (size_t)T * R), *h_src = malloc(8 * (size_t)n), *h_grow = malloc(4 * (size_t)m);
    uint16_t *h_comb = malloc(2 * (size_t)T * H), *h_recv = malloc(2 * (size_t)n * H), *h_gx = malloc(2 * (size_t)m * H);
    CHECK_HIP(hipMemcpy(&h_status, status, 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&h_m, num_grouped, 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_slot, send_slot, 4 * (size_t)T * R, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_src, src_info, 8 * (size_t)n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_comb, combined, 2 * (size_t)T * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_recv, recv_x, 2 * (size_t)n * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_grow, grouped_row, 4 * (size_t)m, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_gx, grouped_x, 2 * (size_t)m * H, hipMemcpyDeviceToHost));
    if (h_status != 0) FAIL("device status %d", h_status);

    /* send_slot: a bijection onto [0, n); src_info points back */
    char *seen = calloc((size_t)n, 1);
    for (int t = 0; t < T; ++t) {
        int routed = 0;
        for (int r = 0; r < R; ++r) {
            int on = 0;
            for (int j = 0; j < K; ++j) on |= idx[t * K + j] >= 0 && idx[t * K + j] / (E / R) == r;
            const int s = h_slot[t * R + r];
            if (on != (s >= 0)) FAIL("send_slot[%d][%d] = %d disagrees with the routing", t, r, s);
            if (s < 0) continue;
            routed = 1;
            if (s >= n || seen[s]) FAIL("send_slot[%d][%d] = %d repeated or out of range", t, r, s);
            seen[s] = 1;
            if (h_src[2 * s + 1] != t) FAIL("src_info of row %d names token %d, not %d", s, h_src[2 * s + 1], t);
        }
        /* identity experts: combined row = x (weights of a routed token sum to 0.25 * slots on each rank,
           so compare against sum_r W_r * x = (0.25 * valid slots) * x) */
        int vs = 0;
        for (int j = 0; j < K; ++j) vs += idx[t * K + j] >= 0;
        for (int i = 0; i < H; ++i) {
            const float want = routed ? 0.25f * (float)vs * bf16_value(x[t * H + i]) : 0.0f;
            if (bf16_value(h_comb[t * H + i]) != want)
                FAIL("combined[%d][%d] = %g, want %g", t, i, bf16_value(h_comb[t * H + i]), want);
        }
    }
    for (int s = 0; s < n; ++s)
        if (!seen[s]) FAIL("row %d never assigned", s);

    /* grouping: one entry per valid slot, rows copied bit for bit, padding zero */
    if (h_m != m) FAIL("num_grouped_rows %d, want %d", h_m, m);
    int entries = 0;
    for (int g = 0; g < m; ++g) {
        const int row = h_grow[g];
        if (row < -1 || row >= n) FAIL("grouped_row[%d] = %d", g, row);
        if (row >= 0) ++entries;
        for (int i = 0; i < H; ++i) {
            const uint16_t want = row >= 0 ? h_recv[(size_t)row * H + i] : 0;
            if (h_gx[(size_t)g * H + i] != want) FAIL("grouped_x[%d][%d] differs from its receive row", g, i);
        }
    }
    if (entries != valid_slots) FAIL("%d grouped entries, %d valid slots", entries, valid_slots);

    /* the fp8 path: quantiser, quantising dispatch (and its cached mode), dequantiser */
    const int S = H / 128;
    uint8_t *d_q = dev_alloc((size_t)T * H), *d_rq = dev_alloc((size_t)n * H), *d_cq = dev_alloc((size_t)n * H);
    float *d_qs = dev_alloc(4 * (size_t)T * S), *d_rs = dev_alloc(4 * (size_t)n * S), *d_cs = dev_alloc(4 * (size_t)n * S);
    int32_t *send_slot8 = dev_alloc(4 * (size_t)T * R);
    void *back = dev_alloc((size_t)n * H * 2);
    CHECK_EP(ep_quantize_fp8(d_x, T, H, S, d_q, d_qs, stream));
    CHECK_EP(ep_dispatch_to_fp8(&shape, d_x, S, d_idx, d_w, in_rank, gbl, recv_gbl, ws, ws_bytes, n, d_rq, d_rs, recv_w,
                                recv_idx, src_info, send_slot8, status, stream));
    CHECK_EP(ep_dispatch_cached_to_fp8(&shape, d_x, S, send_slot8, n, d_cq, d_cs, status, stream));
    CHECK_EP(ep_dequantize_fp8(d_rq, d_rs, n, H, S, back, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    uint8_t *h_q = malloc((size_t)T * H), *h_rq = malloc((size_t)n * H), *h_cq = malloc((size_t)n * H);
    float *h_qs = malloc(4 * (size_t)T * S), *h_rs = malloc(4 * (size_t)n * S), *h_cs = malloc(4 * (size_t)n * S);
    int32_t *h_slot8 = malloc(4 * (size_t)T * R);
    uint16_t *h_back = malloc(2 * (size_t)n * H);
    CHECK_HIP(hipMemcpy(h_q, d_q, (size_t)T * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_rq, d_rq, (size_t)n * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_cq, d_cq, (size_t)n * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_qs, d_qs, 4 * (size_t)T * S, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_rs, d_rs, 4 * (size_t)n * S, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_cs, d_cs, 4 * (size_t)n * S, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_slot8, send_slot8, 4 * (size_t)T * R, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_back, back, 2 * (size_t)n * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&h_status, status, 4, hipMemcpyDeviceToHost));
    if (h_status != 0) FAIL("device status %d after the fp8 path", h_status);
    for (int t = 0; t < T; ++t) {
        for (int q = 0; q < S; ++q) { /* the group's largest magnitude (first one) is coded +-448 */
            int at = q * 128;
            for (int i = q * 128; i < (q + 1) * 128; ++i)
                if (fabsf(bf16_value(x[t * H + i])) > fabsf(bf16_value(x[t * H + at]))) at = i;
            if (bf16_value(x[t * H + at]) != 0.0f && (h_q[(size_t)t * H + at] & 0x7f) != 0x7e)
                FAIL("quantiser: largest magnitude of token %d group %d coded 0x%02x", t, q, h_q[(size_t)t * H + at]);
        }
        for (int r = 0; r < R; ++r) {
            const int s = h_slot8[t * R + r];
            if (s != h_slot[t * R + r]) FAIL("quantising dispatch: send_slot[%d][%d] = %d, ep_dispatch %d", t, r, s,
                                             h_slot[t * R + r]);
            if (s < 0) continue;
            if (memcmp(h_rq + (size_t)s * H, h_q + (size_t)t * H, H) || memcmp(h_cq + (size_t)s * H, h_q + (size_t)t * H, H))
                FAIL("row %d does not hold token %d's codes", s, t);
            if (memcmp(h_rs + (size_t)s * S, h_qs + (size_t)t * S, 4 * S) ||
                memcmp(h_cs + (size_t)s * S, h_qs + (size_t)t * S, 4 * S))
                FAIL("row %d does not hold token %d's scales", s, t);
            for (int i = 0; i < H; ++i) { /* half an E4M3 step (1/16) plus the bf16 rounding (1/256) */
                const float xv = bf16_value(x[t * H + i]), bv = bf16_value(h_back[(size_t)s * H + i]);
                if (fabsf(bv - xv) > fabsf(xv) * (1.0f / 16 + 1.0f / 256) + 1e-6f)
                    FAIL("dequantised row %d channel %d = %g, x = %g", s, i, bv, xv);
            }
        }
    }

    /* host-side argument checks answer without touching the device */
    ep_shape_t bad = shape;
    bad.num_ranks = 3; /* not a multiple of 8 and E % R != 0 */
    if (ep_get_layout(&bad, d_idx, per_rank, per_node, per_expert, in_rank, ws, ws_bytes, NULL, stream) !=
        EP_ERR_INVALID_ARG)
        FAIL("malformed shape accepted");

    printf("c abi roundtrip ok: t=%d N=%d grouped rows=%d entries=%d\n", T, n, m, entries);
    return 0;
}
