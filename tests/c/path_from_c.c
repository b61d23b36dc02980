/* The whole flat path driven from plain C99 through libep.so, with device
 * buffers from the HIP runtime's C API and one caller-created stream:
 * ep_get_layout -> ep_dispatch -> ep_combine (identity expert: the combine
 * reads the dispatched rows back). The results are compared bit for bit with
 * the CPU oracle (liboracle.so, test infrastructure), called from the same
 * program. Inputs come from a fixed xorshift generator: ids in [-1, E) with
 * repeats, bf16 rows in [-2, 2), weights in [0, 1).
 * Prints one line per step and exits non-zero on the first mismatch. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"

/* oracle/oracle.c (no header: test infrastructure) */
int oracle_layout(int T, int K, int E, int R, int G, const int64_t *topk_idx, int32_t *tokens_per_expert,
                  int32_t *tokens_per_rank, int32_t *tokens_per_group, int32_t *expert_offsets,
                  int32_t *rank_offsets, int32_t *group_offsets, uint8_t *in_rank, uint8_t *in_group,
                  int32_t *slot, int32_t *group_slot, uint32_t *err);
void oracle_dispatch(int T, int H, int K, int E, int R, const int64_t *topk_idx, const float *topk_w,
                     const uint16_t *x, const uint8_t *x_fp8, const float *x_scales,
                     const int32_t *rank_offsets, int64_t capacity, uint16_t *recv_x, uint8_t *recv_fp8,
                     float *recv_scales, int32_t *recv_src, int32_t *recv_topk_idx, float *recv_topk_w,
                     uint32_t *err);
void oracle_combine(int T, int H, int K, const int32_t *slot, const float *topk_w, const uint8_t *y,
                    int64_t y_rows, int64_t row_stride, int chunked, uint32_t epoch, uint16_t *out,
                    uint32_t *err);

#define T 1000
#define H 512
#define K 4
#define E 32
#define R 8

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 32);
}
static float next_unit(void) { return (float)(next_u32() >> 8) / 16777216.0f; }

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));                \
            return 1;                                                             \
        }                                                                         \
    } while (0)
#define EP_OK_(call)                                                              \
    do {                                                                          \
        int r_ = (call);                                                          \
        if (r_ != EP_OK) {                                                        \
            printf("FAIL %s: %s\n", #call, ep_status_string(r_));                 \
            return 1;                                                             \
        }                                                                         \
    } while (0)

static int same(const char *what, const void *a, const void *b, size_t bytes) {
    int ok = memcmp(a, b, bytes) == 0;
    printf("%s %s\n", ok ? "ok" : "FAIL", what);
    return ok;
}

int main(void) {
    static int64_t ids[T * K];
    static float w[T * K];
    static uint16_t x[T * H];
    for (int i = 0; i < T * K; i++) {
        ids[i] = (int64_t)(next_u32() % (E + 1)) - 1;
        w[i] = next_unit();
    }
    for (int i = 0; i < T * H; i++) {
        float f = next_unit() * 4.0f - 2.0f;
        uint32_t u;
        memcpy(&u, &f, 4);
        x[i] = (uint16_t)(u >> 16);
    }

    /* oracle */
    static int32_t o_tpe[E], o_tpr[R], o_tpg[1], o_eo[E + 1], o_ro[R + 1], o_go[2], o_slot[T * K],
        o_gslot[T * K];
    static uint8_t o_in_rank[T * R], o_in_group[T];
    uint32_t o_err = 0;
    if (oracle_layout(T, K, E, R, 1, ids, o_tpe, o_tpr, o_tpg, o_eo, o_ro, o_go, o_in_rank, o_in_group,
                      o_slot, o_gslot, &o_err) != 0) {
        printf("FAIL oracle_layout\n");
        return 1;
    }
    const int N = o_ro[R];
    uint16_t *o_recv = malloc(sizeof(uint16_t) * (size_t)N * H);
    int32_t *o_src = malloc(sizeof(int32_t) * (size_t)N);
    int32_t *o_ridx = malloc(sizeof(int32_t) * (size_t)N * K);
    float *o_rw = malloc(sizeof(float) * (size_t)N * K);
    static uint16_t o_out[T * H];
    oracle_dispatch(T, H, K, E, R, ids, w, x, NULL, NULL, o_ro, N, o_recv, NULL, NULL, o_src, o_ridx, o_rw,
                    &o_err);
    oracle_combine(T, H, K, o_slot, w, (const uint8_t *)o_recv, N, 2 * H, 0, 0, o_out, &o_err);
    printf("oracle done: %d receive rows\n", N);

    /* device */
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    ep_shape s = {T, H, K, E, R, 1};
    size_t ws_bytes = ep_workspace_bytes(&s);
    void *ws;
    int64_t *d_ids;
    float *d_w;
    uint16_t *d_x, *d_recv, *d_out;
    int32_t *d_tpe, *d_tpr, *d_eo, *d_ro, *d_slot, *d_src, *d_ridx;
    float *d_rw;
    uint8_t *d_in_rank;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    HIP_OK(hipMalloc((void **)&d_ids, sizeof ids));
    HIP_OK(hipMalloc((void **)&d_w, sizeof w));
    HIP_OK(hipMalloc((void **)&d_x, sizeof x));
    HIP_OK(hipMalloc((void **)&d_out, sizeof o_out));
    HIP_OK(hipMalloc((void **)&d_tpe, sizeof o_tpe));
    HIP_OK(hipMalloc((void **)&d_tpr, sizeof o_tpr));
    HIP_OK(hipMalloc((void **)&d_eo, sizeof o_eo));
    HIP_OK(hipMalloc((void **)&d_ro, sizeof o_ro));
    HIP_OK(hipMalloc((void **)&d_slot, sizeof o_slot));
    HIP_OK(hipMalloc((void **)&d_in_rank, sizeof o_in_rank));
    HIP_OK(hipMemcpy(d_ids, ids, sizeof ids, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));

    ep_layout L;
    memset(&L, 0, sizeof L);
    L.tokens_per_expert = d_tpe;
    L.tokens_per_rank = d_tpr;
    L.expert_offsets = d_eo;
    L.rank_offsets = d_ro;
    L.is_token_in_rank = d_in_rank;
    L.slot = d_slot;
    EP_OK_(ep_get_layout(&s, d_ids, &L, ws, ws_bytes, st));
    int32_t ro[R + 1];
    HIP_OK(hipMemcpyAsync(ro, d_ro, sizeof ro, hipMemcpyDeviceToHost, st));
    HIP_OK(hipStreamSynchronize(st));
    printf("layout done: %d receive rows\n", ro[R]);
    if (ro[R] != N) {
        printf("FAIL receive rows %d != %d\n", ro[R], N);
        return 1;
    }

    HIP_OK(hipMalloc((void **)&d_recv, sizeof(uint16_t) * (size_t)N * H));
    HIP_OK(hipMalloc((void **)&d_src, sizeof(int32_t) * (size_t)N));
    HIP_OK(hipMalloc((void **)&d_ridx, sizeof(int32_t) * (size_t)N * K));
    HIP_OK(hipMalloc((void **)&d_rw, sizeof(float) * (size_t)N * K));
    ep_tokens tk = {d_x, NULL, NULL, d_ids, d_w};
    ep_recv rv = {d_recv, NULL, NULL, d_src, d_ridx, d_rw, N};
    EP_OK_(ep_dispatch(&s, &L, &tk, &rv, ws, ws_bytes, st));
    EP_OK_(ep_combine(&s, &L, d_recv, N, 2 * H, EP_FMT_PLAIN, 0, d_w, d_out, ws, ws_bytes, st));
    uint32_t bits = 0;
    EP_OK_(ep_check_errors(ws, st, &bits));
    printf("path done: device error bits %u\n", bits);

    static int32_t g_tpe[E], g_tpr[R], g_eo[E + 1], g_slot[T * K];
    static uint8_t g_in_rank[T * R];
    static uint16_t g_out[T * H];
    uint16_t *g_recv = malloc(sizeof(uint16_t) * (size_t)N * H);
    int32_t *g_src = malloc(sizeof(int32_t) * (size_t)N);
    int32_t *g_ridx = malloc(sizeof(int32_t) * (size_t)N * K);
    float *g_rw = malloc(sizeof(float) * (size_t)N * K);
    HIP_OK(hipMemcpy(g_tpe, d_tpe, sizeof g_tpe, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_tpr, d_tpr, sizeof g_tpr, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_eo, d_eo, sizeof g_eo, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_slot, d_slot, sizeof g_slot, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_in_rank, d_in_rank, sizeof g_in_rank, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_recv, d_recv, sizeof(uint16_t) * (size_t)N * H, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_src, d_src, sizeof(int32_t) * (size_t)N, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_ridx, d_ridx, sizeof(int32_t) * (size_t)N * K, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_rw, d_rw, sizeof(float) * (size_t)N * K, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_out, d_out, sizeof g_out, hipMemcpyDeviceToHost));

    int ok = 1;
    ok &= same("tokens_per_expert", g_tpe, o_tpe, sizeof o_tpe);
    ok &= same("tokens_per_rank", g_tpr, o_tpr, sizeof o_tpr);
    ok &= same("expert_offsets", g_eo, o_eo, sizeof o_eo);
    ok &= same("rank_offsets", ro, o_ro, sizeof o_ro);
    ok &= same("is_token_in_rank", g_in_rank, o_in_rank, sizeof o_in_rank);
    ok &= same("slot", g_slot, o_slot, sizeof o_slot);
    ok &= same("recv_x", g_recv, o_recv, sizeof(uint16_t) * (size_t)N * H);
    ok &= same("recv_src", g_src, o_src, sizeof(int32_t) * (size_t)N);
    ok &= same("recv_topk_idx", g_ridx, o_ridx, sizeof(int32_t) * (size_t)N * K);
    ok &= same("recv_topk_weights", g_rw, o_rw, sizeof(float) * (size_t)N * K);
    ok &= same("combine out", g_out, o_out, sizeof o_out);
    uint32_t want_bits = o_err;  /* ids are in [-1, E): no error expected on either side */
    if (bits != want_bits) {
        printf("FAIL error bits %u != %u\n", bits, want_bits);
        ok = 0;
    }
    HIP_OK(hipStreamDestroy(st));
    printf("%s\n", ok ? "path ok" : "path FAILED");
    return ok ? 0 : 1;
}
