/* The path driven from plain C99 through libep.so, with device buffers from
 * the HIP runtime's C API and one caller-created stream:
 *   flat: ep_get_layout -> ep_dispatch -> ep_combine (identity expert: the
 *         combine reads the dispatched rows back);
 *   two-level (2 groups of 4 ranks): ep_get_layout with groups ->
 *         ep_hierarchical_dispatch (both steps) -> ep_combine on the chunked
 *         rows and ep_combine_two_level; the fused one-launch two-level
 *         dispatch; the allocation-free layout;
 *   several sources: ep_source_layout -> ep_source_dispatch_fused (send and
 *         copy epilogue in one launch), whose dense rows equal the flat
 *         dispatch's.
 * The results are compared bit for bit with the CPU oracle (liboracle.so,
 * test infrastructure), called from the same program. Inputs come from a fixed xorshift generator: ids in [-1, E) with
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
int oracle_hier_dispatch(int T, int H, int K, int E, int R, int G, const int64_t *topk_idx,
                         const float *topk_w, const uint16_t *x, const uint8_t *x_fp8,
                         const float *x_scales, const int32_t *slot, const int32_t *group_offsets,
                         uint32_t epoch, uint8_t *group_buf, int64_t group_cap, uint8_t *peer_buf,
                         int64_t peer_cap, int steps, uint32_t *err);
int oracle_source_counts(int T, int K, int E, int R, int S, const int64_t *topk_idx, int32_t *counts,
                         int32_t *recv_offsets);
void oracle_combine_two_level(int T, int H, int K, int E, int R, int G, const int64_t *topk_idx,
                              const int32_t *slot, const int32_t *group_slot, const float *topk_w,
                              const uint8_t *y, int64_t y_rows, int64_t row_stride, int chunked,
                              uint32_t epoch, uint8_t *group_buf, int64_t group_cap, int steps,
                              uint16_t *out, uint32_t *err);

#define T 1000
#define H 512
#define K 4
#define E 32
#define R 8
#define G2 2
#define EPOCH 7u

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
    /* error reporting: an invalid id makes ep_check_errors return
     * EP_ERR_DEVICE with the id bit; a clean pass after it clears word 0,
     * while word 1 keeps the bit until ep_clear_errors. */
    {
        const int64_t bad_id = E + 3, good_id = ids[5];
        uint32_t b0 = 99, b1 = 99;
        EP_OK_(ep_clear_errors(ws, st));
        HIP_OK(hipMemcpy(d_ids + 5, &bad_id, sizeof bad_id, hipMemcpyHostToDevice));
        EP_OK_(ep_get_layout(&s, d_ids, &L, ws, ws_bytes, st));
        int rc = ep_check_errors(ws, st, &b0);
        ok &= rc == EP_ERR_DEVICE && b0 == EP_DEVERR_EXPERT_ID;
        printf("%s invalid id: status %d, bits %u\n", rc == EP_ERR_DEVICE && b0 == EP_DEVERR_EXPERT_ID ? "ok" : "FAIL",
               rc, b0);
        HIP_OK(hipMemcpy(d_ids + 5, &good_id, sizeof good_id, hipMemcpyHostToDevice));
        EP_OK_(ep_get_layout(&s, d_ids, &L, ws, ws_bytes, st));
        rc = ep_check_errors(ws, st, &b0);
        const int rc1 = ep_check_sticky_errors(ws, st, &b1);
        const int pass_ok = rc == EP_OK && b0 == 0 && rc1 == EP_ERR_DEVICE && b1 == EP_DEVERR_EXPERT_ID;
        ok &= pass_ok;
        printf("%s clean pass after it: status %d bits %u, since clear: status %d bits %u\n",
               pass_ok ? "ok" : "FAIL", rc, b0, rc1, b1);
        EP_OK_(ep_clear_errors(ws, st));
        rc = ep_check_sticky_errors(ws, st, &b1);
        ok &= rc == EP_OK && b1 == 0;
        printf("%s cleared: status %d bits %u\n", rc == EP_OK && b1 == 0 ? "ok" : "FAIL", rc, b1);
    }
    /* the allocation-free layout: same outputs, error words in ws */
    {
        static int32_t n_tpr[R], n_ro[R + 1], n_slot[T * K];
        int32_t *dn_tpr, *dn_ro, *dn_slot;
        HIP_OK(hipMalloc((void **)&dn_tpr, sizeof n_tpr));
        HIP_OK(hipMalloc((void **)&dn_ro, sizeof n_ro));
        HIP_OK(hipMalloc((void **)&dn_slot, sizeof n_slot));
        ep_layout Ln;
        memset(&Ln, 0, sizeof Ln);
        Ln.tokens_per_rank = dn_tpr;
        Ln.rank_offsets = dn_ro;
        Ln.slot = dn_slot;
        EP_OK_(ep_get_layout_noalloc(&s, d_ids, &Ln, (uint32_t *)ws, st));
        uint32_t bn = 99;
        EP_OK_(ep_check_errors(ws, st, &bn));
        HIP_OK(hipMemcpy(n_tpr, dn_tpr, sizeof n_tpr, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(n_ro, dn_ro, sizeof n_ro, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(n_slot, dn_slot, sizeof n_slot, hipMemcpyDeviceToHost));
        ok &= same("noalloc tokens_per_rank", n_tpr, o_tpr, sizeof o_tpr);
        ok &= same("noalloc rank_offsets", n_ro, o_ro, sizeof o_ro);
        ok &= same("noalloc slot", n_slot, o_slot, sizeof o_slot);
        ok &= bn == 0;
    }
    /* several sources (S3 source ranks): source layout, then the send and the
     * copy epilogue in one launch; the dense rows equal the flat dispatch's */
    {
        enum { S3 = 3 };
        static int32_t c_counts[S3 * R], c_offs[R * S3 + 1];
        if (oracle_source_counts(T, K, E, R, S3, ids, c_counts, c_offs) != 0) {
            printf("FAIL oracle_source_counts\n");
            return 1;
        }
        int cap = 1;
        for (int i = 0; i < S3 * R; i++) cap = c_counts[i] > cap ? c_counts[i] : cap;
        size_t ws3_bytes = ep_source_workspace_bytes(&s, S3);
        const int64_t stride3 = ep_chunked_record_bytes(&s, EP_SEG_BF16);
        void *ws3;
        int32_t *d3_counts, *d3_offs, *d3_sslot, *d3_src, *d3_ridx;
        uint8_t *d3_staging;
        uint16_t *d3_recv;
        float *d3_rw;
        HIP_OK(hipMalloc(&ws3, ws3_bytes));
        HIP_OK(hipMalloc((void **)&d3_counts, sizeof c_counts));
        HIP_OK(hipMalloc((void **)&d3_offs, sizeof c_offs));
        HIP_OK(hipMalloc((void **)&d3_sslot, sizeof(int32_t) * T * K));
        HIP_OK(hipMalloc((void **)&d3_staging, (size_t)R * S3 * cap * stride3));
        HIP_OK(hipMalloc((void **)&d3_recv, sizeof(uint16_t) * (size_t)N * H));
        HIP_OK(hipMalloc((void **)&d3_src, sizeof(int32_t) * (size_t)N));
        HIP_OK(hipMalloc((void **)&d3_ridx, sizeof(int32_t) * (size_t)N * K));
        HIP_OK(hipMalloc((void **)&d3_rw, sizeof(float) * (size_t)N * K));
        ep_sources src3 = {S3, cap, d3_counts, d3_offs, d3_sslot};
        ep_recv rv3 = {d3_recv, NULL, NULL, d3_src, d3_ridx, d3_rw, N};
        EP_OK_(ep_source_layout(&s, d_ids, &src3, ws3, ws3_bytes, st));
        EP_OK_(ep_source_dispatch_fused(&s, &src3, &tk, EPOCH, d3_staging, &rv3, ws3, ws3_bytes, st));
        uint32_t b3 = 99;
        EP_OK_(ep_check_errors(ws3, st, &b3));
        static int32_t g3_offs[R * S3 + 1];
        HIP_OK(hipMemcpy(g3_offs, d3_offs, sizeof g3_offs, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_recv, d3_recv, sizeof(uint16_t) * (size_t)N * H, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_src, d3_src, sizeof(int32_t) * (size_t)N, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_ridx, d3_ridx, sizeof(int32_t) * (size_t)N * K, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_rw, d3_rw, sizeof(float) * (size_t)N * K, hipMemcpyDeviceToHost));
        ok &= same("sources: recv_offsets", g3_offs, c_offs, sizeof c_offs);
        ok &= same("sources, one launch: recv_x", g_recv, o_recv, sizeof(uint16_t) * (size_t)N * H);
        ok &= same("sources, one launch: recv_src", g_src, o_src, sizeof(int32_t) * (size_t)N);
        ok &= same("sources, one launch: recv_topk_idx", g_ridx, o_ridx, sizeof(int32_t) * (size_t)N * K);
        ok &= same("sources, one launch: recv_topk_weights", g_rw, o_rw, sizeof(float) * (size_t)N * K);
        ok &= b3 == 0;
    }
    /* two-level path on the same tokens, R ranks in G2 groups */
    {
        static int32_t p_tpe[E], p_tpr[R], p_tpg[G2], p_eo[E + 1], p_ro[R + 1], p_go[G2 + 1], p_slot[T * K],
            p_gslot[T * K];
        static uint8_t p_in_rank[T * R], p_in_group[T * G2];
        uint32_t p_err = 0;
        if (oracle_layout(T, K, E, R, G2, ids, p_tpe, p_tpr, p_tpg, p_eo, p_ro, p_go, p_in_rank, p_in_group,
                          p_slot, p_gslot, &p_err) != 0) {
            printf("FAIL oracle_layout with groups\n");
            return 1;
        }
        ep_shape s2 = {T, H, K, E, R, G2};
        const int64_t stride = ep_chunked_record_bytes(&s2, EP_SEG_BF16);
        const int64_t pstride = ep_partial_row_bytes(&s2);
        const int GR = p_go[G2], N2 = p_ro[R];
        uint8_t *o_gbuf = calloc((size_t)GR, (size_t)stride), *o_pbuf = calloc((size_t)N2, (size_t)stride);
        uint8_t *o_part = calloc((size_t)GR, (size_t)pstride);
        static uint16_t o_out2[T * H], o_out3[T * H], g_out2[T * H], g_out3[T * H];
        oracle_hier_dispatch(T, H, K, E, R, G2, ids, w, x, NULL, NULL, p_slot, p_go, EPOCH, o_gbuf, GR, o_pbuf,
                             N2, 3, &p_err);
        oracle_combine(T, H, K, p_slot, w, o_pbuf, N2, stride, 1, EPOCH, o_out2, &p_err);
        oracle_combine_two_level(T, H, K, E, R, G2, ids, p_slot, p_gslot, w, o_pbuf, N2, stride, 1, EPOCH,
                                 o_part, GR, 3, o_out3, &p_err);
        printf("oracle two-level done: %d group rows, %d peer rows\n", GR, N2);

        size_t ws2_bytes = ep_workspace_bytes(&s2);
        void *ws2;
        int32_t *d2_tpg, *d2_go, *d2_slot, *d2_gslot, *d2_ro;
        uint8_t *d2_gbuf, *d2_pbuf, *d2_part;
        uint16_t *d2_out;
        HIP_OK(hipMalloc(&ws2, ws2_bytes));
        HIP_OK(hipMalloc((void **)&d2_tpg, sizeof p_tpg));
        HIP_OK(hipMalloc((void **)&d2_go, sizeof p_go));
        HIP_OK(hipMalloc((void **)&d2_ro, sizeof p_ro));
        HIP_OK(hipMalloc((void **)&d2_slot, sizeof p_slot));
        HIP_OK(hipMalloc((void **)&d2_gslot, sizeof p_gslot));
        HIP_OK(hipMalloc((void **)&d2_gbuf, (size_t)GR * stride));
        HIP_OK(hipMalloc((void **)&d2_pbuf, (size_t)N2 * stride));
        HIP_OK(hipMalloc((void **)&d2_part, (size_t)GR * pstride));
        HIP_OK(hipMalloc((void **)&d2_out, sizeof g_out2));
        HIP_OK(hipMemset(d2_gbuf, 0, (size_t)GR * stride));
        HIP_OK(hipMemset(d2_pbuf, 0, (size_t)N2 * stride));
        HIP_OK(hipMemset(d2_part, 0, (size_t)GR * pstride));
        ep_layout L2;
        memset(&L2, 0, sizeof L2);
        L2.tokens_per_group = d2_tpg;
        L2.group_offsets = d2_go;
        L2.rank_offsets = d2_ro;
        L2.slot = d2_slot;
        L2.group_slot = d2_gslot;
        EP_OK_(ep_get_layout(&s2, d_ids, &L2, ws2, ws2_bytes, st));
        EP_OK_(ep_hierarchical_dispatch(&s2, &L2, &tk, EPOCH, EP_HIER_SCALEOUT | EP_HIER_FORWARD, d2_gbuf, GR,
                                        d2_pbuf, N2, ws2, ws2_bytes, st));
        EP_OK_(ep_combine(&s2, &L2, d2_pbuf, N2, stride, EP_FMT_CHUNKED, EPOCH, d_w, d2_out, ws2, ws2_bytes, st));
        HIP_OK(hipMemcpyAsync(g_out2, d2_out, sizeof g_out2, hipMemcpyDeviceToHost, st));
        EP_OK_(ep_combine_two_level(&s2, &L2, d_ids, d2_pbuf, N2, stride, EP_FMT_CHUNKED, EPOCH, d_w, d2_part,
                                    GR, 3, d2_out, ws2, ws2_bytes, st));
        HIP_OK(hipMemcpyAsync(g_out3, d2_out, sizeof g_out3, hipMemcpyDeviceToHost, st));
        uint32_t bits2 = 0;
        EP_OK_(ep_check_errors(ws2, st, &bits2));
        printf("two-level path done: device error bits %u\n", bits2);
        static int32_t g2_tpg[G2], g2_go[G2 + 1], g2_gslot[T * K];
        uint8_t *g_gbuf = malloc((size_t)GR * stride), *g_pbuf = malloc((size_t)N2 * stride);
        uint8_t *g_part = malloc((size_t)GR * pstride);
        HIP_OK(hipMemcpy(g2_tpg, d2_tpg, sizeof g2_tpg, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g2_go, d2_go, sizeof g2_go, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g2_gslot, d2_gslot, sizeof g2_gslot, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_gbuf, d2_gbuf, (size_t)GR * stride, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_pbuf, d2_pbuf, (size_t)N2 * stride, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_part, d2_part, (size_t)GR * pstride, hipMemcpyDeviceToHost));
        ok &= same("tokens_per_group", g2_tpg, p_tpg, sizeof p_tpg);
        ok &= same("group_offsets", g2_go, p_go, sizeof p_go);
        ok &= same("group_slot", g2_gslot, p_gslot, sizeof p_gslot);
        ok &= same("group rows (scale-out step)", g_gbuf, o_gbuf, (size_t)GR * stride);
        ok &= same("peer rows (forward step)", g_pbuf, o_pbuf, (size_t)N2 * stride);
        ok &= same("combine out, chunked rows", g_out2, o_out2, sizeof o_out2);
        ok &= same("two-level partial rows", g_part, o_part, (size_t)GR * pstride);
        ok &= same("two-level combine out", g_out3, o_out3, sizeof o_out3);
        /* the fused one-launch form (16-token batches), fresh buffers, next epoch */
        {
            uint8_t *o_gbuf2 = calloc((size_t)GR, (size_t)stride), *o_pbuf2 = calloc((size_t)N2, (size_t)stride);
            uint32_t f_err = 0;
            oracle_hier_dispatch(T, H, K, E, R, G2, ids, w, x, NULL, NULL, p_slot, p_go, EPOCH + 1, o_gbuf2, GR,
                                 o_pbuf2, N2, 3, &f_err);
            HIP_OK(hipMemset(d2_gbuf, 0, (size_t)GR * stride));
            HIP_OK(hipMemset(d2_pbuf, 0, (size_t)N2 * stride));
            ep_fused_opts fo;
            memset(&fo, 0, sizeof fo);
            fo.tile_tokens = 16;
            EP_OK_(ep_hierarchical_dispatch_fused(&s2, &L2, &tk, EPOCH + 1, d2_gbuf, GR, d2_pbuf, N2, &fo, ws2,
                                                  ws2_bytes, st));
            uint32_t fb = 99;
            EP_OK_(ep_check_errors(ws2, st, &fb));
            HIP_OK(hipMemcpy(g_gbuf, d2_gbuf, (size_t)GR * stride, hipMemcpyDeviceToHost));
            HIP_OK(hipMemcpy(g_pbuf, d2_pbuf, (size_t)N2 * stride, hipMemcpyDeviceToHost));
            ok &= same("fused group rows", g_gbuf, o_gbuf2, (size_t)GR * stride);
            ok &= same("fused peer rows", g_pbuf, o_pbuf2, (size_t)N2 * stride);
            ok &= fb == 0 && f_err == 0;
            /* ring mode: one-token batches, group rows through a ring of 65 batches */
            f_err = 0;
            oracle_hier_dispatch(T, H, K, E, R, G2, ids, w, x, NULL, NULL, p_slot, p_go, EPOCH + 2, o_gbuf2, GR,
                                 o_pbuf2, N2, 3, &f_err);
            HIP_OK(hipMemset(d2_pbuf, 0, (size_t)N2 * stride));
            memset(&fo, 0, sizeof fo);
            fo.tile_tokens = 1;
            fo.ring_batches = 65;
            EP_OK_(ep_hierarchical_dispatch_fused(&s2, &L2, &tk, EPOCH + 2, d2_gbuf, GR, d2_pbuf, N2, &fo, ws2,
                                                  ws2_bytes, st));
            fb = 99;
            EP_OK_(ep_check_errors(ws2, st, &fb));
            HIP_OK(hipMemcpy(g_pbuf, d2_pbuf, (size_t)N2 * stride, hipMemcpyDeviceToHost));
            ok &= same("fused peer rows, ring of 65 batches", g_pbuf, o_pbuf2, (size_t)N2 * stride);
            ok &= fb == 0 && f_err == 0;
        }
        if (bits2 != p_err) {
            printf("FAIL two-level error bits %u != %u\n", bits2, p_err);
            ok = 0;
        }
    }

    HIP_OK(hipStreamDestroy(st));
    printf("%s\n", ok ? "path ok" : "path FAILED");
    return ok ? 0 : 1;
}
