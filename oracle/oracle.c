/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for the expert-parallel
 * MoE dispatch / combine path (layout, dispatch, two-level dispatch with
 * 512 B data-as-flag chunks, weighted combine).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the HIP implementation, and the HIP
 * implementation never calls it.
 *
 * Sources (web pages; cited by title and section):
 *   [V2]   "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK 复制机制"
 *          §3.3 阶段1 (notify warps: expert counts, rank dedup, prefix sum),
 *          §3.3 阶段2 (dispatch warps: per-token copy, rank -> slot),
 *          §3.4 (TokenLayout: hidden | sf | metadata, 16 B aligned pieces),
 *          §3.5 (inputs x / topk_idx / topk_weights, outputs recv_*),
 *          §3.6 (hybrid dispatch: scale-out write, then forward).
 *   [PIPE] "07: DeepEP Intra/Inter-node 协调 — NVLink Scale-up + RDMA
 *          Scale-out 三阶段流水线的代码实证": hybrid scale-out stage (one
 *          store per destination group), forward warps (scale-up rank =
 *          expert / experts_per_rank), is_nvlink_accessible (rank numbering).
 *   [ASC]  "Ascend Send Ordering": 导言 and 能省多少，又不能省什么 (512 B
 *          block = 480 B payload + 32 B flag; blocks = ceil(P / 480)).
 *   [MEGA] "06_06: NVLink Scale-up + RDMA Scale-out — DeepEP 三阶段流水线 vs
 *          DeepGEMM 对称内存": combine write of BF16 expert outputs.
 *
 * Readings where the pages leave a step open (all deterministic):
 *   - Receive rows inside one destination region follow ascending source
 *     token: the order a single dispatch warp walking tokens in order would
 *     produce with its atomic counter ([V2] §3.3 阶段2).
 *   - Destination regions are compact and laid end to end in rank order,
 *     starting at the exclusive prefix sum of the per-rank counts.
 *   - Expert id -1 means "no expert"; any other id outside [0, E) sets
 *     error bit 0 and is then treated as -1.
 *   - slot[t][k] is the absolute receive row of (t, rank of k) for every
 *     valid k (repeated ranks share a row), -1 for skipped k.
 *   - The chunk flag is 32 B = eight u32 words, each equal to the caller's
 *     epoch (>= 1); a chunk is accepted only if all eight match.
 *   - Combine: out[t][h] = bf16_rne(sum over valid k in ascending k of
 *     fmaf(w[t][k], y[slot[t][k]][h], acc)), acc starting at +0.0f.
 *
 * Error bits: 1 = bad expert id, 2 = capacity exceeded, 4 = flag mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_ERR_EXPERT 1u
#define ORC_ERR_CAPACITY 2u
#define ORC_ERR_FLAG 4u

#define ORC_CHUNK_BYTES 512
#define ORC_CHUNK_PAYLOAD 480
#define ORC_FLAG_WORDS 8

/* ----------------------------------------------------------------------- */
/* Number helpers written from their definitions.                          */
/* ----------------------------------------------------------------------- */

/* bfloat16 is the upper half of an IEEE binary32; widening is exact. */
static float bf16_bits_to_float(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 to bfloat16, nearest with ties to even. The kept part is
 * the upper 16 bits; the dropped lower 16 bits decide the rounding. NaN maps
 * to the canonical quiet NaN 0x7FC0. */
static uint16_t float_to_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return 0x7FC0;
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1; /* carries into the exponent correctly, up to infinity */
    return (uint16_t)upper;
}

static int64_t round_up16(int64_t n) { return (n + 15) / 16 * 16; }

/* An expert id as the path uses it: -1 stays -1 (no expert); anything else
 * outside [0, E) is reported and treated as -1. */
static int64_t checked_expert(int64_t e, int E, uint32_t *err) {
    if (e == -1) return -1;
    if (e < -1 || e >= E) {
        *err |= ORC_ERR_EXPERT;
        return -1;
    }
    return e;
}

/* Is rank r already produced by an earlier valid lane k' < k of token t? */
static int rank_seen_before(const int64_t *row, int k, int E, int epr, int64_t r) {
    uint32_t dummy = 0;
    for (int j = 0; j < k; j++) {
        int64_t e = checked_expert(row[j], E, &dummy);
        if (e >= 0 && e / epr == r) return 1;
    }
    return 0;
}

/* Same test for scale-out groups: group of expert e is (e / epr) / P. */
static int group_seen_before(const int64_t *row, int k, int E, int epr, int P, int64_t g) {
    uint32_t dummy = 0;
    for (int j = 0; j < k; j++) {
        int64_t e = checked_expert(row[j], E, &dummy);
        if (e >= 0 && (e / epr) / P == g) return 1;
    }
    return 0;
}

/* ----------------------------------------------------------------------- */
/* Layout ([V2] §3.3 阶段1 + the slot assignment of 阶段2).                */
/* ----------------------------------------------------------------------- */

/* Computes, for T tokens with K expert choices each:
 *   tokens_per_expert[E]  per valid lane (not deduplicated),
 *   tokens_per_rank[R]    per token, rank deduplicated,
 *   tokens_per_group[G]   per token, group deduplicated (group = rank / P),
 *   *_offsets[n+1]        exclusive prefix sums of the counts,
 *   in_rank[T*R], in_group[T*G]  0/1 membership masks,
 *   slot[T*K], group_slot[T*K]   absolute receive row of (t, rank(k)) and
 *                                (t, group(k)), -1 for skipped lanes.
 * All output arrays must be provided. Returns 0, or -1 on a bad shape. */
int oracle_layout(int T, int K, int E, int R, int G, const int64_t *topk_idx,
                  int32_t *tokens_per_expert, int32_t *tokens_per_rank,
                  int32_t *tokens_per_group, int32_t *expert_offsets,
                  int32_t *rank_offsets, int32_t *group_offsets, uint8_t *in_rank,
                  uint8_t *in_group, int32_t *slot, int32_t *group_slot,
                  uint32_t *err) {
    if (T < 0 || K < 1 || E < 1 || R < 1 || G < 1 || E % R != 0 || R % G != 0)
        return -1;
    const int epr = E / R, P = R / G;
    memset(tokens_per_expert, 0, sizeof(int32_t) * (size_t)E);
    memset(tokens_per_rank, 0, sizeof(int32_t) * (size_t)R);
    memset(tokens_per_group, 0, sizeof(int32_t) * (size_t)G);
    memset(in_rank, 0, (size_t)T * (size_t)R);
    memset(in_group, 0, (size_t)T * (size_t)G);

    /* Counting: every valid lane counts its expert; a rank (group) counts a
     * token once however many of its lanes land there. */
    for (int t = 0; t < T; t++) {
        const int64_t *row = topk_idx + (size_t)t * K;
        for (int k = 0; k < K; k++) {
            int64_t e = checked_expert(row[k], E, err);
            if (e < 0) continue;
            tokens_per_expert[e] += 1;
            int64_t r = e / epr, g = r / P;
            if (!in_rank[(size_t)t * R + r]) {
                in_rank[(size_t)t * R + r] = 1;
                tokens_per_rank[r] += 1;
            }
            if (!in_group[(size_t)t * G + g]) {
                in_group[(size_t)t * G + g] = 1;
                tokens_per_group[g] += 1;
            }
        }
    }

    /* Exclusive prefix sums. */
    expert_offsets[0] = 0;
    for (int e = 0; e < E; e++) expert_offsets[e + 1] = expert_offsets[e] + tokens_per_expert[e];
    rank_offsets[0] = 0;
    for (int r = 0; r < R; r++) rank_offsets[r + 1] = rank_offsets[r] + tokens_per_rank[r];
    group_offsets[0] = 0;
    for (int g = 0; g < G; g++) group_offsets[g + 1] = group_offsets[g] + tokens_per_group[g];

    /* Slots: walk tokens in order, hand out the next row of each destination
     * region the first time a token reaches it; later lanes of the same token
     * reuse that row. */
    int32_t *next_r = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    int32_t *next_g = (int32_t *)malloc(sizeof(int32_t) * (size_t)G);
    if (!next_r || !next_g) { free(next_r); free(next_g); return -1; }
    for (int r = 0; r < R; r++) next_r[r] = rank_offsets[r];
    for (int g = 0; g < G; g++) next_g[g] = group_offsets[g];
    for (int t = 0; t < T; t++) {
        const int64_t *row = topk_idx + (size_t)t * K;
        for (int k = 0; k < K; k++) {
            uint32_t dummy = 0;
            int64_t e = checked_expert(row[k], E, &dummy);
            int32_t *s = slot + (size_t)t * K + k;
            int32_t *gs = group_slot + (size_t)t * K + k;
            if (e < 0) { *s = -1; *gs = -1; continue; }
            int64_t r = e / epr, g = r / P;
            if (!rank_seen_before(row, k, E, epr, r)) {
                *s = next_r[r]++;
            } else {
                for (int j = 0; j < k; j++) {
                    int64_t ej = checked_expert(row[j], E, &dummy);
                    if (ej >= 0 && ej / epr == r) { *s = slot[(size_t)t * K + j]; break; }
                }
            }
            if (!group_seen_before(row, k, E, epr, P, g)) {
                *gs = next_g[g]++;
            } else {
                for (int j = 0; j < k; j++) {
                    int64_t ej = checked_expert(row[j], E, &dummy);
                    if (ej >= 0 && (ej / epr) / P == g) { *gs = group_slot[(size_t)t * K + j]; break; }
                }
            }
        }
    }
    free(next_r);
    free(next_g);
    return 0;
}

/* ----------------------------------------------------------------------- */
/* Expand-mode rows ([V2] §3.3 阶段3, copy epilogue with expand: one row    */
/* per (token, lane), grouped by expert).                                  */
/* ----------------------------------------------------------------------- */

/* expert_slot[t][k] = row of lane k of token t in the expert-major receive
 * buffer: expert e's rows start at expert_offsets[e] and follow the lanes
 * (t, k) that chose e in ascending t, then ascending k (the order one copy
 * warp walking the received tokens and lanes in order would hand out with
 * its per-expert atomic counter). -1 for lanes without a valid expert. */
int oracle_expert_slots(int T, int K, int E, const int64_t *topk_idx,
                        const int32_t *expert_offsets, int32_t *expert_slot) {
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!next) return -1;
    for (int e = 0; e < E; e++) next[e] = expert_offsets[e];
    for (int t = 0; t < T; t++) {
        for (int k = 0; k < K; k++) {
            uint32_t dummy = 0;
            int64_t e = checked_expert(topk_idx[(size_t)t * K + k], E, &dummy);
            expert_slot[(size_t)t * K + k] = e < 0 ? -1 : next[e]++;
        }
    }
    free(next);
    return 0;
}

/* ----------------------------------------------------------------------- */
/* Several source ranks on one GPU: the counts exchange ([V2] §3.3 阶段3,   */
/* psum_num_recv_tokens_per_scaleup_rank; §3.5 handle).                    */
/* ----------------------------------------------------------------------- */

/* S source ranks own consecutive token ranges of Ts = ceil(T / S) tokens
 * (the last may be shorter). Each source counts its tokens per destination
 * rank: counts[s][r] = #{t of source s : t sends to r}. The exchange hands
 * destination r the column counts[.][r]; recv_offsets[r][s] = rank_offsets[r]
 * + sum_{s' < s} counts[s'][r] is where source s's tokens start in r's
 * region (rank-major, recv_offsets[R * S] = N). Returns -1 on bad args. */
int oracle_source_counts(int T, int K, int E, int R, int S, const int64_t *topk_idx,
                         int32_t *counts, int32_t *recv_offsets) {
    if (S < 1 || R < 1 || E % R != 0) return -1;
    const int epr = E / R;
    const int Ts = (T + S - 1) / S;
    uint8_t *seen = (uint8_t *)calloc((size_t)R, 1);
    if (!seen) return -1;
    memset(counts, 0, sizeof(int32_t) * (size_t)S * (size_t)R);
    for (int t = 0; t < T; t++) {
        const int src = Ts ? t / Ts : 0;
        memset(seen, 0, (size_t)R);
        for (int k = 0; k < K; k++) {
            uint32_t dummy = 0;
            int64_t e = checked_expert(topk_idx[(size_t)t * K + k], E, &dummy);
            if (e < 0) continue;
            int64_t r = e / epr;
            if (!seen[r]) { seen[r] = 1; counts[(size_t)src * R + r] += 1; }
        }
    }
    int32_t run = 0;
    for (int r = 0; r < R; r++)
        for (int src = 0; src < S; src++) {
            recv_offsets[(size_t)r * S + src] = run;
            run += counts[(size_t)src * R + r];
        }
    recv_offsets[(size_t)R * S] = run;
    free(seen);
    return 0;
}

/* Staging row of every lane: src_slot[t*K+k] = (r*S + s)*cap + j for a
 * valid lane of rank r, j = #{earlier tokens of source s that send to r}
 * (lanes of one rank share the row); -1 for an invalid lane, and -1 with
 * error bit 1 when j >= cap. Returns -1 on bad args. */
int oracle_source_slots(int T, int K, int E, int R, int S, const int64_t *topk_idx, int64_t cap,
                        int32_t *src_slot, uint32_t *err) {
    if (S < 1 || R < 1 || E % R != 0 || cap < 0) return -1;
    const int epr = E / R;
    const int Ts = (T + S - 1) / S;
    int64_t *next = (int64_t *)malloc(sizeof(int64_t) * (size_t)R);
    if (!next) return -1;
    for (int t = 0; t < T; t++) {
        const int src = t / Ts;
        if (t == src * Ts)
            for (int r = 0; r < R; r++) next[r] = 0;
        const int64_t *row = topk_idx + (size_t)t * K;
        for (int k = 0; k < K; k++) {
            int64_t e = checked_expert(row[k], E, err);
            int32_t v = -1;
            if (e >= 0) {
                int64_t r = e / epr;
                int64_t j = next[r];
                for (int q = 0; q < k; q++)
                    if (row[q] >= 0 && row[q] < E && row[q] / epr == r) j = next[r] - 1;
                int first = (j == next[r]);
                if (first) next[r]++;
                if (j < cap) v = (int32_t)((r * S + src) * cap + j);
                else if (first) *err |= ORC_ERR_CAPACITY;
            }
            src_slot[(size_t)t * K + k] = v;
        }
    }
    free(next);
    return 0;
}

/* ----------------------------------------------------------------------- */
/* Direct dispatch ([V2] §3.3 阶段2, §3.5; [PIPE] NVL receivers).          */
/* ----------------------------------------------------------------------- */

/* For each token t (ascending) and each lane k (ascending) whose rank r has
 * not been seen earlier in the token, the token's record is written to the
 * next free row of r's region (rows start at rank_offsets[r]). The record is:
 *   recv_x[row]        = x[t]            (H bf16, optional)
 *   recv_fp8[row]      = x_fp8[t]        (H bytes, optional)
 *   recv_scales[row]   = x_scales[t]     (H/128 fp32, optional)
 *   recv_src[row]      = t               (optional)
 *   recv_topk_idx[row] = topk_idx[t] as int32, invalid ids as -1 (optional)
 *   recv_topk_w[row]   = topk_w[t] bit for bit (optional)
 * Rows at or beyond `capacity` are not written and set error bit 1. */
void oracle_dispatch(int T, int H, int K, int E, int R, const int64_t *topk_idx,
                     const float *topk_w, const uint16_t *x, const uint8_t *x_fp8,
                     const float *x_scales, const int32_t *rank_offsets, int64_t capacity,
                     uint16_t *recv_x, uint8_t *recv_fp8, float *recv_scales,
                     int32_t *recv_src, int32_t *recv_topk_idx, float *recv_topk_w,
                     uint32_t *err) {
    const int epr = E / R;
    const int S = H / 128;
    int64_t *next = (int64_t *)malloc(sizeof(int64_t) * (size_t)R);
    if (!next) return;
    for (int r = 0; r < R; r++) next[r] = rank_offsets[r];
    for (int t = 0; t < T; t++) {
        const int64_t *row = topk_idx + (size_t)t * K;
        for (int k = 0; k < K; k++) {
            int64_t e = checked_expert(row[k], E, err);
            if (e < 0) continue;
            int64_t r = e / epr;
            if (rank_seen_before(row, k, E, epr, r)) continue;
            int64_t dst = next[r]++;
            if (dst >= capacity) { *err |= ORC_ERR_CAPACITY; continue; }
            if (recv_x && x)
                memcpy(recv_x + dst * H, x + (size_t)t * H, sizeof(uint16_t) * (size_t)H);
            if (recv_fp8 && x_fp8)
                memcpy(recv_fp8 + dst * H, x_fp8 + (size_t)t * H, (size_t)H);
            if (recv_scales && x_scales)
                memcpy(recv_scales + dst * S, x_scales + (size_t)t * S, sizeof(float) * (size_t)S);
            if (recv_src) recv_src[dst] = t;
            if (recv_topk_idx) {
                uint32_t dummy = 0;
                for (int j = 0; j < K; j++)
                    recv_topk_idx[dst * K + j] = (int32_t)checked_expert(row[j], E, &dummy);
            }
            if (recv_topk_w && topk_w)
                memcpy(recv_topk_w + dst * K, topk_w + (size_t)t * K, sizeof(float) * (size_t)K);
        }
    }
    free(next);
}

/* ----------------------------------------------------------------------- */
/* Token record and 512 B data-as-flag chunks ([V2] §3.4; [ASC]).          */
/* ----------------------------------------------------------------------- */

/* Record = [bf16 hidden][fp8 hidden][fp32 scales][topk_idx i32 x K]
 *          [topk_w f32 x K][src i32], each present piece padded to 16 B.
 * The metadata pieces are always present. Returns its byte length P. */
int64_t oracle_record_bytes(int H, int K, int with_bf16, int with_fp8, int with_scales) {
    int64_t p = 0;
    if (with_bf16) p += round_up16(2 * (int64_t)H);
    if (with_fp8) p += round_up16((int64_t)H);
    if (with_scales) p += round_up16(4 * (int64_t)(H / 128));
    p += round_up16(4 * (int64_t)K);
    p += round_up16(4 * (int64_t)K);
    p += round_up16(4);
    return p;
}

/* A payload of P bytes occupies ceil(P / 480) blocks of 512 B. */
int64_t oracle_chunked_bytes(int64_t payload_bytes) {
    int64_t blocks = (payload_bytes + ORC_CHUNK_PAYLOAD - 1) / ORC_CHUNK_PAYLOAD;
    return blocks * ORC_CHUNK_BYTES;
}

/* Serialise token t's record into rec[0 .. P). */
void oracle_pack_record(int t, int H, int K, int E, const int64_t *topk_idx,
                        const float *topk_w, const uint16_t *x, const uint8_t *x_fp8,
                        const float *x_scales, uint8_t *rec) {
    const int S = H / 128;
    int64_t off = 0;
    int64_t P = oracle_record_bytes(H, K, x != NULL, x_fp8 != NULL, x_scales != NULL);
    memset(rec, 0, (size_t)P);
    if (x) {
        memcpy(rec + off, x + (size_t)t * H, 2 * (size_t)H);
        off += round_up16(2 * (int64_t)H);
    }
    if (x_fp8) {
        memcpy(rec + off, x_fp8 + (size_t)t * H, (size_t)H);
        off += round_up16((int64_t)H);
    }
    if (x_scales) {
        memcpy(rec + off, x_scales + (size_t)t * S, 4 * (size_t)S);
        off += round_up16(4 * (int64_t)S);
    }
    uint32_t dummy = 0;
    for (int k = 0; k < K; k++) {
        int32_t v = (int32_t)checked_expert(topk_idx[(size_t)t * K + k], E, &dummy);
        memcpy(rec + off + 4 * k, &v, 4);
    }
    off += round_up16(4 * (int64_t)K);
    if (topk_w) memcpy(rec + off, topk_w + (size_t)t * K, 4 * (size_t)K);
    off += round_up16(4 * (int64_t)K);
    int32_t src = t;
    memcpy(rec + off, &src, 4);
}

/* Cut a P-byte record into 512 B blocks: block c carries record bytes
 * [480c, 480c + 480) (zero past the end) followed by 32 B of flag, eight u32
 * words each equal to `epoch`. */
void oracle_chunk(const uint8_t *rec, int64_t P, uint32_t epoch, uint8_t *out) {
    int64_t nblk = oracle_chunked_bytes(P) / ORC_CHUNK_BYTES;
    for (int64_t c = 0; c < nblk; c++) {
        uint8_t *blk = out + c * ORC_CHUNK_BYTES;
        int64_t begin = c * ORC_CHUNK_PAYLOAD;
        int64_t n = P - begin < ORC_CHUNK_PAYLOAD ? P - begin : ORC_CHUNK_PAYLOAD;
        memset(blk, 0, ORC_CHUNK_PAYLOAD);
        memcpy(blk, rec + begin, (size_t)n);
        for (int w = 0; w < ORC_FLAG_WORDS; w++)
            memcpy(blk + ORC_CHUNK_PAYLOAD + 4 * w, &epoch, 4);
    }
}

/* Does block c of a chunked row carry all eight flag words == epoch? */
static int block_flag_ok(const uint8_t *chunked_row, int64_t c, uint32_t epoch) {
    const uint8_t *f = chunked_row + c * ORC_CHUNK_BYTES + ORC_CHUNK_PAYLOAD;
    for (int w = 0; w < ORC_FLAG_WORDS; w++) {
        uint32_t v;
        memcpy(&v, f + 4 * w, 4);
        if (v != epoch) return 0;
    }
    return 1;
}

/* Inverse of oracle_chunk: copies the payload back into rec[0 .. P) and
 * returns 0 if every block's flag equals epoch, 1 otherwise. */
int oracle_unchunk(const uint8_t *in, int64_t P, uint32_t epoch, uint8_t *rec) {
    int64_t nblk = oracle_chunked_bytes(P) / ORC_CHUNK_BYTES;
    int bad = 0;
    for (int64_t c = 0; c < nblk; c++) {
        int64_t begin = c * ORC_CHUNK_PAYLOAD;
        int64_t n = P - begin < ORC_CHUNK_PAYLOAD ? P - begin : ORC_CHUNK_PAYLOAD;
        memcpy(rec + begin, in + c * ORC_CHUNK_BYTES, (size_t)n);
        if (!block_flag_ok(in, c, epoch)) bad = 1;
    }
    return bad;
}

/* ----------------------------------------------------------------------- */
/* Two-level dispatch ([V2] §3.6; [PIPE] hybrid scale-out stage, forward). */
/* ----------------------------------------------------------------------- */

/* Step 1 (scale-out write): for each token t and each destination group g
 * (first lane reaching g), the chunked record goes once to the next row of
 * g's region in group_buf (rows start at group_offsets[g]).
 * Step 2 (forward): the rows of group_buf are read in row order; a row whose
 * flags do not all equal epoch sets error bit 2 and is dropped. Otherwise the
 * record's src and topk_idx say which ranks of g (rank / P == g; first lane
 * per rank) receive it; rank r of lane k gets it at row slot[src][k] of
 * peer_buf (the row the layout gave the pair (src, r), so a dropped record
 * leaves a hole instead of shifting later rows), re-chunked with the same
 * epoch.
 * Row strides are oracle_chunked_bytes(P). Rows at or beyond a buffer's
 * capacity are not written and set error bit 1. */
int oracle_hier_dispatch(int T, int H, int K, int E, int R, int G, const int64_t *topk_idx,
                         const float *topk_w, const uint16_t *x, const uint8_t *x_fp8,
                         const float *x_scales, const int32_t *slot,
                         const int32_t *group_offsets, uint32_t epoch, uint8_t *group_buf,
                         int64_t group_cap, uint8_t *peer_buf, int64_t peer_cap, int steps,
                         uint32_t *err) {
    const int epr = E / R, P = R / G;
    if (K > 64) return -1;
    const int64_t Prec = oracle_record_bytes(H, K, x != NULL, x_fp8 != NULL, x_scales != NULL);
    const int64_t stride = oracle_chunked_bytes(Prec);
    uint8_t *rec = (uint8_t *)malloc((size_t)Prec);
    int64_t *next_g = (int64_t *)malloc(sizeof(int64_t) * (size_t)G);
    if (!rec || !next_g) { free(rec); free(next_g); return -1; }

    /* Step 1. */
    for (int g = 0; g < G; g++) next_g[g] = group_offsets[g];
    for (int t = 0; t < T && (steps & 1); t++) {
        const int64_t *row = topk_idx + (size_t)t * K;
        int packed = 0;
        for (int k = 0; k < K; k++) {
            int64_t e = checked_expert(row[k], E, err);
            if (e < 0) continue;
            int64_t g = (e / epr) / P;
            if (group_seen_before(row, k, E, epr, P, g)) continue;
            int64_t dst = next_g[g]++;
            if (dst >= group_cap) { *err |= ORC_ERR_CAPACITY; continue; }
            if (!packed) {
                oracle_pack_record(t, H, K, E, topk_idx, topk_w, x, x_fp8, x_scales, rec);
                packed = 1;
            }
            oracle_chunk(rec, Prec, epoch, group_buf + dst * stride);
        }
    }

    /* Step 2. Record offsets of the metadata pieces. */
    int64_t off_idx = 0;
    if (x) off_idx += round_up16(2 * (int64_t)H);
    if (x_fp8) off_idx += round_up16((int64_t)H);
    if (x_scales) off_idx += round_up16(4 * (int64_t)(H / 128));
    const int64_t off_src = off_idx + 2 * round_up16(4 * (int64_t)K);
    int64_t n_group_rows = group_offsets[G];
    if (n_group_rows > group_cap) n_group_rows = group_cap;
    int g = 0;
    if (!(steps & 2)) n_group_rows = 0;
    for (int64_t n = 0; n < n_group_rows; n++) {
        while (n >= group_offsets[g + 1]) g++;
        if (oracle_unchunk(group_buf + n * stride, Prec, epoch, rec)) {
            *err |= ORC_ERR_FLAG;
            continue;
        }
        int32_t src;
        memcpy(&src, rec + off_src, 4);
        if (src < 0 || src >= T) { *err |= ORC_ERR_FLAG; continue; }
        int32_t ids[64];
        for (int k = 0; k < K; k++) memcpy(&ids[k], rec + off_idx + 4 * k, 4);
        for (int k = 0; k < K; k++) {
            if (ids[k] < 0 || ids[k] >= E) continue;
            int64_t r = ids[k] / epr;
            if (r / P != g) continue;
            int seen = 0;
            for (int j = 0; j < k; j++)
                if (ids[j] >= 0 && ids[j] < E && ids[j] / epr == r) seen = 1;
            if (seen) continue;
            int64_t dst = slot[(size_t)src * K + k];
            if (dst >= peer_cap) { *err |= ORC_ERR_CAPACITY; continue; }
            oracle_chunk(rec, Prec, epoch, peer_buf + dst * stride);
        }
    }
    free(rec);
    free(next_g);
    return 0;
}

/* Unpack `rows` chunked records into the plain receive arrays (any may be
 * NULL). Returns the number of rows whose flags did not all equal epoch. */
int64_t oracle_unpack_rows(const uint8_t *buf, int64_t rows, int H, int K, int with_bf16,
                           int with_fp8, int with_scales, uint32_t epoch, uint16_t *recv_x,
                           uint8_t *recv_fp8, float *recv_scales, int32_t *recv_src,
                           int32_t *recv_topk_idx, float *recv_topk_w) {
    const int S = H / 128;
    const int64_t Prec = oracle_record_bytes(H, K, with_bf16, with_fp8, with_scales);
    const int64_t stride = oracle_chunked_bytes(Prec);
    uint8_t *rec = (uint8_t *)malloc((size_t)Prec);
    if (!rec) return -1;
    int64_t bad = 0;
    for (int64_t n = 0; n < rows; n++) {
        bad += oracle_unchunk(buf + n * stride, Prec, epoch, rec);
        int64_t off = 0;
        if (with_bf16) {
            if (recv_x) memcpy(recv_x + n * H, rec + off, 2 * (size_t)H);
            off += round_up16(2 * (int64_t)H);
        }
        if (with_fp8) {
            if (recv_fp8) memcpy(recv_fp8 + n * H, rec + off, (size_t)H);
            off += round_up16((int64_t)H);
        }
        if (with_scales) {
            if (recv_scales) memcpy(recv_scales + n * S, rec + off, 4 * (size_t)S);
            off += round_up16(4 * (int64_t)S);
        }
        if (recv_topk_idx) memcpy(recv_topk_idx + n * K, rec + off, 4 * (size_t)K);
        off += round_up16(4 * (int64_t)K);
        if (recv_topk_w) memcpy(recv_topk_w + n * K, rec + off, 4 * (size_t)K);
        off += round_up16(4 * (int64_t)K);
        if (recv_src) memcpy(recv_src + n, rec + off, 4);
    }
    free(rec);
    return bad;
}

/* ----------------------------------------------------------------------- */
/* Several source ranks: send into per-source regions, then the copy       */
/* epilogue ([V2] §3.3 阶段2 slot per destination rank, 阶段3 copy         */
/* epilogue walking psum_num_recv_tokens_per_scaleup_rank).                */
/* ----------------------------------------------------------------------- */

/* Send step. Source s (tokens [s*Ts, min((s+1)*Ts, T)), Ts = ceil(T / S))
 * sends each token once per distinct destination rank r, in token order, to
 * the next row of the region (r, s) of `staging`: row (r*S + s)*cap + j with
 * j = #{earlier tokens of s that send to r}. Rows are chunked records (row
 * stride oracle_chunked_bytes(P)) carrying `epoch`. j >= cap sets error bit 1
 * and the row is not written. Returns -1 on bad args. */
int oracle_source_dispatch(int T, int H, int K, int E, int R, int S, const int64_t *topk_idx,
                           const float *topk_w, const uint16_t *x, const uint8_t *x_fp8,
                           const float *x_scales, uint32_t epoch, uint8_t *staging, int64_t cap,
                           uint32_t *err) {
    if (S < 1 || R < 1 || E % R != 0 || cap < 0) return -1;
    const int epr = E / R;
    const int Ts = (T + S - 1) / S;
    const int64_t Prec = oracle_record_bytes(H, K, x != NULL, x_fp8 != NULL, x_scales != NULL);
    const int64_t stride = oracle_chunked_bytes(Prec);
    uint8_t *rec = (uint8_t *)malloc((size_t)Prec);
    int64_t *next = (int64_t *)malloc(sizeof(int64_t) * (size_t)R);
    if (!rec || !next) { free(rec); free(next); return -1; }
    for (int src = 0; src < S; src++) {
        for (int r = 0; r < R; r++) next[r] = 0;
        const int t_end = (src + 1) * Ts < T ? (src + 1) * Ts : T;
        for (int t = src * Ts; t < t_end; t++) {
            const int64_t *row = topk_idx + (size_t)t * K;
            oracle_pack_record(t, H, K, E, topk_idx, topk_w, x, x_fp8, x_scales, rec);
            for (int k = 0; k < K; k++) {
                int64_t e = checked_expert(row[k], E, err);
                if (e < 0) continue;
                int64_t r = e / epr;
                int seen = 0;
                for (int j = 0; j < k; j++)
                    if (row[j] >= 0 && row[j] < E && row[j] / epr == r) seen = 1;
                if (seen) continue;
                int64_t j = next[r]++;
                if (j >= cap) { *err |= ORC_ERR_CAPACITY; continue; }
                oracle_chunk(rec, Prec, epoch, staging + (((int64_t)r * S + src) * cap + j) * stride);
            }
        }
    }
    free(rec);
    free(next);
    return 0;
}

/* Copy epilogue. Dense receive row i in [0, N), N = recv_offsets[R*S],
 * comes from the region (r, s) found by walking recv_offsets (rank-major)
 * until recv_offsets[r*S + s] <= i < recv_offsets[r*S + s + 1]; its staging
 * row is (r*S + s)*cap + (i - recv_offsets[r*S + s]). The record's fields
 * go to row i of the receive arrays (any may be NULL). Rows left unwritten:
 * i >= recv_cap or a region row beyond cap (error bit 1), a staging row
 * whose flags are not all `epoch` (error bit 2). Returns -1 on bad args. */
int oracle_copy_epilogue(int H, int K, int R, int S, const int32_t *recv_offsets,
                         const uint8_t *staging, int64_t cap, int with_bf16, int with_fp8,
                         int with_scales, uint32_t epoch, int64_t recv_cap, uint16_t *recv_x,
                         uint8_t *recv_fp8, float *recv_scales, int32_t *recv_src,
                         int32_t *recv_topk_idx, float *recv_topk_w, uint32_t *err) {
    if (S < 1 || R < 1 || cap < 0 || recv_cap < 0) return -1;
    const int S8 = H / 128;
    const int64_t Prec = oracle_record_bytes(H, K, with_bf16, with_fp8, with_scales);
    const int64_t stride = oracle_chunked_bytes(Prec);
    uint8_t *rec = (uint8_t *)malloc((size_t)Prec);
    if (!rec) return -1;
    const int64_t n_rows = recv_offsets[(size_t)R * S];
    int64_t region = 0;  /* r*S + s of the current region */
    for (int64_t i = 0; i < n_rows; i++) {
        while (i >= recv_offsets[region + 1]) region++;
        const int64_t j = i - recv_offsets[region];
        if (j >= cap || i >= recv_cap) { *err |= ORC_ERR_CAPACITY; continue; }
        if (oracle_unchunk(staging + (region * cap + j) * stride, Prec, epoch, rec)) {
            *err |= ORC_ERR_FLAG;
            continue;
        }
        int64_t off = 0;
        if (with_bf16) {
            if (recv_x) memcpy(recv_x + i * H, rec + off, 2 * (size_t)H);
            off += round_up16(2 * (int64_t)H);
        }
        if (with_fp8) {
            if (recv_fp8) memcpy(recv_fp8 + i * H, rec + off, (size_t)H);
            off += round_up16((int64_t)H);
        }
        if (with_scales) {
            if (recv_scales) memcpy(recv_scales + i * S8, rec + off, 4 * (size_t)S8);
            off += round_up16(4 * (int64_t)S8);
        }
        if (recv_topk_idx) memcpy(recv_topk_idx + i * K, rec + off, 4 * (size_t)K);
        off += round_up16(4 * (int64_t)K);
        if (recv_topk_w) memcpy(recv_topk_w + i * K, rec + off, 4 * (size_t)K);
        off += round_up16(4 * (int64_t)K);
        if (recv_src) memcpy(recv_src + i, rec + off, 4);
    }
    free(rec);
    return 0;
}

/* ----------------------------------------------------------------------- */
/* Combine ([MEGA] combine write; [ASC] BF16 hidden + FP32 weights).       */
/* ----------------------------------------------------------------------- */

/* Element h of row s of y: plain rows hold H bf16 back to back; chunked rows
 * hold the record, whose first piece is the bf16 hidden, cut into blocks. */
static uint16_t y_elem(const uint8_t *y, int64_t row_stride, int chunked, int64_t s, int64_t h) {
    int64_t b = 2 * h;
    int64_t at = chunked ? (b / ORC_CHUNK_PAYLOAD) * ORC_CHUNK_BYTES + b % ORC_CHUNK_PAYLOAD : b;
    uint16_t v;
    memcpy(&v, y + s * row_stride + at, 2);
    return v;
}

/* out[t][h] = bf16_rne(acc), acc = +0.0f, then for k = 0..K-1 with a usable
 * row s = slot[t][k]: acc = fmaf(w[t][k], y[s][h], acc). A lane is unusable
 * if s < 0; s >= y_rows sets error bit 1 and skips it; in chunked format a
 * row whose hidden-carrying blocks do not all have flag == epoch sets error
 * bit 2 and skips it. A token with no usable lane gets zeros. */
void oracle_combine(int T, int H, int K, const int32_t *slot, const float *topk_w,
                    const uint8_t *y, int64_t y_rows, int64_t row_stride, int chunked,
                    uint32_t epoch, uint16_t *out, uint32_t *err) {
    const int64_t hidden_blocks = (2 * (int64_t)H + ORC_CHUNK_PAYLOAD - 1) / ORC_CHUNK_PAYLOAD;
    int *use = (int *)malloc(sizeof(int) * (size_t)K);
    if (!use) return;
    for (int t = 0; t < T; t++) {
        for (int k = 0; k < K; k++) {
            int32_t s = slot[(size_t)t * K + k];
            use[k] = 0;
            if (s < 0) continue;
            if (s >= y_rows) { *err |= ORC_ERR_CAPACITY; continue; }
            if (chunked) {
                int ok = 1;
                for (int64_t c = 0; c < hidden_blocks; c++)
                    if (!block_flag_ok(y + (int64_t)s * row_stride, c, epoch)) ok = 0;
                if (!ok) { *err |= ORC_ERR_FLAG; continue; }
            }
            use[k] = 1;
        }
        for (int h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int k = 0; k < K; k++) {
                if (!use[k]) continue;
                int32_t s = slot[(size_t)t * K + k];
                float v = bf16_bits_to_float(y_elem(y, row_stride, chunked, s, h));
                acc = fmaf(topk_w[(size_t)t * K + k], v, acc);
            }
            out[(size_t)t * H + h] = float_to_bf16_bits(acc);
        }
    }
    free(use);
}

/* ----------------------------------------------------------------------- */
/* Two-level combine: the two-level dispatch run backwards ([PIPE] combine  */
/* roles kNVLSender -> kNVLAndRDMAForwarder -> kRDMAReceiver on the legacy  */
/* internode page; [V2] §3.6 hybrid path).                                 */
/* ----------------------------------------------------------------------- */

/* Byte stride of a partial row: the bf16 hidden row alone, cut into 512 B
 * blocks of 480 B payload + 32 B flag. */
int64_t oracle_partial_row_bytes(int H) { return oracle_chunked_bytes(2 * (int64_t)H); }

/* Is lane k of a token usable for combine (valid slot, in range, flags)? */
static int combine_lane_ok(int32_t s, const uint8_t *y, int64_t y_rows, int64_t row_stride,
                           int chunked, int64_t hidden_blocks, uint32_t epoch, uint32_t *err) {
    if (s < 0) return 0;
    if (s >= y_rows) { *err |= ORC_ERR_CAPACITY; return 0; }
    if (chunked) {
        for (int64_t c = 0; c < hidden_blocks; c++)
            if (!block_flag_ok(y + (int64_t)s * row_stride, c, epoch)) { *err |= ORC_ERR_FLAG; return 0; }
    }
    return 1;
}

/* steps & 1 (intra-group reduce): for every token t and every group g it
 * sends to, partial[t, g][h] = bf16_rne(acc), acc = +0.0f, then for the
 * usable lanes k of t whose rank lies in g, in ascending k:
 * acc = fmaf(w[t][k], y[slot[t][k]][h], acc). The partial is written, as a
 * chunked row with flags = epoch, to row group_slot[t][k0] of group_buf (k0 =
 * the first lane of g); rows >= group_cap are not written (error bit 1).
 * steps & 2 (cross-group reduce): out[t][h] = bf16_rne(acc), acc = +0.0f,
 * then for the groups g of t in ascending g whose partial row has all flags
 * == epoch (else error bit 2, skipped): acc = acc + partial[t, g][h].
 * Lanes of y are usable as in oracle_combine. */
void oracle_combine_two_level(int T, int H, int K, int E, int R, int G, const int64_t *topk_idx,
                              const int32_t *slot, const int32_t *group_slot, const float *topk_w,
                              const uint8_t *y, int64_t y_rows, int64_t row_stride, int chunked,
                              uint32_t epoch, uint8_t *group_buf, int64_t group_cap, int steps,
                              uint16_t *out, uint32_t *err) {
    const int epr = E / R, P = R / G;
    const int64_t hidden_blocks = (2 * (int64_t)H + ORC_CHUNK_PAYLOAD - 1) / ORC_CHUNK_PAYLOAD;
    const int64_t pstride = oracle_partial_row_bytes(H);
    int *use = (int *)malloc(sizeof(int) * (size_t)K);
    int *grp = (int *)malloc(sizeof(int) * (size_t)K);
    uint16_t *prow = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)H);
    if (!use || !grp || !prow) { free(use); free(grp); free(prow); return; }
    for (int t = 0; t < T; t++) {
        for (int k = 0; k < K; k++) {
            uint32_t dummy = 0;
            int64_t e = checked_expert(topk_idx[(size_t)t * K + k], E, &dummy);
            grp[k] = e < 0 ? -1 : (int)((e / epr) / P);
        }
        if (steps & 1) {
            for (int k = 0; k < K; k++)
                use[k] = combine_lane_ok(slot[(size_t)t * K + k], y, y_rows, row_stride, chunked,
                                         hidden_blocks, epoch, err);
            for (int k0 = 0; k0 < K; k0++) {
                int g = grp[k0];
                if (g < 0) continue;
                int first = 1;
                for (int j = 0; j < k0; j++)
                    if (grp[j] == g) first = 0;
                if (!first) continue;
                int64_t dst = group_slot[(size_t)t * K + k0];
                if (dst >= group_cap) { *err |= ORC_ERR_CAPACITY; continue; }
                for (int h = 0; h < H; h++) {
                    float acc = 0.0f;
                    for (int k = 0; k < K; k++) {
                        if (!use[k] || grp[k] != g) continue;
                        int32_t s = slot[(size_t)t * K + k];
                        acc = fmaf(topk_w[(size_t)t * K + k],
                                   bf16_bits_to_float(y_elem(y, row_stride, chunked, s, h)), acc);
                    }
                    prow[h] = float_to_bf16_bits(acc);
                }
                oracle_chunk((const uint8_t *)prow, 2 * (int64_t)H, epoch, group_buf + dst * pstride);
            }
        }
        if (steps & 2) {
            float *acc = (float *)calloc((size_t)H, sizeof(float));
            if (!acc) break;
            for (int g = 0; g < G; g++) {
                int k0 = -1;
                for (int k = 0; k < K; k++)
                    if (grp[k] == g) { k0 = k; break; }
                if (k0 < 0) continue;
                int64_t row = group_slot[(size_t)t * K + k0];
                if (row >= group_cap) { *err |= ORC_ERR_CAPACITY; continue; }
                const uint8_t *pr = group_buf + row * pstride;
                int ok = 1;
                for (int64_t c = 0; c < hidden_blocks; c++)
                    if (!block_flag_ok(pr, c, epoch)) ok = 0;
                if (!ok) { *err |= ORC_ERR_FLAG; continue; }
                for (int h = 0; h < H; h++)
                    acc[h] = acc[h] + bf16_bits_to_float(y_elem(pr, 0, 1, 0, h));
            }
            for (int h = 0; h < H; h++) out[(size_t)t * H + h] = float_to_bf16_bits(acc[h]);
            free(acc);
        }
    }
    free(use);
    free(grp);
    free(prow);
}

/* Exposed for the pin tests of the number helpers. */
uint16_t oracle_f32_to_bf16(float f) { return float_to_bf16_bits(f); }
float oracle_bf16_to_f32(uint16_t h) { return bf16_bits_to_float(h); }
