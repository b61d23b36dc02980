/*
 * ep.h -- C ABI of libep.so: the single-GPU data-parallel core of
 * expert-parallel MoE dispatch and combine on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [V2]   "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK 复制机制"
 *   [PIPE] "07: DeepEP Intra/Inter-node 协调 — NVLink Scale-up + RDMA
 *          Scale-out 三阶段流水线的代码实证"
 *   [MEGA] "06_06: NVLink Scale-up + RDMA Scale-out — DeepEP 三阶段流水线 vs
 *          DeepGEMM 对称内存"
 *   [ASC]  "Ascend Send Ordering"
 *
 * Model. One GPU holds T tokens of one source rank. R logical destination
 * ranks (E / R experts each, rank of expert e = e / (E / R)) are partitions of
 * this GPU's HBM; for the two-level path the R ranks form G scale-out groups
 * of P = R / G scale-up peers, rank r = g * P + peer ([PIPE]
 * is_nvlink_accessible). Each destination rank owns a compact region of
 * receive rows; regions are laid end to end in rank order (rank_offsets), and
 * inside a region rows follow ascending source token.
 *
 * Conventions for every entry point:
 *   - Every pointer is a DEVICE pointer unless stated, allocated and owned by
 *     the caller. The library allocates and frees no device memory and keeps
 *     no global state; calls on distinct workspaces are independent.
 *   - Work is enqueued asynchronously on `stream` (NULL = default stream).
 *     Inputs must stay valid until the work completes.
 *   - Arrays are row-major and densely packed. bf16 values are passed as their
 *     16-bit patterns (uint16_t), FP8 values as e4m3 bytes.
 *   - Alignment: hidden rows (bf16, FP8), receive rows and chunk buffers need
 *     16 B aligned base pointers; other arrays their element alignment.
 *   - With T = 0 the per-token arrays (topk_idx, x, weights, slot, ...) and
 *     buffers of zero capacity may be NULL; the layout calls then write zero
 *     counts and offsets, and no call writes a row.
 *   - Return value: EP_OK, or a negative EP_ERR_* status. Nothing is enqueued
 *     when a host-side check fails. Problems only visible on the device set
 *     bits in the workspace's error words (read with ep_check_errors and
 *     ep_check_sticky_errors, which return EP_ERR_DEVICE when a bit is set).
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define EP_OK 0
#define EP_ERR_ARG (-1)         /* null / misaligned pointer, bad shape, bad size */
#define EP_ERR_UNSUPPORTED (-2) /* shape outside the supported limits below */
#define EP_ERR_HIP (-3)         /* a HIP runtime call or launch failed */
#define EP_ERR_DEVICE (-4)      /* the device reported an error: ep_check_errors /
                                   ep_check_sticky_errors return it when error bits are
                                   set and write the bits (EP_DEVERR_*) to *bits */
#define EP_ERR_SCRATCH (-5)     /* ep_get_layout_noalloc: the shape's count tables do not
                                   fit the static scratch (EP_LAYOUT_SCRATCH_BYTES) */

/* Device error bits (workspace error words). */
#define EP_DEVERR_EXPERT_ID 1u  /* an expert id < -1 or >= E (treated as -1) */
#define EP_DEVERR_CAPACITY 2u   /* a row index >= the given buffer capacity (not written / not read) */
#define EP_DEVERR_FLAG 4u       /* a 512 B chunk flag != epoch (row dropped / skipped) */
#define EP_DEVERR_TIMEOUT 8u    /* a bounded wait for a batch flag gave up (batch not forwarded) */

/* Payload pieces present in a token record (ep_record_bytes). */
#define EP_SEG_BF16 1
#define EP_SEG_FP8 2
#define EP_SEG_SCALES 4

/* Row formats accepted by ep_combine. */
#define EP_FMT_PLAIN 0    /* rows of H bf16 values at a fixed byte stride */
#define EP_FMT_CHUNKED 1  /* chunked token records (see ep_hierarchical_dispatch) */

/* Two-level dispatch steps. */
#define EP_HIER_SCALEOUT 1 /* step 1: one write per (token, destination group) */
#define EP_HIER_FORWARD 2  /* step 2: forward group rows to scale-up peers */

/* Supported limits (EP_ERR_UNSUPPORTED beyond them). */
#define EP_MAX_TOPK 64
#define EP_MAX_RANKS 1024
#define EP_MAX_GROUPS 256
#define EP_MAX_EXPERTS 4096

/* Problem shape. T >= 0 tokens; H hidden size (H % 8 == 0; H % 128 == 0 when
 * FP8 scales are used); K in [1, 64] experts per token; E experts; R ranks
 * with E % R == 0; G groups with R % G == 0 (G = 1 for the flat path). */
typedef struct ep_shape {
    int32_t T, H, K, E, R, G;
} ep_shape;

/* Layout arrays written by ep_get_layout and read by the other calls
 * ([V2] §3.3 阶段1: per-expert counts, per-rank counts after rank
 * deduplication, prefix sums; [V2] §3.3 阶段2: one slot per token and
 * destination; the is-token-in-rank mask of [PIPE]'s RDMA sender). */
typedef struct ep_layout {
    int32_t *tokens_per_expert;  /* [E]   valid lanes per expert (not deduplicated) */
    int32_t *tokens_per_rank;    /* [R]   tokens per rank, each token counted once */
    int32_t *tokens_per_group;   /* [G]   tokens per group, each token counted once */
    int32_t *expert_offsets;     /* [E+1] exclusive prefix sum of tokens_per_expert */
    int32_t *rank_offsets;       /* [R+1] exclusive prefix sum; rank_offsets[R] = N rows */
    int32_t *group_offsets;      /* [G+1] exclusive prefix sum of tokens_per_group */
    uint8_t *is_token_in_rank;   /* [T*R] 1 if token t sends to rank r, else 0 */
    uint8_t *is_token_in_group;  /* [T*G] 1 if token t sends to group g, else 0 */
    int32_t *slot;               /* [T*K] receive row of (t, rank of lane k); -1 if lane skipped */
    int32_t *group_slot;         /* [T*K] group-region row of (t, group of lane k); -1 if skipped */
    int32_t *expert_slot;        /* [T*K] expand-mode row of (t, k); -1 if skipped (needs
                                    expert_offsets) */
} ep_layout;

/* Send side: per-token payload and routing of the T local tokens ([V2] §3.5). */
typedef struct ep_tokens {
    const uint16_t *x;            /* [T*H] bf16 hidden rows, or NULL */
    const uint8_t *x_fp8;         /* [T*H] e4m3 hidden rows, or NULL */
    const float *x_scales;        /* [T*H/128] one fp32 scale per 128 channels, or NULL */
    const int64_t *topk_idx;      /* [T*K] expert ids, -1 = no expert (required) */
    const float *topk_weights;    /* [T*K] routing weights, or NULL */
} ep_tokens;

/* Receive side of the direct dispatch: `capacity` rows each ([V2] §3.5
 * outputs recv_x / recv_topk_idx / recv_topk_weights; [PIPE] NVL receivers
 * write recv_x[row] and recv_x_scales[row * H/128]). */
typedef struct ep_recv {
    uint16_t *x;               /* [cap*H] or NULL (needs ep_tokens.x) */
    uint8_t *x_fp8;            /* [cap*H] or NULL (needs ep_tokens.x_fp8) */
    float *x_scales;           /* [cap*H/128] or NULL (needs ep_tokens.x_scales) */
    int32_t *src_idx;          /* [cap] source token of each row, or NULL */
    int32_t *topk_idx;         /* [cap*K] the token's expert ids as int32 (invalid -> -1), or NULL */
    float *topk_weights;       /* [cap*K] the token's weights, bit for bit, or NULL */
    int64_t capacity;          /* rows available; rows >= capacity are not written */
} ep_recv;

/* Bytes of workspace the calls need for `shape` (host only, no GPU work).
 * Layout: two u32 error words at offset 0 (word 0: errors of the current
 * pass of calls, cleared by the layout calls; word 1: errors since the last
 * ep_clear_errors, cleared by nothing else; undefined in a new workspace
 * until its first ep_clear_errors), then per-block partial counts. The
 * workspace may be reused by successive calls on one stream. */
size_t ep_workspace_bytes(const ep_shape *shape);

/* Byte length P of a packed token record with pieces `seg_flags`
 * (EP_SEG_*): [bf16 H*2][fp8 H][scales (H/128)*4][topk_idx K*4][topk_w K*4]
 * [src 4], each present piece padded to 16 B ([V2] §3.4 TokenLayout; the
 * metadata pieces are always present). Host only. Returns -1 on bad args. */
int64_t ep_record_bytes(const ep_shape *shape, int seg_flags);

/* Row stride of a chunked record: 512 * ceil(P / 480) bytes ([ASC] 导言 and
 * 能省多少: 512 B blocks of 480 B payload + 32 B flag). Host only. */
int64_t ep_chunked_record_bytes(const ep_shape *shape, int seg_flags);

/* Layout ([V2] §3.3 阶段1 notify warps and the slot rule of 阶段2).
 * For each token t and lane k with a valid expert e = topk_idx[t*K+k]:
 * rank r = e / (E/R), group g = r / (R/G). Counts: tokens_per_expert per lane;
 * tokens_per_rank / tokens_per_group once per token. Offsets: exclusive
 * prefix sums. Slot: slot[t*K+k] = rank_offsets[r] + #{t' < t : token t'
 * sends to r} (repeated ranks in a token share the row); group_slot likewise
 * with groups. Every output pointer except the workspace may be NULL to skip
 * that output. Also clears workspace error word 0 first, so a pass of
 * calls starts with a clean word. Ids < -1 or >= E set EP_DEVERR_EXPERT_ID
 * and count as -1. ws: at least ep_workspace_bytes(shape) bytes, 256 B
 * aligned. */
int ep_get_layout(const ep_shape *shape, const int64_t *topk_idx, const ep_layout *layout,
                  void *ws, size_t ws_bytes, void *stream);

/* Allocation-free layout, for callers that cannot allocate device memory at
 * call time (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): ep_get_layout with the same outputs, bit for bit,
 * but its per-workgroup count tables live in a static device array of
 * EP_LAYOUT_SCRATCH_BYTES inside the library instead of a workspace. Each GPU
 * the library runs on holds one such array until the process ends (its
 * address is looked up on the first call on that GPU); every call on a GPU
 * shares it, so calls that overlap on one GPU (several streams, several host
 * threads) race and must be serialised by the caller. The call allocates and
 * frees nothing. Limit: the count tables, 256 + a(4 * (nb + 1) * (2 * R4 + G4))
 * + a(4 * (nb + 1) * E) bytes (nb = ceil(T / 256), R4 and G4 = R and G rounded up to
 * multiples of 4, a() rounds up to a multiple of 256), must not exceed
 * EP_LAYOUT_SCRATCH_BYTES (4 MiB: e.g. 262,144 tokens with E = 256 and R =
 * 64 need 1.6 MB, 16,384 tokens with E = 2048 and R = 256 need 0.66 MB),
 * else EP_ERR_SCRATCH and nothing is enqueued.
 * errors: device pointer to two u32 error words with the meaning of the
 * workspace's (word 0 cleared by this call, then EP_DEVERR_EXPERT_ID set for
 * invalid ids in both); passing a workspace's base makes ep_check_errors on
 * that workspace read them. Other arguments and checks as ep_get_layout. */
#define EP_LAYOUT_SCRATCH_BYTES (4u << 20)
int ep_get_layout_noalloc(const ep_shape *shape, const int64_t *topk_idx, const ep_layout *layout,
                          uint32_t *errors, void *stream);

/* Expand-mode rows ([V2] §3.3 阶段3: the copy epilogue with expand, where a
 * received token gets one row per chosen expert, grouped by expert for the
 * expert GEMMs). When layout->expert_slot is non-NULL, ep_get_layout also
 * writes expert_slot[t*K+k] = expert_offsets[e] + #{lanes (t', k') before
 * (t, k) in token-then-lane order with the same expert e}, -1 for skipped
 * lanes; the rows of expert e are [expert_offsets[e], expert_offsets[e+1]),
 * expert_offsets[E] rows in all. Requires layout->expert_offsets
 * (EP_ERR_ARG without it). */

/* Direct dispatch ([V2] §3.3 阶段2 and §3.5; [PIPE] RDMA sender / NVL
 * sender record fields). Each token is read once and its record (present
 * pieces of ep_tokens plus src index, topk ids and weights) is written to
 * every receive row it owns: recv row layout->slot[t*K+k] for the first lane
 * k of each distinct rank. Needs layout->slot from ep_get_layout with the
 * same topk_idx. Receive pointers may be NULL to skip that piece. Rows >=
 * recv->capacity are not written and set EP_DEVERR_CAPACITY. */
int ep_dispatch(const ep_shape *shape, const ep_layout *layout, const ep_tokens *tokens,
                const ep_recv *recv, void *ws, size_t ws_bytes, void *stream);

/* Expand-mode dispatch: like ep_dispatch, but the token's record goes to the
 * row layout->expert_slot[t*K+k] of every valid lane k (one row per lane, no
 * rank deduplication). recv->capacity counts expand rows. */
int ep_dispatch_expand(const ep_shape *shape, const ep_layout *layout, const ep_tokens *tokens,
                       const ep_recv *recv, void *ws, size_t ws_bytes, void *stream);

/* Two-level dispatch ([V2] §3.6; [PIPE] hybrid scale-out stage and forward
 * warps) with chunked records ([ASC] data-as-flag 512 B blocks).
 * A record (ep_record_bytes, pieces = the non-NULL ones among x, x_fp8,
 * x_scales; x is required, topk_weights required) is cut into 512 B blocks:
 * block c holds record bytes [480c, 480c+480) (zero past the end) and then
 * eight u32 flag words equal to `epoch`. Row stride = ep_chunked_record_bytes.
 *  step EP_HIER_SCALEOUT: each token writes its chunked record once per
 *    destination group g, at row layout->group_slot of group_buf.
 *  step EP_HIER_FORWARD: each row n < min(group_offsets[G], group_cap) of
 *    group_buf is read once; if any block flag != epoch the row is dropped
 *    (EP_DEVERR_FLAG); else its record is written, flags = epoch, to
 *    peer_buf row layout->slot[src*K+k] for the first lane k of each distinct
 *    rank of the row's group.
 * `steps` is EP_HIER_SCALEOUT, EP_HIER_FORWARD or both (two launches, stream
 * ordered). epoch >= 1 (zeroed memory never passes the flag check). Needs
 * layout->slot, group_slot and group_offsets. Rows >= a buffer's capacity are
 * not written (EP_DEVERR_CAPACITY). After both steps the unpacked peer rows
 * equal what ep_dispatch writes for the same pieces. */
int ep_hierarchical_dispatch(const ep_shape *shape, const ep_layout *layout,
                             const ep_tokens *tokens, uint32_t epoch, int steps,
                             void *group_buf, int64_t group_cap, void *peer_buf,
                             int64_t peer_cap, void *ws, size_t ws_bytes, void *stream);

/* Both two-level steps in one persistent launch, forwarders consuming each
 * batch of records once its flag is published ([ASC] 方案一 and the
 * hierarchical Stage1: the batch's payload written without ordering, then
 * one ordered flag per batch; [PIPE] forward warps: records taken from the
 * scale-out buffer as they arrive, each wait bounded by a time limit).
 * Batch b = tokens [b * tile, (b+1) * tile). A workgroup writing batch b's
 * group rows (as step EP_HIER_SCALEOUT) stores them with device scope, waits
 * until they are acknowledged, then stores flag b = epoch; a workgroup
 * forwarding batch b waits for that flag (at most timeout_us; then the
 * batch's rows are not forwarded and EP_DEVERR_TIMEOUT is set) and forwards
 * the group rows of the batch's tokens (as step EP_HIER_FORWARD, block flags
 * checked). Jobs are handed out in order and job i writes batch i, then
 * forwards batch i - 64, so each group row is read back shortly after it was
 * written. The results are those of ep_hierarchical_dispatch with both
 * steps, byte for byte. Same arguments and requirements as
 * ep_hierarchical_dispatch with steps = 3; the workspace (ep_workspace_bytes)
 * also holds the batch flags, the ring's batch-freed words and the work
 * counters, which the call zeroes first with a small kernel (no memset), so
 * calls on one workspace must not overlap. opts may be NULL (defaults);
 * all-zero fields mean the defaults. */
typedef struct ep_fused_opts {
    int32_t tile_tokens;    /* tokens per batch, 1..64 (0: 2) */
    uint32_t timeout_us;    /* longest wait for one batch flag (0: 100000 us; in ring
                               mode scaled by the batch's generation, below) */
    uint32_t test_flags;    /* EP_FUSED_WITHHOLD: batch `withhold_batch`'s flag is never
                               published, to test the bounded wait (its group rows are
                               still written; it is not forwarded; EP_DEVERR_TIMEOUT) */
    int32_t withhold_batch;
    int32_t ring_batches;   /* 0: group rows at their group-region rows (group_slot), as
                               ep_hierarchical_dispatch writes them. > 64: group_buf is a
                               ring of this many batches instead ([PIPE] the scale-out
                               receive buffer with flow control: a sender waits until the
                               forwarder has freed the slots it reuses). Token i of batch b
                               puts its j-th distinct group's record at row
                               ((b mod ring) * tile + i) * min(K, G) + j; the producer of
                               batch b waits until batch b - ring was forwarded. With
                               n = b / ring, the producer waits at most (n + 1/2) *
                               timeout_us (then writes anyway and sets
                               EP_DEVERR_TIMEOUT) and the forwarder (n + 1) * timeout_us,
                               so a lost flag stops only its own batch, and a broken run
                               lasts at most about (nbatch / ring + 1) * timeout_us.
                               Needs group_cap >= ring * tile * min(K, G) (< 2^31); the
                               peer rows are those of ring 0, byte for byte; group_buf's
                               contents afterwards are unspecified (the last pass over the
                               ring), and group_slot's capacity check does not apply.
                               A ring too short for the whole grid runs with a shorter
                               lag (down to 16 batches) and at most ring - lag
                               workgroups, so it also bounds the work in flight (slower).
                               Other values: EP_ERR_ARG. */
} ep_fused_opts;
#define EP_FUSED_WITHHOLD 1u
int ep_hierarchical_dispatch_fused(const ep_shape *shape, const ep_layout *layout,
                                   const ep_tokens *tokens, uint32_t epoch, void *group_buf,
                                   int64_t group_cap, void *peer_buf, int64_t peer_cap,
                                   const ep_fused_opts *opts, void *ws, size_t ws_bytes,
                                   void *stream);

/* Combine ([MEGA] combine write of BF16 expert outputs per (token, top-k);
 * [ASC] BF16 hidden with FP32 top-k weights): the inverse gather plus a
 * weighted reduction back to token order:
 *   out[t][h] = bf16_rne(acc), acc = +0.0f, then for k = 0..K-1 with
 *   s = layout->slot[t*K+k] >= 0:  acc = fmaf(topk_weights[t*K+k], y[s][h], acc)
 * (fp32, one rounding per step, ascending k; a row shared by two lanes is read
 * once and used twice). y: `y_rows` rows at `y_row_stride` bytes; format
 * EP_FMT_PLAIN (H bf16 at the start of each row; stride % 16 == 0) or
 * EP_FMT_CHUNKED (chunked records whose first piece is the bf16 hidden;
 * stride % 512 == 0; a row whose hidden-carrying blocks do not all have
 * flag == epoch is skipped with EP_DEVERR_FLAG). s >= y_rows is skipped with
 * EP_DEVERR_CAPACITY. A token with no usable lane gets zeros. */
int ep_combine(const ep_shape *shape, const ep_layout *layout, const void *y, int64_t y_rows,
               int64_t y_row_stride, int y_format, uint32_t epoch, const float *topk_weights,
               uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* Expand-mode combine: ep_combine over expand rows, s = layout->expert_slot
 * instead of layout->slot (each lane has its own row). */
int ep_combine_expand(const ep_shape *shape, const ep_layout *layout, const void *y,
                      int64_t y_rows, int64_t y_row_stride, int y_format, uint32_t epoch,
                      const float *topk_weights, uint16_t *out, void *ws, size_t ws_bytes,
                      void *stream);

/* Byte stride of a partial row of the two-level combine: the bf16 hidden row
 * alone in 512 B data-as-flag blocks, 512 * ceil(2H / 480). Host only. */
int64_t ep_partial_row_bytes(const ep_shape *shape);

/* Two-level combine: the two-level dispatch run backwards (the combine roles
 * of [MEGA]'s legacy internode walk-through: scale-up reduce, then
 * scale-out; [V2] §3.6 groups). y holds the per-(token, rank) expert outputs
 * at layout->slot rows (EP_FMT_PLAIN or EP_FMT_CHUNKED as for ep_combine).
 *  step 1 (steps & 1): for each token t and group g it sends to, partial =
 *    bf16_rne(acc), acc = +0.0f, then for the usable lanes k of t whose rank
 *    lies in g, ascending k: acc = fmaf(topk_weights[t*K+k], y[slot][h], acc);
 *    written with flags = epoch as a chunked row (stride
 *    ep_partial_row_bytes) at row layout->group_slot[t*K+k0] of group_buf (k0
 *    = first lane of g). Rows >= group_cap are not written
 *    (EP_DEVERR_CAPACITY).
 *  step 2 (steps & 2): out[t][h] = bf16_rne(acc), acc = +0.0f, then for the
 *    groups of t in ascending g: acc = acc + partial[t, g][h] (fp32 add); a
 *    partial row with a flag != epoch is skipped (EP_DEVERR_FLAG).
 * Needs layout->slot, layout->group_slot, tokens' topk_idx; epoch >= 1.
 * Usable lanes are as in ep_combine. With G = 1 the result equals
 * ep_combine bit for bit. With steps = 3, K <= 8, H <= 3,840 or
 * 5,760 < H <= 7,680 (a row's 512 B blocks cut into 1, 2 or 4 slices of 8
 * blocks) and group_cap partial rows of at least 512 MB (smaller ones stay
 * in the MALL between two launches anyway), both steps run as one persistent
 * launch with one flag per batch of tokens in the workspace (as for
 * ep_hierarchical_dispatch_fused; calls on one workspace must not overlap):
 * job i reduces batch i's groups, publishes it, then sums batch i - 128
 * across groups, so the partial rows are read back shortly after they were
 * written. A batch whose flag does not come
 * within 100 ms is not summed (EP_DEVERR_TIMEOUT). The results equal the two
 * launches' bit for bit. */
int ep_combine_two_level(const ep_shape *shape, const ep_layout *layout, const int64_t *topk_idx,
                         const void *y, int64_t y_rows, int64_t y_row_stride, int y_format,
                         uint32_t epoch, const float *topk_weights, void *group_buf,
                         int64_t group_cap, int steps, uint16_t *out, void *ws, size_t ws_bytes,
                         void *stream);

/* Several source ranks on one GPU ([V2] §3.3 阶段2: each source hands out,
 * per destination rank, the next slot of its own region there, addressed as
 * rank * capacity + slot; 阶段3: the copy epilogue finds each received row's
 * source from the prefix sum of tokens received per source rank
 * (psum_num_recv_tokens_per_scaleup_rank) and copies the row out of that
 * source's region). Source s owns tokens [s*Ts, min((s+1)*Ts, T)), Ts =
 * ceil(T / S). The staging buffer holds one region of `capacity` chunked
 * rows per (destination rank r, source s), region index r*S + s. */
typedef struct ep_sources {
    int32_t S;               /* source ranks, 1 <= S <= EP_MAX_RANKS */
    int64_t capacity;        /* rows per (rank, source) region; R*S*capacity <= INT32_MAX */
    int32_t *counts;         /* [S*R] tokens source s sends to rank r, each token once */
    int32_t *recv_offsets;   /* [R*S+1] rank-major exclusive prefix of counts: the dense rows
                                of region (r, s) start at recv_offsets[r*S+s]; [R*S] = N */
    int32_t *src_slot;       /* [T*K] staging row (r*S+s)*capacity + j of (t, rank r of lane
                                k), j = #{earlier tokens of s sending to r}; -1 if skipped */
} ep_sources;

/* Workspace bytes of the several-source calls (>= ep_workspace_bytes; the
 * error word is at the same place). Host only; 0 on bad args. */
size_t ep_source_workspace_bytes(const ep_shape *shape, int32_t S);

/* Per-source counts, the counts exchange (recv_offsets, what every
 * destination learns from an all-to-all of counts) and src_slot. Clears the
 * workspace error word 0 first. j >= capacity sets EP_DEVERR_CAPACITY and the
 * lane gets -1; invalid ids set EP_DEVERR_EXPERT_ID. Deterministic: with
 * contiguous sources, region (r, s) of the dense rows is exactly the part of
 * rank r's region (ep_get_layout) that holds source s's tokens, so dense row
 * recv_offsets[r*S+s] + j == layout slot of the same (t, r). */
int ep_source_layout(const ep_shape *shape, const int64_t *topk_idx, const ep_sources *sources,
                     void *ws, size_t ws_bytes, void *stream);

/* Send step: each token's chunked record (pieces as for
 * ep_hierarchical_dispatch; x and topk_weights required) goes once to each
 * distinct staging row src_slot[t*K+k] >= 0, flags = epoch (>= 1). staging:
 * R*S*capacity rows of ep_chunked_record_bytes. */
int ep_source_dispatch(const ep_shape *shape, const ep_sources *sources, const ep_tokens *tokens,
                       uint32_t epoch, void *staging, void *ws, size_t ws_bytes, void *stream);

/* Copy epilogue: dense row i < N = recv_offsets[R*S] of region (r, s)
 * (recv_offsets[r*S+s] <= i < recv_offsets[r*S+s+1]) is staging row
 * (r*S+s)*capacity + (i - recv_offsets[r*S+s]); its record (pieces
 * `seg_flags`, as written by ep_source_dispatch) is unpacked into row i of
 * the receive arrays (NULL ones skipped; a piece must be in the record to be
 * asked for). A row whose flags are not all epoch is skipped
 * (EP_DEVERR_FLAG); rows >= recv->capacity and region rows >= capacity are
 * skipped (EP_DEVERR_CAPACITY). The result equals ep_dispatch's receive
 * rows. The combine of this layout is ep_combine with layout->slot =
 * src_slot over y rows indexed like the staging buffer. */
int ep_copy_epilogue(const ep_shape *shape, const ep_sources *sources, const void *staging,
                     uint32_t epoch, int seg_flags, const ep_recv *recv, void *ws,
                     size_t ws_bytes, void *stream);

/* Send and copy epilogue in one persistent launch: the same staging rows and
 * receive rows as ep_source_dispatch followed by ep_copy_epilogue with the
 * pieces of `tokens` (EP_SEG_BF16, plus EP_SEG_FP8 / EP_SEG_SCALES when
 * tokens carry them), with the destinations consuming each batch of records
 * once its flag is published ([V2] §3.3 阶段2 and 阶段3; [ASC] 方案一: a
 * batch's records written without ordering, then one ordered flag). Jobs are
 * handed out in order: job i sends the records of tokens [4i, 4i+4) and
 * publishes the batch, then unpacks the staging rows of batch i - 64 into
 * their dense rows recv_offsets[r*S+s] + j, while those rows are still in the
 * MALL. That pays off only when the staging rows are well past the MALL:
 * at 4,096 tokens over 32 ranks and 32 sources, 0.95 times the two calls'
 * time at H = 7,168 (473 MB of staging rows), 1.05 times at H = 4,096 and
 * up to 1.26 times at H = 1,024. A batch whose flag does not come within
 * 100 ms is not unpacked (EP_DEVERR_TIMEOUT); rows >= recv->capacity are skipped
 * (EP_DEVERR_CAPACITY). Needs the arguments of both calls; the workspace
 * (ep_source_workspace_bytes) also holds the batch flags, which the call
 * zeroes first with a small kernel, so calls on one workspace must not
 * overlap. */
int ep_source_dispatch_fused(const ep_shape *shape, const ep_sources *sources, const ep_tokens *tokens,
                             uint32_t epoch, void *staging, const ep_recv *recv, void *ws,
                             size_t ws_bytes, void *stream);

/* Clear both workspace error words (a stream-ordered kernel, no memset
 * node). */
int ep_clear_errors(void *ws, void *stream);

/* Synchronise `stream`, then copy error word 0 (the errors since the last
 * ep_get_layout / ep_source_layout call on this workspace) to *bits (host
 * pointer). Returns EP_OK when no bit is set, EP_ERR_DEVICE when one is
 * ([V2] §3.5: the caller learns of a failed pass from the call, not only
 * from the data), EP_ERR_ARG / EP_ERR_HIP when the word could not be read
 * (*bits is then left unchanged). */
int ep_check_errors(void *ws, void *stream, uint32_t *bits);

/* As ep_check_errors, for error word 1: every error any call on this
 * workspace reported since the last ep_clear_errors, across passes (a pass
 * that follows a failed one does not hide it). */
int ep_check_sticky_errors(void *ws, void *stream, uint32_t *bits);

/* Static description of a status code. */
const char *ep_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
