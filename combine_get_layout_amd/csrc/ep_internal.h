// ep_internal.h -- launch entry points of the kernels behind the C ABI.
// Host-side argument checks live in api.hip; these functions assume a shape and
// pointers that passed them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

constexpr int kLayoutTokens = 256;  // tokens per layout workgroup (one per thread)
constexpr int kFusedMinTile = 1;    // smallest batch of the fused two-level dispatch (tokens)
constexpr int kFusedMaxTile = 64;   // largest batch
constexpr int kFusedLag = 64;       // fixed lag of the fused two-level dispatch (batches)
constexpr int kFusedDefaultTile = 2;  // one token per wave of a 2-wave workgroup (measured best of 1-16)
constexpr int kFusedCounters = 64;  // u32 words before the batch flags (two used)

// Workspace carve-up (byte offsets from the workspace base).
struct WsLayout {
    int nb;                 // layout workgroups = max(1, ceil(T / kLayoutTokens))
    int rp, gp;             // R and G rounded up to multiples of 4
    int wrow;               // ints per row of the rank/lane/group table: 2 * rp + gp
    size_t err;             // uint32 error word
    // Per-workgroup count tables, one row per layout workgroup (row-major),
    // plus one row for the column totals when many workgroups are scanned:
    size_t part_rlg;        // int32 [nb + 1][wrow]: deduplicated tokens per rank (columns
                            // [0, R)), valid lanes per rank ([rp, rp + R)) and
                            // deduplicated tokens per group ([2 rp, 2 rp + G))
    size_t part_expert;     // int32 [nb + 1][E] lanes per expert
    size_t tables_end;      // end of the count tables (all the layout kernels use)
    size_t fused;           // fused two-level dispatch: u32 [kFusedCounters] work counters,
                            // then u32 [ceil(T / kFusedMinTile)] batch flags, then as
                            // many batch-freed words (ring mode)
    size_t total;
};
WsLayout ws_layout(const ep_shape& s);

// Workspace of the several-source calls: the layout workspace, then per-tile
// counts [S][nbs][R] (nbs = tiles of 256 tokens per source).
struct WsSource {
    int Ts;       // tokens per source, ceil(T / S)
    int nbs;      // tiles per source, max(1, ceil(Ts / 256))
    size_t part;  // int32 [S][nbs][R]
    size_t total;
};
WsSource ws_source(const ep_shape& s, int S);

// Record geometry of a packed token record (vectors are 16 B).
struct RecordGeom {
    int nv_x, nv_fp8, nv_scales, nv_idx, nv_w;  // vectors per piece (0 if absent)
    int q_fp8, q_scales, q_idx, q_w, q_src;     // first vector of each piece
    int nv;                                     // total vectors = P / 16
    int64_t bytes;                              // P
    int nchunks;                                // ceil(P / 480)
    int64_t stride;                             // 512 * nchunks
};
RecordGeom record_geom(const ep_shape& s, int seg_flags);

// Launch facts of a persistent kernel on the device of stream `st`: the
// wall-clock rate (kHz, for bounded waits), the CU count and how many
// workgroups of `block_threads` threads of `kernel` one CU holds at once.
// Queried on the first call for each (device, kernel) and kept, so later calls
// (also under stream capture) make no queries.
struct LaunchInfo {
    int rate_khz, cus, per_cu;
};
hipError_t launch_info(hipStream_t st, const void* kernel, int block_threads, LaunchInfo* out);
// Zero n consecutive u32 words with a small kernel on `st` (the persistent
// launches' counters and batch flags: a kernel, not a memset, so that the
// call can be captured into a graph).
hipError_t launch_zero_words(uint32_t* words, int n, hipStream_t st);

hipError_t launch_layout(const ep_shape& s, const int64_t* topk, const ep_layout& L, char* ws,
                         hipStream_t st);
// The allocation-free variant: count tables in the library's per-device
// scratch array (needs ws_layout(s).total <= EP_LAYOUT_SCRATCH_BYTES), error
// words at `err`.
hipError_t launch_layout_noalloc(const ep_shape& s, const int64_t* topk, const ep_layout& L,
                                 uint32_t* err, hipStream_t st);
hipError_t launch_dispatch(const ep_shape& s, const ep_layout& L, const ep_tokens& tk,
                           const ep_recv& rv, char* ws, hipStream_t st);
hipError_t launch_hier(const ep_shape& s, const ep_layout& L, const ep_tokens& tk,
                       uint32_t epoch, int steps, void* group_buf, int64_t group_cap,
                       void* peer_buf, int64_t peer_cap, char* ws, hipStream_t st);
hipError_t launch_hier_fused(const ep_shape& s, const ep_layout& L, const ep_tokens& tk,
                             uint32_t epoch, void* group_buf, int64_t group_cap, void* peer_buf,
                             int64_t peer_cap, int tile, uint32_t timeout_us, int withhold, int ring,
                             char* ws, hipStream_t st);
hipError_t launch_combine(const ep_shape& s, const ep_layout& L, const void* y, int64_t y_rows,
                          int64_t y_stride, int fmt, uint32_t epoch, const float* w,
                          uint16_t* out, char* ws, hipStream_t st);
hipError_t launch_combine_two_level(const ep_shape& s, const ep_layout& L, const int64_t* topk,
                                    const void* y, int64_t y_rows, int64_t y_stride, int fmt,
                                    uint32_t epoch, const float* w, void* group_buf,
                                    int64_t group_cap, int steps, uint16_t* out, char* ws,
                                    hipStream_t st);
hipError_t launch_send_rows(const ep_shape& s, const ep_tokens& tk, const int32_t* rows,
                            int64_t n_rows, uint32_t epoch, void* buf, char* ws, hipStream_t st);
hipError_t launch_source_layout(const ep_shape& s, const int64_t* topk, const ep_sources& src,
                                char* ws, hipStream_t st);
hipError_t launch_copy_epilogue(const ep_shape& s, const ep_sources& src, const void* staging,
                                uint32_t epoch, int seg, const ep_recv& rv, char* ws,
                                hipStream_t st);
// Send and copy epilogue in one launch (records' pieces as in tokens).
hipError_t launch_source_fused(const ep_shape& s, const ep_sources& src, const ep_tokens& tk,
                               uint32_t epoch, void* staging, const ep_recv& rv, char* ws, hipStream_t st);
constexpr uint32_t kSourceFusedTimeoutUs = 100000;  // longest wait for one batch flag of that launch

}  // namespace ep
