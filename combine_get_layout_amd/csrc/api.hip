// api.hip -- the extern "C" boundary of libep.so: argument checks, workspace
// and record sizing, and the kernel launches (declared in include/ep.h).
#include <hip/hip_runtime.h>

#include <mutex>

#include "ep.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

WsLayout ws_layout(const ep_shape& s) {
    WsLayout w;
    w.nb = s.T > 0 ? (s.T + kLayoutTokens - 1) / kLayoutTokens : 1;
    w.rp = (s.R + 3) / 4 * 4;
    w.gp = (s.G + 3) / 4 * 4;
    w.wrow = 2 * w.rp + w.gp;
    size_t off = 0;
    w.err = off;
    off += 256;
    w.part_rlg = off;
    off += align256(sizeof(int32_t) * (size_t)(w.nb + 1) * w.wrow);
    w.part_expert = off;
    off += align256(sizeof(int32_t) * (size_t)(w.nb + 1) * s.E);
    w.tables_end = off;
    w.fused = off;
    off += align256(sizeof(uint32_t) * (kFusedCounters + 2 * ((size_t)(s.T + kFusedMinTile - 1) / kFusedMinTile)));
    w.total = off;
    return w;
}

static int pad16_vecs(int64_t bytes) { return (int)((bytes + 15) / 16); }

hipError_t launch_info(hipStream_t st, const void* kernel, int block_threads, LaunchInfo* out) {
    struct Entry {
        int dev;
        const void* kernel;
        int threads;
        LaunchInfo info;
    };
    constexpr int kMaxEntries = 256;  // (device, kernel) pairs: a few kernels on up to 64 devices
    static Entry cache[kMaxEntries];
    static int n_cache = 0;
    static std::mutex mu;
    int dev = 0;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cache; ++i) {
        if (cache[i].dev == dev && cache[i].kernel == kernel && cache[i].threads == block_threads) {
            *out = cache[i].info;
            return hipSuccess;
        }
    }
    LaunchInfo d = {0, 0, 0};
    if ((e = hipDeviceGetAttribute(&d.rate_khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.per_cu, kernel, block_threads, 0)) != hipSuccess)
        return e;
    if (n_cache < kMaxEntries) cache[n_cache++] = {dev, kernel, block_threads, d};
    *out = d;
    return hipSuccess;
}

RecordGeom record_geom(const ep_shape& s, int seg) {
    RecordGeom g;
    g.nv_x = (seg & EP_SEG_BF16) ? pad16_vecs(2 * (int64_t)s.H) : 0;
    g.nv_fp8 = (seg & EP_SEG_FP8) ? pad16_vecs(s.H) : 0;
    g.nv_scales = (seg & EP_SEG_SCALES) ? pad16_vecs(4 * (int64_t)(s.H / 128)) : 0;
    g.nv_idx = pad16_vecs(4 * (int64_t)s.K);
    g.nv_w = pad16_vecs(4 * (int64_t)s.K);
    g.q_fp8 = g.nv_x;
    g.q_scales = g.q_fp8 + g.nv_fp8;
    g.q_idx = g.q_scales + g.nv_scales;
    g.q_w = g.q_idx + g.nv_idx;
    g.q_src = g.q_w + g.nv_w;
    g.nv = g.q_src + 1;
    g.bytes = 16 * (int64_t)g.nv;
    g.nchunks = (int)((g.bytes + kChunkPayload - 1) / kChunkPayload);
    g.stride = (int64_t)kChunkBytes * g.nchunks;
    return g;
}

namespace {

__global__ void clear_error_kernel(uint32_t* err) {
    err[0] = 0u;  // current pass
    err[1] = 0u;  // since the last clear
}

// One thread per word (a single workgroup looping over 8,192 batch flags took
// 4.5 us).
__global__ void zero_words_kernel(uint32_t* words, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) words[i] = 0u;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape check shared by all entry points.
int check_shape(const ep_shape* s) {
    if (!s) return EP_ERR_ARG;
    if (s->T < 0 || s->H <= 0 || s->K < 1 || s->E < 1 || s->R < 1 || s->G < 1) return EP_ERR_ARG;
    if (s->E % s->R != 0 || s->R % s->G != 0 || s->H % 8 != 0) return EP_ERR_ARG;
    if (s->K > EP_MAX_TOPK || s->R > EP_MAX_RANKS || s->G > EP_MAX_GROUPS || s->E > EP_MAX_EXPERTS)
        return EP_ERR_UNSUPPORTED;
    if ((int64_t)s->T * s->K > INT32_MAX || (int64_t)s->T * s->R > ((int64_t)1 << 40))
        return EP_ERR_UNSUPPORTED;
    return EP_OK;
}

int check_ws(const ep_shape* s, void* ws, size_t ws_bytes) {
    if (!ws || !aligned(ws, 256)) return EP_ERR_ARG;
    if (ws_bytes < ws_layout(*s).total) return EP_ERR_ARG;
    return EP_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

}  // namespace

hipError_t launch_zero_words(uint32_t* words, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + kBlockThreads - 1) / kBlockThreads), dim3(kBlockThreads), 0, st,
                       words, n);
    return hipSuccess;
}
}  // namespace ep

using namespace ep;

extern "C" {

size_t ep_workspace_bytes(const ep_shape* shape) {
    if (check_shape(shape) != EP_OK) return 0;
    return ws_layout(*shape).total;
}

int64_t ep_record_bytes(const ep_shape* shape, int seg_flags) {
    if (check_shape(shape) != EP_OK || (seg_flags & ~7)) return -1;
    if ((seg_flags & EP_SEG_SCALES) && shape->H % 128 != 0) return -1;
    if ((seg_flags & EP_SEG_FP8) && shape->H % 16 != 0) return -1;
    return record_geom(*shape, seg_flags).bytes;
}

int64_t ep_chunked_record_bytes(const ep_shape* shape, int seg_flags) {
    if (ep_record_bytes(shape, seg_flags) < 0) return -1;
    return record_geom(*shape, seg_flags).stride;
}

int ep_get_layout(const ep_shape* shape, const int64_t* topk_idx, const ep_layout* layout,
                  void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(shape);
    if (rc != EP_OK) return rc;
    if ((rc = check_ws(shape, ws, ws_bytes)) != EP_OK) return rc;
    if (!layout || (shape->T > 0 && !topk_idx) || !aligned(topk_idx, 8)) return EP_ERR_ARG;
    const ep_layout& L = *layout;
    if (!aligned(L.is_token_in_rank, 16) || !aligned(L.is_token_in_group, 16)) return EP_ERR_ARG;
    if (L.expert_slot && !L.expert_offsets) return EP_ERR_ARG;
    const void* i32s[] = {L.tokens_per_expert, L.tokens_per_rank, L.tokens_per_group,
                          L.expert_offsets, L.rank_offsets, L.group_offsets, L.slot,
                          L.group_slot, L.expert_slot};
    for (const void* p : i32s)
        if (!aligned(p, 4)) return EP_ERR_ARG;
    return hip_status(launch_layout(*shape, topk_idx, L, static_cast<char*>(ws),
                                    static_cast<hipStream_t>(stream)));
}

int ep_get_layout_noalloc(const ep_shape* shape, const int64_t* topk_idx, const ep_layout* layout,
                          uint32_t* errors, void* stream) {
    int rc = check_shape(shape);
    if (rc != EP_OK) return rc;
    if (ws_layout(*shape).tables_end > (size_t)EP_LAYOUT_SCRATCH_BYTES) return EP_ERR_SCRATCH;
    if (!layout || !errors || !aligned(errors, 4) || (shape->T > 0 && !topk_idx) || !aligned(topk_idx, 8))
        return EP_ERR_ARG;
    const ep_layout& L = *layout;
    if (!aligned(L.is_token_in_rank, 16) || !aligned(L.is_token_in_group, 16)) return EP_ERR_ARG;
    if (L.expert_slot && !L.expert_offsets) return EP_ERR_ARG;
    const void* i32s[] = {L.tokens_per_expert, L.tokens_per_rank, L.tokens_per_group,
                          L.expert_offsets, L.rank_offsets, L.group_offsets, L.slot,
                          L.group_slot, L.expert_slot};
    for (const void* p : i32s)
        if (!aligned(p, 4)) return EP_ERR_ARG;
    return hip_status(launch_layout_noalloc(*shape, topk_idx, L, errors,
                                            static_cast<hipStream_t>(stream)));
}

int ep_dispatch(const ep_shape* shape, const ep_layout* layout, const ep_tokens* tokens,
                const ep_recv* recv, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(shape);
    if (rc != EP_OK) return rc;
    if ((rc = check_ws(shape, ws, ws_bytes)) != EP_OK) return rc;
    if (!layout || !tokens || !recv || recv->capacity < 0) return EP_ERR_ARG;
    if (shape->T > 0 && (!layout->slot || !tokens->topk_idx)) return EP_ERR_ARG;
    if (shape->T > 0 &&
        ((recv->x && !tokens->x) || (recv->x_fp8 && !tokens->x_fp8) ||
         (recv->x_scales && !tokens->x_scales) || (recv->topk_weights && !tokens->topk_weights)))
        return EP_ERR_ARG;
    if ((tokens->x_fp8 || recv->x_fp8) && shape->H % 16 != 0) return EP_ERR_ARG;
    if ((tokens->x_scales || recv->x_scales) && shape->H % 128 != 0) return EP_ERR_ARG;
    if (!aligned(tokens->x, 16) || !aligned(tokens->x_fp8, 16) || !aligned(recv->x, 16) ||
        !aligned(recv->x_fp8, 16) || !aligned(tokens->x_scales, 4) || !aligned(recv->x_scales, 4) ||
        !aligned(tokens->topk_idx, 8) || !aligned(tokens->topk_weights, 4) ||
        !aligned(recv->src_idx, 4) || !aligned(recv->topk_idx, 4) ||
        !aligned(recv->topk_weights, 4) || !aligned(layout->slot, 4))
        return EP_ERR_ARG;
    return hip_status(launch_dispatch(*shape, *layout, *tokens, *recv, static_cast<char*>(ws),
                                      static_cast<hipStream_t>(stream)));
}

int ep_dispatch_expand(const ep_shape* shape, const ep_layout* layout, const ep_tokens* tokens,
                       const ep_recv* recv, void* ws, size_t ws_bytes, void* stream) {
    if (!layout) return EP_ERR_ARG;
    ep_layout rows = *layout;
    rows.slot = layout->expert_slot;
    return ep_dispatch(shape, &rows, tokens, recv, ws, ws_bytes, stream);
}

int ep_hierarchical_dispatch(const ep_shape* shape, const ep_layout* layout,
                             const ep_tokens* tokens, uint32_t epoch, int steps,
                             void* group_buf, int64_t group_cap, void* peer_buf,
                             int64_t peer_cap, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(shape);
    if (rc != EP_OK) return rc;
    if ((rc = check_ws(shape, ws, ws_bytes)) != EP_OK) return rc;
    if (!layout || !tokens || epoch == 0 || steps < 1 || steps > 3) return EP_ERR_ARG;
    if (group_cap < 0 || peer_cap < 0) return EP_ERR_ARG;
    if ((steps & EP_HIER_SCALEOUT) && shape->T > 0 &&
        (!tokens->x || !tokens->topk_idx || !tokens->topk_weights || !layout->group_slot ||
         (group_cap > 0 && !group_buf)))
        return EP_ERR_ARG;
    if ((steps & EP_HIER_FORWARD) &&
        (!layout->group_offsets || (shape->T > 0 && !layout->slot) || (group_cap > 0 && !group_buf) ||
         (peer_cap > 0 && !peer_buf)))
        return EP_ERR_ARG;
    if (tokens->x_fp8 && shape->H % 16 != 0) return EP_ERR_ARG;
    if (tokens->x_scales && shape->H % 128 != 0) return EP_ERR_ARG;
    if (!aligned(tokens->x, 16) || !aligned(tokens->x_fp8, 16) || !aligned(tokens->x_scales, 4) ||
        !aligned(tokens->topk_idx, 8) || !aligned(tokens->topk_weights, 4) ||
        !aligned(group_buf, 16) || !aligned(peer_buf, 16))
        return EP_ERR_ARG;
    return hip_status(launch_hier(*shape, *layout, *tokens, epoch, steps, group_buf, group_cap,
                                  peer_buf, peer_cap, static_cast<char*>(ws),
                                  static_cast<hipStream_t>(stream)));
}

int ep_hierarchical_dispatch_fused(const ep_shape* shape, const ep_layout* layout,
                                   const ep_tokens* tokens, uint32_t epoch, void* group_buf,
                                   int64_t group_cap, void* peer_buf, int64_t peer_cap,
                                   const ep_fused_opts* opts, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(shape);
    if (rc != EP_OK) return rc;
    if ((rc = check_ws(shape, ws, ws_bytes)) != EP_OK) return rc;
    if (!layout || !tokens || epoch == 0 || group_cap < 0 || peer_cap < 0) return EP_ERR_ARG;
    if (shape->T > 0 &&
        (!tokens->x || !tokens->topk_idx || !tokens->topk_weights || !layout->group_slot ||
         !layout->slot || (group_cap > 0 && !group_buf) || (peer_cap > 0 && !peer_buf)))
        return EP_ERR_ARG;
    if (tokens->x_fp8 && shape->H % 16 != 0) return EP_ERR_ARG;
    if (tokens->x_scales && shape->H % 128 != 0) return EP_ERR_ARG;
    if (!aligned(tokens->x, 16) || !aligned(tokens->x_fp8, 16) || !aligned(tokens->x_scales, 4) ||
        !aligned(tokens->topk_idx, 8) || !aligned(tokens->topk_weights, 4) ||
        !aligned(group_buf, 16) || !aligned(peer_buf, 16) || !aligned(layout->slot, 4) ||
        !aligned(layout->group_slot, 4))
        return EP_ERR_ARG;
    ep_fused_opts o = {0, 0, 0, 0, 0};
    if (opts) o = *opts;
    const int tile = o.tile_tokens ? o.tile_tokens : kFusedDefaultTile;
    if (tile < kFusedMinTile || tile > kFusedMaxTile || (o.test_flags & ~EP_FUSED_WITHHOLD)) return EP_ERR_ARG;
    // Ring mode: more batches than the fixed lag (the producer of batch b
    // waits for the forwarding of batch b - ring), and room for all of them.
    if (o.ring_batches < 0 || (o.ring_batches > 0 && o.ring_batches <= kFusedLag)) return EP_ERR_ARG;
    // Ring rows are 32-bit indices on the device.
    const int64_t ring_rows = (int64_t)o.ring_batches * tile * std::min(shape->K, shape->G);
    if (o.ring_batches > 0 && (group_cap < ring_rows || ring_rows > INT32_MAX)) return EP_ERR_ARG;
    const uint32_t timeout = o.timeout_us ? o.timeout_us : 100000u;
    const int withhold = (o.test_flags & EP_FUSED_WITHHOLD) ? o.withhold_batch : -1;
    return hip_status(launch_hier_fused(*shape, *layout, *tokens, epoch, group_buf, group_cap, peer_buf,
                                        peer_cap, tile, timeout, withhold, o.ring_batches,
                                        static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

int ep_combine(const ep_shape* shape, const ep_layout* layout, const void* y, int64_t y_rows,
               int64_t y_row_stride, int y_format, uint32_t epoch, const float* topk_weights,
               uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(shape);
    if (rc != EP_OK) return rc;
    if ((rc = check_ws(shape, ws, ws_bytes)) != EP_OK) return rc;
    if (!layout || y_rows < 0) return EP_ERR_ARG;
    if (y_format != EP_FMT_PLAIN && y_format != EP_FMT_CHUNKED) return EP_ERR_ARG;
    if (shape->T > 0 && (!layout->slot || !topk_weights || !out || (y_rows > 0 && !y)))
        return EP_ERR_ARG;
    if (y_format == EP_FMT_PLAIN && (y_row_stride % 16 != 0 || y_row_stride < 2 * (int64_t)shape->H))
        return EP_ERR_ARG;
    if (y_format == EP_FMT_CHUNKED) {
        const int64_t hidden_blocks = (2 * (int64_t)shape->H + kChunkPayload - 1) / kChunkPayload;
        if (epoch == 0 || y_row_stride % kChunkBytes != 0 || y_row_stride < hidden_blocks * kChunkBytes)
            return EP_ERR_ARG;
    }
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(topk_weights, 4) || !aligned(layout->slot, 4))
        return EP_ERR_ARG;
    return hip_status(launch_combine(*shape, *layout, y, y_rows, y_row_stride, y_format, epoch,
                                     topk_weights, out, static_cast<char*>(ws),
                                     static_cast<hipStream_t>(stream)));
}

int ep_combine_expand(const ep_shape* shape, const ep_layout* layout, const void* y,
                      int64_t y_rows, int64_t y_row_stride, int y_format, uint32_t epoch,
                      const float* topk_weights, uint16_t* out, void* ws, size_t ws_bytes,
                      void* stream) {
    if (!layout) return EP_ERR_ARG;
    ep_layout rows = *layout;
    rows.slot = layout->expert_slot;
    return ep_combine(shape, &rows, y, y_rows, y_row_stride, y_format, epoch, topk_weights, out, ws,
                      ws_bytes, stream);
}

int64_t ep_partial_row_bytes(const ep_shape* shape) {
    if (check_shape(shape) != EP_OK) return -1;
    return (int64_t)kChunkBytes * ((2 * (int64_t)shape->H + kChunkPayload - 1) / kChunkPayload);
}

int ep_combine_two_level(const ep_shape* shape, const ep_layout* layout, const int64_t* topk_idx,
                         const void* y, int64_t y_rows, int64_t y_row_stride, int y_format,
                         uint32_t epoch, const float* topk_weights, void* group_buf,
                         int64_t group_cap, int steps, uint16_t* out, void* ws, size_t ws_bytes,
                         void* stream) {
    int rc = check_shape(shape);
    if (rc != EP_OK) return rc;
    if ((rc = check_ws(shape, ws, ws_bytes)) != EP_OK) return rc;
    if (!layout || y_rows < 0 || group_cap < 0 || epoch == 0 || steps < 1 || steps > 3) return EP_ERR_ARG;
    if (y_format != EP_FMT_PLAIN && y_format != EP_FMT_CHUNKED) return EP_ERR_ARG;
    if (shape->T > 0) {
        if (!topk_idx || !layout->group_slot || (group_cap > 0 && !group_buf)) return EP_ERR_ARG;
        if ((steps & 1) && (!layout->slot || !topk_weights || (y_rows > 0 && !y))) return EP_ERR_ARG;
        if ((steps & 2) && !out) return EP_ERR_ARG;
    }
    const int64_t hidden_blocks = (2 * (int64_t)shape->H + kChunkPayload - 1) / kChunkPayload;
    if ((steps & 1) && y_format == EP_FMT_PLAIN && (y_row_stride % 16 != 0 || y_row_stride < 2 * (int64_t)shape->H))
        return EP_ERR_ARG;
    if ((steps & 1) && y_format == EP_FMT_CHUNKED &&
        (y_row_stride % kChunkBytes != 0 || y_row_stride < hidden_blocks * kChunkBytes))
        return EP_ERR_ARG;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(group_buf, 16) || !aligned(topk_weights, 4) ||
        !aligned(topk_idx, 8) || !aligned(layout->slot, 4) || !aligned(layout->group_slot, 4))
        return EP_ERR_ARG;
    return hip_status(launch_combine_two_level(*shape, *layout, topk_idx, y, y_rows, y_row_stride,
                                               y_format, epoch, topk_weights, group_buf, group_cap,
                                               steps, out, static_cast<char*>(ws),
                                               static_cast<hipStream_t>(stream)));
}

size_t ep_source_workspace_bytes(const ep_shape* shape, int32_t S) {
    if (check_shape(shape) != EP_OK || S < 1 || S > EP_MAX_RANKS) return 0;
    return ws_source(*shape, S).total;
}

static int check_sources(const ep_shape* shape, const ep_sources* src, void* ws, size_t ws_bytes) {
    int rc = check_shape(shape);
    if (rc != EP_OK) return rc;
    if (!src || src->S < 1 || src->capacity < 0) return EP_ERR_ARG;
    if (src->S > EP_MAX_RANKS) return EP_ERR_UNSUPPORTED;
    if ((int64_t)shape->R * src->S * src->capacity > INT32_MAX) return EP_ERR_UNSUPPORTED;
    if (!ws || !aligned(ws, 256) || ws_bytes < ws_source(*shape, src->S).total) return EP_ERR_ARG;
    return EP_OK;
}

int ep_source_layout(const ep_shape* shape, const int64_t* topk_idx, const ep_sources* sources,
                     void* ws, size_t ws_bytes, void* stream) {
    int rc = check_sources(shape, sources, ws, ws_bytes);
    if (rc != EP_OK) return rc;
    const ep_sources& X = *sources;
    if (!X.counts || !X.recv_offsets || (shape->T > 0 && (!topk_idx || !X.src_slot))) return EP_ERR_ARG;
    if (!aligned(topk_idx, 8) || !aligned(X.counts, 4) || !aligned(X.recv_offsets, 4) ||
        !aligned(X.src_slot, 4))
        return EP_ERR_ARG;
    return hip_status(launch_source_layout(*shape, topk_idx, X, static_cast<char*>(ws),
                                           static_cast<hipStream_t>(stream)));
}

int ep_source_dispatch(const ep_shape* shape, const ep_sources* sources, const ep_tokens* tokens,
                       uint32_t epoch, void* staging, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_sources(shape, sources, ws, ws_bytes);
    if (rc != EP_OK) return rc;
    if (!tokens || epoch == 0) return EP_ERR_ARG;
    const int64_t rows = (int64_t)shape->R * sources->S * sources->capacity;
    if (shape->T > 0 && (!tokens->x || !tokens->topk_idx || !tokens->topk_weights ||
                         !sources->src_slot || (rows > 0 && !staging)))
        return EP_ERR_ARG;
    if (tokens->x_fp8 && shape->H % 16 != 0) return EP_ERR_ARG;
    if (tokens->x_scales && shape->H % 128 != 0) return EP_ERR_ARG;
    if (!aligned(tokens->x, 16) || !aligned(tokens->x_fp8, 16) || !aligned(tokens->x_scales, 4) ||
        !aligned(tokens->topk_idx, 8) || !aligned(tokens->topk_weights, 4) ||
        !aligned(staging, 16) || !aligned(sources->src_slot, 4))
        return EP_ERR_ARG;
    return hip_status(launch_send_rows(*shape, *tokens, sources->src_slot, rows, epoch, staging,
                                       static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

int ep_copy_epilogue(const ep_shape* shape, const ep_sources* sources, const void* staging,
                     uint32_t epoch, int seg_flags, const ep_recv* recv, void* ws,
                     size_t ws_bytes, void* stream) {
    int rc = check_sources(shape, sources, ws, ws_bytes);
    if (rc != EP_OK) return rc;
    if (!recv || recv->capacity < 0 || epoch == 0 || !sources->recv_offsets) return EP_ERR_ARG;
    if (!(seg_flags & EP_SEG_BF16) || (seg_flags & ~7)) return EP_ERR_ARG;
    if ((seg_flags & EP_SEG_FP8) && shape->H % 16 != 0) return EP_ERR_ARG;
    if ((seg_flags & EP_SEG_SCALES) && shape->H % 128 != 0) return EP_ERR_ARG;
    if ((recv->x_fp8 && !(seg_flags & EP_SEG_FP8)) || (recv->x_scales && !(seg_flags & EP_SEG_SCALES)))
        return EP_ERR_ARG;
    if (sources->capacity > 0 && !staging) return EP_ERR_ARG;
    if (!aligned(staging, 16) || !aligned(recv->x, 16) || !aligned(recv->x_fp8, 16) ||
        !aligned(recv->x_scales, 4) || !aligned(recv->src_idx, 4) || !aligned(recv->topk_idx, 4) ||
        !aligned(recv->topk_weights, 4) || !aligned(sources->recv_offsets, 4))
        return EP_ERR_ARG;
    return hip_status(launch_copy_epilogue(*shape, *sources, staging, epoch, seg_flags, *recv,
                                           static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

int ep_source_dispatch_fused(const ep_shape* shape, const ep_sources* sources, const ep_tokens* tokens,
                             uint32_t epoch, void* staging, const ep_recv* recv, void* ws, size_t ws_bytes,
                             void* stream) {
    int rc = check_sources(shape, sources, ws, ws_bytes);
    if (rc != EP_OK) return rc;
    if (!tokens || !recv || recv->capacity < 0 || epoch == 0 || !sources->recv_offsets) return EP_ERR_ARG;
    const int64_t rows = (int64_t)shape->R * sources->S * sources->capacity;
    if (shape->T > 0 && (!tokens->x || !tokens->topk_idx || !tokens->topk_weights ||
                         !sources->src_slot || (rows > 0 && !staging)))
        return EP_ERR_ARG;
    if (tokens->x_fp8 && shape->H % 16 != 0) return EP_ERR_ARG;
    if (tokens->x_scales && shape->H % 128 != 0) return EP_ERR_ARG;
    if ((recv->x_fp8 && !tokens->x_fp8) || (recv->x_scales && !tokens->x_scales)) return EP_ERR_ARG;
    if (!aligned(tokens->x, 16) || !aligned(tokens->x_fp8, 16) || !aligned(tokens->x_scales, 4) ||
        !aligned(tokens->topk_idx, 8) || !aligned(tokens->topk_weights, 4) || !aligned(staging, 16) ||
        !aligned(sources->src_slot, 4) || !aligned(recv->x, 16) || !aligned(recv->x_fp8, 16) ||
        !aligned(recv->x_scales, 4) || !aligned(recv->src_idx, 4) || !aligned(recv->topk_idx, 4) ||
        !aligned(recv->topk_weights, 4) || !aligned(sources->recv_offsets, 4))
        return EP_ERR_ARG;
    return hip_status(launch_source_fused(*shape, *sources, *tokens, epoch, staging, *recv,
                                          static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

int ep_clear_errors(void* ws, void* stream) {
    if (!ws || !aligned(ws, 256)) return EP_ERR_ARG;
    hipLaunchKernelGGL(clear_error_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<uint32_t*>(ws));
    return hip_status(hipGetLastError());
}

// Reads error word `which` (0: current pass, 1: since the last clear).
static int read_error_word(void* ws, void* stream, uint32_t* bits, int which) {
    if (!ws || !bits || !aligned(ws, 256)) return EP_ERR_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t v[2] = {0u, 0u};
    if (hipMemcpyAsync(v, ws, sizeof v, hipMemcpyDeviceToHost, st) != hipSuccess) return EP_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return EP_ERR_HIP;
    *bits = v[which];
    return v[which] ? EP_ERR_DEVICE : EP_OK;
}

int ep_check_errors(void* ws, void* stream, uint32_t* bits) {
    return read_error_word(ws, stream, bits, 0);
}

int ep_check_sticky_errors(void* ws, void* stream, uint32_t* bits) {
    return read_error_word(ws, stream, bits, 1);
}

const char* ep_status_string(int status) {
    switch (status) {
        case EP_OK: return "ok";
        case EP_ERR_ARG: return "invalid argument (null or misaligned pointer, bad shape or size)";
        case EP_ERR_UNSUPPORTED: return "shape outside the supported limits";
        case EP_ERR_HIP: return "HIP runtime or launch error";
        case EP_ERR_SCRATCH:
            return "shape too large for the allocation-free call's static scratch "
                   "(ep_workspace_bytes(shape) > EP_LAYOUT_SCRATCH_BYTES); use ep_get_layout";
        case EP_ERR_DEVICE:
            return "device-detected error: bad expert id, capacity exceeded or flag/epoch mismatch "
                   "(the bits are in the workspace error word)";
        default: return "unknown status";
    }
}

}  // extern "C"
