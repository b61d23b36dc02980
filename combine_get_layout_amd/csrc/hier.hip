// hier.hip -- ep_hierarchical_dispatch on gfx950: two-level dispatch with
// 512-byte data-as-flag chunked records.
//
// What is computed follows "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK
// 复制机制" §3.6 (scale-out warps write each token to the destination group's
// receive buffer, forward warps store it from there to the scale-up peer) and
// "07: DeepEP Intra/Inter-node 协调 — NVLink Scale-up + RDMA Scale-out 三阶段流水
// 线的代码实证" (hybrid scale-out stage: one store per destination group; forward
// warps: scale-up rank = expert / experts_per_rank). The record is the
// TokenLayout of the V2 page, §3.4 (hidden | scales | metadata, 16 B pieces),
// cut into the blocks of "Ascend Send Ordering", 导言: 512 B = 480 B payload +
// 32 B flag.
//
// CDNA4 mapping: a 512 B block is 32 16-byte vectors, so one wave64 store of a
// 16-byte vector per lane covers exactly two blocks: lanes 0-29 carry payload
// vectors of block 2i, lanes 30-31 its flag, lanes 32-61 and 62-63 the same
// for block 2i+1. Record vector q sits in block q / 30, vector q % 30.
//   step 1: four waves per token, each assembling a run of its chunked
//           record's blocks in VGPRs, stream it once to each destination
//           group's row.
//   step 2: one wave per group-region row (the row count is read on the
//           device; grid-stride past 262,144 rows): check every block's flag,
//           read src and top-k ids from the record, then stream the row to
//           each scale-up peer's row.
//   fused : both steps in one persistent launch; job i writes batch i of the
//           tokens' records and publishes its flag, then forwards batch
//           i - lag, whose records are then still in the MALL.
// Step 1 also serves several source ranks on one GPU: given one staging row
// per (token, destination rank) instead of per group, it is their send.
#include <algorithm>

#include "ep_device.h"
#include "ep_epilogue.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kPieceIters = 16;  // wave iterations (2 blocks each) held in VGPRs

#ifndef EP_SO_SPLIT
#define EP_SO_SPLIT 4  // scale-out: waves per token, each writing a run of the record's blocks (measured best of 1, 2, 4)
#endif
constexpr int kSoSplit = EP_SO_SPLIT;
#ifndef EP_SO_NTSTORE
#define EP_SO_NTSTORE 1  // scale-out: non-temporal stores of the group rows (else plain stores)
#endif
#ifndef EP_FWD_NTSTORE
#define EP_FWD_NTSTORE 1  // forward: non-temporal stores of the peer rows (else plain stores)
#endif
#ifndef EP_FUSED_WAVE
#define EP_FUSED_WAVE 0  // fused kernel: each wave takes its own batches (else each workgroup;
                         // measured slower: the counters' atomics serialise at small batches)
#endif
#ifndef EP_FUSED_COHERENT
#define EP_FUSED_COHERENT 1  // fused kernel: device-scope stores and loads of group rows (else fences)
#endif

// How a scale-out wave stores its record: non-temporal, plain, or with
// device scope (written through the XCD's L2, so that once the wave's stores
// are acknowledged every CU of the device reads them).
constexpr int kStoreStream = 0, kStorePlain = 1, kStoreDevice = 2;

// Device-scope 16-byte store / load at byte `off` of a row of `bytes` bytes
// (a buffer resource over the row: an access past its end is dropped by the
// hardware). Cache-policy 16 is the device-scope bit (sc1).
constexpr int kDeviceScope = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void st16_device(void* row, int64_t bytes, int64_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, row_rsrc(row, bytes), (int)off, 0, kDeviceScope);
}
__device__ __forceinline__ u32x4 ld16_device(const void* row, int64_t bytes, int64_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(row, bytes), (int)off, 0, kDeviceScope);
}
__device__ __forceinline__ uint32_t ld4_device(const void* row, int64_t bytes, int64_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(row_rsrc(row, bytes), (int)off, 0, kDeviceScope);
}
// Wait until every vector memory access of this wave has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
constexpr int kSoPiece = kPieceIters / kSoSplit;  // wave iterations a scale-out wave holds

struct HierArgs {
    int T, H, K, E, R, G, epr, P;
    RecordGeom geom;
    const int32_t* slot;
    const int32_t* group_slot;
    const int32_t* group_offsets;
    const int64_t* topk;
    const float* topk_w;
    const uint8_t* x;
    const uint8_t* x_fp8;
    const float* x_scales;
    uint8_t* group_buf;
    int64_t group_cap;
    uint8_t* peer_buf;
    int64_t peer_cap;
    uint32_t epoch;
    uint32_t* err;
};

// Record vector q >= q_scales of token t (16 bytes): scales, expert ids,
// weights, source index, or zero past the end of the record. Every
// candidate value is loaded (indices clamped into the token's arrays) and
// the vector is then selected by q: loads under per-lane branches were
// issued one round trip at a time.
__device__ __forceinline__ u32x4 meta_vector(const HierArgs& a, int t, int q) {
    const RecordGeom& g = a.geom;
    const int ns = a.H / 128;
    const int i0 = max(0, (q - g.q_scales) * 4);
    const int k0 = max(0, (q - g.q_idx) * 4), kw0 = max(0, (q - g.q_w) * 4);
    float sc[4] = {0.f, 0.f, 0.f, 0.f}, wt[4];
    int64_t e[4];
    if (a.x_scales) {  // present whenever the record has scales (then ns >= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = a.x_scales[(int64_t)t * ns + min(i0 + j, ns - 1)];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        e[j] = a.topk[(int64_t)t * a.K + min(k0 + j, a.K - 1)];
        wt[j] = a.topk_w[(int64_t)t * a.K + min(kw0 + j, a.K - 1)];
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (q < g.q_idx) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i0 + j < ns) v[j] = __float_as_uint(sc[j]);
    } else if (q < g.q_w) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (k0 + j < a.K) v[j] = (uint32_t)(expert_ok(e[j], a.E) ? (int32_t)e[j] : -1);
    } else if (q < g.q_src) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (kw0 + j < a.K) v[j] = __float_as_uint(wt[j]);
    } else if (q == g.q_src) {
        v[0] = (uint32_t)t;
    }
    return v;
}

// Scale-out write of wave-slice `part` (of SPLIT) of token t's chunked record
// to each destination group's row, PIECE wave-iterations held at a time.
// Wave-slice `part` (of SPLIT) of token t's chunked record, PIECE
// wave-iterations held at a time, stored to group row gs (lane k's value)
// for every lane k in dest.
template <int SPLIT, int PIECE, int STORE>
__device__ __forceinline__ void write_record(const HierArgs& a, int t, int part, uint64_t dest, int gs) {
    const int lane = lane_id();
    const int nchunks = a.geom.nchunks;
    const int iters = (nchunks + 1) / 2;
    const int64_t stride = a.geom.stride;
    const u32x4 flag = {a.epoch, a.epoch, a.epoch, a.epoch};
    const int c_half = lane >> 5, w = lane & 31;
    const int q_fp8 = a.geom.q_fp8, q_meta = a.geom.q_scales;
    const uint8_t* x_row = a.x + (int64_t)t * a.H * 2;
    const uint8_t* f_row = a.x_fp8 ? a.x_fp8 + (int64_t)t * a.H : x_row;
    // This wave's run of wave-iterations of the record.
    const int per = (iters + SPLIT - 1) / SPLIT;
    const int it_lo = min(iters, part * per), it_hi = min(iters, it_lo + per);
    for (int it0 = it_lo; it0 < it_hi; it0 += PIECE) {
        u32x4 v[PIECE];
        // 1. Hidden vectors (bf16, then fp8): one unconditional load per
        //    iteration; lanes holding anything else load the row's first
        //    vector (in bounds, cached) and are overwritten below.
#pragma unroll
        for (int j = 0; j < PIECE; ++j) {
            const int q = (2 * (it0 + j) + c_half) * kChunkPayloadVecs + w;
            const uint8_t* src = q < q_fp8 ? x_row + (int64_t)q * 16
                                 : (q < q_meta ? f_row + (int64_t)(q - q_fp8) * 16 : x_row);
            v[j] = ld16(src);
        }
        // 2. Metadata and padding: only in the iterations that reach them.
#pragma unroll
        for (int j = 0; j < PIECE; ++j) {
            const int q = (2 * (it0 + j) + c_half) * kChunkPayloadVecs + w;
            const int q_last = (2 * (it0 + j) + 2) * kChunkPayloadVecs - 1;  // wave-uniform
            if (q_last >= q_meta && w < kChunkPayloadVecs && q >= q_meta) v[j] = meta_vector(a, t, q);
        }
        // 3. Flags.
#pragma unroll
        for (int j = 0; j < PIECE; ++j)
            if (w >= kChunkPayloadVecs) v[j] = flag;
        for (uint64_t m = dest; m; m &= m - 1) {
            const int k = __ffsll((unsigned long long)m) - 1;
            uint8_t* row = a.group_buf + (int64_t)readlane(gs, k) * stride;
#pragma unroll
            for (int j = 0; j < PIECE; ++j) {
                const int c = 2 * (it0 + j) + c_half;
                if (it0 + j < it_hi && c < nchunks) {
                    if constexpr (STORE == kStoreStream) st16_stream(row + chunk_lane_offset(it0 + j, lane), v[j]);
                    else if constexpr (STORE == kStorePlain) st16(row + chunk_lane_offset(it0 + j, lane), v[j]);
                    else st16_device(row, stride, chunk_lane_offset(it0 + j, lane), v[j]);
                }
            }
        }
    }
}

// Scale-out write of wave-slice `part` of token t's record to each
// destination group's row (the first lane of each group).
template <int SPLIT, int PIECE, int STORE = kStoreStream>
__device__ __forceinline__ void scaleout_token(const HierArgs& a, int t, int part) {
    const int lane = lane_id();
    int gs = -1;
    if (lane < a.K) gs = a.group_slot[(int64_t)t * a.K + lane];
    bool first = gs >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int sj = readlane(gs, j);
        if (j < lane && sj == gs) first = false;
    }
    const bool over = first && gs >= a.group_cap;
    if (over && part == 0) report(a.err, EP_DEVERR_CAPACITY);
    const uint64_t dest = __ballot(first && !over);
    if (!dest) return;
    write_record<SPLIT, PIECE, STORE>(a, t, part, dest, gs);
}

__global__ __launch_bounds__(kBlockThreads) void scaleout_kernel(HierArgs a) {
    const int gw = blockIdx.x * kWavesPerBlock + wave_in_block();
    const int t = gw / kSoSplit, part = gw % kSoSplit;
    if (t >= a.T) return;
    scaleout_token<kSoSplit, kSoPiece, EP_SO_NTSTORE ? kStoreStream : kStorePlain>(a, t, part);
}

// Address of record byte b (4-byte aligned, never straddling a block) in a
// chunked row.
__device__ __forceinline__ const uint8_t* record_byte(const uint8_t* row, int64_t b) {
    return row + (b / kChunkPayload) * kChunkBytes + b % kChunkPayload;
}

// Forward of group row n (of group g) to each of its scale-up peers: the
// whole record is loaded together with src and this lane's expert id (its
// flag lanes load the flags); every block's flag must equal epoch, else the
// row is dropped with EP_DEVERR_FLAG. Destinations: the first lane of each
// distinct rank of group g among the record's ids, at the layout's slot of
// (src, lane).
// t_known >= 0: the caller knows the row's token, so the slots are loaded
// together with the record and the record's src must equal it.
template <bool DEVICE_LOADS = false>
__device__ __forceinline__ void forward_row(const HierArgs& a, int64_t n, int g, int t_known = -1) {
    const int lane = lane_id();
    const int nchunks = a.geom.nchunks;
    const int iters = (nchunks + 1) / 2;
    const int64_t stride = a.geom.stride;
    const int64_t off_idx = (int64_t)a.geom.q_idx * 16;
    const int64_t off_src = (int64_t)a.geom.q_src * 16;
    const int c_half = lane >> 5, wv = lane & 31;
    const uint8_t* src_row = a.group_buf + n * stride;
    // The first piece (the whole record when it fits) is requested at once,
    // together with the metadata. In the fused launch (device-scope loads)
    // also for longer records, with the flags of the later pieces: one round
    // trip before the flag check instead of two (the fused launch at H = 8,192
    // 1,094 -> 976 us, at 16,384 1,929 -> 1,829 us). The forward launch keeps
    // a flag pre-pass for those: there the change took its registers from 193
    // to 166, and the forward of one-piece records (hier8x8) got 34 us slower.
    const bool one_piece = iters <= kPieceIters;
    const bool hold_first = DEVICE_LOADS || one_piece;
    u32x4 v[kPieceIters];
    if (hold_first) {
#pragma unroll
        for (int j = 0; j < kPieceIters; ++j) {
            const int c = min(2 * j + c_half, nchunks - 1);
            const int64_t off = (int64_t)c * kChunkBytes + (int64_t)wv * 16;
            if constexpr (DEVICE_LOADS) v[j] = ld16_device(src_row, stride, off);
            else v[j] = ld16_stream(src_row + off);  // read once: non-temporal (-7 us per hier8x8 step)
        }
    }
    int32_t src, id, d_early = -1;
    if (t_known >= 0 && lane < a.K) d_early = a.slot[(int64_t)t_known * a.K + lane];
    if constexpr (DEVICE_LOADS) {
        src = (int32_t)ld4_device(src_row, stride, record_byte(src_row, off_src) - src_row);
        id = (int32_t)ld4_device(src_row, stride, record_byte(src_row, off_idx + 4 * min(lane, a.K - 1)) - src_row);
    } else {
        src = *reinterpret_cast<const int32_t*>(record_byte(src_row, off_src));
        id = *reinterpret_cast<const int32_t*>(record_byte(src_row, off_idx + 4 * min(lane, a.K - 1)));
    }
    bool ok = true;
    if (hold_first) {
        if constexpr (DEVICE_LOADS) {
            // Flags of the blocks past the first piece (flag vector i: block i / 2).
            for (int i = 4 * kPieceIters + lane; i < 2 * nchunks; i += kWave) {
                const int64_t off = (int64_t)(i >> 1) * kChunkBytes + kChunkPayload + (i & 1) * 16;
                const u32x4 f = ld16_device(src_row, stride, off);
                ok &= f[0] == a.epoch && f[1] == a.epoch && f[2] == a.epoch && f[3] == a.epoch;
            }
        }
#pragma unroll
        for (int j = 0; j < kPieceIters; ++j) {
            const bool is_flag = wv >= kChunkPayloadVecs && j < iters && 2 * j + c_half < nchunks;
            const u32x4 f = v[j];
            ok &= !is_flag || (f[0] == a.epoch && f[1] == a.epoch && f[2] == a.epoch && f[3] == a.epoch);
        }
    } else {
        for (int i = lane; i < 2 * nchunks; i += kWave) {
            const int64_t off = (int64_t)(i >> 1) * kChunkBytes + kChunkPayload + (i & 1) * 16;
            const u32x4 f = DEVICE_LOADS ? ld16_device(src_row, stride, off) : ld16(src_row + off);
            ok &= f[0] == a.epoch && f[1] == a.epoch && f[2] == a.epoch && f[3] == a.epoch;
        }
    }
    if (__ballot(!ok) || src < 0 || src >= a.T || (t_known >= 0 && src != t_known)) {
        if (lane == 0) report(a.err, EP_DEVERR_FLAG);
        return;
    }
    int32_t r = -1, d = -1;
    if (lane < a.K && id >= 0 && id < a.E && (id / a.epr) / a.P == g) {
        r = id / a.epr;
        d = t_known >= 0 ? d_early : a.slot[(int64_t)src * a.K + lane];
    }
    bool first = r >= 0 && d >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int rj = readlane(r, j);
        if (j < lane && rj == r) first = false;
    }
    const bool over = first && d >= a.peer_cap;
    if (over) report(a.err, EP_DEVERR_CAPACITY);
    const uint64_t dest = __ballot(first && !over);
    if (!dest) return;

    for (int it0 = 0; it0 < iters; it0 += kPieceIters) {
        if (DEVICE_LOADS ? it0 > 0 : !one_piece) {  // else this piece is already held
#pragma unroll
            for (int j = 0; j < kPieceIters; ++j) {
                const int c = 2 * (it0 + j) + c_half;
                if (it0 + j < iters && c < nchunks)
                    v[j] = DEVICE_LOADS ? ld16_device(src_row, stride, chunk_lane_offset(it0 + j, lane))
                                        : ld16_stream(src_row + chunk_lane_offset(it0 + j, lane));
            }
        }
        for (uint64_t m = dest; m; m &= m - 1) {
            const int k = __ffsll((unsigned long long)m) - 1;
            uint8_t* row = a.peer_buf + (int64_t)readlane(d, k) * stride;
#pragma unroll
            for (int j = 0; j < kPieceIters; ++j) {
                const int c = 2 * (it0 + j) + c_half;
                if (it0 + j < iters && c < nchunks) {
                    if constexpr (EP_FWD_NTSTORE) st16_stream(row + chunk_lane_offset(it0 + j, lane), v[j]);
                    else st16(row + chunk_lane_offset(it0 + j, lane), v[j]);
                }
            }
        }
    }
}

constexpr int kForwardMaxBlocks = 65536;  // workgroups of the forward launch at most

// One wave per group-region row (grid-stride when the grid is capped); the
// row count is read on the device. The row's group is the number of groups g >= 1 whose region starts
// at or before n (empty groups have equal starts).
__global__ __launch_bounds__(kBlockThreads) void forward_kernel(HierArgs a) {
    __shared__ int32_t goff[EP_MAX_GROUPS + 1];
    for (int i = threadIdx.x; i <= a.G; i += kBlockThreads) goff[i] = a.group_offsets[i];
    __syncthreads();
    const int lane = lane_id();
    const int64_t n_rows = min((int64_t)goff[a.G], a.group_cap);
    const int64_t wave_stride = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block(); n < n_rows;
         n += wave_stride) {
        int g = 0;
        for (int base = 1; base <= a.G; base += kWave) {
            const int j = base + lane;
            g += __popcll(__ballot(j <= a.G && goff[j] <= n));
        }
        forward_row(a, n, g);
    }
}

// ---------------------------------------------------------------------------
// Both steps in one persistent launch, with one flag per batch of tokens
// ("Ascend Send Ordering", 方案一: the payload of a batch is written without
// ordering, then one ordered flag publishes the whole batch; Stage1 of the
// hierarchical path the same; "07: DeepEP Intra/Inter-node 协调": forward
// warps take records from the scale-out buffer as they arrive, waiting with
// a time limit). Batch b = tokens [b*tile, (b+1)*tile).
//   * Production of batch b: its tokens' scale-out records are written with
//     device-scope stores (through the XCD's L2 to the device's coherence
//     point); each wave waits until its stores are acknowledged, and after a
//     barrier one thread stores the batch's flag = epoch (device scope).
//   * Forwarding of batch b: one thread waits for the flag (device-scope
//     polls, bounded by `timeout` clock ticks, after which the batch is
//     skipped with EP_DEVERR_TIMEOUT); after a barrier the group rows of the
//     batch's tokens are read with device-scope loads and forwarded as in
//     step 2 (block flags checked, record's src and ids, the layout's
//     slots).
// Default schedule (EP_FUSED_LAG > 0), a fixed lag: one counter hands out
// jobs 0 .. nbatch + lag - 1 in order, and job i produces batch i, then
// forwards batch i - lag. A group row is therefore read back a bounded
// number of batches after it was written, while it is still in the
// memory-side cache (the 256 MB MALL) instead of being fetched from HBM;
// with the grid sized to hold about 20 MB of records at once, the records
// in flight stay well inside that cache. The other schedule (EP_FUSED_LAG = 0) hands
// out forwarding as soon as a flag is seen and otherwise production, from
// two counters; production then runs far ahead of forwarding and the rows
// come back from HBM.
// Either way a workgroup waits only for a batch whose production another
// running workgroup has already taken on, and production never waits, so
// every wait ends even if the grid is not co-resident; the time limit covers
// the rest. Counters and flags live in the workspace and are zeroed by a
// one-workgroup kernel launched just before (stream ordered, no memset node).
// ---------------------------------------------------------------------------
#ifndef EP_FUSED_WPB
#define EP_FUSED_WPB 2  // waves per workgroup of the workgroup-level fused kernel
#endif
#ifndef EP_FUSED_WG_PER_CU
#define EP_FUSED_WG_PER_CU 0  // > 0: at most this many fused workgroups per CU (0: from the record size)
#endif
#ifndef EP_FUSED_INFLIGHT_BYTES
#define EP_FUSED_INFLIGHT_BYTES (20ll << 20)  // records the fused grid's waves hold at once (about)
#endif
#ifndef EP_FUSED_LAG
#define EP_FUSED_LAG 64  // > 0: job i produces batch i, then forwards batch i - EP_FUSED_LAG
#endif
constexpr int kRingMinLag = 16;  // shortest lag the ring mode takes (batches)
// The host accepts ring sizes above kFusedLag; the ring's waits point at
// earlier jobs only while the ring is longer than the lag.
static_assert(EP_FUSED_LAG <= kFusedLag, "ring sizes are checked against kFusedLag");
constexpr int kFusedWaves = EP_FUSED_WPB;
constexpr int kFusedThreads = kFusedWaves * kWave;

struct FusedArgs {
    HierArgs h;
    int tile;               // tokens per batch
    int nbatch;             // ceil(T / tile)
    int withhold;           // batch whose flag is never published (-1: none)
    int lag;                // fixed-lag schedule: batches between production and forwarding
    int ring;               // > 0: group rows in a ring of this many batches (released by forwarding)
    int gmax;               // ring rows per token: min(K, G)
    uint32_t* freed;        // [nbatch] epoch once batch b's ring rows are read (ring mode)
    uint64_t timeout;       // wall-clock ticks a batch wait may last
    uint32_t* ctr;          // [0] next batch to produce, [1] next batch to forward
    uint32_t* flags;        // [nbatch] epoch once batch b is written
};


__device__ __forceinline__ uint32_t flag_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Take the next job: a published batch to forward if there is one, else a
// batch to produce, else (production all handed out) the next batch to
// forward, to be waited for. kind: 0 produce, 1 forward (flag seen), 2
// forward (wait), 3 done. Called by one thread.
__device__ __forceinline__ int take_job(const FusedArgs& f, int& job) {
    // Both counters are read together (one round trip instead of two: a
    // claim's device-scope accesses are its cost, several microseconds each
    // under contention).
    const uint32_t fb = flag_load(&f.ctr[1]);
    const uint32_t pb = flag_load(&f.ctr[0]);
    if ((int)fb < f.nbatch && flag_load(&f.flags[fb]) == f.h.epoch) {
        uint32_t want = fb;
        if (__hip_atomic_compare_exchange_strong(&f.ctr[1], &want, fb + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
            job = (int)fb;
            return 1;
        }
    }
    if (pb < (uint32_t)f.nbatch) {
        const uint32_t b = atomicAdd(&f.ctr[0], 1u);
        if ((int)b < f.nbatch) {
            job = (int)b;
            return 0;
        }
    }
    const uint32_t b = atomicAdd(&f.ctr[1], 1u);
    if ((int)b < f.nbatch) {
        job = (int)b;
        return 2;
    }
    return 3;
}

// Wait (one thread) until batch `job`'s flag is out, at most f.timeout
// wall-clock ticks; false (and EP_DEVERR_TIMEOUT) if it never comes.
__device__ __forceinline__ bool wait_batch(const FusedArgs& f, int job, uint64_t limit = 0) {
    if (wait_flag_bounded(&f.flags[job], f.h.epoch, limit ? limit : f.timeout)) return true;
    report(f.h.err, EP_DEVERR_TIMEOUT);
    return false;
}

// The group rows of token t, forwarded in ascending lane order (the first
// lane of each group).
template <bool DEVICE_LOADS>
__device__ __forceinline__ void forward_token(const HierArgs& a, int t) {
    const int lane = lane_id();
    int gs = -1, g = -1;
    if (lane < a.K) {
        gs = a.group_slot[(int64_t)t * a.K + lane];
        const int64_t e = a.topk[(int64_t)t * a.K + lane];
        if (gs >= 0 && expert_ok(e, a.E)) g = ((int)e / a.epr) / a.P;
    }
    bool first = gs >= 0 && g >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int sj = readlane(gs, j);
        if (j < lane && sj == gs) first = false;
    }
    for (uint64_t m = __ballot(first && gs < a.group_cap); m; m &= m - 1) {
        const int k = __ffsll((unsigned long long)m) - 1;
        forward_row<DEVICE_LOADS>(a, readlane(gs, k), readlane(g, k), t);
    }
}

#if EP_FUSED_WAVE
// Each wave takes its own jobs: no barrier, no LDS; a batch is written (or
// forwarded) by one wave, and the flag is stored by that wave's lane 0 after
// the wave's stores are acknowledged.
__global__ __launch_bounds__(kBlockThreads) void fused_hier_kernel(FusedArgs f) {
    const HierArgs& a = f.h;
    const int lane = lane_id();
    for (;;) {
        int kind = 3, job = 0;
        if (lane == 0) kind = take_job(f, job);
        kind = readlane(kind, 0);
        job = readlane(job, 0);
        if (kind == 3) return;
        const int t0 = job * f.tile, t1 = min(a.T, t0 + f.tile);
        if (kind == 0) {
            for (int t = t0; t < t1; ++t) scaleout_token<1, kPieceIters, kStoreDevice>(a, t, 0);
            wait_vmem();
            if (lane == 0 && job != f.withhold)
                __hip_atomic_store(&f.flags[job], a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        int ok = 1;
        if (kind == 2 && lane == 0) ok = wait_batch(f, job) ? 1 : 0;
        if (!readlane(ok, 0)) continue;
        for (int t = t0; t < t1; ++t) forward_token<true>(a, t);
    }
}
#elif EP_FUSED_LAG > 0
// Fixed-lag schedule: one counter hands out jobs 0 .. nbatch + lag - 1 in
// order; job i writes batch i (if i < nbatch) and publishes its flag, then
// forwards batch i - lag (if i >= lag), waiting for its flag. Batch i - lag
// was handed out before job i to a running workgroup that writes it before
// it waits for anything, so every wait ends; a group row is read about `lag`
// jobs after it was written.
//
// Ring mode (ring > 0): the group rows are not kept at their group-region
// rows but pass through a ring of `ring` batches, the scale-out receive
// buffer with flow control of "07: DeepEP Intra/Inter-node 协调" (the RDMA
// sender waits until the receiver's ring has free slots; the forwarder
// releases them). The j-th distinct group of the i-th token of batch b goes
// to ring row (b mod ring) * tile * gmax + i * gmax + j. Before writing batch
// b >= ring, the producer waits until batch b - ring's rows were read
// (`freed`); a forwarder marks its batch freed once its loads are done, also
// after a timed-out wait. Batch b - ring was forwarded by job
// b - ring + lag < b (ring > lag), handed out earlier, so every wait still
// points at an earlier job. The rows then stay in a few hundred MB that the
// MALL can hold instead of all G_rows.
// The waits of one slot chain through the generations n = b / ring: the
// producer of batch b waits for the forwarder of b - ring, which waits for
// its producer, and so on. Since every wait may start at about the same
// time, each limit grows with n: a forwarder waits at most (n + 1) * timeout,
// a producer at most (n + 1/2) * timeout. A flag lost in generation n then
// stops only its own batch: its forwarder gives up at (n + 1) * timeout,
// before the next producer's limit, whose flag comes before its forwarder's.
__device__ __forceinline__ int ring_row(const FusedArgs& f, int batch, int i, uint64_t firsts, int lane) {
    const int base = (batch % f.ring) * f.tile * f.gmax + i * f.gmax;
    return base + __popcll(firsts & ((1ull << lane) - 1));
}

// The distinct groups of token t (first lane of each, as in scaleout_token
// and forward_token): group slot, group and the mask of first lanes.
__device__ __forceinline__ uint64_t token_groups(const HierArgs& a, int t, int& gs, int& g) {
    const int lane = lane_id();
    gs = -1;
    g = -1;
    if (lane < a.K) {
        gs = a.group_slot[(int64_t)t * a.K + lane];
        const int64_t e = a.topk[(int64_t)t * a.K + lane];
        if (gs >= 0 && expert_ok(e, a.E)) g = ((int)e / a.epr) / a.P;
    }
    bool first = gs >= 0 && g >= 0;
    for (int j = 0; j < a.K; ++j)
        if (j < lane && readlane(gs, j) == gs) first = false;
    return __ballot(first);
}

__global__ __launch_bounds__(kFusedThreads) void fused_hier_kernel(FusedArgs f) {
    const HierArgs& a = f.h;
    __shared__ int sh_job, sh_ok;
    const int wave = wave_in_block(), lane = lane_id();
    const int njobs = f.nbatch + f.lag;
    for (;;) {
        if (threadIdx.x == 0) sh_job = (int)atomicAdd(&f.ctr[0], 1u);
        __syncthreads();
        const int job = sh_job;
        __syncthreads();
        if (job >= njobs) return;
        if (job < f.nbatch) {
            const int t0 = job * f.tile, t1 = min(a.T, t0 + f.tile);
            if (f.ring > 0) {
                if (job >= f.ring && threadIdx.x == 0 &&
                    !wait_flag_bounded(&f.freed[job - f.ring], a.epoch,
                                       (uint64_t)(job / f.ring) * f.timeout + f.timeout / 2))
                    report(a.err, EP_DEVERR_TIMEOUT);
                __syncthreads();
                for (int t = t0 + wave; t < t1; t += kFusedWaves) {
                    int gs, g;
                    const uint64_t fm = token_groups(a, t, gs, g);
                    write_record<1, kPieceIters, kStoreDevice>(a, t, 0, fm, ring_row(f, job, t - t0, fm, lane));
                }
            } else {
                for (int t = t0 + wave; t < t1; t += kFusedWaves)
                    scaleout_token<1, kPieceIters, kStoreDevice>(a, t, 0);
            }
            wait_vmem();
            __syncthreads();
            if (threadIdx.x == 0 && job != f.withhold)
                __hip_atomic_store(&f.flags[job], a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const int fb = job - f.lag;
        if (fb < 0) continue;
        if (threadIdx.x == 0)
            sh_ok = wait_batch(f, fb, f.ring > 0 ? (uint64_t)(fb / f.ring + 1) * f.timeout : 0) ? 1 : 0;
        __syncthreads();
        const int ok = sh_ok;
        __syncthreads();
        const int t0 = fb * f.tile, t1 = min(a.T, t0 + f.tile);
        if (ok) {
            for (int t = t0 + wave; t < t1; t += kFusedWaves) {
                if (f.ring > 0) {
                    int gs, g;
                    const uint64_t fm = token_groups(a, t, gs, g);
                    const int rr = ring_row(f, fb, t - t0, fm, lane);
                    for (uint64_t m = fm; m; m &= m - 1) {
                        const int k = __ffsll((unsigned long long)m) - 1;
                        forward_row<true>(a, readlane(rr, k), readlane(g, k), t);
                    }
                } else {
                    forward_token<true>(a, t);
                }
            }
        }
        if (f.ring > 0) {  // release the batch's ring rows (its loads are done)
            wait_vmem();
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_store(&f.freed[fb], a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}
#else
__global__ __launch_bounds__(kFusedThreads) void fused_hier_kernel(FusedArgs f) {
    const HierArgs& a = f.h;
    __shared__ int sh_job, sh_kind;  // kind: 0 produce, 1 forward (flag seen), 2 forward (wait), 3 done
    __shared__ int sh_ok;
    const int wave = wave_in_block();
    for (;;) {
        if (threadIdx.x == 0) {
            int job = 0;
            sh_kind = take_job(f, job);
            sh_job = job;
        }
        __syncthreads();
        const int kind = sh_kind, job = sh_job;
        __syncthreads();
        if (kind == 3) return;
        const int t0 = job * f.tile, t1 = min(a.T, t0 + f.tile);
        if (kind == 0) {
            // Wave w writes whole records of tokens t0 + w, t0 + w + W, ... (W waves per workgroup)
            // (the kernel's register budget is set by the forward part, so a
            // wave holds a 32-block piece of the record at once).
            for (int t = t0 + wave; t < t1; t += kFusedWaves)
                scaleout_token<1, kPieceIters, EP_FUSED_COHERENT ? kStoreDevice : kStorePlain>(a, t, 0);
#if EP_FUSED_COHERENT
            // Publish: the rows were stored with device scope; each wave waits
            // until its stores are acknowledged, and after the barrier thread
            // 0 stores the flag (device scope). No L2 write-back is needed.
            wait_vmem();
            __syncthreads();
            if (threadIdx.x == 0 && job != f.withhold)
                __hip_atomic_store(&f.flags[job], a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
            // Release: the barrier orders every wave's stores before thread
            // 0's flag store, whose agent-scope release makes them visible
            // device-wide (an L2 write-back, then the store).
            __syncthreads();
            if (threadIdx.x == 0 && job != f.withhold)
                __hip_atomic_store(&f.flags[job], a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
#endif
            continue;
        }
        // Acquire: thread 0 sees the flag (kind 1: seen while claiming; kind
        // 2: waited for, with a time limit); after the barrier every wave
        // reads the batch's rows (with device-scope loads, or after an
        // agent-scope acquire fence).
        if (threadIdx.x == 0) {
            const bool ok = kind == 1 || wait_batch(f, job);
#if !EP_FUSED_COHERENT
            if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#endif
            sh_ok = ok ? 1 : 0;
        }
        __syncthreads();
        const int ok = sh_ok;
        __syncthreads();
        if (!ok) continue;
        // Forward the group rows of the batch's tokens: wave w takes tokens
        // t0 + w, t0 + w + W, ... (W waves per workgroup)
        for (int t = t0 + wave; t < t1; t += kFusedWaves) forward_token<EP_FUSED_COHERENT != 0>(a, t);
    }
}

#endif  // EP_FUSED_WAVE

// ---------------------------------------------------------------------------
// Several sources, send and copy epilogue in one persistent launch: the
// receivers take each batch of records as soon as its flag is out ("DeepEP V2
// 深度深潜", §3.3 阶段2 and 阶段3; "Ascend Send Ordering", 方案一: the batch's
// records written without ordering, then one flag). The same fixed-lag
// schedule as the fused two-level dispatch: job i sends batch i's records to
// their staging rows (device-scope stores, then the batch's flag), then
// unpacks the staging rows of batch i - lag into their dense receive rows
// (device-scope loads), shortly after they were written, so they come from
// the MALL. The staging row (r*S + s)*capacity + j of (t, r) holds dense row
// recv_offsets[r*S + s] + j, which is the copy epilogue's row; every dense row
// of a region below its capacity is some (t, r)'s, so the receive rows equal
// those of the send followed by the copy epilogue. A batch's records are
// written one token per wave; its staging rows (about D per token) are then
// listed in LDS and spread over all the workgroup's waves, so that each wave
// unpacks one or two rows, not a token's D rows one after another: at ep32
// with 32 sources 251 us against 264 us for the two launches (one token per
// wave for the unpacking as well: 270-323 us).
// ---------------------------------------------------------------------------
#ifndef EP_SRCF_WPB
#define EP_SRCF_WPB 8  // waves per workgroup
#endif
#ifndef EP_SRCF_WG_PER_CU
#define EP_SRCF_WG_PER_CU 0  // at most this many workgroups per CU (0: all resident, 1 at 162 VGPRs)
#endif
#ifndef EP_SRCF_LAG
#define EP_SRCF_LAG 64  // job i sends batch i, then unpacks batch i - EP_SRCF_LAG
#endif
#ifndef EP_SRCF_TILE
#define EP_SRCF_TILE 4  // tokens per batch (at most EP_SRCF_WPB: one listing wave per token)
#endif
constexpr int kSrcFusedWaves = EP_SRCF_WPB;
static_assert(EP_SRCF_TILE <= EP_SRCF_WPB, "one listing wave per token of a batch");

struct SourceFusedArgs {
    HierArgs h;        // send: group_slot = src_slot, group_buf = staging, group_cap = its rows
    EpilogueArgs e;    // unpack into the receive arrays
    int tile, nbatch, lag;
    uint64_t timeout;  // wall-clock ticks a batch wait may last
    uint32_t* ctr;     // [0] next job
    uint32_t* flags;   // [nbatch] epoch once batch b's records are written
};

__global__ __launch_bounds__(kSrcFusedWaves * kWave) void source_fused_kernel(SourceFusedArgs f) {
    const HierArgs& a = f.h;
    __shared__ int sh_job, sh_ok;
    const int wave = wave_in_block(), lane = lane_id();
    const int njobs = f.nbatch + f.lag;
    for (;;) {
        if (threadIdx.x == 0) sh_job = (int)atomicAdd(&f.ctr[0], 1u);
        __syncthreads();
        const int job = sh_job;
        __syncthreads();
        if (job >= njobs) return;
        if (job < f.nbatch) {
            const int t0 = job * f.tile, t1 = min(a.T, t0 + f.tile);
            for (int t = t0 + wave; t < t1; t += kSrcFusedWaves)
                scaleout_token<1, kPieceIters, kStoreDevice>(a, t, 0);
            wait_vmem();
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_store(&f.flags[job], a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const int fb = job - f.lag;
        if (fb < 0) continue;
        if (threadIdx.x == 0) {
            const bool ok = wait_flag_bounded(&f.flags[fb], a.epoch, f.timeout);
            if (!ok) report(a.err, EP_DEVERR_TIMEOUT);
            sh_ok = ok ? 1 : 0;
        }
        __syncthreads();
        const int ok = sh_ok;
        __syncthreads();
        if (!ok) continue;
        const int t0 = fb * f.tile, t1 = min(a.T, t0 + f.tile);
        // The batch's distinct staging rows go to an LDS list (wave w lists
        // token t0 + w's, at most K each); then every wave takes rows w, w + W, ...
        __shared__ int64_t sh_rows[kSrcFusedWaves][EP_MAX_TOPK];
        __shared__ int sh_n[kSrcFusedWaves];
        {
            const int t = t0 + wave;
            int sr = -1;
            if (t < t1 && lane < a.K) sr = a.group_slot[(int64_t)t * a.K + lane];
            bool first = sr >= 0 && sr < a.group_cap;
            for (int j = 0; j < a.K; ++j)
                if (j < lane && readlane(sr, j) == sr) first = false;
            const uint64_t m = __ballot(first);
            if (first) sh_rows[wave][__popcll(m & ((1ull << lane) - 1))] = sr;
            if (lane == 0) sh_n[wave] = __popcll(m);
        }
        __syncthreads();
        int total = 0;
        for (int w = 0; w < kSrcFusedWaves; ++w) total += sh_n[w];
        for (int e = wave; e < total; e += kSrcFusedWaves) {
            int w = 0, k = e;
            while (k >= sh_n[w]) k -= sh_n[w++];
            const int64_t row = sh_rows[w][k];
            const int64_t q = row / f.e.cap, j = row - q * f.e.cap;
            const int64_t i = (int64_t)f.e.offs[q] + j;
            if (i >= f.e.rcap) {
                if (lane == 0) report(a.err, EP_DEVERR_CAPACITY);
                continue;
            }
            epilogue_row<true>(f.e, i, a.group_buf + row * a.geom.stride);
        }
        __syncthreads();  // the list is rebuilt by the next job
    }
}

HierArgs hier_args(const ep_shape& s, const ep_tokens& tk, uint32_t epoch, char* ws) {
    const WsLayout W = ws_layout(s);
    int seg = EP_SEG_BF16 | (tk.x_fp8 ? EP_SEG_FP8 : 0) | (tk.x_scales ? EP_SEG_SCALES : 0);
    HierArgs a = {};
    a.T = s.T; a.H = s.H; a.K = s.K; a.E = s.E; a.R = s.R; a.G = s.G;
    a.epr = s.E / s.R; a.P = s.R / s.G;
    a.geom = record_geom(s, seg);
    a.topk = tk.topk_idx;
    a.topk_w = tk.topk_weights;
    a.x = reinterpret_cast<const uint8_t*>(tk.x);
    a.x_fp8 = tk.x_fp8;
    a.x_scales = tk.x_scales;
    a.epoch = epoch;
    a.err = reinterpret_cast<uint32_t*>(ws + W.err);
    return a;
}

}  // namespace

hipError_t launch_hier(const ep_shape& s, const ep_layout& L, const ep_tokens& tk,
                       uint32_t epoch, int steps, void* group_buf, int64_t group_cap,
                       void* peer_buf, int64_t peer_cap, char* ws, hipStream_t st) {
    HierArgs a = hier_args(s, tk, epoch, ws);
    a.slot = L.slot;
    a.group_slot = L.group_slot;
    a.group_offsets = L.group_offsets;
    a.group_buf = reinterpret_cast<uint8_t*>(group_buf);
    a.group_cap = group_cap;
    a.peer_buf = reinterpret_cast<uint8_t*>(peer_buf);
    a.peer_cap = peer_cap;
    const dim3 block(kBlockThreads);
    if ((steps & EP_HIER_SCALEOUT) && s.T > 0)
        hipLaunchKernelGGL(scaleout_kernel,
                           dim3((unsigned)(((int64_t)s.T * kSoSplit + kWavesPerBlock - 1) / kWavesPerBlock)), block, 0,
                           st, a);
    if ((steps & EP_HIER_FORWARD) && group_cap > 0) {
        // One wave per row up to 262,144 rows (grid-stride beyond): one-shot
        // waves beat a grid of 8,192 workgroups walking 2-3 rows per wave
        // (hier8x8 forward 645 -> 600 us by rocprofv3). Waves past the row
        // count read on the device exit at once.
        const int64_t want = (group_cap + kWavesPerBlock - 1) / kWavesPerBlock;
        const int blocks = (int)(want < kForwardMaxBlocks ? want : kForwardMaxBlocks);
        hipLaunchKernelGGL(forward_kernel, dim3(blocks), block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_hier_fused(const ep_shape& s, const ep_layout& L, const ep_tokens& tk,
                             uint32_t epoch, void* group_buf, int64_t group_cap, void* peer_buf,
                             int64_t peer_cap, int tile, uint32_t timeout_us, int withhold, int ring,
                             char* ws, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    if (ring > 0 && (EP_FUSED_WAVE || EP_FUSED_LAG == 0)) return hipErrorNotSupported;  // lag kernel only
    const WsLayout W = ws_layout(s);
    FusedArgs f;
    f.h = hier_args(s, tk, epoch, ws);
    f.h.slot = L.slot;
    f.h.group_slot = L.group_slot;
    f.h.group_offsets = L.group_offsets;
    f.h.group_buf = reinterpret_cast<uint8_t*>(group_buf);
    f.h.group_cap = group_cap;
    f.h.peer_buf = reinterpret_cast<uint8_t*>(peer_buf);
    f.h.peer_cap = peer_cap;
    f.tile = tile;
    f.nbatch = (s.T + tile - 1) / tile;
    f.withhold = withhold;
    f.lag = EP_FUSED_LAG;
    f.ring = ring;
    f.gmax = std::min(s.K, s.G);
    f.ctr = reinterpret_cast<uint32_t*>(ws + W.fused);
    f.flags = f.ctr + kFusedCounters;
    f.freed = f.flags + f.nbatch;
    LaunchInfo d;
    const hipError_t e = launch_info(st, reinterpret_cast<const void*>(&fused_hier_kernel),
                                     EP_FUSED_WAVE ? kBlockThreads : kFusedThreads, &d);
    if (e != hipSuccess) return e;
    f.timeout = (uint64_t)timeout_us * (uint64_t)(d.rate_khz > 0 ? d.rate_khz : 100000) / 1000u;
    // No more workgroups than are resident at once (more would find no work),
    // and per CU only as many as keep about EP_FUSED_INFLIGHT_BYTES of records
    // in the waves at once (but at least 2): with more, the rows written
    // between a batch's production and its forwarding push it out of the
    // MALL; with fewer, HBM idles. At hier8x8 (15,872-byte records) that is 2
    // workgroups of 2 waves per CU: 699 us for the launch, against 1,003 us
    // with 1 and 764 us with all 4 resident; with 9,216-byte records
    // (H = 4,096) all 4: 445 against 574 us with 2; with 35,328-byte records
    // (H = 16,384) 2: 1,932 against 2,492 us with 1.
    const int waves_per_wg = EP_FUSED_WAVE ? kWavesPerBlock : kFusedWaves;
    int per_cu = d.per_cu;
    if (EP_FUSED_WG_PER_CU > 0) {
        per_cu = std::min(per_cu, EP_FUSED_WG_PER_CU);
    } else {
        const int64_t fit = (int64_t)EP_FUSED_INFLIGHT_BYTES /
                            ((int64_t)waves_per_wg * std::max(1, d.cus) * std::max<int64_t>(1, f.h.geom.stride));
        per_cu = (int)std::min<int64_t>(per_cu, std::max<int64_t>(2, fit));
    }
    int resident = std::max(1, d.cus * std::max(1, per_cu));
    // Ring mode: a workgroup holds one job at a time, so about `blocks` jobs
    // are in flight; the producer of batch b waits for job b - ring + lag,
    // which is then done only if ring - lag >= blocks. A ring with room for
    // the whole grid keeps the lag of 64; a shorter one takes a lag down to
    // 16, leaving more of the ring to jobs in flight, and caps the grid at
    // ring - lag. At hier8x8 (512 workgroups) that gave 2,088 / 1,085 / 893 /
    // 770 us for rings of 128 / 256 / 384 / 512 batches, against 3,555 /
    // 1,281 / 937 / 783 us with the lag of 64; with 768 batches the lag of
    // 64 is best (695 against 719 us with 16).
    if (ring > 0) {
        f.lag = std::min(EP_FUSED_LAG, std::max(kRingMinLag, ring - resident));
        resident = std::min(resident, std::max(1, ring - f.lag));
    }
    const int jobs_per_block = EP_FUSED_WAVE ? kWavesPerBlock : 1;
    const int blocks = std::min(resident, std::max(1, (2 * f.nbatch + jobs_per_block - 1) / jobs_per_block));
    launch_zero_words(f.ctr, kFusedCounters + 2 * f.nbatch, st);  // then f.flags, then f.freed
    hipLaunchKernelGGL(fused_hier_kernel, dim3(blocks), dim3(EP_FUSED_WAVE ? kBlockThreads : kFusedThreads), 0, st,
                       f);
    return hipGetLastError();
}

hipError_t launch_send_rows(const ep_shape& s, const ep_tokens& tk, const int32_t* rows,
                            int64_t n_rows, uint32_t epoch, void* buf, char* ws, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    HierArgs a = hier_args(s, tk, epoch, ws);
    a.group_slot = rows;
    a.group_buf = reinterpret_cast<uint8_t*>(buf);
    a.group_cap = n_rows;
    hipLaunchKernelGGL(scaleout_kernel,
                       dim3((unsigned)(((int64_t)s.T * kSoSplit + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(kBlockThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_source_fused(const ep_shape& s, const ep_sources& src, const ep_tokens& tk,
                               uint32_t epoch, void* staging, const ep_recv& rv, char* ws, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const int seg = EP_SEG_BF16 | (tk.x_fp8 ? EP_SEG_FP8 : 0) | (tk.x_scales ? EP_SEG_SCALES : 0);
    SourceFusedArgs f;
    f.h = hier_args(s, tk, epoch, ws);
    f.h.group_slot = src.src_slot;
    f.h.group_buf = reinterpret_cast<uint8_t*>(staging);
    f.h.group_cap = (int64_t)s.R * src.S * src.capacity;
    EpilogueArgs& e = f.e;
    e.H = s.H; e.K = s.K; e.RS = s.R * src.S;
    e.cap = src.capacity;
    e.geom = record_geom(s, seg);
    e.offs = src.recv_offsets;
    e.staging = reinterpret_cast<const uint8_t*>(staging);
    e.rx = reinterpret_cast<uint8_t*>(rv.x);
    e.rfp8 = rv.x_fp8;
    e.rscales = rv.x_scales;
    e.rsrc = rv.src_idx;
    e.ridx = rv.topk_idx;
    e.rw = rv.topk_weights;
    e.rcap = rv.capacity;
    e.epoch = epoch;
    e.err = f.h.err;
    f.tile = EP_SRCF_TILE;
    f.nbatch = (s.T + f.tile - 1) / f.tile;
    f.lag = EP_SRCF_LAG;
    f.ctr = reinterpret_cast<uint32_t*>(ws + ws_layout(s).fused);
    f.flags = f.ctr + kFusedCounters;
    LaunchInfo d;
    const hipError_t err = launch_info(st, reinterpret_cast<const void*>(&source_fused_kernel),
                                       kSrcFusedWaves * kWave, &d);
    if (err != hipSuccess) return err;
    f.timeout = (uint64_t)kSourceFusedTimeoutUs * (uint64_t)(d.rate_khz > 0 ? d.rate_khz : 100000) / 1000u;
    const int per_cu = EP_SRCF_WG_PER_CU > 0 ? std::min(d.per_cu, EP_SRCF_WG_PER_CU) : d.per_cu;
    const int blocks = std::min(std::max(1, d.cus * std::max(1, per_cu)), std::max(1, 2 * f.nbatch));
    launch_zero_words(f.ctr, kFusedCounters + f.nbatch, st);  // f.flags follows the counter words
    hipLaunchKernelGGL(source_fused_kernel, dim3(blocks), dim3(kSrcFusedWaves * kWave), 0, st, f);
    return hipGetLastError();
}

}  // namespace ep
