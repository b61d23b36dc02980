// source.hip -- several source ranks on one GPU: per-source counts, the counts
// exchange, per-source staging slots and the copy epilogue.
//
// What is computed follows "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK
// 复制机制": §3.3 阶段2 (a source hands out, per destination rank, the next
// slot of its own region at that rank, and the combine later addresses the
// row as rank * capacity + slot) and 阶段3 (the copy epilogue finds the
// source of each received row from the prefix sum of tokens received per
// source rank and copies the row out of that source's region). Slots are made
// deterministic: inside a source, ascending token order.
//
// S sources own consecutive ranges of Ts = ceil(T / S) tokens. Launches:
//   1. count    : one workgroup per (256-token tile, source); the tile's bit
//                 matrix bits[r][t/32] in LDS (a repeated rank sets the same
//                 bit) gives per-tile counts by popcount.
//   2. exchange : one workgroup. Per (source, rank): tile prefixes and the
//                 total counts[s][r]; then the rank-major scan over (r, s)
//                 gives recv_offsets, i.e. what each destination learns from
//                 the all-to-all of counts.
//   3. assign   : rebuilds the bit matrix; the staging row of (t, rank r) is
//                 (r*S + s) * capacity + tile prefix + popcount of the bits of
//                 earlier tokens of the tile.
//   send        : the scale-out kernel of the two-level dispatch with these
//                 rows (hier.hip).
//   4. epilogue : one wave per dense receive row i: a 64-way search of
//                 recv_offsets finds its region (r, s), the wave loads the
//                 chunked record (its flag lanes load the flags), checks them
//                 and stores every field to row i of the receive arrays.
#include "ep_device.h"
#include "ep_epilogue.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kTile = kLayoutTokens;
constexpr int kTileWords = kTile / 32;
constexpr int kExchangeThreads = 1024;

struct SourceArgs {
    int T, K, E, R, S, Ts, nbs, epr;
    FastDiv div_epr;  // e / epr: rank of an expert
    int64_t cap;
    const int64_t* topk;
    int32_t* part;      // [S][nbs][R] per-tile counts -> per-source exclusive prefix
    int32_t* counts;    // [S][R]
    int32_t* offs;      // [R*S + 1]
    int32_t* src_slot;  // [T][K]
    uint32_t* err;
};

// Tokens [t0, t0 + nt) of this workgroup's tile.
__device__ __forceinline__ void tile_range(const SourceArgs& a, int& t0, int& nt) {
    const int s = blockIdx.y, b = blockIdx.x;
    const int begin = s * a.Ts;
    const int end = min(begin + a.Ts, a.T);
    t0 = begin + b * kTile;
    nt = max(0, min(kTile, end - t0));
}

// A token's expert ids: with K <= 8 all requested at once (lanes past K
// re-read lane K - 1; callers stop at K), else read on use. A loop over a
// run-time K issued one load per round trip.
struct Ids {
    int64_t v[8];
    __device__ __forceinline__ void load(const int64_t* row, int K) {
        if (K <= 8) {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = row[min(k, K - 1)];
        }
    }
    // f(k, id) for k = 0 .. K - 1.
    template <typename F>
    __device__ __forceinline__ void each(const int64_t* row, int K, F f) const {
        if (K <= 8) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (k >= K) break;
                f(k, v[k]);
            }
        } else {
            for (int k = 0; k < K; ++k) f(k, row[k]);
        }
    }
};

// Bit (r, i) of the tile's matrix is set when token t0 + i sends to rank r.
// Returns whether this thread's token holds an invalid id. The caller has
// requested the ids (ids.load) before, so they arrive while the matrix is
// cleared.
__device__ bool tile_bits(const SourceArgs& a, int t0, int nt, uint32_t* bits, const Ids& ids) {
    const int i = threadIdx.x;
    const int64_t* row = a.topk + (int64_t)(t0 + i) * a.K;
    for (int j = threadIdx.x; j < a.R * kTileWords; j += kBlockThreads) bits[j] = 0u;
    __syncthreads();
    bool bad = false;
    if (i < nt) {
        const uint32_t bit = 1u << (i & 31);
        ids.each(row, a.K, [&](int, int64_t e) {
            bad |= expert_bad(e, a.E);
            if (expert_ok(e, a.E)) atomicOr(&bits[a.div_epr((int)e) * kTileWords + (i >> 5)], bit);
        });
    }
    __syncthreads();
    return bad;
}

__global__ __launch_bounds__(kBlockThreads) void source_count_kernel(SourceArgs a) {
    extern __shared__ uint32_t bits[];
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.err = 0u;  // clean word
    int t0, nt;
    tile_range(a, t0, nt);
    Ids ids;
    if ((int)threadIdx.x < nt) ids.load(a.topk + (int64_t)(t0 + threadIdx.x) * a.K, a.K);
    tile_bits(a, t0, nt, bits, ids);
    int32_t* part = a.part + ((int64_t)blockIdx.y * a.nbs + blockIdx.x) * a.R;
    for (int r = threadIdx.x; r < a.R; r += kBlockThreads) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kTileWords; ++w) c += __popc(bits[r * kTileWords + w]);
        part[r] = c;
    }
}

__global__ __launch_bounds__(kExchangeThreads) void source_exchange_kernel(SourceArgs a) {
    __shared__ int32_t scan[kExchangeThreads];
    const int RS = a.R * a.S;
    // Per (source, rank): tile counts -> exclusive prefix over the source's
    // tiles, and the source's total.
    for (int idx = threadIdx.x; idx < RS; idx += kExchangeThreads) {
        const int s = idx / a.R, r = idx - s * a.R;
        int32_t run = 0;
        for (int b = 0; b < a.nbs; ++b) {
            int32_t* p = a.part + ((int64_t)s * a.nbs + b) * a.R + r;
            const int32_t c = *p;
            *p = run;
            run += c;
        }
        a.counts[idx] = run;
    }
    __syncthreads();
    // Rank-major exclusive scan: entry e = r*S + s is counts[s][r]. Each
    // thread owns a contiguous run of entries.
    const int per = (RS + kExchangeThreads - 1) / kExchangeThreads;
    const int e0 = min(RS, (int)threadIdx.x * per), e1 = min(RS, e0 + per);
    int32_t sum = 0;
    for (int e = e0; e < e1; ++e) sum += a.counts[(e % a.S) * a.R + e / a.S];
    scan[threadIdx.x] = sum;
    __syncthreads();
    for (int d = 1; d < kExchangeThreads; d <<= 1) {
        const int32_t v = (int)threadIdx.x >= d ? scan[threadIdx.x - d] : 0;
        __syncthreads();
        scan[threadIdx.x] += v;
        __syncthreads();
    }
    int32_t run = scan[threadIdx.x] - sum;
    for (int e = e0; e < e1; ++e) {
        a.offs[e] = run;
        run += a.counts[(e % a.S) * a.R + e / a.S];
    }
    if (threadIdx.x == kExchangeThreads - 1) a.offs[RS] = scan[kExchangeThreads - 1];
}

__global__ __launch_bounds__(kBlockThreads) void source_assign_kernel(SourceArgs a) {
    extern __shared__ uint32_t bits[];
    // The tile's per-rank prefixes go to LDS after the bit matrix; they are
    // loaded while the matrix is cleared and read once the marking barrier
    // has passed (one round trip instead of one per lane).
    int32_t* base = reinterpret_cast<int32_t*>(bits + a.R * kTileWords);
    const int s = blockIdx.y;
    int t0, nt;
    tile_range(a, t0, nt);
    Ids ids;
    if ((int)threadIdx.x < nt) ids.load(a.topk + (int64_t)(t0 + threadIdx.x) * a.K, a.K);
    constexpr int kPrefixRounds = (EP_MAX_RANKS + kBlockThreads - 1) / kBlockThreads;
    const int32_t* part = a.part + ((int64_t)s * a.nbs + blockIdx.x) * a.R;
    int32_t pv[kPrefixRounds];
#pragma unroll
    for (int q = 0; q < kPrefixRounds; ++q) pv[q] = part[min((int)threadIdx.x + q * kBlockThreads, a.R - 1)];
#pragma unroll
    for (int q = 0; q < kPrefixRounds; ++q)
        if ((int)threadIdx.x + q * kBlockThreads < a.R) base[threadIdx.x + q * kBlockThreads] = pv[q];
    const bool bad = tile_bits(a, t0, nt, bits, ids);
    if (bad) report(a.err, EP_DEVERR_EXPERT_ID);
    const int i = threadIdx.x;
    if (i >= nt) return;
    const int64_t t = t0 + i;
    const int w = i >> 5;
    const uint32_t below = (1u << (i & 31)) - 1u;
    bool over = false;
    const int64_t* row = a.topk + t * a.K;
    ids.each(row, a.K, [&](int k, int64_t e) {
        int32_t v = -1;
        if (expert_ok(e, a.E)) {
            const int r = a.div_epr((int)e);
            int64_t j = base[r] + __popc(bits[r * kTileWords + w] & below);
            for (int q = 0; q < w; ++q) j += __popc(bits[r * kTileWords + q]);
            if (j < a.cap) v = (int32_t)(((int64_t)r * a.S + s) * a.cap + j);
            else over = true;
        }
        a.src_slot[t * a.K + k] = v;
    });
    if (over) report(a.err, EP_DEVERR_CAPACITY);
}

// Region of dense row i: the largest p < RS with offs[p] <= i (offsets are
// non-decreasing and offs[0] = 0). Each round probes 64 evenly spaced
// entries, one per lane, and keeps the interval after the last probe <= i.
__device__ __forceinline__ int find_region(const int32_t* offs, int RS, int64_t i) {
    const int lane = lane_id();
    int lo = 0, hi = RS;  // offs[lo] <= i; the answer lies in [lo, hi)
    while (hi - lo > 1) {
        const int step = (hi - lo + kWave - 1) / kWave;
        const int p = lo + lane * step;
        const bool le = p < hi && offs[p] <= i;
        const int c = __popcll(__ballot(le));  // >= 1: lane 0 probes lo
        lo += (c - 1) * step;
        hi = min(hi, lo + step);
    }
    return lo;
}

__global__ __launch_bounds__(kBlockThreads) void copy_epilogue_kernel(EpilogueArgs a) {
    const int lane = lane_id();
    const int64_t n_rows = a.offs[a.RS];
    const int64_t wave_stride = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t i = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block(); i < n_rows;
         i += wave_stride) {
        const int reg = find_region(a.offs, a.RS, i);
        const int64_t j = i - a.offs[reg];
        if (j >= a.cap || i >= a.rcap) {
            if (lane == 0) report(a.err, EP_DEVERR_CAPACITY);
            continue;
        }
        epilogue_row<false>(a, i, a.staging + ((int64_t)reg * a.cap + j) * a.geom.stride);
    }
}

}  // namespace

WsSource ws_source(const ep_shape& s, int S) {
    WsSource w;
    const WsLayout base = ws_layout(s);
    w.Ts = (s.T + S - 1) / S;
    w.nbs = w.Ts > 0 ? (w.Ts + kTile - 1) / kTile : 1;
    w.part = base.total;
    w.total = base.total + ((sizeof(int32_t) * (size_t)S * w.nbs * s.R + 255) / 256) * 256;
    return w;
}

hipError_t launch_source_layout(const ep_shape& s, const int64_t* topk, const ep_sources& src,
                                char* ws, hipStream_t st) {
    const WsSource W = ws_source(s, src.S);
    SourceArgs a;
    a.T = s.T; a.K = s.K; a.E = s.E; a.R = s.R; a.S = src.S;
    a.Ts = W.Ts; a.nbs = W.nbs; a.epr = s.E / s.R;
    a.div_epr = FastDiv::make(a.epr);
    a.cap = src.capacity;
    a.topk = topk;
    a.part = reinterpret_cast<int32_t*>(ws + W.part);
    a.counts = src.counts;
    a.offs = src.recv_offsets;
    a.src_slot = src.src_slot;
    a.err = reinterpret_cast<uint32_t*>(ws + ws_layout(s).err);
    const dim3 grid(W.nbs, src.S), block(kBlockThreads);
    const size_t lds = sizeof(uint32_t) * (size_t)s.R * kTileWords;
    hipLaunchKernelGGL(source_count_kernel, grid, block, lds, st, a);
    const size_t lds_assign = lds + sizeof(int32_t) * (size_t)s.R;  // + the tile's per-rank prefixes
    hipLaunchKernelGGL(source_exchange_kernel, dim3(1), dim3(kExchangeThreads), 0, st, a);
    if (s.T > 0) hipLaunchKernelGGL(source_assign_kernel, grid, block, lds_assign, st, a);
    return hipGetLastError();
}

hipError_t launch_copy_epilogue(const ep_shape& s, const ep_sources& src, const void* staging,
                                uint32_t epoch, int seg, const ep_recv& rv, char* ws,
                                hipStream_t st) {
    EpilogueArgs a;
    a.H = s.H; a.K = s.K; a.RS = s.R * src.S;
    a.cap = src.capacity;
    a.geom = record_geom(s, seg);
    a.offs = src.recv_offsets;
    a.staging = reinterpret_cast<const uint8_t*>(staging);
    a.rx = reinterpret_cast<uint8_t*>(rv.x);
    a.rfp8 = rv.x_fp8;
    a.rscales = rv.x_scales;
    a.rsrc = rv.src_idx;
    a.ridx = rv.topk_idx;
    a.rw = rv.topk_weights;
    a.rcap = rv.capacity;
    a.epoch = epoch;
    a.err = reinterpret_cast<uint32_t*>(ws + ws_layout(s).err);
    // Waves for at most min(receive capacity, R*S*capacity) rows; the row
    // count itself is read on the device.
    const int64_t bound = (int64_t)a.RS * src.capacity;
    const int64_t rows = rv.capacity < bound ? rv.capacity : bound;
    const int64_t want = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    const int blocks = (int)(want < 1 ? 1 : (want < 8192 ? want : 8192));
    hipLaunchKernelGGL(copy_epilogue_kernel, dim3(blocks), dim3(kBlockThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace ep
