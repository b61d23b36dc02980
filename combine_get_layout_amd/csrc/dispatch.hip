// dispatch.hip -- ep_dispatch on gfx950: read each token once, write its record
// to every destination rank's receive row.
//
// What is computed follows "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK
// 复制机制", §3.3 阶段2 (dispatch warps: load the hidden row, load top-k ids and
// weights, one destination per distinct rank) and §3.5 (recv_x,
// recv_topk_idx, recv_topk_weights), with the record fields of "07: DeepEP
// Intra/Inter-node 协调 — NVLink Scale-up + RDMA Scale-out 三阶段流水线的代码实证"
// (hidden, scales, source index, top-k ids and weights; NVL receivers write
// recv_x[row] and recv_x_scales[row * H/128]).
//
// Mapping on CDNA4: each source token's row is cut into `split` column
// slices of whole 128-byte lines, one wave64 per slice, four waves per
// workgroup (split = EP_DSP_SPLIT, 4, for rows of 2,048 bf16 values and
// more; fewer for narrower rows, so that a slice fills a wave's 64 lanes).
// A wave loads its slice into VGPRs (up to 16 16-byte vectors per lane per
// pass), then streams it to each destination row with non-temporal 16-byte
// stores: one HBM read, D writes, no LDS round trip. Destinations are the
// lanes k whose slot differs from every earlier lane's (the rank
// deduplication), found with one ballot. The first slice's wave also writes
// the scales and the metadata. Rows of at most 32 vectors with K <= 8 take
// a second kernel that holds 2, 4 or 8 tokens per wave.
#include <algorithm>

#include "ep_device.h"
#include "ep_internal.h"

// Compile-time tuning knobs (defaults are the measured best on MI355X).
#ifndef EP_DSP_NVMAX
#define EP_DSP_NVMAX 16     // most 16-byte vectors per lane held per pass
#endif
#ifndef EP_DSP_NTSTORE
#define EP_DSP_NTSTORE 1    // non-temporal stores of receive rows
#endif
#ifndef EP_DSP_NTLOAD
#define EP_DSP_NTLOAD 0     // non-temporal loads of the source rows
#endif
#ifndef EP_DSP_WPB
#define EP_DSP_WPB 4        // waves (tokens) per workgroup
#endif
#ifndef EP_DSP_MINB
#define EP_DSP_MINB 1       // minimum resident workgroups per CU (launch bound)
#endif
#ifndef EP_DSP_SPLIT
#define EP_DSP_SPLIT 4      // most waves per token: the row is cut into this many column slices
#endif
#ifndef EP_DSP_PERSIST
#define EP_DSP_PERSIST 0    // persistent, software-pipelined kernel (experiment)
#endif
#ifndef EP_DSP_PERSIST_BPC
#define EP_DSP_PERSIST_BPC 64  // most workgroups per CU of the persistent grid
#endif

namespace ep {
namespace {

constexpr int kDspWaves = EP_DSP_WPB;
constexpr int kDspThreads = kDspWaves * kWave;

__device__ __forceinline__ u32x4 ld_src(const void* p) {
#if EP_DSP_NTLOAD
    return ld16_stream(p);
#else
    return ld16(p);
#endif
}
__device__ __forceinline__ void st_dst(void* p, u32x4 v) {
#if EP_DSP_NTSTORE
    st16_stream(p, v);
#else
    st16(p, v);
#endif
}

struct DispatchArgs {
    int T, H, K, E;
    const int32_t* slot;
    const int64_t* topk;
    const float* topk_w;
    const uint8_t* x;       // bf16 rows as bytes
    const uint8_t* x_fp8;
    const float* x_scales;
    uint8_t* rx;
    uint8_t* rfp8;
    float* rscales;
    int32_t* rsrc;
    int32_t* ridx;
    float* rw;
    int64_t cap;
    uint32_t* err;
    int split;              // waves (column slices) per token
};

// Vectors of one wave's column slice of a row of `nvec` vectors: a multiple of
// 8 (128 bytes), so that no two waves write parts of one cache line of a
// receive row whose bytes are a multiple of 128 (the last slice is shorter).
// Slices that split lines cost 16-22% (H = 7232: 115.7 vs 100.1 us; H =
// 4160 at 16,384 tokens: 288.9 vs 236.6 us).
__host__ __device__ __forceinline__ int slice_vecs(int64_t nvec, int split) {
    return (int)((((nvec + split - 1) / split) + 7) & ~(int64_t)7);
}

// Vectors [v0, v1) of a row of `nvec` vectors: column slice `part` of `split`.
__device__ __forceinline__ void slice_range(int nvec, int part, int split, int& v0, int& v1) {
    const int per = (((nvec + split - 1) / split) + 7) & ~7;  // slice_vecs in 32-bit arithmetic
    v0 = min(nvec, part * per);
    v1 = min(nvec, v0 + per);
}

// One pass of a slice: v[j] = vector base + j * 64 + lane of the row at src.
// Every load is issued; addresses past the slice are clamped to its last
// vector (or to vector 0 of an empty slice) and the stores mask them.
template <int NV>
__device__ __forceinline__ void load_pass(const uint8_t* src, int base, int v1, u32x4 (&v)[NV]) {
    const int lane = lane_id();
    const int last = max(v1 - 1, 0);
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = ld_src(src + (int64_t)min(base + j * kWave + lane, last) * 16);
}

// Copy vectors [v0, v1) of the row at src to the rows dst + slot_k * row_bytes
// of every destination lane k in `dest`. v holds the first pass (loaded by
// the caller); later passes of slices wider than 64 NV vectors load here.
template <int NV>
__device__ __forceinline__ void fan_out_row(const uint8_t* src, int64_t row_bytes, uint8_t* dst,
                                            uint64_t dest, int slot, int v0, int v1, u32x4 (&v)[NV]) {
    const int lane = lane_id();
    for (int base = v0; base < v1; base += kWave * NV) {
        if (base != v0) load_pass<NV>(src, base, v1, v);
        for (uint64_t m = dest; m; m &= m - 1) {
            const int k = __ffsll((unsigned long long)m) - 1;
            uint8_t* row = dst + (int64_t)readlane(slot, k) * row_bytes;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int i = base + j * kWave + lane;
                if (i < v1) st_dst(row + (int64_t)i * 16, v[j]);
            }
        }
    }
}

// FP8: the launch moves an FP8 payload (its first pass is then loaded with
// the bf16 one; without it the kernel holds no registers for it).
template <int NV, bool FP8>
__global__ __launch_bounds__(kDspThreads, EP_DSP_MINB) void dispatch_kernel(DispatchArgs a) {
    const int lane = lane_id();
    const int gw = blockIdx.x * kDspWaves + wave_in_block();
    const int t = gw / a.split, part = gw % a.split;
    if (t >= a.T) return;

    // Lanes 0..K-1 hold this token's slots, ids and weights (the other lanes
    // load lane 0's and drop them). The first pass of the bf16 (and FP8)
    // slice is requested together with them, so the wave waits for one
    // round trip, not two (measured 1-2 us at 4,096 tokens x 7,168).
    const int kl = lane < a.K ? lane : 0;
    int s = a.slot[(int64_t)t * a.K + kl];
    int64_t e = a.topk[(int64_t)t * a.K + kl];
    float wk = a.topk_w ? a.topk_w[(int64_t)t * a.K + kl] : 0.f;
    const bool bf16 = a.x && a.rx;
    const int64_t xrow = (int64_t)a.H * 2;
    const uint8_t* xsrc = bf16 ? a.x + (int64_t)t * xrow : nullptr;
    int xv0 = 0, xv1 = 0;
    slice_range((int)(xrow / 16), part, a.split, xv0, xv1);
    // The FP8 slice's first pass too, in registers of its own when that
    // keeps the occupancy (up to 4 vectors per lane); wider slices load it
    // into v after the bf16 stores.
    constexpr bool kEarlyFp8 = FP8 && NV <= 4;
    u32x4 v[NV], vf[kEarlyFp8 ? NV : 1];
    if (bf16) load_pass<NV>(xsrc, xv0, xv1, v);
    const uint8_t* fsrc = FP8 ? a.x_fp8 + (int64_t)t * a.H : nullptr;
    int fv0 = 0, fv1 = 0;
    slice_range(a.H / 16, part, a.split, fv0, fv1);
    if constexpr (kEarlyFp8) load_pass<NV>(fsrc, fv0, fv1, vf);
    if (lane >= a.K) {
        s = -1;
        e = -1;
        wk = 0.f;
    }

    // A lane is a destination if its slot is valid and no lower lane has the
    // same slot (same rank).
    bool first = s >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int sj = readlane(s, j);
        if (j < lane && sj == s) first = false;
    }
    const bool over = first && s >= a.cap;
    if (over && part == 0) report(a.err, EP_DEVERR_CAPACITY);
    const uint64_t dest = __ballot(first && !over);
    if (!dest) return;

    if (bf16) fan_out_row<NV>(xsrc, xrow, a.rx, dest, s, xv0, xv1, v);
    if constexpr (kEarlyFp8) {
        fan_out_row<NV>(fsrc, a.H, a.rfp8, dest, s, fv0, fv1, vf);
    } else if constexpr (FP8) {
        load_pass<NV>(fsrc, fv0, fv1, v);
        fan_out_row<NV>(fsrc, a.H, a.rfp8, dest, s, fv0, fv1, v);
    }
    if (part != 0) return;  // scales and metadata: written once per row
    if (a.x_scales && a.rscales) {
        const int ns = a.H / 128;
        for (int base = 0; base < ns; base += kWave) {
            const int i = base + lane;
            const float sv = i < ns ? a.x_scales[(int64_t)t * ns + i] : 0.f;
            for (uint64_t m = dest; m; m &= m - 1) {
                const int k = __ffsll((unsigned long long)m) - 1;
                if (i < ns) a.rscales[(int64_t)readlane(s, k) * ns + i] = sv;
            }
        }
    }
    // Metadata: source token, the token's expert ids (invalid -> -1) and weights.
    const int32_t id = expert_ok(e, a.E) ? (int32_t)e : -1;
    for (uint64_t m = dest; m; m &= m - 1) {
        const int k = __ffsll((unsigned long long)m) - 1;
        const int64_t row = readlane(s, k);
        if (a.rsrc && lane == 0) a.rsrc[row] = t;
        if (lane < a.K) {
            if (a.ridx) a.ridx[row * a.K + lane] = id;
            if (a.rw && a.topk_w) a.rw[row * a.K + lane] = wk;
        }
    }
}

// Narrow rows (every present payload row at most 32 vectors: H <= 256 for
// the bf16 row) with K <= 8: one token per wave would leave most lanes idle,
// so a wave holds TPW tokens, one per group of G = 64 / TPW lanes, and lane
// v of a group holds vector v of each payload row of its token (G >= K, so
// lanes v < K also hold the token's id and weight of lane v). Every lane
// reads its token's K slots (the same addresses within a group) and walks
// the destinations in ascending k: one store instruction then writes the
// vector of every group whose token has k as a destination.
template <int TPW>
__global__ __launch_bounds__(kDspThreads) void dispatch_narrow_kernel(DispatchArgs a) {
    constexpr int G = kWave / TPW;
    const int lane = lane_id();
    const int v = lane % G;
    const int t = (blockIdx.x * kDspWaves + wave_in_block()) * TPW + lane / G;
    if (t >= a.T) return;  // no cross-lane operations below
    int s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = a.slot[(int64_t)t * a.K + min(k, a.K - 1)];
    const int kv = min(v, a.K - 1);
    const int64_t e = a.topk[(int64_t)t * a.K + kv];
    const float wk = a.topk_w ? a.topk_w[(int64_t)t * a.K + kv] : 0.f;
    const int nvx = a.H / 8, nvf = a.H / 16, ns = a.H / 128;
    const bool bf16 = a.x && a.rx, fp8 = a.x_fp8 && a.rfp8, scales = a.x_scales && a.rscales && ns > 0;
    u32x4 vx = {0u, 0u, 0u, 0u}, vf = {0u, 0u, 0u, 0u};
    float sc = 0.f;
    if (bf16) vx = ld_src(a.x + (int64_t)t * a.H * 2 + (int64_t)min(v, nvx - 1) * 16);
    if (fp8) vf = ld_src(a.x_fp8 + (int64_t)t * a.H + (int64_t)min(v, nvf - 1) * 16);
    if (scales) sc = a.x_scales[(int64_t)t * ns + min(v, ns - 1)];
    const int32_t id = expert_ok(e, a.E) ? (int32_t)e : -1;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (k >= a.K) break;
        bool first = s[k] >= 0;  // a rank reached by an earlier lane is written once
#pragma unroll
        for (int j = 0; j < k; ++j) first = first && s[j] != s[k];
        if (!first) continue;
        if (s[k] >= a.cap) {
            if (v == 0) report(a.err, EP_DEVERR_CAPACITY);
            continue;
        }
        const int64_t row = s[k];
        if (bf16 && v < nvx) st_dst(a.rx + row * a.H * 2 + (int64_t)v * 16, vx);
        if (fp8 && v < nvf) st_dst(a.rfp8 + row * a.H + (int64_t)v * 16, vf);
        if (scales && v < ns) a.rscales[row * ns + v] = sc;
        if (a.rsrc && v == 0) a.rsrc[row] = t;
        if (v < a.K) {
            if (a.ridx) a.ridx[row * a.K + v] = id;
            if (a.rw && a.topk_w) a.rw[row * a.K + v] = wk;
        }
    }
}

// Persistent form (EP_DSP_PERSIST, off by default: measured slower than the
// one-shot kernel on every workload). A grid of at most the resident waves;
// wave w takes the items (token, slice) w, w + W, w + 2W, ... (W = waves in
// the grid) with two register sets. EP_DSP_PERSIST=1 issues the next item's
// loads before the current item's stores; =2 after them (loads and stores
// share one in-order counter, so with 1 the wave waits for the next loads
// before its first store, and with 2 it waits once for both). Needs the
// widest slice to fit in one pass (NV vectors per lane).
struct Item {
    int t, part;
    int s;        // slot of lane k < K
    int64_t e;    // expert id of lane k
    float wk;     // weight of lane k
};

template <int NV>
__device__ __forceinline__ void load_item(const DispatchArgs& a, int item, Item& it, u32x4 (&v)[NV],
                                          u32x4 (&f)[NV]) {
    const int lane = lane_id();
    it.t = item / a.split;
    it.part = item % a.split;
    it.s = -1;
    it.e = -1;
    it.wk = 0.f;
    if (lane < a.K) {
        it.s = a.slot[(int64_t)it.t * a.K + lane];
        it.e = a.topk[(int64_t)it.t * a.K + lane];
        if (a.topk_w) it.wk = a.topk_w[(int64_t)it.t * a.K + lane];
    }
    if (a.x && a.rx) {
        const int64_t row_bytes = (int64_t)a.H * 2;
        const int nvec_all = (int)(row_bytes / 16);
        const int per = slice_vecs(nvec_all, a.split);
        const int v0 = min(nvec_all, it.part * per), v1 = min(nvec_all, v0 + per);
        const uint8_t* src = a.x + (int64_t)it.t * row_bytes;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = v0 + j * kWave + lane;
            v[j] = ld_src(src + (int64_t)min(i, max(v1 - 1, 0)) * 16);
        }
    }
    if (a.x_fp8 && a.rfp8) {
        const int64_t row_bytes = a.H;
        const int nvec_all = (int)(row_bytes / 16);
        const int per = slice_vecs(nvec_all, a.split);
        const int v0 = min(nvec_all, it.part * per), v1 = min(nvec_all, v0 + per);
        const uint8_t* src = a.x_fp8 + (int64_t)it.t * row_bytes;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = v0 + j * kWave + lane;
            f[j] = ld_src(src + (int64_t)min(i, max(v1 - 1, 0)) * 16);
        }
    }
}

template <int NV>
__device__ __forceinline__ void store_slice(const u32x4 (&v)[NV], int64_t row_bytes, uint8_t* dst,
                                            uint64_t dest, int slot, int part, int split) {
    const int lane = lane_id();
    const int nvec_all = (int)(row_bytes / 16);
    const int per = slice_vecs(nvec_all, split);
    const int v0 = min(nvec_all, part * per), v1 = min(nvec_all, v0 + per);
    for (uint64_t m = dest; m; m &= m - 1) {
        const int k = __ffsll((unsigned long long)m) - 1;
        uint8_t* row = dst + (int64_t)readlane(slot, k) * row_bytes;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = v0 + j * kWave + lane;
            if (i < v1) st_dst(row + (int64_t)i * 16, v[j]);
        }
    }
}

template <int NV>
__device__ __forceinline__ void store_item(const DispatchArgs& a, const Item& it, const u32x4 (&v)[NV],
                                           const u32x4 (&f)[NV]) {
    const int lane = lane_id();
    bool first = it.s >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int sj = readlane(it.s, j);
        if (j < lane && sj == it.s) first = false;
    }
    const bool over = first && it.s >= a.cap;
    if (over && it.part == 0) report(a.err, EP_DEVERR_CAPACITY);
    const uint64_t dest = __ballot(first && !over);
    if (!dest) return;
    if (a.x && a.rx) store_slice<NV>(v, (int64_t)a.H * 2, a.rx, dest, it.s, it.part, a.split);
    if (a.x_fp8 && a.rfp8) store_slice<NV>(f, a.H, a.rfp8, dest, it.s, it.part, a.split);
    if (it.part != 0) return;
    if (a.x_scales && a.rscales) {
        const int ns = a.H / 128;
        for (int base = 0; base < ns; base += kWave) {
            const int i = base + lane;
            const float sv = i < ns ? a.x_scales[(int64_t)it.t * ns + i] : 0.f;
            for (uint64_t m = dest; m; m &= m - 1) {
                const int k = __ffsll((unsigned long long)m) - 1;
                if (i < ns) a.rscales[(int64_t)readlane(it.s, k) * ns + i] = sv;
            }
        }
    }
    const int32_t id = expert_ok(it.e, a.E) ? (int32_t)it.e : -1;
    for (uint64_t m = dest; m; m &= m - 1) {
        const int k = __ffsll((unsigned long long)m) - 1;
        const int64_t row = readlane(it.s, k);
        if (a.rsrc && lane == 0) a.rsrc[row] = it.t;
        if (lane < a.K) {
            if (a.ridx) a.ridx[row * a.K + lane] = id;
            if (a.rw && a.topk_w) a.rw[row * a.K + lane] = it.wk;
        }
    }
}

template <int NV>
__global__ __launch_bounds__(kDspThreads) void dispatch_persistent_kernel(DispatchArgs a, int nitems) {
    const int gw = blockIdx.x * kDspWaves + wave_in_block();
    const int nw = gridDim.x * kDspWaves;
    int item = gw;
    if (item >= nitems) return;
    Item cur;
    u32x4 v[NV], f[NV];
    load_item<NV>(a, item, cur, v, f);
    for (;;) {
        const int next = item + nw;
        Item nx;
        u32x4 vn[NV], fn[NV];
        const bool more = next < nitems;
#if EP_DSP_PERSIST == 2
        // The current item's stores first, then the next item's loads: the
        // wave then waits once for both, the loads in flight while the
        // stores drain.
        store_item<NV>(a, cur, v, f);
        if (more) load_item<NV>(a, next, nx, vn, fn);
#else
        if (more) load_item<NV>(a, next, nx, vn, fn);
        store_item<NV>(a, cur, v, f);
#endif
        if (!more) break;
        cur = nx;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            v[j] = vn[j];
            f[j] = fn[j];
        }
        item = next;
    }
}

// The instantiation holding enough vectors per lane for the widest slice.
template <bool FP8>
hipError_t launch_nv(int64_t per_lane, dim3 grid, dim3 block, const DispatchArgs& a, hipStream_t st) {
    if (per_lane <= 1)
        hipLaunchKernelGGL((dispatch_kernel<1, FP8>), grid, block, 0, st, a);
    else if (per_lane <= 2)
        hipLaunchKernelGGL((dispatch_kernel<2, FP8>), grid, block, 0, st, a);
    else if (per_lane <= 4 || EP_DSP_NVMAX <= 4)
        hipLaunchKernelGGL((dispatch_kernel<4, FP8>), grid, block, 0, st, a);
    else if (per_lane <= 8 || EP_DSP_NVMAX <= 8)
        hipLaunchKernelGGL((dispatch_kernel<8, FP8>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((dispatch_kernel<16, FP8>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const ep_shape& s, const ep_layout& L, const ep_tokens& tk,
                           const ep_recv& rv, char* ws, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const WsLayout W = ws_layout(s);
    DispatchArgs a;
    a.T = s.T; a.H = s.H; a.K = s.K; a.E = s.E;
    a.slot = L.slot;
    a.topk = tk.topk_idx;
    a.topk_w = tk.topk_weights;
    a.x = reinterpret_cast<const uint8_t*>(tk.x);
    a.x_fp8 = tk.x_fp8;
    a.x_scales = tk.x_scales;
    a.rx = reinterpret_cast<uint8_t*>(rv.x);
    a.rfp8 = rv.x_fp8;
    a.rscales = rv.x_scales;
    a.rsrc = rv.src_idx;
    a.ridx = rv.topk_idx;
    a.rw = rv.topk_weights;
    a.cap = rv.capacity;
    a.err = reinterpret_cast<uint32_t*>(ws + W.err);
    // Narrow rows: several tokens per wave, one per power-of-two group of
    // lanes wide enough for the widest present row (in 16-byte vectors) and
    // for the K lanes of the metadata.
    {
        int widest_v = 1;
        if (tk.x) widest_v = std::max(widest_v, s.H / 8);
        if (tk.x_fp8) widest_v = std::max(widest_v, s.H / 16);
        if (tk.x_scales) widest_v = std::max(widest_v, s.H / 128);
        if (s.K <= 8 && widest_v <= kWave / 2) {
            const int g = std::max(widest_v, s.K);
            int G = 8;  // groups of 8, 16 or 32 lanes: 8, 4 or 2 tokens per wave
            while (G < g) G *= 2;
            const int tpw = kWave / G;
            const int64_t nw = ((int64_t)s.T + tpw - 1) / tpw;
            const dim3 g2((unsigned)((nw + kDspWaves - 1) / kDspWaves)), b2(kDspThreads);
            switch (tpw) {
                case 2: hipLaunchKernelGGL(dispatch_narrow_kernel<2>, g2, b2, 0, st, a); break;
                case 4: hipLaunchKernelGGL(dispatch_narrow_kernel<4>, g2, b2, 0, st, a); break;
                default: hipLaunchKernelGGL(dispatch_narrow_kernel<8>, g2, b2, 0, st, a); break;
            }
            return hipGetLastError();
        }
    }
    // Slices per token: EP_DSP_SPLIT, halved while a slice of the widest
    // present row would not fill a wave's 64 lanes.
    const int64_t widest = tk.x ? 2 * (int64_t)s.H : (int64_t)s.H;
    a.split = EP_DSP_SPLIT;
    while (a.split > 1 && slice_vecs(widest / 16, a.split) < kWave) a.split = (a.split + 1) / 2;
    const int64_t waves = (int64_t)s.T * a.split;
    const dim3 grid((unsigned)((waves + kDspWaves - 1) / kDspWaves)), block(kDspThreads);
    // Vectors per lane held in registers: enough for the widest present slice.
    const int64_t slice = slice_vecs(widest / 16, a.split);
    const int64_t per_lane = (slice + kWave - 1) / kWave;
#if EP_DSP_PERSIST
    if (per_lane <= 4 && waves <= INT32_MAX) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dispatch_persistent_kernel<4>,
                                                              kDspThreads, 0)) != hipSuccess)
            return e;
        const int64_t resident = (int64_t)cus * std::max(1, std::min(per_cu, EP_DSP_PERSIST_BPC));
        const int64_t blocks = std::min<int64_t>(resident, (waves + kDspWaves - 1) / kDspWaves);
        hipLaunchKernelGGL(dispatch_persistent_kernel<4>, dim3((unsigned)blocks), block, 0, st, a, (int)waves);
        return hipGetLastError();
    }
#endif
    if (a.x_fp8 && a.rfp8) return launch_nv<true>(per_lane, grid, block, a, st);
    return launch_nv<false>(per_lane, grid, block, a, st);
}

}  // namespace ep
