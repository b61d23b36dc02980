// layout.hip -- ep_get_layout on gfx950: counts, offsets, masks and slots.
//
// What is computed follows "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK
// 复制机制", §3.3 阶段1 (notify warps: per-lane expert counts, per-token rank
// deduplication, prefix sums) and the slot hand-out of §3.3 阶段2, with slots
// made deterministic: the row of (token t, rank r) is
//     rank_offsets[r] + #{t' < t : token t' sends to r}.
//
// Two stream-ordered launches, all integer work, no waiting between
// workgroups:
//   1. count  : one thread per token, 256 tokens per workgroup. Each token ORs
//               its bit into an LDS bit matrix bits[r][t/32] (a repeated rank
//               sets the same bit: that is the deduplication) and bumps an
//               LDS expert histogram. Per-workgroup counts are popcounts of
//               the bit rows; the is-token-in-rank mask is expanded from the
//               same bits with 16-byte stores.
//   2. assign : every workgroup rebuilds its bit matrix, sums the count table
//               of the earlier workgroups (and of all of them) for each rank
//               and group, scans the totals in LDS (wave shuffles), and gives
//               every lane its slot = region start + earlier workgroups +
//               popcount of the bits of earlier tokens in its own workgroup.
//               Expert totals and offsets are split by rank: workgroup b owns
//               the experts of a slice of ranks, and the offset of a slice's
//               first expert is the prefix of the per-rank lane counts, which
//               every workgroup already sums. Workgroups never wait for each
//               other and no grid-wide fence is needed (the launch boundary
//               orders the two kernels).
#include <rocprim/block/block_radix_sort.hpp>

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kWords = kLayoutTokens / 32;  // bit-matrix words per rank per workgroup

struct LayoutArgs {
    int T, K, E, R, G, epr, P, nb;
    const int64_t* topk;
    uint32_t* err;
    int32_t* part_rank;      // [nb][R] per-workgroup counts
    int32_t* part_group;     // [nb][G]
    int32_t* part_expert;    // [nb][E]
    int32_t* part_lanes;     // [nb][R] valid lanes per rank (not deduplicated)
    ep_layout out;
};

// The expert ids of one token: lanes k < K of its row, held in registers when
// K <= KMAX (KMAX > 0), else re-read from memory on use (KMAX == 0).
template <int KMAX>
struct TokenIds {
    int64_t v[KMAX > 0 ? KMAX : 1];
    __device__ __forceinline__ void load(const int64_t* row, int K) {
        if constexpr (KMAX > 0) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k) v[k] = k < K ? row[k] : -1;
        }
    }
    __device__ __forceinline__ int64_t get(const int64_t* row, int k) const {
        if constexpr (KMAX > 0) return v[k];
        else return row[k];
    }
};

// Set this token's bit for every rank (and group) its valid lanes reach and
// count its experts. Returns whether any lane held an invalid id.
template <int KMAX>
__device__ __forceinline__ bool mark_token(const LayoutArgs& a, const TokenIds<KMAX>& ids,
                                           const int64_t* row, uint32_t* bits_r, uint32_t* bits_g,
                                           int32_t* cnt_e) {
    const int w = threadIdx.x / 32;
    const uint32_t bit = 1u << (threadIdx.x & 31);
    const int kn = KMAX > 0 ? KMAX : a.K;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < kn; ++k) {
        if (KMAX > 0 && k >= a.K) break;
        const int64_t e = ids.get(row, k);
        bad |= expert_bad(e, a.E);
        if (!expert_ok(e, a.E)) continue;
        const int r = (int)e / a.epr;
        atomicOr(&bits_r[r * kWords + w], bit);
        if (bits_g) atomicOr(&bits_g[(r / a.P) * kWords + w], bit);
        if (cnt_e) atomicAdd(&cnt_e[(int)e], 1);
    }
    return bad;
}

// Expand bits[c][t/32] into this workgroup's rows of a [T, C] uint8 mask, one
// token per thread: all lanes of a 32-token group read the same LDS word
// (a broadcast), and each lane writes its own row with 16-byte stores when C
// is a multiple of 16 (rows then stay 16-byte aligned), else byte stores.
__device__ void write_mask(const uint32_t* bits, int C, int t0, int nt, uint8_t* mask) {
    const int lt = threadIdx.x;
    if (lt >= nt) return;
    const int w = lt >> 5, sh = lt & 31;
    uint8_t* row = mask + (int64_t)(t0 + lt) * C;
    if ((C & 15) == 0) {
        for (int c0 = 0; c0 < C; c0 += 16) {
            uint32_t word[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 16; ++j)
                word[j >> 2] |= ((bits[(c0 + j) * kWords + w] >> sh) & 1u) << (8 * (j & 3));
            u32x4 out = {word[0], word[1], word[2], word[3]};
            st16(row + c0, out);
        }
    } else {
        for (int c = 0; c < C; ++c) row[c] = (uint8_t)((bits[c * kWords + w] >> sh) & 1u);
    }
}

__device__ __forceinline__ int popc_row(const uint32_t* bits, int c) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) s += __popc(bits[c * kWords + w]);
    return s;
}

template <int KMAX>
__global__ __launch_bounds__(kBlockThreads) void layout_count_kernel(LayoutArgs a) {
    extern __shared__ uint32_t lds[];
    uint32_t* bits_r = lds;
    uint32_t* bits_g = bits_r + a.R * kWords;
    int32_t* cnt_e = reinterpret_cast<int32_t*>(bits_g + a.G * kWords);
    const int b = blockIdx.x;
    const int t0 = b * kLayoutTokens;
    const int t = t0 + threadIdx.x;
    const int64_t* row = a.topk + (int64_t)t * a.K;
    TokenIds<KMAX> ids;
    if (t < a.T) ids.load(row, a.K);
    if (b == 0 && threadIdx.x == 0) *a.err = 0u;  // a pass of calls starts with a clean word
    const int n_lds = (a.R + a.G) * kWords + a.E;
    for (int i = threadIdx.x; i < n_lds; i += kBlockThreads) lds[i] = 0u;
    __syncthreads();
    if (t < a.T) mark_token<KMAX>(a, ids, row, bits_r, bits_g, cnt_e);
    __syncthreads();

    for (int c = threadIdx.x; c < a.R; c += kBlockThreads)
        a.part_rank[(int64_t)b * a.R + c] = popc_row(bits_r, c);
    for (int c = threadIdx.x; c < a.G; c += kBlockThreads)
        a.part_group[(int64_t)b * a.G + c] = popc_row(bits_g, c);
    for (int c = threadIdx.x; c < a.E; c += kBlockThreads)
        a.part_expert[(int64_t)b * a.E + c] = cnt_e[c];
    for (int c = threadIdx.x; c < a.R; c += kBlockThreads) {
        int lanes = 0;
        for (int e = c * a.epr; e < (c + 1) * a.epr; ++e) lanes += cnt_e[e];
        a.part_lanes[(int64_t)b * a.R + c] = lanes;
    }

    const int nt = min(kLayoutTokens, a.T - t0);
    if (nt > 0 && a.out.is_token_in_rank) write_mask(bits_r, a.R, t0, nt, a.out.is_token_in_rank);
    if (nt > 0 && a.out.is_token_in_group) write_mask(bits_g, a.G, t0, nt, a.out.is_token_in_group);
}

// Inclusive scan of one int across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Workgroup-wide exclusive scan where thread i owns the contiguous elements
// [i*per, min(n, (i+1)*per)) through get(i) / put(i, prefix). Returns the
// total. scratch: kWavesPerBlock ints of LDS. Contains two barriers.
template <typename Get, typename Put>
__device__ int block_scan(int n, Get get, Put put, int* scratch) {
    const int tid = threadIdx.x;
    const int per = (n + kBlockThreads - 1) / kBlockThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += get(i);
    const int inc = wave_inclusive_scan(s);
    if (lane_id() == kWave - 1) scratch[wave_in_block()] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        const int v = scratch[w];
        before += w < wave_in_block() ? v : 0;
        total += v;
    }
    int run = before + inc - s;
    for (int i = lo; i < hi; ++i) {
        const int v = get(i);
        put(i, run);
        run += v;
    }
    __syncthreads();
    return total;
}

constexpr int kMaxSliceRounds = EP_MAX_EXPERTS / kBlockThreads;

template <int KMAX>
__global__ __launch_bounds__(kBlockThreads) void layout_assign_kernel(LayoutArgs a) {
    extern __shared__ uint32_t lds[];
    uint32_t* bits_r = lds;
    uint32_t* bits_g = bits_r + a.R * kWords;
    int32_t* base_r = reinterpret_cast<int32_t*>(bits_g + a.G * kWords);  // [R]
    int32_t* tot_r = base_r + a.R;                                        // [R]
    int32_t* lane_base = tot_r + a.R;                                     // [R]
    int32_t* base_g = lane_base + a.R;                                    // [G]
    int32_t* tot_g = base_g + a.G;                                        // [G]
    int32_t* scratch = tot_g + a.G;                                       // [waves + 1]
    const int b = blockIdx.x;
    const bool groups = a.out.group_slot != nullptr;
    const int t0 = b * kLayoutTokens;
    const int t = t0 + threadIdx.x;
    const int64_t* row = a.topk + (int64_t)t * a.K;

    // Every global read this workgroup needs is issued first and together: the
    // token's ids, and for column c of each count table (ranks, lanes, groups,
    // this workgroup's slice of experts) the sums over the earlier workgroups
    // and over all of them. Column and row indices are clamped so that every
    // load is unconditional; out-of-range terms are masked from the sums.
    TokenIds<KMAX> ids;
    if (t < a.T) ids.load(row, a.K);
    int32_t* te = a.out.tokens_per_expert;
    int32_t* eo = a.out.expert_offsets;
    const bool experts = te || eo;
    const int rpb = (a.R + a.nb - 1) / a.nb;
    const int r0 = min(a.R, b * rpb), r1 = min(a.R, r0 + rpb);
    const int e0 = r0 * a.epr, ne = experts ? (r1 - r0) * a.epr : 0;
    const int ncols = max(max(a.R, a.G), ne);
    int etot[kMaxSliceRounds];
#pragma unroll
    for (int j = 0; j < kMaxSliceRounds; ++j) etot[j] = 0;
    for (int c = threadIdx.x, round = 0; c < ncols; c += kBlockThreads, ++round) {
        const int cr = min(c, a.R - 1), cg = min(c, a.G - 1);
        const int ce = min(e0 + c, a.E - 1);
        constexpr int kBatch = 16;
        const bool own_e = c < ne && a.out.expert_slot != nullptr;
        int rb = 0, ra = 0, la = 0, gb = 0, ga = 0, ea = 0;
        for (int b0 = 0; b0 < a.nb; b0 += kBatch) {
            int32_t vr[kBatch], vl[kBatch], vg[kBatch], ve[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int64_t rowj = min(b0 + j, a.nb - 1);
                vr[j] = a.part_rank[rowj * a.R + cr];
                vl[j] = a.part_lanes[rowj * a.R + cr];
                vg[j] = a.part_group[rowj * a.G + cg];
                ve[j] = a.part_expert[rowj * a.E + ce];
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const bool in = b0 + j < a.nb, early = b0 + j < b;
                rb += early ? vr[j] : 0;
                ra += in ? vr[j] : 0;
                la += in ? vl[j] : 0;
                gb += early ? vg[j] : 0;
                ga += in ? vg[j] : 0;
                // Expand mode: this column becomes the exclusive prefix over
                // workgroups (each expert column is owned by one workgroup).
                if (own_e && in) a.part_expert[(int64_t)(b0 + j) * a.E + ce] = ea;
                ea += in ? ve[j] : 0;
            }
        }
        if (c < a.R) {
            base_r[c] = rb;
            tot_r[c] = ra;
            lane_base[c] = la;
        }
        if (c < a.G) {
            base_g[c] = gb;
            tot_g[c] = ga;
        }
        if (c < ne) {
#pragma unroll
            for (int j = 0; j < kMaxSliceRounds; ++j)
                if (j == round) etot[j] = ea;
            if (te) te[e0 + c] = ea;
        }
    }

    for (int i = threadIdx.x; i < (a.R + a.G) * kWords; i += kBlockThreads) lds[i] = 0u;
    __syncthreads();
    bool bad = false;
    if (t < a.T) bad = mark_token<KMAX>(a, ids, row, bits_r, groups ? bits_g : nullptr, nullptr);

    // Region starts = exclusive scan of the totals; workgroup 0 publishes the
    // counts and offsets.
    const bool pub = b == 0;
    int32_t* ro = a.out.rank_offsets;
    int32_t* go = a.out.group_offsets;
    const int n_rows = block_scan(
        a.R, [&](int i) { return tot_r[i]; },
        [&](int i, int p) {
            base_r[i] += p;
            if (pub && ro) ro[i] = p;
            if (pub && a.out.tokens_per_rank) a.out.tokens_per_rank[i] = tot_r[i];
        },
        scratch);
    const int n_grows = block_scan(
        a.G, [&](int i) { return tot_g[i]; },
        [&](int i, int p) {
            base_g[i] += p;
            if (pub && go) go[i] = p;
            if (pub && a.out.tokens_per_group) a.out.tokens_per_group[i] = tot_g[i];
        },
        scratch);
    // lane_base: lane totals -> exclusive prefix (in place; each thread owns its chunk)
    const int n_lanes = block_scan(
        a.R, [&](int i) { return lane_base[i]; }, [&](int i, int p) { lane_base[i] = p; }, scratch);
    if (pub && threadIdx.x == 0) {
        if (ro) ro[a.R] = n_rows;
        if (go) go[a.G] = n_grows;
        if (eo) eo[a.E] = n_lanes;
    }

    if (bad) report(a.err, EP_DEVERR_EXPERT_ID);
    if (t < a.T) {
        const int w = threadIdx.x / 32;
        const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
        const int kn = KMAX > 0 ? KMAX : a.K;
#pragma unroll
        for (int k = 0; k < kn; ++k) {
            if (KMAX > 0 && k >= a.K) break;
            const int64_t e = ids.get(row, k);
            int32_t s = -1, gs = -1;
            if (expert_ok(e, a.E)) {
                const int r = (int)e / a.epr;
                int pre = __popc(bits_r[r * kWords + w] & below);
                for (int j = 0; j < w; ++j) pre += __popc(bits_r[r * kWords + j]);
                s = base_r[r] + pre;
                if (groups) {
                    const int g = r / a.P;
                    int gpre = __popc(bits_g[g * kWords + w] & below);
                    for (int j = 0; j < w; ++j) gpre += __popc(bits_g[g * kWords + j]);
                    gs = base_g[g] + gpre;
                }
            }
            if (a.out.slot) a.out.slot[(int64_t)t * a.K + k] = s;
            if (groups) a.out.group_slot[(int64_t)t * a.K + k] = gs;
        }
    }

    // Expert offsets of this workgroup's slice of ranks: lanes of the earlier
    // ranks + prefix inside the slice (column c of the slice sits in round
    // c / 256 of thread c % 256).
    if (!eo || ne == 0) return;
    int carry = lane_base[r0];
#pragma unroll
    for (int j = 0; j < kMaxSliceRounds; ++j) {
        if (j * kBlockThreads >= ne) break;
        const int v = etot[j];
        const int inc = wave_inclusive_scan(v);
        if (lane_id() == kWave - 1) scratch[wave_in_block()] = inc;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) {
            before += w < wave_in_block() ? scratch[w] : 0;
            total += scratch[w];
        }
        const int c = j * kBlockThreads + threadIdx.x;
        if (c < ne) eo[e0 + c] = carry + before + inc - v;
        carry += total;
        __syncthreads();
    }
}

// Expand-mode rows: the (token, lane) entries of a 256-token workgroup are
// sorted by expert, stably (entries keep token-then-lane order inside an
// expert), with a block radix sort in LDS. The row of an entry is
//   expert_offsets[e] + (lanes of e in earlier workgroups) + (position of the
//   entry among the workgroup's entries of e).
// The middle term is the count table turned into per-workgroup prefixes by
// the assign launch.
template <int ITEMS>
__global__ __launch_bounds__(kBlockThreads) void layout_expand_kernel(LayoutArgs a, int key_bits) {
    using sort_t = rocprim::block_radix_sort<int, kBlockThreads, ITEMS, int>;
    __shared__ union {
        typename sort_t::storage_type sort;
        int keys[kBlockThreads * ITEMS];
    } sh;
    const int b = blockIdx.x;
    const int t0 = b * kLayoutTokens;
    const int t = t0 + threadIdx.x;
    int keys[ITEMS], vals[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        int64_t e = -1;
        if (t < a.T && k < a.K) e = a.topk[(int64_t)t * a.K + k];
        keys[k] = expert_ok(e, a.E) ? (int)e : a.E;  // no expert: sorted last
        vals[k] = threadIdx.x * ITEMS + k;
    }
    sort_t().sort(keys, vals, sh.sort, 0, key_bits);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) sh.keys[threadIdx.x * ITEMS + j] = keys[j];
    __syncthreads();
    const int n = kBlockThreads * ITEMS;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int pos = threadIdx.x * ITEMS + j;
        const int key = keys[j];
        const int lt = vals[j] / ITEMS, k = vals[j] % ITEMS;
        if (k >= a.K || t0 + lt >= a.T) continue;  // padding entry
        int32_t row = -1;
        if (key < a.E) {
            int lo = 0, hi = pos;  // first position holding `key`
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (sh.keys[mid] < key) lo = mid + 1; else hi = mid;
            }
            row = a.out.expert_offsets[key] + a.part_expert[(int64_t)b * a.E + key] + (pos - lo);
        }
        a.out.expert_slot[(int64_t)(t0 + lt) * a.K + k] = row;
        (void)n;
    }
}

}  // namespace

hipError_t launch_layout(const ep_shape& s, const int64_t* topk, const ep_layout& L, char* ws,
                         hipStream_t st) {
    const WsLayout W = ws_layout(s);
    LayoutArgs a;
    a.T = s.T; a.K = s.K; a.E = s.E; a.R = s.R; a.G = s.G;
    a.epr = s.E / s.R; a.P = s.R / s.G; a.nb = W.nb;
    a.topk = topk;
    a.err = reinterpret_cast<uint32_t*>(ws + W.err);
    a.part_rank = reinterpret_cast<int32_t*>(ws + W.part_rank);
    a.part_group = reinterpret_cast<int32_t*>(ws + W.part_group);
    a.part_expert = reinterpret_cast<int32_t*>(ws + W.part_expert);
    a.part_lanes = reinterpret_cast<int32_t*>(ws + W.part_lanes);
    a.out = L;

    const size_t lds_count = sizeof(uint32_t) * ((size_t)(s.R + s.G) * kWords + s.E);
    const size_t lds_assign = sizeof(uint32_t) * ((size_t)(s.R + s.G) * kWords + 3 * (size_t)s.R +
                                                  2 * (size_t)s.G + kWavesPerBlock + 1);
    const dim3 grid(W.nb), block(kBlockThreads);
#define EP_LAYOUT_LAUNCH(KM)                                                          \
    do {                                                                              \
        hipLaunchKernelGGL(layout_count_kernel<KM>, grid, block, lds_count, st, a);   \
        hipLaunchKernelGGL(layout_assign_kernel<KM>, grid, block, lds_assign, st, a); \
    } while (0)
    if (s.K <= 2)
        EP_LAYOUT_LAUNCH(2);
    else if (s.K <= 4)
        EP_LAYOUT_LAUNCH(4);
    else if (s.K <= 8)
        EP_LAYOUT_LAUNCH(8);
    else
        EP_LAYOUT_LAUNCH(0);
#undef EP_LAYOUT_LAUNCH
    if (L.expert_slot) {
        int bits = 1;
        while ((1 << bits) <= s.E) ++bits;  // keys 0..E
        if (s.K <= 8)
            hipLaunchKernelGGL(layout_expand_kernel<8>, grid, block, 0, st, a, bits);
        else
            hipLaunchKernelGGL(layout_expand_kernel<16>, grid, block, 0, st, a, bits);
    }
    return hipGetLastError();
}

}  // namespace ep
