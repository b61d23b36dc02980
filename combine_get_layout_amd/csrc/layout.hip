// layout.hip -- ep_get_layout on gfx950: counts, offsets, masks and slots.
//
// What is computed follows "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK
// 复制机制", §3.3 阶段1 (notify warps: per-lane expert counts, per-token rank
// deduplication, prefix sums) and the slot hand-out of §3.3 阶段2, with slots
// made deterministic: the row of (token t, rank r) is
//     rank_offsets[r] + #{t' < t : token t' sends to r}.
//
// Two stream-ordered launches (three with expand rows), all integer work, no
// waiting between workgroups:
//   1. count  : one thread per token, 256 tokens per workgroup. Each token ORs
//               its bit into an LDS bit matrix bits[r][t/32] (a repeated rank
//               sets the same bit: that is the deduplication) and bumps an
//               LDS expert histogram; with one group, the group bits are one
//               wave ballot. Per-workgroup counts are popcounts of the bit
//               rows, written as one row per workgroup of two tables
//               ([ranks | lanes per rank | groups] and [experts]); the
//               is-token-in-rank mask is expanded from the same bits with
//               16-byte stores.
//   2. assign : every workgroup rebuilds its bit matrix and reads every row of
//               the rank/lane/group table as 16-byte vectors, keeping for each
//               column the sum over the earlier workgroups and over all of
//               them. The section totals go through DPP wave scans and one
//               barrier; each lane's slot = region start + earlier
//               workgroups + this workgroup's tokens to the rank in earlier
//               32-token words (a u8 table) + popcount of the earlier bits of
//               its own word. Expert totals and offsets are split by rank:
//               workgroup b owns the experts of a slice of ranks, and the
//               offset of a slice's first expert is the prefix of the
//               per-rank lane counts, which every workgroup already sums.
//   3. expand : (only when expand rows are asked for) the row of each
//               (token, lane) inside its expert's region.
// With many workgroups (kScanMinBlocks or more) the assign launch would read
// nb rows in each of nb workgroups; a scan launch between count and assign
// then turns every column of both tables into its exclusive prefix over the
// workgroup rows (in place, totals in an extra row nb), and each assign
// workgroup reads two rows: O(nb * columns) work in all instead of
// O(nb^2 * columns).
// Workgroups never wait for each other and no grid-wide fence is needed (the
// launch boundaries order the kernels).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include <rocprim/block/block_radix_sort.hpp>
#include <rocprim/warp/warp_scan.hpp>

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kWords = kLayoutTokens / 32;  // bit-matrix words per rank per workgroup

struct LayoutArgs {
    int T, K, E, R, G, epr, P, nb;
    FastDiv div_epr, div_P;  // e / epr (rank of an expert), r / P (group of a rank)
    int rp, wrow;            // rank/lane/group table: lanes start at column rp, groups at 2 rp
    const int64_t* topk;
    uint32_t* err;
    // Per-workgroup count tables, one row per workgroup:
    int32_t* part_rlg;       // [nb][wrow] ranks | lanes per rank | groups
    int32_t* part_expert;    // [nb][E] lanes per expert
    ep_layout out;
};

// The expert ids of one token: lanes k < K of its row, held in registers when
// K <= KMAX (KMAX > 0), else re-read from memory on use (KMAX == 0).
template <int KMAX>
struct TokenIds {
    int64_t v[KMAX > 0 ? KMAX : 1];
    __device__ __forceinline__ void load(const int64_t* row, int K) {
        if constexpr (KMAX > 0) {
            // Every load issued (lanes k >= K re-read lane K - 1; callers
            // stop at K): loads under a branch were sunk past the LDS
            // clearing and the barrier to their first use.
#pragma unroll
            for (int k = 0; k < KMAX; ++k) v[k] = row[min(k, K - 1)];
        }
    }
    // Callers ask for lanes k < K only.
    __device__ __forceinline__ int64_t get(const int64_t* row, int k) const {
        if constexpr (KMAX > 0) return v[k];
        else return row[k];
    }
};

// Set this token's bit for every rank its valid lanes reach (LDS atomics: a
// repeated rank sets the same bit) and, with cnt_e, count its experts. The
// group bits: with one group, bit (0, t) is "the token has a valid lane",
// written by the wave from one ballot (lane 0 holds the word of lanes 0-31,
// lane 32 that of lanes 32-63; tokens past T form a suffix of inactive
// lanes, so both writers are active whenever their half has a token); with
// several groups, LDS atomics as for ranks. Returns whether any lane held an
// invalid id.
template <int KMAX>
__device__ __forceinline__ bool mark_token(const LayoutArgs& a, const TokenIds<KMAX>& ids,
                                           const int64_t* row, uint32_t* bits_r, uint32_t* bits_g,
                                           int32_t* cnt_e) {
    const int w = threadIdx.x / 32;
    const uint32_t bit = 1u << (threadIdx.x & 31);
    const int kn = KMAX > 0 ? KMAX : a.K;
    const bool group_atomics = bits_g && a.G > 1;
    bool bad = false, any = false;
#pragma unroll
    for (int k = 0; k < kn; ++k) {
        if (KMAX > 0 && k >= a.K) break;
        const int64_t e = ids.get(row, k);
        bad |= expert_bad(e, a.E);
        if (!expert_ok(e, a.E)) continue;
        any = true;
        const int r = a.div_epr((int)e);
        atomicOr(&bits_r[r * kWords + w], bit);
        if (group_atomics) atomicOr(&bits_g[a.div_P(r) * kWords + w], bit);
        if (cnt_e) atomicAdd(&cnt_e[(int)e], 1);
    }
    if (bits_g && a.G == 1) {
        const uint64_t m = __ballot(any);
        const int lane = lane_id();
        if (lane == 0 || lane == 32) bits_g[w] = (uint32_t)(m >> lane);
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

    int32_t* rlg = a.part_rlg + (int64_t)b * a.wrow;
    for (int c = threadIdx.x; c < a.R; c += kBlockThreads) {
        rlg[c] = popc_row(bits_r, c);
        int lanes = 0;
        for (int e = c * a.epr; e < (c + 1) * a.epr; ++e) lanes += cnt_e[e];
        rlg[a.rp + c] = lanes;
    }
    for (int c = threadIdx.x; c < a.G; c += kBlockThreads) rlg[2 * a.rp + c] = popc_row(bits_g, c);
    for (int c = threadIdx.x; c < a.E; c += kBlockThreads)
        a.part_expert[(int64_t)b * a.E + c] = cnt_e[c];

    const int nt = min(kLayoutTokens, a.T - t0);
    if (nt > 0 && a.out.is_token_in_rank) write_mask(bits_r, a.R, t0, nt, a.out.is_token_in_rank);
    if (nt > 0 && a.out.is_token_in_group) write_mask(bits_g, a.G, t0, nt, a.out.is_token_in_group);
}

// Inclusive scan of one int across the 64 lanes of a wave (rocPRIM's
// cross-lane scan: DPP row shifts and row broadcasts, no LDS round trips).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    using scan_t = rocprim::warp_scan<int, kWave>;
    static_assert(sizeof(scan_t::storage_type) <= 1, "cross-lane scan: no shared storage");
    scan_t::storage_type none;
    int y;
    scan_t().inclusive_scan(x, y, none, rocprim::plus<int>());
    return y;
}

// The assign kernel's ownership of table columns:
//   * vector v = q*256 + thread (round q) of a rank/lane/group row: columns
//     4v .. 4v+3, all in one section since rp and gp are multiples of 4;
//   * column q*256 + thread of this workgroup's slice of experts.
constexpr int kVecRounds = (2 * EP_MAX_RANKS + EP_MAX_GROUPS + 4 * kBlockThreads - 1) / (4 * kBlockThreads);
constexpr int kSliceRounds = EP_MAX_EXPERTS / kBlockThreads;
#ifndef EP_LAYOUT_ROWBATCH
#define EP_LAYOUT_ROWBATCH 8  // table rows (workgroups) loaded per batch
#endif
constexpr int kRowBatch = EP_LAYOUT_ROWBATCH;
constexpr int kSpreadStride = 17;  // ints per (thread group, column) partial: 2 x (4 + 4) + 1
// Scan slots of the LDS scratch, one int per wave each.
constexpr int kScRank = 0;                          // rank totals, per vector round
constexpr int kScLane = kScRank + kVecRounds;       // lane totals, per vector round
constexpr int kScGroup = kScLane + kVecRounds;      // group totals, per vector round
constexpr int kScSlice = kScGroup + kVecRounds;     // expert slice totals, per slice round
constexpr int kScLaneStart = kScSlice + kSliceRounds;  // lanes of the ranks before the slice
constexpr int kScSlots = kScLaneStart + 1;

// Workgroup-wide exclusive prefix of the value x that this thread holds in
// round q, from its wave-inclusive scan `inc` and the per-wave totals of
// every round in sc[round * waves + wave]. Also returns the grand total.
template <int NR>
__device__ __forceinline__ int round_prefix(const int32_t* sc, int nr, int q, int inc, int x,
                                            int& total) {
    int before = 0;
    total = 0;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        if (j >= nr) break;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) {
            const int y = sc[j * kWavesPerBlock + w];
            total += y;
            before += (j < q || (j == q && w < wave_in_block())) ? y : 0;
        }
    }
    return before + inc - x;
}

// Running sums over the rows of a batch: rows < b (earlier workgroups) and
// rows < nb (all); clamped repeats past the last row are masked.
__device__ __forceinline__ void add_rows(const u32x4* x, int b0, int b, int nb, int (&bef)[4],
                                         int (&all)[4]) {
#pragma unroll
    for (int j = 0; j < kRowBatch; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bef[i] += b0 + j < b ? (int)x[j][i] : 0;
            all[i] += b0 + j < nb ? (int)x[j][i] : 0;
        }
    }
}

// SPREAD: the launch has more than 2 batches of table rows and no expand
// rows, so the spread loads below may apply (a separate instantiation keeps
// the code of the other launches as it is). SCANNED: the scan launch has
// already turned the tables into per-workgroup prefixes with the totals in
// row nb, so only rows b and nb are read.
template <int KMAX, bool SPREAD, bool SCANNED>
__global__ __launch_bounds__(kBlockThreads) void layout_assign_kernel(LayoutArgs a) {
    extern __shared__ __align__(16) uint32_t lds[];
    uint32_t* bits_r = lds;                                                // [R][kWords]
    uint32_t* bits_g = bits_r + a.R * kWords;                              // [G][kWords]
    int32_t* base_r = reinterpret_cast<int32_t*>(bits_g + a.G * kWords);  // [R]
    int32_t* base_g = base_r + a.R;                                        // [G]
    int32_t* scratch = base_g + a.G;                                       // [kScSlots][waves]
    uint8_t* pre_r = reinterpret_cast<uint8_t*>(scratch + kScSlots * kWavesPerBlock);  // [R][kWords]
    uint8_t* pre_g = pre_r + a.R * kWords;                                 // [G][kWords]
    int32_t* red = reinterpret_cast<int32_t*>(pre_g + a.G * kWords);       // [kBlockThreads][kSpreadStride]
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const bool groups = a.out.group_slot != nullptr;
    const int t0 = b * kLayoutTokens;
    const int t = t0 + tid;
    const int64_t* row = a.topk + (int64_t)t * a.K;

    // The token's ids first; the bit matrices are cleared while they are in
    // flight.
    TokenIds<KMAX> ids;
    if (t < a.T) ids.load(row, a.K);
    for (int i = tid; i < (a.R + a.G) * kWords; i += kBlockThreads) lds[i] = 0u;
    for (int i = tid; i < kScSlots * kWavesPerBlock; i += kBlockThreads) scratch[i] = 0;

    // Count tables. The rank/lane/group rows are read as 16-byte vectors,
    // thread v taking vector v of every row, so a wave's load is 1 KiB of one
    // row. The slice of experts this workgroup owns (the experts of ranks
    // [r0, r1)) is read one column per thread. Round 0 of both is loaded in
    // the same batches; every load of a batch is unconditional (rows clamped,
    // repeats masked). For each column the sums over the earlier workgroups
    // (bef) and over all of them (all, etot) are kept.
    int32_t* te = a.out.tokens_per_expert;
    int32_t* eo = a.out.expert_offsets;
    const bool experts = te || eo;
    const int rpb = (a.R + a.nb - 1) / a.nb;
    const int r0 = min(a.R, b * rpb), r1 = min(a.R, r0 + rpb);
    const int e0 = r0 * a.epr, ne = experts ? (r1 - r0) * a.epr : 0;
    const int nvec = a.wrow / 4;
    const int vec_rounds = (nvec + kBlockThreads - 1) / kBlockThreads;
    const int slice_rounds = (ne + kBlockThreads - 1) / kBlockThreads;
    const bool expand = a.out.expert_slot != nullptr;
    int bef[kVecRounds][4], all[kVecRounds][4], etot[kSliceRounds];
#pragma unroll
    for (int q = 0; q < kVecRounds; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) bef[q][i] = all[q][i] = 0;
#pragma unroll
    for (int q = 0; q < kSliceRounds; ++q) etot[q] = 0;
    // Expert column c of the slice: its total; in expand mode the column is
    // rewritten in place as the exclusive prefix over workgroups (each expert
    // column is owned by one workgroup).
    auto expert_rows = [&](const int32_t* x, int32_t* pe, int b0, bool own, int& ea) {
#pragma unroll
        for (int j = 0; j < kRowBatch; ++j) {
            if (own && b0 + j < a.nb) pe[(int64_t)(b0 + j) * a.E] = ea;
            ea += b0 + j < a.nb ? x[j] : 0;
        }
    };
    // Many rows of a table of at most 256 vectors, no expand rows: a thread
    // takes vpt (1 or 2) neighbouring vectors and one expert column, and the
    // threads form J = 256 / cols groups, group j reading rows j, j + J,
    // j + 2J, ..., so each thread follows about nb / J rows instead of nb.
    // The groups' partial sums (per vector: 4 columns before b and 4 over all
    // rows; the expert column's total) meet in LDS at the barrier after the
    // loads. Measured: 22.2 -> 18.8 us per layout call at 64 workgroups and
    // 34 vectors per row; with 2 batches of rows or fewer the extra LDS pass
    // costs more than it saves.
    const int vpt = nvec > 128 ? 2 : 1;
    const int cols = max(max((nvec + vpt - 1) / vpt, ne), 1);
    const int J = kBlockThreads / cols;
    const bool spread = SPREAD && !SCANNED && !expand && vec_rounds == 1 && slice_rounds <= 1 &&
                        J >= 2 && a.nb > 2 * kRowBatch;
    auto spread_loads = [&](auto vpt_c) {
        constexpr int VPT = decltype(vpt_c)::value;
        const int c = tid % cols, j = tid / cols;
        if (j >= J) return;
        const int32_t* pv[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) pv[u] = a.part_rlg + 4 * min(c * VPT + u, nvec - 1);
        const int32_t* pcol = a.part_expert + min(e0 + c, a.E - 1);
        int pb[VPT][4] = {}, pa[VPT][4] = {}, pe_sum = 0;
        for (int rb = j; rb < a.nb; rb += J * kRowBatch) {
            u32x4 x[VPT][kRowBatch];
            int32_t xe[kRowBatch];
#pragma unroll
            for (int i = 0; i < kRowBatch; ++i) {
                const int64_t rr = min(rb + i * J, a.nb - 1);
#pragma unroll
                for (int u = 0; u < VPT; ++u) x[u][i] = ld16(pv[u] + rr * a.wrow);
                xe[i] = pcol[rr * a.E];
            }
#pragma unroll
            for (int i = 0; i < kRowBatch; ++i) {
                const int rr = rb + i * J;
                const bool in = rr < a.nb, before = rr < b;
#pragma unroll
                for (int u = 0; u < VPT; ++u)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        pa[u][q] += in ? (int)x[u][i][q] : 0;
                        pb[u][q] += before ? (int)x[u][i][q] : 0;
                    }
                pe_sum += in ? xe[i] : 0;
            }
        }
        int32_t* o = red + (j * cols + c) * kSpreadStride;
#pragma unroll
        for (int u = 0; u < VPT; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o[8 * u + q] = pb[u][q];
                o[8 * u + 4 + q] = pa[u][q];
            }
        o[16] = pe_sum;
    };
    if constexpr (SCANNED) {
        // This workgroup's prefix row and the totals row, every round at once.
        const int32_t* pb = a.part_rlg + (int64_t)b * a.wrow;
        const int32_t* pa = a.part_rlg + (int64_t)a.nb * a.wrow;
        const int32_t* ea = a.part_expert + (int64_t)a.nb * a.E;
        u32x4 xb[kVecRounds], xa[kVecRounds];
        int32_t xe[kSliceRounds];
#pragma unroll
        for (int q = 0; q < kVecRounds; ++q) {
            const int v = min(q * kBlockThreads + tid, nvec - 1);
            xb[q] = ld16(pb + 4 * v);
            xa[q] = ld16(pa + 4 * v);
        }
#pragma unroll
        for (int q = 0; q < kSliceRounds; ++q) xe[q] = ea[min(e0 + q * kBlockThreads + tid, a.E - 1)];
#pragma unroll
        for (int q = 0; q < kVecRounds; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bef[q][i] = q < vec_rounds ? (int)xb[q][i] : 0;
                all[q][i] = q < vec_rounds ? (int)xa[q][i] : 0;
            }
#pragma unroll
        for (int q = 0; q < kSliceRounds; ++q) {
            const int c = q * kBlockThreads + tid;
            if (q < slice_rounds && c < ne) {
                etot[q] = xe[q];
                if (te) te[e0 + c] = xe[q];
            }
        }
    } else if (spread) {
        if (vpt == 2)
            spread_loads(std::integral_constant<int, 2>{});
        else
            spread_loads(std::integral_constant<int, 1>{});
    } else {
        const int v = min(tid, nvec - 1);
        const int32_t* pv = a.part_rlg + 4 * v;
        const bool own = tid < ne && expand;
        int32_t* pe = a.part_expert + min(e0 + tid, a.E - 1);
        int ea = 0;
        for (int b0 = 0; b0 < a.nb; b0 += kRowBatch) {
            u32x4 x[kRowBatch];
            int32_t xe[kRowBatch];
#pragma unroll
            for (int j = 0; j < kRowBatch; ++j) {
                const int64_t rj = min(b0 + j, a.nb - 1);
                x[j] = ld16(pv + rj * a.wrow);
                xe[j] = pe[rj * a.E];
            }
            add_rows(x, b0, b, a.nb, bef[0], all[0]);
            expert_rows(xe, pe, b0, own, ea);
        }
        if (tid < ne) {
            etot[0] = ea;
            if (te) te[e0 + tid] = ea;
        }
    }
    // Further rounds: only for tables wider than 1,024 columns or slices
    // wider than 256 experts.
#pragma unroll
    for (int q = 1; q < kVecRounds; ++q) {
        if (!SCANNED && q < vec_rounds) {
            const int32_t* pv = a.part_rlg + 4 * min(q * kBlockThreads + tid, nvec - 1);
            for (int b0 = 0; b0 < a.nb; b0 += kRowBatch) {
                u32x4 x[kRowBatch];
#pragma unroll
                for (int j = 0; j < kRowBatch; ++j) x[j] = ld16(pv + (int64_t)min(b0 + j, a.nb - 1) * a.wrow);
                add_rows(x, b0, b, a.nb, bef[q], all[q]);
            }
        }
    }
#pragma unroll
    for (int q = 1; q < kSliceRounds; ++q) {
        if (!SCANNED && q < slice_rounds) {
            const int c = q * kBlockThreads + tid;
            const bool own = c < ne && expand;
            int32_t* pe = a.part_expert + min(e0 + c, a.E - 1);
            int ea = 0;
            for (int b0 = 0; b0 < a.nb; b0 += kRowBatch) {
                int32_t xe[kRowBatch];
#pragma unroll
                for (int j = 0; j < kRowBatch; ++j) xe[j] = pe[(int64_t)min(b0 + j, a.nb - 1) * a.E];
                expert_rows(xe, pe, b0, own, ea);
            }
            if (c < ne) {
                etot[q] = ea;
                if (te) te[e0 + c] = ea;
            }
        }
    }
    __syncthreads();
    if (spread) {
        if (tid < nvec) {  // vector tid = neighbour tid % vpt of column tid / vpt
            const int c = tid / vpt, u = tid % vpt;
            int sb[4] = {0, 0, 0, 0}, sa[4] = {0, 0, 0, 0};
            for (int j = 0; j < J; ++j) {
                const int32_t* o = red + (j * cols + c) * kSpreadStride + 8 * u;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    sb[q] += o[q];
                    sa[q] += o[4 + q];
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bef[0][q] = sb[q];
                all[0][q] = sa[q];
            }
        }
        if (tid < ne) {
            int se = 0;
            for (int j = 0; j < J; ++j) se += red[(j * cols + tid) * kSpreadStride + 16];
            etot[0] = se;
            if (te) te[e0 + tid] = se;
        }
    }

    bool bad = false;
    if (t < a.T) bad = mark_token<KMAX>(a, ids, row, bits_r, groups ? bits_g : nullptr, nullptr);

    // The section of this thread's vector in round q (0 ranks, 1 lanes,
    // 2 groups, -1 none), its first column inside the section, and whether
    // column i of the vector is a real column (padding columns are masked).
    auto section = [&](int q, int& col0) {
        const int v = q * kBlockThreads + tid;
        const int c4 = 4 * v;
        if (v >= nvec) { col0 = 0; return -1; }
        if (c4 < a.rp) { col0 = c4; return 0; }
        if (c4 < 2 * a.rp) { col0 = c4 - a.rp; return 1; }
        col0 = c4 - 2 * a.rp;
        return 2;
    };
    auto col_ok = [&](int sec, int col) { return sec >= 0 && col < (sec == 2 ? a.G : a.R); };

    // Wave scans of the section totals and of the expert slice; the wave
    // totals go to the scratch slots. The lanes of the ranks before this
    // workgroup's slice (r < r0) are one more workgroup-wide sum.
    int inc[kVecRounds], tot[kVecRounds], inc_e[kSliceRounds];
    int before_slice = 0;
    const bool last_lane = lane_id() == kWave - 1;
    const int wv = wave_in_block();
#pragma unroll
    for (int q = 0; q < kVecRounds; ++q) {
        inc[q] = tot[q] = 0;
        if (q >= vec_rounds) continue;
        int col0;
        const int sec = section(q, col0);
        int x = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = col_ok(sec, col0 + i) ? all[q][i] : 0;
            x += v;
            before_slice += sec == 1 && col0 + i < r0 ? v : 0;
        }
        tot[q] = x;
        const int xr = wave_inclusive_scan(sec == 0 ? x : 0);
        const int xl = wave_inclusive_scan(sec == 1 ? x : 0);
        const int xg = wave_inclusive_scan(sec == 2 ? x : 0);
        inc[q] = sec == 0 ? xr : (sec == 1 ? xl : xg);
        if (last_lane) {
            scratch[(kScRank + q) * kWavesPerBlock + wv] = xr;
            scratch[(kScLane + q) * kWavesPerBlock + wv] = xl;
            scratch[(kScGroup + q) * kWavesPerBlock + wv] = xg;
        }
    }
#pragma unroll
    for (int q = 0; q < kSliceRounds; ++q) {
        inc_e[q] = 0;
        if (q >= slice_rounds) continue;
        inc_e[q] = wave_inclusive_scan(etot[q]);
        if (last_lane) scratch[(kScSlice + q) * kWavesPerBlock + wv] = inc_e[q];
    }
    before_slice = wave_inclusive_scan(before_slice);
    if (last_lane) scratch[kScLaneStart * kWavesPerBlock + wv] = before_slice;
    __syncthreads();

    // Region starts. Each owned rank (group) column gets its first row for
    // this workgroup, base = region start + earlier workgroups, and the u8
    // count of this workgroup's tokens to it before each 32-token word.
    // Workgroup 0 publishes the counts and offsets.
    const bool pub = b == 0;
    int32_t* ro = a.out.rank_offsets;
    int32_t* go = a.out.group_offsets;
#pragma unroll
    for (int q = 0; q < kVecRounds; ++q) {
        if (q >= vec_rounds) break;
        int col0;
        const int sec = section(q, col0);
        if (sec < 0) continue;
        const int sc = sec == 0 ? kScRank : (sec == 1 ? kScLane : kScGroup);
        // Exclusive prefix of this thread's vector within its section, over
        // the rounds and waves before it, and the section total.
        int run = 0, total = 0;
        for (int j = 0; j < vec_rounds; ++j) {
#pragma unroll
            for (int w = 0; w < kWavesPerBlock; ++w) {
                const int y = scratch[(sc + j) * kWavesPerBlock + w];
                total += y;
                run += (j < q || (j == q && w < wv)) ? y : 0;
            }
        }
        run += inc[q] - tot[q];
        if (sec == 1) {
            if (pub && eo && col_ok(sec, col0) && col0 + 4 >= a.R && col0 < a.R) eo[a.E] = total;
            continue;
        }
        uint32_t* bits = sec == 0 ? bits_r : bits_g;
        int32_t* base = sec == 0 ? base_r : base_g;
        uint8_t* pre = sec == 0 ? pre_r : pre_g;
        int32_t* off = sec == 0 ? ro : go;
        int32_t* cnt = sec == 0 ? a.out.tokens_per_rank : a.out.tokens_per_group;
        const int n = sec == 0 ? a.R : a.G;
        const bool want_pre = sec == 0 || groups;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = col0 + i;
            if (c >= n) break;
            base[c] = run + bef[q][i];
            if (want_pre) {
                // The column's 8 words in two 16-byte LDS reads (rows of the
                // bit matrix are 32-byte aligned), then its 8 u8 prefixes in
                // two 4-byte writes: no read waits behind a write.
                static_assert(kWords == 8, "pre table packing assumes 8 words per column");
                const u32x4 w0 = *reinterpret_cast<const u32x4*>(bits + c * kWords);
                const u32x4 w1 = *reinterpret_cast<const u32x4*>(bits + c * kWords + 4);
                const uint32_t n0 = __popc(w0[0]), n1 = n0 + __popc(w0[1]), n2 = n1 + __popc(w0[2]),
                               n3 = n2 + __popc(w0[3]), n4 = n3 + __popc(w1[0]), n5 = n4 + __popc(w1[1]),
                               n6 = n5 + __popc(w1[2]);
                uint32_t* pw = reinterpret_cast<uint32_t*>(pre + c * kWords);
                pw[0] = (n0 << 8) | (n1 << 16) | (n2 << 24);
                pw[1] = n3 | (n4 << 8) | (n5 << 16) | (n6 << 24);
            }
            if (pub) {
                if (off) off[c] = run;
                if (cnt) cnt[c] = all[q][i];
                if (off && c == n - 1) off[n] = total;
            }
            run += all[q][i];
        }
    }
    // Expert offsets of this workgroup's slice: lanes of the ranks before the
    // slice + prefix inside the slice.
    if (eo && ne > 0) {
        int lane_start = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) lane_start += scratch[kScLaneStart * kWavesPerBlock + w];
#pragma unroll
        for (int q = 0; q < kSliceRounds; ++q) {
            const int c = q * kBlockThreads + tid;
            if (q >= slice_rounds) break;
            int unused;
            const int p = round_prefix<kSliceRounds>(scratch + kScSlice * kWavesPerBlock, slice_rounds, q,
                                                      inc_e[q], etot[q], unused);
            if (c < ne) eo[e0 + c] = lane_start + p;
        }
    }
    __syncthreads();

    if (bad) report(a.err, EP_DEVERR_EXPERT_ID);
    if (t >= a.T) return;
    // Slot of lane k = base of its rank + tokens of this workgroup to that
    // rank in earlier words + earlier tokens of its own word.
    const int w = tid / 32;
    const uint32_t below = (1u << (tid & 31)) - 1u;
    auto slot_of = [&](int64_t e, int32_t& s, int32_t& gs) {
        s = gs = -1;
        if (!expert_ok(e, a.E)) return;
        const int r = a.div_epr((int)e);
        s = base_r[r] + pre_r[r * kWords + w] + __popc(bits_r[r * kWords + w] & below);
        if (groups) {
            const int g = a.div_P(r);
            gs = base_g[g] + pre_g[g * kWords + w] + __popc(bits_g[g * kWords + w] & below);
        }
    };
    if constexpr (KMAX == 4 || KMAX == 8) {
        // Whole rows of 16-byte vectors when they are aligned (t*K*4 bytes is
        // a multiple of 16 for K = 4 and 8).
        const bool vec = a.K == KMAX && (reinterpret_cast<uintptr_t>(a.out.slot) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(a.out.group_slot) & 15) == 0;
        if (vec) {
            int32_t s[KMAX], gs[KMAX];
#pragma unroll
            for (int k = 0; k < KMAX; ++k) slot_of(ids.get(row, k), s[k], gs[k]);
#pragma unroll
            for (int v = 0; v < KMAX / 4; ++v) {
                if (a.out.slot) {
                    u32x4 o = {(uint32_t)s[4 * v], (uint32_t)s[4 * v + 1], (uint32_t)s[4 * v + 2],
                               (uint32_t)s[4 * v + 3]};
                    st16(a.out.slot + (int64_t)t * a.K + 4 * v, o);
                }
                if (groups) {
                    u32x4 o = {(uint32_t)gs[4 * v], (uint32_t)gs[4 * v + 1],
                               (uint32_t)gs[4 * v + 2], (uint32_t)gs[4 * v + 3]};
                    st16(a.out.group_slot + (int64_t)t * a.K + 4 * v, o);
                }
            }
            return;
        }
    }
    const int kn = KMAX > 0 ? KMAX : a.K;
#pragma unroll
    for (int k = 0; k < kn; ++k) {
        if (KMAX > 0 && k >= a.K) break;
        int32_t s, gs;
        slot_of(ids.get(row, k), s, gs);
        if (a.out.slot) a.out.slot[(int64_t)t * a.K + k] = s;
        if (groups) a.out.group_slot[(int64_t)t * a.K + k] = gs;
    }
}

// Column scan for launches with many workgroups. The columns of both tables
// ([rank | lane | group] columns, then expert columns) are cut into tiles of
// 64, one workgroup of 16 waves per tile, one column per lane (a wave's load
// of a row is 256 contiguous bytes). Wave w sums its segment of rows
// [w nb / 16, (w + 1) nb / 16); the segment sums meet in LDS; the wave then
// rewrites its rows as exclusive prefixes and the last wave writes the
// column total into row nb. Padding columns are scanned like the others and
// never read as counts.
#ifndef EP_LAYOUT_SCAN_MIN
#define EP_LAYOUT_SCAN_MIN 512  // workgroups from which the scan pays for its launch
#endif
constexpr int kScanMinBlocks = EP_LAYOUT_SCAN_MIN;
constexpr int kScanWaves = 16;
constexpr int kScanRows = 16;        // rows loaded per batch

__global__ __launch_bounds__(kScanWaves * kWave) void layout_scan_kernel(LayoutArgs a) {
    __shared__ int seg[kScanWaves][kWave];
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    const int c = blockIdx.x * kWave + lane;
    const bool in = c < a.wrow + a.E;
    const bool rlg = c < a.wrow;
    int32_t* col = rlg ? a.part_rlg + c : a.part_expert + min(c - a.wrow, a.E - 1);
    const int64_t stride = rlg ? a.wrow : a.E;
    const int r0 = (int)((int64_t)a.nb * w / kScanWaves), r1 = (int)((int64_t)a.nb * (w + 1) / kScanWaves);
    int sum = 0;
    for (int rb = r0; rb < r1; rb += kScanRows) {
        int x[kScanRows];
#pragma unroll
        for (int j = 0; j < kScanRows; ++j) x[j] = col[(int64_t)min(rb + j, r1 - 1) * stride];
#pragma unroll
        for (int j = 0; j < kScanRows; ++j) sum += rb + j < r1 ? x[j] : 0;
    }
    seg[w][lane] = sum;
    __syncthreads();
    int run = 0, total = 0;
#pragma unroll
    for (int j = 0; j < kScanWaves; ++j) {
        const int y = seg[j][lane];
        total += y;
        run += j < w ? y : 0;
    }
    for (int rb = r0; rb < r1; rb += kScanRows) {
        int x[kScanRows];
#pragma unroll
        for (int j = 0; j < kScanRows; ++j) x[j] = col[(int64_t)min(rb + j, r1 - 1) * stride];
#pragma unroll
        for (int j = 0; j < kScanRows; ++j) {
            if (in && rb + j < r1) col[(int64_t)(rb + j) * stride] = run;
            run += rb + j < r1 ? x[j] : 0;
        }
    }
    if (in && w == kScanWaves - 1) col[(int64_t)a.nb * stride] = total;
}

// Expand-mode rows. The row of entry (t, k) with expert e is
//   expert_offsets[e] + (lanes of e in earlier workgroups)
//                     + (entries of e before (t, k) in this workgroup, in
//                        token-then-lane order).
// The middle term is the count table turned into per-workgroup prefixes by
// the assign launch. The last term has two ways:
//   * bit matrix (E <= 2048 and no token of the workgroup names an expert on
//     two lanes): each entry ORs its token's bit into bits[e][t/32] in LDS;
//     the term is the popcount of the bits of earlier tokens;
//   * otherwise the entries are sorted by expert, stably, with a block radix
//     sort in LDS, and the term is the entry's distance from the first
//     position holding e.
constexpr int kExpandBitsMaxE = 2048;  // E * kWords words of LDS = 64 KiB

template <int ITEMS>
using ExpandSort = rocprim::block_radix_sort<int, kBlockThreads, ITEMS, int>;

template <int ITEMS>
__global__ __launch_bounds__(kBlockThreads) void layout_expand_kernel(LayoutArgs a, int key_bits,
                                                                      int use_bits) {
    using sort_t = ExpandSort<ITEMS>;
    extern __shared__ __align__(16) uint32_t lds_x[];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int t0 = b * kLayoutTokens;
    const int t = t0 + tid;
    // Every id load issued (token and lane clamped, the extra entries masked
    // to key E afterwards): loads under a branch were issued one by one.
    const int tc = min(t, a.T - 1);
    int64_t raw[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) raw[k] = a.topk[(int64_t)tc * a.K + min(k, a.K - 1)];
    int keys[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const int64_t e = t < a.T && k < a.K ? raw[k] : -1;
        keys[k] = expert_ok(e, a.E) ? (int)e : a.E;  // no expert: key E
    }
    bool dup = false;
#pragma unroll
    for (int k = 1; k < ITEMS; ++k)
#pragma unroll
        for (int j = 0; j < k; ++j) dup |= keys[k] < a.E && keys[k] == keys[j];

    if (use_bits) {
        // Both global terms of every lane (clamped ids), requested before the
        // bit matrix is built so that they arrive during it.
        int base[ITEMS];
#pragma unroll
        for (int k = 0; k < ITEMS; ++k) {
            const int e = min(keys[k], a.E - 1);
            base[k] = a.out.expert_offsets[e] + a.part_expert[(int64_t)b * a.E + e];
        }
        if (!__syncthreads_or(dup)) {
            uint32_t* bits = lds_x;  // [E][kWords]
            for (int i = tid; i < a.E * kWords; i += kBlockThreads) bits[i] = 0u;
            __syncthreads();
            const int w = tid / 32;
            const uint32_t bit = 1u << (tid & 31);
#pragma unroll
            for (int k = 0; k < ITEMS; ++k)
                if (keys[k] < a.E) atomicOr(&bits[keys[k] * kWords + w], bit);
            __syncthreads();
            if (t >= a.T) return;
            const uint32_t below = bit - 1u;
#pragma unroll
            for (int k = 0; k < ITEMS; ++k) {
                if (k >= a.K) break;
                const int e = min(keys[k], a.E - 1);
                int rank = __popc(bits[e * kWords + w] & below);
#pragma unroll
                for (int j = 0; j < kWords; ++j) rank += j < w ? __popc(bits[e * kWords + j]) : 0;
                a.out.expert_slot[(int64_t)t * a.K + k] = keys[k] < a.E ? base[k] + rank : -1;
            }
            return;
        }
    }

    typename sort_t::storage_type& sort_st = *reinterpret_cast<typename sort_t::storage_type*>(lds_x);
    int* sorted = reinterpret_cast<int*>(lds_x);  // [kBlockThreads * ITEMS], after the sort
    int vals[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) vals[k] = tid * ITEMS + k;
    sort_t().sort(keys, vals, sort_st, 0, key_bits);
    __syncthreads();
    // The global terms of every sorted entry (clamped keys), requested
    // together before the searches.
    int sbase[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int e = min(keys[j], a.E - 1);
        sbase[j] = a.out.expert_offsets[e] + a.part_expert[(int64_t)b * a.E + e];
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) sorted[tid * ITEMS + j] = keys[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int pos = tid * ITEMS + j;
        const int key = keys[j];
        const int lt = vals[j] / ITEMS, k = vals[j] % ITEMS;
        if (k >= a.K || t0 + lt >= a.T) continue;  // padding entry
        int32_t row = -1;
        if (key < a.E) {
            int lo = 0, hi = pos;  // first position holding `key`
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (sorted[mid] < key) lo = mid + 1; else hi = mid;
            }
            row = sbase[j] + (pos - lo);
        }
        a.out.expert_slot[(int64_t)(t0 + lt) * a.K + k] = row;
    }
}

// Expand-mode rows for K > 16: the workgroup's entries, in token-then-lane
// order (entry i = token i / K, lane i % K), are taken in passes of
// kBlockThreads * 16; each pass is sorted stably by expert as above and an
// LDS histogram carries, per expert, the entries of the earlier passes.
constexpr int kWideItems = 16;
constexpr int kWidePass = kBlockThreads * kWideItems;
using WideSort = rocprim::block_radix_sort<int, kBlockThreads, kWideItems, int>;

__global__ __launch_bounds__(kBlockThreads) void layout_expand_wide_kernel(LayoutArgs a, int key_bits) {
    extern __shared__ __align__(16) uint32_t lds_x[];
    typename WideSort::storage_type& sort_st = *reinterpret_cast<typename WideSort::storage_type*>(lds_x);
    int* sorted = reinterpret_cast<int*>(lds_x);  // [kWidePass], after each sort
    const size_t hist_off = std::max(sizeof(typename WideSort::storage_type), sizeof(int) * kWidePass);
    int* hist = reinterpret_cast<int*>(reinterpret_cast<char*>(lds_x) + hist_off);  // [E]
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int t0 = b * kLayoutTokens;
    const int nt = min(kLayoutTokens, a.T - t0);
    const int n = nt * a.K;  // entries of this workgroup
    for (int e = tid; e < a.E; e += kBlockThreads) hist[e] = 0;
    for (int base = 0; base < n; base += kWidePass) {
        int keys[kWideItems], vals[kWideItems];
#pragma unroll
        for (int j = 0; j < kWideItems; ++j) {
            const int i = base + tid * kWideItems + j;
            int key = a.E;  // no expert, or past the last entry
            if (i < n) {
                const int64_t e = a.topk[(int64_t)t0 * a.K + i];
                if (expert_ok(e, a.E)) key = (int)e;
            }
            keys[j] = key;
            vals[j] = i;
        }
        __syncthreads();  // the previous pass is done with `sorted` and `hist`
        WideSort().sort(keys, vals, sort_st, 0, key_bits);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kWideItems; ++j) sorted[tid * kWideItems + j] = keys[j];
        __syncthreads();
        int run_end[kWideItems];  // entries of the key up to here, at the last of its run
#pragma unroll
        for (int j = 0; j < kWideItems; ++j) {
            const int pos = tid * kWideItems + j;
            const int key = keys[j];
            run_end[j] = 0;
            if (key >= a.E) continue;
            int lo = 0, hi = pos;  // first position holding `key`
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (sorted[mid] < key) lo = mid + 1; else hi = mid;
            }
            const int i = vals[j];
            a.out.expert_slot[(int64_t)t0 * a.K + i] =
                a.out.expert_offsets[key] + a.part_expert[(int64_t)b * a.E + key] + hist[key] + (pos - lo);
            if (pos + 1 == kWidePass || sorted[pos + 1] != key) run_end[j] = pos - lo + 1;
        }
        __syncthreads();  // every row of this pass has read hist
#pragma unroll
        for (int j = 0; j < kWideItems; ++j)
            if (run_end[j]) hist[keys[j]] += run_end[j];
    }
    // Lanes with no expert.
    for (int i = tid; i < n; i += kBlockThreads) {
        const int64_t e = a.topk[(int64_t)t0 * a.K + i];
        if (!expert_ok(e, a.E)) a.out.expert_slot[(int64_t)t0 * a.K + i] = -1;
    }
}

}  // namespace

// The count tables of the launches below sit at the offsets ws_layout gives,
// from `tables` (a workspace, or the scratch array of the allocation-free
// entry point); the error words are at `err`.
static hipError_t launch_layout_tables(const ep_shape& s, const int64_t* topk, const ep_layout& L,
                                       uint32_t* err, char* tables, hipStream_t st) {
    const WsLayout W = ws_layout(s);
    LayoutArgs a;
    a.T = s.T; a.K = s.K; a.E = s.E; a.R = s.R; a.G = s.G;
    a.epr = s.E / s.R; a.P = s.R / s.G; a.nb = W.nb;
    a.div_epr = FastDiv::make(a.epr);
    a.div_P = FastDiv::make(a.P);
    a.rp = W.rp; a.wrow = W.wrow;
    a.topk = topk;
    a.err = err;
    a.part_rlg = reinterpret_cast<int32_t*>(tables + W.part_rlg);
    a.part_expert = reinterpret_cast<int32_t*>(tables + W.part_expert);
    a.out = L;

    const size_t lds_count = sizeof(uint32_t) * ((size_t)(s.R + s.G) * kWords + s.E);
    const bool scanned = W.nb >= kScanMinBlocks;
    const bool spread_launch = !scanned && W.nb > 2 * kRowBatch && !L.expert_slot;
    const size_t lds_assign = sizeof(uint32_t) * ((size_t)(s.R + s.G) * kWords + s.R + s.G +
                                                  (size_t)kScSlots * kWavesPerBlock) +
                              (size_t)(s.R + s.G) * kWords +
                              // partial sums of the spread table loads (only used with many rows)
                              (spread_launch ? sizeof(int32_t) * kBlockThreads * kSpreadStride : 0);
    const dim3 grid(W.nb), block(kBlockThreads);
#define EP_LAYOUT_LAUNCH(KM)                                                                  \
    do {                                                                                      \
        hipLaunchKernelGGL(layout_count_kernel<KM>, grid, block, lds_count, st, a);           \
        if (scanned) {                                                                        \
            hipLaunchKernelGGL(layout_scan_kernel, dim3((unsigned)((W.wrow + s.E + kWave - 1) / kWave)), \
                               dim3(kScanWaves * kWave), 0, st, a);                           \
            hipLaunchKernelGGL((layout_assign_kernel<KM, false, true>), grid, block, lds_assign, st, a); \
        } else if (spread_launch)                                                             \
            hipLaunchKernelGGL((layout_assign_kernel<KM, true, false>), grid, block, lds_assign, st, a); \
        else                                                                                  \
            hipLaunchKernelGGL((layout_assign_kernel<KM, false, false>), grid, block, lds_assign, st, a); \
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
        const int use_bits = s.E <= kExpandBitsMaxE;
        const size_t bit_lds = use_bits ? sizeof(uint32_t) * (size_t)s.E * kWords : 0;
        if (s.K <= 8) {
            const size_t lds = std::max({sizeof(typename ExpandSort<8>::storage_type),
                                         sizeof(int) * kBlockThreads * 8, bit_lds});
            hipLaunchKernelGGL(layout_expand_kernel<8>, grid, block, lds, st, a, bits, use_bits);
        } else if (s.K <= 16) {
            const size_t lds = std::max({sizeof(typename ExpandSort<16>::storage_type),
                                         sizeof(int) * kBlockThreads * 16, bit_lds});
            hipLaunchKernelGGL(layout_expand_kernel<16>, grid, block, lds, st, a, bits, use_bits);
        } else {
            const size_t lds = std::max(sizeof(typename WideSort::storage_type), sizeof(int) * kWidePass) +
                               sizeof(int) * (size_t)s.E;
            hipLaunchKernelGGL(layout_expand_wide_kernel, grid, block, lds, st, a, bits);
        }
    }
    return hipGetLastError();
}

hipError_t launch_layout(const ep_shape& s, const int64_t* topk, const ep_layout& L, char* ws,
                         hipStream_t st) {
    return launch_layout_tables(s, topk, L, reinterpret_cast<uint32_t*>(ws + ws_layout(s).err), ws, st);
}

// ---------------------------------------------------------------------------
// Allocation-free layout: the count tables in a file-scope device array
// instead of the caller's workspace. Each GPU the library runs on holds its
// own copy of the array until the process ends; every call on that GPU uses
// it, so calls that overlap on one GPU race. In host code `scratch` names a
// host-side stand-in, not a device address: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current
// and kept in scratch_addr[]. Only that address is passed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[EP_LAYOUT_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
char* scratch_addr[kMaxDevices];
std::mutex scratch_mutex;

// Device address of `scratch` on device `dev`, looked up on first use.
hipError_t scratch_on(int dev, char** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_addr[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_addr[dev] = static_cast<char*>(p);
    }
    *out = scratch_addr[dev];
    return hipSuccess;
}
}  // namespace

hipError_t launch_layout_noalloc(const ep_shape& s, const int64_t* topk, const ep_layout& L,
                                 uint32_t* err, hipStream_t st) {
    int dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    char* tables = nullptr;
    if ((e = scratch_on(dev, &tables)) != hipSuccess) return e;
    return launch_layout_tables(s, topk, L, err, tables, st);
}

}  // namespace ep
