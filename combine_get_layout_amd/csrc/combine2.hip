// combine2.hip -- ep_combine_two_level on gfx950: the two-level dispatch run
// backwards.
//
// What is computed follows the combine roles of "06_06: NVLink Scale-up +
// RDMA Scale-out — DeepEP 三阶段流水线 vs DeepGEMM 对称内存" (combine warps
// kNVLSender -> kNVLAndRDMAForwarder -> kRDMAReceiver: reduce inside the
// scale-up domain first, then across scale-out groups) on the rows of the
// hybrid path of "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK 复制机制"
// §3.6:
//   step 1 (group reduce): for every token t and group g it sends to,
//     partial[t, g] = bf16_rne(fp32 fused multiply-adds of the lanes of t whose
//     rank is in g, ascending k, from +0), written as a chunked row (512 B
//     blocks of 480 B payload + 32 B flag = epoch, "Ascend Send Ordering",
//     导言) at the token's group-region row;
//   step 2 (cross-group reduce): out[t] = bf16_rne(fp32 sum of the token's
//     partial rows in ascending g, from +0); a partial row whose flags are not
//     all epoch is skipped.
//
// CDNA4 mapping: with K <= 8 both steps cut a token into slices of 4
// wave-iterations, one wave per slice (the slices of a token in one
// workgroup), and stream its rows one burst at a time with the next burst
// requested first; otherwise one wave64 per token. Both use the chunked lane
// mapping (wave iteration i covers blocks 2i and 2i+1; lane L holds
// hidden vector 30 * (2i + L/32) + L%32 when L%32 < 30, else a flag vector),
// so a partial row is produced and consumed with whole-wave 1 KiB stores and
// loads. The flags of every chunked row read are checked by the flag lanes of
// the same loads that bring in its values; a row with a bad flag makes the
// token run a second pass without it (error path only). Past 16 top-k lanes,
// any-K kernels check each row's flags in a short pass before its values are
// used and take the token's groups one at a time.
#include <algorithm>

#include "ep_device.h"
#include "ep_internal.h"

#ifndef EP_C2_ROWS
#define EP_C2_ROWS 1  // both steps: row-streaming kernels when K <= 8 (0 = one wave per token)
#endif
#ifndef EP_C2_FUSED
#define EP_C2_FUSED 1  // both steps asked for, row-streaming shapes: one persistent launch (fixed lag)
#endif
#ifndef EP_C2F_TILE
#define EP_C2F_TILE 1  // fused launch: tokens per batch
#endif
#ifndef EP_C2F_LAG
#define EP_C2F_LAG 128  // fused launch: job i reduces batch i's groups, then batch i - EP_C2F_LAG across groups
#endif
#ifndef EP_C2F_MINW
#define EP_C2F_MINW 1  // fused launch: minimum waves per SIMD the compiler must allow (launch bound)
#endif
#ifndef EP_C2F_WG_PER_CU
#define EP_C2F_WG_PER_CU 0  // fused launch: at most this many workgroups per CU (0: all resident)
#endif

namespace ep {
namespace {

struct Combine2Args {
    int T, H, K, E, R, G, epr, P;
    const int64_t* topk;
    const int32_t* slot;
    const int32_t* group_slot;
    const float* w;
    const uint8_t* y;
    int64_t y_rows, y_stride;
    int y_chunked;
    uint32_t epoch;
    uint8_t* group_buf;
    int64_t group_cap, pstride;
    uint16_t* out;
    uint32_t* err;
};

// This lane's vector of wave iteration `it` in the chunked mapping: block c,
// slot wv; p = hidden vector index. Returns whether it is a hidden vector.
__device__ __forceinline__ bool chunk_vec(int it, int lane, int nvh, int& c, int& wv, int& p) {
    c = 2 * it + (lane >> 5);
    wv = lane & 31;
    p = c * kChunkPayloadVecs + wv;
    return wv < kChunkPayloadVecs && p < nvh;
}

__device__ __forceinline__ u32x4 pack8(const float (&acc)[8]) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = f32_to_bf16(acc[2 * q]) | (f32_to_bf16(acc[2 * q + 1]) << 16);
    return o;
}

__device__ __forceinline__ bool flag_ok(u32x4 f, uint32_t epoch) {
    return f[0] == epoch && f[1] == epoch && f[2] == epoch && f[3] == epoch;
}

template <int KMAX>
__global__ __launch_bounds__(kBlockThreads) void combine_group_kernel(Combine2Args a) {
    const int lane = lane_id();
    const int t = blockIdx.x * kWavesPerBlock + wave_in_block();
    if (t >= a.T) return;
    int s = -1, g = -1, gs = -1;
    float wt = 0.f;
    if (lane < a.K) {
        const int64_t e = a.topk[(int64_t)t * a.K + lane];
        s = a.slot[(int64_t)t * a.K + lane];
        gs = a.group_slot[(int64_t)t * a.K + lane];
        wt = a.w[(int64_t)t * a.K + lane];
        if (expert_ok(e, a.E)) g = ((int)e / a.epr) / a.P;
    }
    bool use = s >= 0 && g >= 0;
    if (use && s >= a.y_rows) {
        report(a.err, EP_DEVERR_CAPACITY);
        use = false;
    }
    uint64_t um = __ballot(use);
    const int nvh = a.H / 8;
    const int nblk = (2 * a.H + kChunkPayload - 1) / kChunkPayload;  // blocks of a hidden row
    const int iters = (nblk + 1) / 2;
    // Groups of this token: the first lane of each, numbered in lane order.
    bool first = g >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int gj = readlane(g, j);
        if (j < lane && gj == g) first = false;
    }
    const uint64_t fm = __ballot(first);
    // gpos: position of this lane's group among the token's groups.
    int gpos = -1;
    for (uint64_t m = fm; m; m &= m - 1) {
        const int k0 = __ffsll((unsigned long long)m) - 1;
        if (readlane(g, k0) == g) gpos = __popcll(fm & ((1ull << k0) - 1));
    }
    const int ng = __popcll(fm);
    // Partial row of each group (its first lane's group slot); rows past the
    // capacity are not written.
    uint8_t* prow[KMAX];
    uint32_t wmask = 0;  // groups whose partial row is written
#pragma unroll
    for (int gi = 0; gi < KMAX; ++gi) {
        prow[gi] = a.group_buf;
        if (gi >= ng) continue;
        int k0 = -1, cnt = 0;
        for (uint64_t m = fm; m; m &= m - 1, ++cnt)
            if (cnt == gi) { k0 = __ffsll((unsigned long long)m) - 1; break; }
        const int64_t dst = readlane(gs, k0);
        if (dst >= a.group_cap) {
            if (lane == 0) report(a.err, EP_DEVERR_CAPACITY);
            continue;
        }
        prow[gi] = a.group_buf + dst * a.pstride;
        wmask |= 1u << gi;
    }
    if (!wmask) return;
    // One pass over the hidden row: every lane's row is read once and feeds
    // its group's accumulator (ascending k inside each group). With chunked
    // rows, the lanes on a block's 32-byte flag load that flag with the same
    // instruction and check it; a row with a bad flag is found only after
    // its values were used, so the token is then computed again without it
    // (an error path only; the second pass rewrites the partial rows).
    const u32x4 flagv = {a.epoch, a.epoch, a.epoch, a.epoch};
    for (int pass = 0; pass < 2; ++pass) {
        const int s_any = um ? readlane(s, __ffsll((unsigned long long)um) - 1) : 0;
        const uint8_t* rowp[KMAX];
        float wk[KMAX];
        int gk[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int kk = min(k, a.K - 1);
            rowp[k] = a.y + (int64_t)(((um >> k) & 1) ? readlane(s, kk) : s_any) * a.y_stride;
            wk[k] = readlane_f(wt, kk);
            gk[k] = readlane(gpos, kk);
        }
        uint32_t bad = 0;  // per lane: bit k = a flag of row k checked by this lane is wrong
        for (int it = 0; it < iters; ++it) {
            int c, wv, p;
            const bool hv = chunk_vec(it, lane, nvh, c, wv, p);
            const bool fl = a.y_chunked && wv >= kChunkPayloadVecs && c < nblk;
            const int64_t blk = (int64_t)c * kChunkBytes + (int64_t)wv * 16;
            const int64_t off = hv ? (a.y_chunked ? blk : (int64_t)p * 16) : (fl ? blk : 0);
            u32x4 v[KMAX];
            if (um) {
#pragma unroll
                for (int k = 0; k < KMAX; ++k) v[k] = ld16(rowp[k] + off);
            }
            if (fl) {
#pragma unroll
                for (int k = 0; k < KMAX; ++k)
                    if (((um >> k) & 1) && !flag_ok(v[k], a.epoch)) bad |= 1u << k;
            }
            float acc[KMAX][8];
#pragma unroll
            for (int gi = 0; gi < KMAX; ++gi)
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[gi][q] = 0.f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (!((um >> k) & 1)) continue;
#pragma unroll
                for (int gi = 0; gi < KMAX; ++gi) {
                    if (gk[k] != gi) continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[gi][2 * q] = __builtin_fmaf(wk[k], bf16_lo(v[k][q]), acc[gi][2 * q]);
                        acc[gi][2 * q + 1] = __builtin_fmaf(wk[k], bf16_hi(v[k][q]), acc[gi][2 * q + 1]);
                    }
                }
            }
            if (c >= nblk) continue;
            const int64_t o_off = (int64_t)c * kChunkBytes + (int64_t)wv * 16;
#pragma unroll
            for (int gi = 0; gi < KMAX; ++gi) {
                if (!((wmask >> gi) & 1)) continue;
                u32x4 o = {0u, 0u, 0u, 0u};
                if (hv) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        o[q] = f32_to_bf16(acc[gi][2 * q]) | (f32_to_bf16(acc[gi][2 * q + 1]) << 16);
                }
                if (wv >= kChunkPayloadVecs) o = flagv;
                st16_stream(prow[gi] + o_off, o);
            }
        }
        if (!a.y_chunked) return;
        uint64_t drop = 0;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (((um >> k) & 1) && __ballot((bad >> k) & 1)) drop |= 1ull << k;
        if (!drop) return;
        if (lane == 0) report(a.err, EP_DEVERR_FLAG);
        um &= ~drop;
    }
}

// Row-streaming group step (K <= 8): a token is cut into slices of VPW
// wave-iterations, one wave per slice, the slices of a token in one
// workgroup. The token's used lanes are walked in (group, lane) order, the
// order of the set bits of seq = sum over groups gi of (lanes of gi) << 8 gi.
// Each lane's slice of its row is read once as one burst, the next lane's
// burst requested before the current one is used, and accumulated into one
// VPW x 8 fp32 set; when the next lane belongs to another group (or none is
// left) the set is rounded and stored as the group's partial slice. Groups
// with no usable lane get a zero partial. Chunked rows: each slice checks the
// flags of its own blocks with the same loads; the slices post the rows whose
// flags failed to LDS and meet at one barrier (reached once by every wave of
// the workgroup), and a token with a dropped row is computed again without
// it (error path only; the second pass rewrites the partial slices).
// Device-scope 16-byte store / load at byte `off` of a row of `bytes` bytes
// (a buffer resource over the row; cache-policy 16 is the device-scope bit,
// sc1): stores go through the XCD's L2 to the device's coherence point, and
// loads do not hit stale lines of another XCD's writes.
constexpr int kC2DeviceScope = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t c2_rsrc(const void* row, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, (int)bytes, 0x00020000);
}

// One token's group step, slice `part` of `slices` (the slices of a token are
// consecutive waves of one workgroup). DEV: the partial rows are stored with
// device scope (the fused launch reads them back in the same kernel);
// otherwise non-temporal stores.
template <int VPW, bool DEV>
__device__ __forceinline__ void group_rows_token(const Combine2Args& a, int t, int part, int slices, bool live,
                                                 uint32_t* drop_lds) {
    constexpr int KMAX = 8;
    const int lane = lane_id(), wave = wave_in_block();
    int s = -1, g = -1, gs = -1;
    float wt = 0.f;
    if (live && lane < a.K) {
        const int64_t e = a.topk[(int64_t)t * a.K + lane];
        s = a.slot[(int64_t)t * a.K + lane];
        gs = a.group_slot[(int64_t)t * a.K + lane];
        wt = a.w[(int64_t)t * a.K + lane];
        if (expert_ok(e, a.E)) g = ((int)e / a.epr) / a.P;
    }
    bool use = s >= 0 && g >= 0;
    if (use && s >= a.y_rows) {
        if (part == 0) report(a.err, EP_DEVERR_CAPACITY);
        use = false;
    }
    uint64_t um = __ballot(use);
    const int nvh = a.H / 8;
    const int nblk = (2 * a.H + kChunkPayload - 1) / kChunkPayload;
    const int iters = (nblk + 1) / 2;
    const int it0 = part * VPW;
    // Groups of this token (first lane of each, in lane order) and the
    // position of each lane's group.
    bool first = g >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int gj = readlane(g, j);
        if (j < lane && gj == g) first = false;
    }
    const uint64_t fm = __ballot(first);
    int gpos = -1;
    for (uint64_t m = fm; m; m &= m - 1) {
        const int k0 = __ffsll((unsigned long long)m) - 1;
        if (readlane(g, k0) == g) gpos = __popcll(fm & ((1ull << k0) - 1));
    }
    // Partial row of each group position; rows past the capacity are not written.
    int64_t pdst[KMAX];
    uint32_t wmask = 0;
#pragma unroll
    for (int gi = 0; gi < KMAX; ++gi) {
        pdst[gi] = 0;
        const uint64_t who = __ballot(((fm >> lane) & 1) && gpos == gi);
        if (!who) continue;
        const int64_t dst = readlane(gs, __ffsll((unsigned long long)who) - 1);
        if (dst >= a.group_cap) {
            if (lane == 0 && part == 0) report(a.err, EP_DEVERR_CAPACITY);
            continue;
        }
        pdst[gi] = dst;
        wmask |= 1u << gi;
    }
    // This lane's vectors of the slice: read offset in a row, whether it is a
    // hidden vector or a flag vector of a hidden block, and whether the
    // partial row has a vector there.
    int p[VPW];
    int64_t off[VPW], o_off[VPW];
    bool hv[VPW], fl[VPW], st[VPW], fw[VPW];
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
        int c, wv;
        const bool in = live && it0 + j < iters;
        const bool hvec = chunk_vec(it0 + j, lane, nvh, c, wv, p[j]);
        hv[j] = in && hvec;
        fl[j] = in && a.y_chunked && wv >= kChunkPayloadVecs && c < nblk;
        const int64_t blk = (int64_t)c * kChunkBytes + (int64_t)wv * 16;
        off[j] = hv[j] ? (a.y_chunked ? blk : (int64_t)p[j] * 16) : (fl[j] ? blk : 0);
        st[j] = in && c < nblk;
        fw[j] = wv >= kChunkPayloadVecs;
        o_off[j] = blk;
    }
    const u32x4 flagv = {a.epoch, a.epoch, a.epoch, a.epoch};
    auto store_partial = [&](int gi, const float (&acc)[VPW][8], bool zero) {
        if (!((wmask >> gi) & 1)) return;
        int64_t dst = 0;
#pragma unroll
        for (int q = 0; q < KMAX; ++q) dst = q == gi ? pdst[q] : dst;
        uint8_t* prow = a.group_buf + dst * a.pstride;
#pragma unroll
        for (int j = 0; j < VPW; ++j) {
            if (!st[j]) continue;
            u32x4 o = {0u, 0u, 0u, 0u};
            if (hv[j] && !zero) o = pack8(acc[j]);
            if (fw[j]) o = flagv;
            if constexpr (DEV) __builtin_amdgcn_raw_buffer_store_b128(o, c2_rsrc(prow, a.pstride), (int)o_off[j], 0,
                                                                      kC2DeviceScope);
            else st16_stream(prow + o_off[j], o);
        }
    };
    for (int pass = 0; pass < 2; ++pass) {
        uint32_t bad = 0;  // per lane: bit k = a flag of row k checked by this lane is wrong
        // Lanes in (group, lane) order.
        uint64_t seq = 0;
#pragma unroll
        for (int gi = 0; gi < KMAX; ++gi)
            seq |= (uint64_t)(__ballot(((um >> lane) & 1) && gpos == gi) & 0xFFu) << (8 * gi);
        uint32_t stored = 0;
        if (seq && live) {
            float acc[VPW][8];
#pragma unroll
            for (int j = 0; j < VPW; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
            int cur = __ffsll((unsigned long long)seq) - 1;
            uint64_t rest = seq & (seq - 1);
            // Two register sets in turn (the loop is unrolled over the at
            // most 8 usable lanes, so no set is copied into the other).
            u32x4 vb[2][VPW];
            {
                const uint8_t* r0 = a.y + (int64_t)readlane(s, cur & 7) * a.y_stride;
#pragma unroll
                for (int j = 0; j < VPW; ++j) vb[0][j] = ld16_stream(r0 + off[j]);
            }
            // The next row's burst is always requested; after the last row
            // it reads the workspace's first 256 bytes (the error words: in
            // bounds and cached). Every step then issues the same loads, so
            // the compiler waits for the current row alone, not for the
            // next one too (a request under a branch made it wait for all).
            // Rows are read once: non-temporal loads (the two-level combine
            // at hier8x8: 915 -> 884 us).
            const uint8_t* spare = reinterpret_cast<const uint8_t*>(a.err) + (lane & 15) * 16;
#pragma unroll
            for (int i = 0; i < KMAX; ++i) {
                const int nxt = rest ? __ffsll((unsigned long long)rest) - 1 : -1;
                {
                    const uint8_t* rn = a.y + (int64_t)readlane(s, (nxt < 0 ? cur : nxt) & 7) * a.y_stride;
#pragma unroll
                    for (int j = 0; j < VPW; ++j) vb[(i + 1) & 1][j] = ld16_stream(nxt >= 0 ? rn + off[j] : spare);
                }
                const int k = cur & 7, gi = cur >> 3;
                const float wk = readlane_f(wt, k);
#pragma unroll
                for (int j = 0; j < VPW; ++j) {
                    if (fl[j] && !flag_ok(vb[i & 1][j], a.epoch)) bad |= 1u << k;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[j][2 * q] = __builtin_fmaf(wk, bf16_lo(vb[i & 1][j][q]), acc[j][2 * q]);
                        acc[j][2 * q + 1] = __builtin_fmaf(wk, bf16_hi(vb[i & 1][j][q]), acc[j][2 * q + 1]);
                    }
                }
                if (nxt < 0 || (nxt >> 3) != gi) {
                    store_partial(gi, acc, false);
                    stored |= 1u << gi;
#pragma unroll
                    for (int j = 0; j < VPW; ++j)
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
                }
                if (nxt < 0) break;
                cur = nxt;
                rest &= rest - 1;
            }
        }
        if (live) {
            float none[VPW][8];
            for (uint32_t z = wmask & ~stored; z; z &= z - 1) store_partial(__ffs(z) - 1, none, true);
        }
        if (!a.y_chunked || pass == 1) return;
        uint32_t drop = 0;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (((um >> k) & 1) && __ballot((bad >> k) & 1)) drop |= 1u << k;
        if (lane == 0) drop_lds[wave] = drop;
        __syncthreads();
        const int w0 = wave - part;
        for (int q = 0; q < slices; ++q) drop |= drop_lds[w0 + q];
        if (!drop || !live) return;
        if (lane == 0 && part == 0) report(a.err, EP_DEVERR_FLAG);
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if ((drop >> k) & 1) drop |= (uint32_t)__ballot(use && s == readlane(s, min(k, a.K - 1)));
        um &= ~(uint64_t)drop;
    }
}

template <int VPW>
__global__ __launch_bounds__(kBlockThreads) void combine_group_rows_kernel(Combine2Args a, int slices) {
    __shared__ uint32_t drop_lds[kWavesPerBlock];
    const int gw = blockIdx.x * kWavesPerBlock + wave_in_block();
    const int t = gw / slices;
    group_rows_token<VPW, false>(a, t, gw % slices, slices, t < a.T, drop_lds);
}

template <int GMAX>
__global__ __launch_bounds__(kBlockThreads) void combine_cross_kernel(Combine2Args a) {
    const int lane = lane_id();
    const int t = blockIdx.x * kWavesPerBlock + wave_in_block();
    if (t >= a.T) return;
    int g = -1, gs = -1;
    if (lane < a.K) {
        const int64_t e = a.topk[(int64_t)t * a.K + lane];
        gs = a.group_slot[(int64_t)t * a.K + lane];
        if (expert_ok(e, a.E)) g = ((int)e / a.epr) / a.P;
    }
    bool first = g >= 0 && gs >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int gj = readlane(g, j);
        if (j < lane && gj == g) first = false;
    }
    if (first && gs >= a.group_cap) {
        report(a.err, EP_DEVERR_CAPACITY);
        first = false;
    }
    uint64_t fm = __ballot(first);
    const int nvh = a.H / 8;
    const int nblk = (2 * a.H + kChunkPayload - 1) / kChunkPayload;
    const int iters = (nblk + 1) / 2;
    uint8_t* out_row = reinterpret_cast<uint8_t*>(a.out) + (int64_t)t * a.H * 2;
    // Partial rows whose flags are checked with the same loads as their
    // values (the lanes on a block's 32-byte flag load the flag); a bad flag
    // drops the row and the token is summed again without it (error path
    // only; the second pass rewrites the output row).
    for (int pass = 0; pass < 2; ++pass) {
        // The token's partial rows in ascending group: position = number of
        // partials with a smaller group; unused positions point at a used row.
        int rank = 0;
        for (uint64_t m = fm; m; m &= m - 1) {
            const int j = __ffsll((unsigned long long)m) - 1;
            rank += readlane(g, j) < g ? 1 : 0;
        }
        const int ng = __popcll(fm);
        const int row_any = fm ? readlane(gs, __ffsll((unsigned long long)fm) - 1) : 0;
        const uint8_t* rowp[GMAX];
#pragma unroll
        for (int pos = 0; pos < GMAX; ++pos) {
            const uint64_t who = __ballot(((fm >> lane) & 1) && rank == pos);
            const int row = who ? readlane(gs, __ffsll((unsigned long long)who) - 1) : row_any;
            rowp[pos] = a.group_buf + (int64_t)row * a.pstride;
        }
        uint32_t bad = 0;  // per lane: bit pos = a flag of partial `pos` checked by this lane is wrong
        constexpr int NB = 2;
        for (int it0 = 0; it0 < iters; it0 += NB) {
            int c[NB], wv[NB], p[NB];
            bool hv[NB], fl[NB];
            int64_t off[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const bool in = it0 + j < iters;
                hv[j] = in && chunk_vec(it0 + j, lane, nvh, c[j], wv[j], p[j]);
                fl[j] = in && wv[j] >= kChunkPayloadVecs && c[j] < nblk;
                off[j] = (hv[j] || fl[j]) ? (int64_t)c[j] * kChunkBytes + (int64_t)wv[j] * 16 : 0;
            }
            u32x4 v[GMAX][NB];
            if (fm) {
#pragma unroll
                for (int pos = 0; pos < GMAX; ++pos)
#pragma unroll
                    for (int j = 0; j < NB; ++j) v[pos][j] = ld16(rowp[pos] + off[j]);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (fl[j]) {
#pragma unroll
                    for (int pos = 0; pos < GMAX; ++pos)
                        if (pos < ng && !flag_ok(v[pos][j], a.epoch)) bad |= 1u << pos;
                }
                float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int pos = 0; pos < GMAX; ++pos) {
                    if (pos >= ng) break;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[2 * q] = acc[2 * q] + bf16_lo(v[pos][j][q]);
                        acc[2 * q + 1] = acc[2 * q + 1] + bf16_hi(v[pos][j][q]);
                    }
                }
                if (hv[j]) {
                    u32x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) o[q] = f32_to_bf16(acc[2 * q]) | (f32_to_bf16(acc[2 * q + 1]) << 16);
                    st16_stream(out_row + (int64_t)p[j] * 16, o);
                }
            }
        }
        uint32_t badpos = 0;
#pragma unroll
        for (int pos = 0; pos < GMAX; ++pos)
            if (pos < ng && __ballot((bad >> pos) & 1)) badpos |= 1u << pos;
        if (!badpos) return;
        if (lane == 0) report(a.err, EP_DEVERR_FLAG);
        fm &= ~__ballot(((fm >> lane) & 1) && ((badpos >> rank) & 1));
    }
}

// Row-streaming cross-group step: slices of VPW wave-iterations, one wave per
// slice, the slices of a token in one workgroup. The token's partial rows are
// read in ascending group, one burst per row with the next row's burst
// requested first, and summed in fp32; flags are checked by the flag lanes of
// the same loads and exchanged between the slices through LDS at one barrier,
// as in the group step.
// One token's cross step, slice `part` of `slices`. DEV: the partial rows are
// read with device scope (written by other workgroups of the same launch);
// otherwise non-temporal loads.
template <int VPW, bool DEV>
__device__ __forceinline__ void cross_rows_token(const Combine2Args& a, int t, int part, int slices, bool live,
                                                 uint32_t* drop_lds) {
    constexpr int GMAX = 8;
    const int lane = lane_id(), wave = wave_in_block();
    int g = -1, gs = -1;
    if (live && lane < a.K) {
        const int64_t e = a.topk[(int64_t)t * a.K + lane];
        gs = a.group_slot[(int64_t)t * a.K + lane];
        if (expert_ok(e, a.E)) g = ((int)e / a.epr) / a.P;
    }
    bool first = g >= 0 && gs >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int gj = readlane(g, j);
        if (j < lane && gj == g) first = false;
    }
    if (first && gs >= a.group_cap) {
        if (part == 0) report(a.err, EP_DEVERR_CAPACITY);
        first = false;
    }
    uint64_t fm = __ballot(first);
    const int nvh = a.H / 8;
    const int nblk = (2 * a.H + kChunkPayload - 1) / kChunkPayload;
    const int iters = (nblk + 1) / 2;
    const int it0 = part * VPW;
    uint8_t* out_row = reinterpret_cast<uint8_t*>(a.out) + (int64_t)(live ? t : 0) * a.H * 2;
    int p[VPW];
    int64_t off[VPW];
    bool hv[VPW], fl[VPW];
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
        int c, wv;
        const bool in = live && it0 + j < iters;
        const bool hvec = chunk_vec(it0 + j, lane, nvh, c, wv, p[j]);
        hv[j] = in && hvec;
        fl[j] = in && wv >= kChunkPayloadVecs && c < nblk;
        off[j] = (hv[j] || fl[j]) ? (int64_t)c * kChunkBytes + (int64_t)wv * 16 : 0;
    }
    for (int pass = 0; pass < 2; ++pass) {
        // Partial rows in ascending group: position = number of the token's
        // partials with a smaller group.
        int rank = 0;
        for (uint64_t m = fm; m; m &= m - 1) {
            const int j = __ffsll((unsigned long long)m) - 1;
            rank += readlane(g, j) < g ? 1 : 0;
        }
        uint32_t posmask = 0;  // bit pos: a partial at position pos exists
        int prow_lane[GMAX];   // lane holding the partial of each position
#pragma unroll
        for (int pos = 0; pos < GMAX; ++pos) {
            const uint64_t who = __ballot(((fm >> lane) & 1) && rank == pos);
            prow_lane[pos] = who ? __ffsll((unsigned long long)who) - 1 : 0;
            posmask |= who ? (1u << pos) : 0u;
        }
        uint32_t bad = 0;  // per lane: bit pos = a flag of partial `pos` checked by this lane is wrong
        float acc[VPW][8];
#pragma unroll
        for (int j = 0; j < VPW; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
        if (posmask && live) {
            auto row_at = [&](int pos) {
                int ln = 0;
#pragma unroll
                for (int q = 0; q < GMAX; ++q) ln = q == pos ? prow_lane[q] : ln;
                return a.group_buf + (int64_t)readlane(gs, ln) * a.pstride;
            };
            int cur = __ffs(posmask) - 1;
            uint32_t rest = posmask & (posmask - 1);
            // As in the group step: two register sets in turn, and the next
            // burst always requested (the workspace's error words after the
            // last row).
            u32x4 vb[2][VPW];
            {
                const uint8_t* r0 = row_at(cur);
#pragma unroll
                for (int j = 0; j < VPW; ++j) {
                    if constexpr (DEV) vb[0][j] = __builtin_amdgcn_raw_buffer_load_b128(c2_rsrc(r0, a.pstride), (int)off[j], 0,
                                                                                        kC2DeviceScope);
                    else vb[0][j] = ld16_stream(r0 + off[j]);
                }
            }
            const uint8_t* spare = reinterpret_cast<const uint8_t*>(a.err) + (lane & 15) * 16;
#pragma unroll
            for (int i = 0; i < GMAX; ++i) {
                const int nxt = rest ? __ffs(rest) - 1 : -1;
                {
                    const uint8_t* rn = row_at(nxt < 0 ? cur : nxt);
                    if constexpr (DEV) {
                        // After the last row the request reads the workspace's
                        // error words (in bounds; the values are not used).
                        const __amdgpu_buffer_rsrc_t rs =
                            c2_rsrc(nxt >= 0 ? static_cast<const void*>(rn) : static_cast<const void*>(a.err),
                                    nxt >= 0 ? a.pstride : 256);
#pragma unroll
                        for (int j = 0; j < VPW; ++j)
                            vb[(i + 1) & 1][j] = __builtin_amdgcn_raw_buffer_load_b128(
                                rs, nxt >= 0 ? (int)off[j] : (lane & 15) * 16, 0, kC2DeviceScope);
                    } else {
#pragma unroll
                        for (int j = 0; j < VPW; ++j) vb[(i + 1) & 1][j] = ld16_stream(nxt >= 0 ? rn + off[j] : spare);
                    }
                }
#pragma unroll
                for (int j = 0; j < VPW; ++j) {
                    if (fl[j] && !flag_ok(vb[i & 1][j], a.epoch)) bad |= 1u << cur;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[j][2 * q] = acc[j][2 * q] + bf16_lo(vb[i & 1][j][q]);
                        acc[j][2 * q + 1] = acc[j][2 * q + 1] + bf16_hi(vb[i & 1][j][q]);
                    }
                }
                if (nxt < 0) break;
                cur = nxt;
                rest &= rest - 1;
            }
        }
#pragma unroll
        for (int j = 0; j < VPW; ++j)
            if (hv[j]) st16_stream(out_row + (int64_t)p[j] * 16, pack8(acc[j]));
        if (pass == 1) return;
        uint32_t badpos = 0;
#pragma unroll
        for (int pos = 0; pos < GMAX; ++pos)
            if (((posmask >> pos) & 1) && __ballot((bad >> pos) & 1)) badpos |= 1u << pos;
        // Exchange as lane masks (positions depend on which rows survive).
        uint32_t drop = (uint32_t)__ballot(((fm >> lane) & 1) && ((badpos >> rank) & 1));
        if (lane == 0) drop_lds[wave] = drop;
        __syncthreads();
        const int w0 = wave - part;
        for (int q = 0; q < slices; ++q) drop |= drop_lds[w0 + q];
        if (!drop || !live) return;
        if (lane == 0 && part == 0) report(a.err, EP_DEVERR_FLAG);
        fm &= ~(uint64_t)drop;
    }
}

template <int VPW>
__global__ __launch_bounds__(kBlockThreads) void combine_cross_rows_kernel(Combine2Args a, int slices) {
    __shared__ uint32_t drop_lds[kWavesPerBlock];
    const int gw = blockIdx.x * kWavesPerBlock + wave_in_block();
    const int t = gw / slices;
    cross_rows_token<VPW, false>(a, t, gw % slices, slices, t < a.T, drop_lds);
}

// ---------------------------------------------------------------------------
// Both steps in one persistent launch, with one flag per batch of tokens (the
// per-batch publication of "Ascend Send Ordering", 方案一, applied to the
// partial rows). One counter hands out jobs 0 .. nbatch + lag - 1 in order;
// job i runs the group step for the tokens of batch i (partial rows stored
// with device scope), waits until its stores are acknowledged and publishes
// flag i = epoch, then runs the cross step for batch i - lag (waiting for its
// flag, bounded by `timeout` clock ticks; on expiry EP_DEVERR_TIMEOUT and the
// batch's outputs are not written), reading the partial rows with device
// scope. A partial row is read back shortly after it was written, while it is
// still in the memory-side cache (the MALL) rather than in HBM alone. Unlike
// the fused dispatch, whose waves each hold a whole record in flight, a
// combine wave streams one or two rows at a time, so this launch wants every
// resident workgroup (3 per CU at its register count) and batches of one
// token per workgroup pass (4 / slices tokens, so that rows of 1 or 2
// slices still keep every wave busy): at hier8x8 746 us against 889 us for
// the two launches (2-token batches: 783 us, 8-token: 1,036 us; one
// workgroup per CU: 1,281 us). The launcher takes this form only for
// partial rows well past the MALL (see kC2FusedMinPartialBytes). Batch i
// - lag was handed out before job i to a running workgroup that writes it
// before it waits for anything, so every wait ends, co-resident or not. The
// arithmetic is that of the two launches, so the results are identical.
// ---------------------------------------------------------------------------
struct C2Fused {
    int tile, nbatch, lag;
    uint64_t timeout;       // wall-clock ticks a batch wait may last
    uint32_t* ctr;          // [0] next job
    uint32_t* flags;        // [nbatch] epoch once batch b's partial rows are written
};

template <int VPW>
__global__ __launch_bounds__(kBlockThreads, EP_C2F_MINW) void combine_two_level_fused_kernel(Combine2Args a, int slices, C2Fused f) {
    __shared__ uint32_t drop_lds[kWavesPerBlock];
    __shared__ int sh_job, sh_ok;
    const int wave = wave_in_block();
    const int per = kWavesPerBlock / slices;  // tokens per pass of the workgroup
    const int sub = wave / slices, part = wave % slices;
    const int njobs = f.nbatch + f.lag;
    for (;;) {
        if (threadIdx.x == 0) sh_job = (int)atomicAdd(&f.ctr[0], 1u);
        __syncthreads();
        const int job = sh_job;
        __syncthreads();
        if (job >= njobs) return;
        if (job < f.nbatch) {
            const int t0 = job * f.tile, t1 = min(a.T, t0 + f.tile);
            for (int tb = t0; tb < t1; tb += per) {
                group_rows_token<VPW, true>(a, tb + sub, part, slices, tb + sub < t1, drop_lds);
                __syncthreads();  // drop_lds is reused by the next token
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are acknowledged
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
        for (int tb = t0; tb < t1; tb += per) {
            cross_rows_token<VPW, true>(a, tb + sub, part, slices, tb + sub < t1, drop_lds);
            __syncthreads();
        }
    }
}

// Whether every flag vector of the first `nblk` blocks of chunked row `row`
// equals epoch; the wave's lanes take the 2 * nblk flag vectors between them.
__device__ __forceinline__ bool row_flags_ok(const uint8_t* row, int nblk, uint32_t epoch, int lane) {
    bool bad = false;
    for (int j = lane; j < 2 * nblk; j += kWave)
        bad |= !flag_ok(ld16(row + (int64_t)(j >> 1) * kChunkBytes + kChunkPayload + (j & 1) * 16), epoch);
    return __ballot(bad) == 0;
}

constexpr int kAnyBatch = 4;  // rows per load batch in the any-K kernels

// Group step for any K (used when K > 16): one wave per token. With chunked
// rows the flags of each usable lane's row are checked first, so a row with
// a bad flag is left out before any of its values is used. Then the token's
// groups are taken one at a time: per wave-iteration the group's lanes are
// read in ascending k, kAnyBatch rows per load batch, accumulated into one
// fp32 set and stored as the group's partial vectors.
__global__ __launch_bounds__(kBlockThreads) void combine_group_any_kernel(Combine2Args a) {
    const int lane = lane_id();
    const int t = blockIdx.x * kWavesPerBlock + wave_in_block();
    if (t >= a.T) return;
    int s = -1, g = -1, gs = -1;
    float wt = 0.f;
    if (lane < a.K) {
        const int64_t e = a.topk[(int64_t)t * a.K + lane];
        s = a.slot[(int64_t)t * a.K + lane];
        gs = a.group_slot[(int64_t)t * a.K + lane];
        wt = a.w[(int64_t)t * a.K + lane];
        if (expert_ok(e, a.E)) g = ((int)e / a.epr) / a.P;
    }
    bool use = s >= 0 && g >= 0;
    if (use && s >= a.y_rows) {
        report(a.err, EP_DEVERR_CAPACITY);
        use = false;
    }
    uint64_t um = __ballot(use);
    const int nvh = a.H / 8;
    const int nblk = (2 * a.H + kChunkPayload - 1) / kChunkPayload;
    const int iters = (nblk + 1) / 2;
    if (a.y_chunked) {
        uint64_t drop = 0;
        for (uint64_t m = um; m; m &= m - 1) {
            const int k = __ffsll((unsigned long long)m) - 1;
            if (!row_flags_ok(a.y + (int64_t)readlane(s, k) * a.y_stride, nblk, a.epoch, lane))
                drop |= 1ull << k;
        }
        if (drop && lane == 0) report(a.err, EP_DEVERR_FLAG);
        um &= ~drop;
    }
    bool first = g >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int gj = readlane(g, j);
        if (j < lane && gj == g) first = false;
    }
    const u32x4 flagv = {a.epoch, a.epoch, a.epoch, a.epoch};
    for (uint64_t fm = __ballot(first); fm; fm &= fm - 1) {
        const int k0 = __ffsll((unsigned long long)fm) - 1;
        const int g0 = readlane(g, k0);
        const int64_t dst = readlane(gs, k0);
        if (dst >= a.group_cap) {
            if (lane == 0) report(a.err, EP_DEVERR_CAPACITY);
            continue;
        }
        uint8_t* prow = a.group_buf + dst * a.pstride;
        const uint64_t gm = um & __ballot(g == g0);
        for (int it = 0; it < iters; ++it) {
            int c, wv, p;
            const bool hv = chunk_vec(it, lane, nvh, c, wv, p);
            const int64_t blk = (int64_t)c * kChunkBytes + (int64_t)wv * 16;
            const int64_t off = a.y_chunked ? blk : (int64_t)p * 16;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (uint64_t m = gm; m;) {
                int kk[kAnyBatch];
                int nk = 0;
                for (; nk < kAnyBatch && m; ++nk, m &= m - 1) kk[nk] = __ffsll((unsigned long long)m) - 1;
                u32x4 v[kAnyBatch];
#pragma unroll
                for (int j = 0; j < kAnyBatch; ++j) {
                    v[j] = u32x4{0u, 0u, 0u, 0u};
                    if (j < nk && hv) v[j] = ld16(a.y + (int64_t)readlane(s, kk[j]) * a.y_stride + off);
                }
#pragma unroll
                for (int j = 0; j < kAnyBatch; ++j) {
                    if (j >= nk) break;
                    const float wk = readlane_f(wt, kk[j]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[2 * q] = __builtin_fmaf(wk, bf16_lo(v[j][q]), acc[2 * q]);
                        acc[2 * q + 1] = __builtin_fmaf(wk, bf16_hi(v[j][q]), acc[2 * q + 1]);
                    }
                }
            }
            if (c >= nblk) continue;
            u32x4 o = hv ? pack8(acc) : u32x4{0u, 0u, 0u, 0u};
            if (wv >= kChunkPayloadVecs) o = flagv;
            st16_stream(prow + blk, o);
        }
    }
}

// Cross-group step for any K (used when K > 16): one wave per token. The
// flags of each partial row are checked first (a bad row is left out); lane
// `pos` then holds the row of the token's pos-th partial in ascending group,
// and per wave-iteration the partials are read kAnyBatch per load batch and
// summed in that order.
__global__ __launch_bounds__(kBlockThreads) void combine_cross_any_kernel(Combine2Args a) {
    const int lane = lane_id();
    const int t = blockIdx.x * kWavesPerBlock + wave_in_block();
    if (t >= a.T) return;
    int g = -1, gs = -1;
    if (lane < a.K) {
        const int64_t e = a.topk[(int64_t)t * a.K + lane];
        gs = a.group_slot[(int64_t)t * a.K + lane];
        if (expert_ok(e, a.E)) g = ((int)e / a.epr) / a.P;
    }
    bool first = g >= 0 && gs >= 0;
    for (int j = 0; j < a.K; ++j) {
        const int gj = readlane(g, j);
        if (j < lane && gj == g) first = false;
    }
    if (first && gs >= a.group_cap) {
        report(a.err, EP_DEVERR_CAPACITY);
        first = false;
    }
    uint64_t fm = __ballot(first);
    const int nvh = a.H / 8;
    const int nblk = (2 * a.H + kChunkPayload - 1) / kChunkPayload;
    const int iters = (nblk + 1) / 2;
    uint64_t drop = 0;
    for (uint64_t m = fm; m; m &= m - 1) {
        const int k = __ffsll((unsigned long long)m) - 1;
        if (!row_flags_ok(a.group_buf + (int64_t)readlane(gs, k) * a.pstride, nblk, a.epoch, lane))
            drop |= 1ull << k;
    }
    if (drop && lane == 0) report(a.err, EP_DEVERR_FLAG);
    fm &= ~drop;
    int rank = 0;  // position of this lane's partial among the token's, by group
    for (uint64_t m = fm; m; m &= m - 1) {
        const int j = __ffsll((unsigned long long)m) - 1;
        rank += readlane(g, j) < g ? 1 : 0;
    }
    const int ng = __popcll(fm);
    int ordrow = 0;  // lane pos: the row of partial pos
    for (int pos = 0; pos < ng; ++pos) {
        const uint64_t who = __ballot(((fm >> lane) & 1) && rank == pos);
        const int row = readlane(gs, __ffsll((unsigned long long)who) - 1);
        if (lane == pos) ordrow = row;
    }
    uint8_t* out_row = reinterpret_cast<uint8_t*>(a.out) + (int64_t)t * a.H * 2;
    for (int it = 0; it < iters; ++it) {
        int c, wv, p;
        const bool hv = chunk_vec(it, lane, nvh, c, wv, p);
        const int64_t blk = (int64_t)c * kChunkBytes + (int64_t)wv * 16;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int pos0 = 0; pos0 < ng; pos0 += kAnyBatch) {
            u32x4 v[kAnyBatch];
#pragma unroll
            for (int j = 0; j < kAnyBatch; ++j) {
                v[j] = u32x4{0u, 0u, 0u, 0u};
                if (pos0 + j < ng && hv)
                    v[j] = ld16(a.group_buf + (int64_t)readlane(ordrow, pos0 + j) * a.pstride + blk);
            }
#pragma unroll
            for (int j = 0; j < kAnyBatch; ++j) {
                if (pos0 + j >= ng) break;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = acc[2 * q] + bf16_lo(v[j][q]);
                    acc[2 * q + 1] = acc[2 * q + 1] + bf16_hi(v[j][q]);
                }
            }
        }
        if (hv) st16_stream(out_row + (int64_t)p * 16, pack8(acc));
    }
}

}  // namespace

constexpr uint32_t kC2FusedTimeoutUs = 100000;  // longest wait for one batch flag
#ifndef EP_C2F_MIN_PARTIAL_BYTES
#define EP_C2F_MIN_PARTIAL_BYTES (512ll << 20)  // one launch from this many bytes of partial rows
#endif
constexpr int64_t kC2FusedMinPartialBytes = EP_C2F_MIN_PARTIAL_BYTES;

hipError_t launch_combine_two_level(const ep_shape& s, const ep_layout& L, const int64_t* topk,
                                    const void* y, int64_t y_rows, int64_t y_stride, int fmt,
                                    uint32_t epoch, const float* w, void* group_buf,
                                    int64_t group_cap, int steps, uint16_t* out, char* ws,
                                    hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const WsLayout W = ws_layout(s);
    Combine2Args a;
    a.T = s.T; a.H = s.H; a.K = s.K; a.E = s.E; a.R = s.R; a.G = s.G;
    a.epr = s.E / s.R; a.P = s.R / s.G;
    a.topk = topk;
    a.slot = L.slot;
    a.group_slot = L.group_slot;
    a.w = w;
    a.y = reinterpret_cast<const uint8_t*>(y);
    a.y_rows = y_rows;
    a.y_stride = y_stride;
    a.y_chunked = fmt == EP_FMT_CHUNKED;
    a.epoch = epoch;
    a.group_buf = reinterpret_cast<uint8_t*>(group_buf);
    a.group_cap = group_cap;
    a.pstride = (int64_t)kChunkBytes * ((2 * (int64_t)s.H + kChunkPayload - 1) / kChunkPayload);
    a.out = out;
    a.err = reinterpret_cast<uint32_t*>(ws + W.err);
    const dim3 grid((s.T + kWavesPerBlock - 1) / kWavesPerBlock), block(kBlockThreads);
    const int nblk = (2 * s.H + kChunkPayload - 1) / kChunkPayload;
    const int iters = (nblk + 1) / 2;
    constexpr int kGroupVpw = 4;
    const int slices = (iters + kGroupVpw - 1) / kGroupVpw;
    // One launch pays off only when the partial rows are well past the MALL:
    // smaller ones are still cached when the cross launch reads them
    // (hier8x8 shapes, T = 16,384, bench.py --hidden: fused / two launches
    // 752 / 885 us at H = 7,168, 421 / 480 us at 3,840 (710 MB of partial
    // rows), 317 / 281 us at 2,048 (400 MB), 168 / 153 us at 1,024).
    const bool big = (int64_t)group_cap * a.pstride >= kC2FusedMinPartialBytes;
    if (steps == 3 && EP_C2_FUSED && big && s.K <= 8 && EP_C2_ROWS && kWavesPerBlock % slices == 0) {
        LaunchInfo d;
        const hipError_t e = launch_info(st, reinterpret_cast<const void*>(&combine_two_level_fused_kernel<kGroupVpw>),
                                         kBlockThreads, &d);
        if (e != hipSuccess) return e;
        C2Fused f;
        f.tile = EP_C2F_TILE * (kWavesPerBlock / slices);  // every wave of a workgroup pass busy
        f.nbatch = (s.T + f.tile - 1) / f.tile;
        f.lag = EP_C2F_LAG;
        f.timeout = (uint64_t)kC2FusedTimeoutUs * (uint64_t)(d.rate_khz > 0 ? d.rate_khz : 100000) / 1000u;
        f.ctr = reinterpret_cast<uint32_t*>(ws + W.fused);
        f.flags = f.ctr + kFusedCounters;
        const int per_cu = EP_C2F_WG_PER_CU > 0 ? std::min(d.per_cu, EP_C2F_WG_PER_CU) : d.per_cu;
        const int blocks = std::min(std::max(1, d.cus * std::max(1, per_cu)), std::max(1, 2 * f.nbatch));
        launch_zero_words(f.ctr, kFusedCounters + f.nbatch, st);  // f.flags follows the counter words
        hipLaunchKernelGGL(combine_two_level_fused_kernel<kGroupVpw>, dim3(blocks), block, 0, st, a, slices, f);
        return hipGetLastError();
    }
    if ((steps & 1) && s.K <= 8 && EP_C2_ROWS && (!a.y_chunked || kWavesPerBlock % slices == 0)) {
        const dim3 g2((unsigned)(((int64_t)s.T * slices + kWavesPerBlock - 1) / kWavesPerBlock));
        hipLaunchKernelGGL(combine_group_rows_kernel<kGroupVpw>, g2, block, 0, st, a, slices);
    } else if (steps & 1) {
        if (s.K <= 2)
            hipLaunchKernelGGL(combine_group_kernel<2>, grid, block, 0, st, a);
        else if (s.K <= 4)
            hipLaunchKernelGGL(combine_group_kernel<4>, grid, block, 0, st, a);
        else if (s.K <= 8)
            hipLaunchKernelGGL(combine_group_kernel<8>, grid, block, 0, st, a);
        else if (s.K <= 16)
            hipLaunchKernelGGL(combine_group_kernel<16>, grid, block, 0, st, a);
        else
            hipLaunchKernelGGL(combine_group_any_kernel, grid, block, 0, st, a);
    }
    if ((steps & 2) && s.K <= 8 && EP_C2_ROWS && kWavesPerBlock % slices == 0) {
        const dim3 g2((unsigned)(((int64_t)s.T * slices + kWavesPerBlock - 1) / kWavesPerBlock));
        hipLaunchKernelGGL(combine_cross_rows_kernel<kGroupVpw>, g2, block, 0, st, a, slices);
    } else if (steps & 2) {
        if (s.K <= 8)
            hipLaunchKernelGGL(combine_cross_kernel<8>, grid, block, 0, st, a);
        else if (s.K <= 16)
            hipLaunchKernelGGL(combine_cross_kernel<16>, grid, block, 0, st, a);
        else
            hipLaunchKernelGGL(combine_cross_any_kernel, grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace ep
