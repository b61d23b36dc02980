// combine.hip -- ep_combine on gfx950: inverse gather plus top-k weighted
// reduction back into token order.
//
// What is computed: out[t] = bf16_rne(sum over valid k, ascending, of
// w[t][k] * y[slot[t][k]]) with one fp32 fused multiply-add per step starting
// from +0. Expert outputs are BF16 rows and the weights FP32, as in "Ascend
// Send Ordering" (改造时按这个顺序检查: BF16 hidden, FP32 top-k weight); the
// rows to gather are the per-(token, destination) rows the dispatch wrote,
// i.e. the combine direction of "06_06: NVLink Scale-up + RDMA Scale-out —
// DeepEP 三阶段流水线 vs DeepGEMM 对称内存" (combine write into
// combine_token_buffer[topk slot][token]).
//
// CDNA4 mapping. A lane owns 16-byte vectors (8 bf16) of the hidden row and
// the fp32 accumulation runs in ascending k with v_fma_f32. Two kernels:
//   * row-streaming (K <= 8, the common case): a token is cut into slices of
//     4 or 8 wave-iterations, one wave per slice; the wave reads its slice of
//     one row at a time as a burst, the next row's burst requested before the
//     current one is summed;
//   * one wave per token (K > 8, or chunked rows whose slices would not fill
//     a workgroup): for a group of NB vectors all K source rows are requested
//     before any arithmetic (K x NB loads in flight per lane, issued without
//     branches or waits in between).
// Chunked rows (512 B blocks, 480 B payload) are read in place: wave
// iteration i covers blocks 2i and 2i+1, lane L holds payload vector
// 30 * (2i + L/32) + L%32 when L%32 < 30; every block that carries hidden
// bytes must have its 32-byte flag equal to epoch.
#include "ep_device.h"
#include "ep_internal.h"

// Compile-time tuning knobs (defaults are the measured best on MI355X).
#ifndef EP_CMB_NB8
#define EP_CMB_NB8 2        // 16-byte vectors per lane per batch when K <= 8
#endif
#ifndef EP_CMB_NTLOAD
#define EP_CMB_NTLOAD 1     // non-temporal loads of the gathered rows
#endif
#ifndef EP_CMB_MINB
#define EP_CMB_MINB 1       // minimum resident workgroups per CU (launch bound)
#endif
#ifndef EP_CMB_WPB
#define EP_CMB_WPB 4        // waves per workgroup
#endif
#ifndef EP_CMB_ROWS
#define EP_CMB_ROWS 2       // row-streaming kernel: 1 = plain rows, 2 = plain and chunked rows
#endif
#ifndef EP_CMB_VPWMAX
#define EP_CMB_VPWMAX 8     // row-streaming kernel: most wave-iterations per slice (4 or 8)
#endif
#ifndef EP_CMB_VPWMAX_CH
#define EP_CMB_VPWMAX_CH 4  // row-streaming kernel on chunked rows: most wave-iterations per slice
#endif
#ifndef EP_CMB_DUP
#define EP_CMB_DUP 1        // row-streaming kernel: keep one repeated row in VGPRs instead of re-reading it
#endif
#ifndef EP_CMB_NTSTORE
#define EP_CMB_NTSTORE 1    // non-temporal stores of the output rows
#endif

namespace ep {
namespace {

constexpr int kCmbWaves = EP_CMB_WPB;
constexpr int kCmbThreads = kCmbWaves * kWave;

__device__ __forceinline__ u32x4 ld_row(const void* p) {
#if EP_CMB_NTLOAD
    return ld16_stream(p);
#else
    return ld16(p);
#endif
}
__device__ __forceinline__ void st_out(void* p, u32x4 v) {
#if EP_CMB_NTSTORE
    st16_stream(p, v);
#else
    st16(p, v);
#endif
}

struct CombineArgs {
    int T, H, K;
    const int32_t* slot;
    const float* w;
    const uint8_t* y;
    int64_t y_rows, stride;
    uint32_t epoch;
    uint16_t* out;
    uint32_t* err;
};

// Byte offset of this lane's vector in wave iteration `it`, and whether the
// lane holds a hidden vector (index p) there.
template <bool CHUNKED>
__device__ __forceinline__ bool lane_vector(int it, int lane, int nvh, int& p, int64_t& off) {
    if (CHUNKED) {
        const int c = 2 * it + (lane >> 5), wv = lane & 31;
        p = c * kChunkPayloadVecs + wv;
        off = (int64_t)c * kChunkBytes + (int64_t)wv * 16;
        return wv < kChunkPayloadVecs && p < nvh;
    }
    p = it * kWave + lane;
    off = (int64_t)p * 16;
    return p < nvh;
}

__device__ __forceinline__ void fma8(float (&acc)[8], float w, u32x4 v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[2 * j] = __builtin_fmaf(w, bf16_lo(v[j]), acc[2 * j]);
        acc[2 * j + 1] = __builtin_fmaf(w, bf16_hi(v[j]), acc[2 * j + 1]);
    }
}

__device__ __forceinline__ u32x4 pack8(const float (&acc)[8]) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16(acc[2 * j]) | (f32_to_bf16(acc[2 * j + 1]) << 16);
    return o;
}

// Flag check of every distinct usable row over its hidden-carrying blocks, as
// a pass of its own (used by the any-K path). Returns the usable lanes left.
__device__ uint64_t check_flags_prepass(const CombineArgs& a, int s, uint64_t um) {
    const int lane = lane_id();
    const int nch = (2 * a.H + kChunkPayload - 1) / kChunkPayload;
    uint64_t keep = um;
    for (uint64_t m = um; m; m &= m - 1) {
        const int k = __ffsll((unsigned long long)m) - 1;
        const int sk = readlane(s, k);
        const uint8_t* row = a.y + (int64_t)sk * a.stride;
        bool ok = true;
        for (int i = lane; i < 2 * nch; i += kWave) {
            const u32x4 f = ld16(row + (int64_t)(i >> 1) * kChunkBytes + kChunkPayload + (i & 1) * 16);
            ok &= f[0] == a.epoch && f[1] == a.epoch && f[2] == a.epoch && f[3] == a.epoch;
        }
        if (__ballot(!ok)) keep &= ~(1ull << k);
    }
    return keep;
}

// KMAX > 0: up to KMAX lanes unrolled with per-lane registers; KMAX == 0:
// any K, one lane at a time.
template <int KMAX, int NB, bool CHUNKED>
__global__ __launch_bounds__(kCmbThreads, EP_CMB_MINB) void combine_kernel(CombineArgs a) {
    const int lane = lane_id();
    const int t = blockIdx.x * kCmbWaves + wave_in_block();
    if (t >= a.T) return;
    int s = -1;
    float wt = 0.f;
    if (lane < a.K) {
        s = a.slot[(int64_t)t * a.K + lane];
        wt = a.w[(int64_t)t * a.K + lane];
    }
    bool use = s >= 0;
    if (use && s >= a.y_rows) {
        report(a.err, EP_DEVERR_CAPACITY);
        use = false;
    }
    uint64_t um = __ballot(use);
    const int nvh = a.H / 8;
    const int nch = (2 * a.H + kChunkPayload - 1) / kChunkPayload;  // hidden-carrying blocks
    const int iters = CHUNKED ? (nch + 1) / 2 : (nvh + kWave - 1) / kWave;
    uint8_t* out_row = reinterpret_cast<uint8_t*>(a.out) + (int64_t)t * a.H * 2;

    if constexpr (KMAX == 0) {
        if (CHUNKED) {
            const uint64_t keep = check_flags_prepass(a, s, um);
            if (keep != um && lane == 0) report(a.err, EP_DEVERR_FLAG);
            um = keep;
        }
        for (int it = 0; it < iters; ++it) {
            int p;
            int64_t off;
            const bool valid = lane_vector<CHUNKED>(it, lane, nvh, p, off);
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int k = 0; k < a.K; ++k) {
                if (!((um >> k) & 1)) continue;
                const int sk = readlane(s, k);
                const float wk = readlane_f(wt, k);
                if (valid) fma8(acc, wk, ld_row(a.y + (int64_t)sk * a.stride + off));
            }
            if (valid) st_out(out_row + (int64_t)p * 16, pack8(acc));
        }
    } else {
        // One uniform row pointer per lane k. Lanes that do not contribute
        // point at a usable row (so every load is in bounds and can be issued
        // unconditionally) and are masked out of the sum; a row shared by two
        // lanes is simply requested twice (the second request is served by
        // the cache), which keeps the load phase free of branches.
        // Chunked rows: the lanes that sit on a block's 32-byte flag (L % 32
        // >= 30) load that flag with the same instruction and check it. A row
        // with a bad flag is found only after its values were used, so the
        // token is then computed again without it (an error path only).
        float wk[KMAX];
        const uint8_t* rowp[KMAX];
        for (int pass = 0; pass < 2; ++pass) {
            if (!um) {
                for (int it = 0; it < iters; ++it) {
                    int p;
                    int64_t off;
                    if (lane_vector<CHUNKED>(it, lane, nvh, p, off))
                        st_out(out_row + (int64_t)p * 16, u32x4{0u, 0u, 0u, 0u});
                }
                return;
            }
            const int s_any = readlane(s, __ffsll((unsigned long long)um) - 1);
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                const int kk = min(k, a.K - 1);
                const int sk = readlane(s, kk);
                rowp[k] = a.y + (int64_t)(((um >> k) & 1) ? sk : s_any) * a.stride;
                wk[k] = readlane_f(wt, kk);
            }
            uint32_t bad = 0;  // per lane: bit k = a flag of row k checked by this lane is wrong
            for (int it0 = 0; it0 < iters; it0 += NB) {
                int p[NB];
                int64_t off[NB];
                bool valid[NB], flag[NB];
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const bool in = it0 + j < iters;
                    valid[j] = in && lane_vector<CHUNKED>(it0 + j, lane, nvh, p[j], off[j]);
                    flag[j] = CHUNKED && in && (lane & 31) >= kChunkPayloadVecs &&
                              2 * (it0 + j) + (lane >> 5) < nch;
                    if (!valid[j] && !flag[j]) off[j] = 0;
                }
                u32x4 v[KMAX][NB];
#pragma unroll
                for (int k = 0; k < KMAX; ++k)
#pragma unroll
                    for (int j = 0; j < NB; ++j) v[k][j] = ld_row(rowp[k] + off[j]);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if (CHUNKED) {
#pragma unroll
                        for (int k = 0; k < KMAX; ++k) {
                            const u32x4 f = v[k][j];
                            const bool ok = f[0] == a.epoch && f[1] == a.epoch && f[2] == a.epoch &&
                                            f[3] == a.epoch;
                            bad |= (flag[j] && !ok) ? (1u << k) : 0u;
                        }
                    }
                    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < KMAX; ++k)
                        if ((um >> k) & 1) fma8(acc, wk[k], v[k][j]);
                    if (valid[j]) st_out(out_row + (int64_t)p[j] * 16, pack8(acc));
                }
            }
            if (!CHUNKED) return;
            uint64_t drop = 0;
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (((um >> k) & 1) && __ballot((bad >> k) & 1)) drop |= 1ull << k;
            if (!drop) return;
            if (lane == 0) report(a.err, EP_DEVERR_FLAG);
            // Every lane reading a dropped row drops with it.
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if ((drop >> k) & 1) drop |= __ballot(use && s == readlane(s, min(k, a.K - 1)));
            um &= ~drop;
        }
    }
}

// Row-streaming variant: a token is cut into slices of VPW wave-iterations,
// one wave per slice. For each lane k in ascending order the wave reads its
// slice of row k as one burst of VPW 16-byte vectors per lane (the next row's
// burst is requested before the current one is used) and accumulates it into
// VPW x 8 fp32 registers. Same sums in the same order as combine_kernel.
// Chunked rows: each slice checks the flags of its own blocks with the loads
// that bring in the values. The slices of a token are waves of one workgroup
// (the launch keeps `slices` a divisor of the waves per workgroup); they post
// the rows whose flags failed to LDS and read each other's after one barrier,
// which every wave of the workgroup reaches exactly once, so a bad row is
// dropped for the whole token and the token is summed again without it (an
// error path only; the second pass rewrites the output).
template <int KMAX, int VPW, bool CHUNKED>
__global__ __launch_bounds__(kCmbThreads, EP_CMB_MINB) void combine_rows_kernel(CombineArgs a, int slices) {
    __shared__ uint32_t drop_lds[CHUNKED ? 2 * kCmbWaves : 1];
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int gw = blockIdx.x * kCmbWaves + wave;
    const int t = gw / slices, part = gw % slices;
    const bool live = t < a.T;
    if (!CHUNKED && !live) return;
    int s = -1;
    float wt = 0.f;
    if (live && lane < a.K) {
        s = a.slot[(int64_t)t * a.K + lane];
        wt = a.w[(int64_t)t * a.K + lane];
    }
    bool use = s >= 0;
    if (use && s >= a.y_rows) {
        if (part == 0) report(a.err, EP_DEVERR_CAPACITY);
        use = false;
    }
    uint64_t um = __ballot(use);
    const int nvh = a.H / 8;
    const int nch = (2 * a.H + kChunkPayload - 1) / kChunkPayload;
    const int iters = CHUNKED ? (nch + 1) / 2 : (nvh + kWave - 1) / kWave;
    const int it0 = part * VPW;
    uint8_t* out_row = reinterpret_cast<uint8_t*>(a.out) + (int64_t)(live ? t : 0) * a.H * 2;
    int p[VPW];
    int64_t off[VPW];
    bool valid[VPW], flag[VPW];
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
        const bool in = live && it0 + j < iters;
        valid[j] = in && lane_vector<CHUNKED>(it0 + j, lane, nvh, p[j], off[j]);
        flag[j] = CHUNKED && in && (lane & 31) >= kChunkPayloadVecs && 2 * (it0 + j) + (lane >> 5) < nch;
        if (!valid[j] && !flag[j]) off[j] = 0;
    }
    for (int pass = 0; pass < 2; ++pass) {
        uint32_t bad = 0;  // per lane: bit k = a flag of row k checked by this lane is wrong
        if (!um) {
#pragma unroll
            for (int j = 0; j < VPW; ++j)
                if (valid[j]) st_out(out_row + (int64_t)p[j] * 16, u32x4{0u, 0u, 0u, 0u});
        } else {
            const int s_any = readlane(s, __ffsll((unsigned long long)um) - 1);
            // A rank reached by two lanes of the token shares one row. The
            // first such row (lowest lane k1) is kept in VGPRs after its use,
            // and the later lanes with the same row take it from there instead
            // of loading it again (kept: lanes that read the kept copy).
            uint64_t kept = 0;
            int k1 = KMAX;
#if EP_CMB_DUP
            {
                bool d = false;
                for (int j = 0; j < a.K; ++j) {
                    const int sj = readlane(s, j);
                    if (j < lane && ((um >> j) & 1) && sj == s) d = true;
                }
                const uint64_t dupm = __ballot(use && d);
                if (dupm) {
                    const int kd = __ffsll((unsigned long long)dupm) - 1;  // first repeating lane
                    const int sd = readlane(s, kd);
                    const uint64_t same = __ballot(use && s == sd);
                    k1 = __ffsll((unsigned long long)same) - 1;
                    kept = same & ~(1ull << k1);
                }
            }
#endif
            float acc[VPW][8];
#pragma unroll
            for (int j = 0; j < VPW; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
            u32x4 buf[2][VPW];
            u32x4 keep[EP_CMB_DUP ? VPW : 1];
            auto row_of = [&](int k) {
                const int kk = min(k, a.K - 1);
                return a.y + (int64_t)(((um >> k) & 1) ? readlane(s, kk) : s_any) * a.stride;
            };
            // A repeated row taken from `keep` is not read again; its load
            // slot reads the workspace's first 256 bytes instead (the error
            // words: in bounds and cached). Every step then issues the same
            // loads whichever rows repeat, so the compiler waits for row k
            // alone before summing it instead of for everything in flight
            // (a request under a branch made it wait for all loads).
            const uint8_t* spare = reinterpret_cast<const uint8_t*>(a.err) + (lane & 15) * 16;
            {
                const uint8_t* r0 = row_of(0);
#pragma unroll
                for (int j = 0; j < VPW; ++j) buf[0][j] = ld_row(r0 + off[j]);
            }
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (k + 1 < KMAX) {
                    const bool again = (kept >> (k + 1)) & 1;
                    const uint8_t* rn = row_of(k + 1);
#pragma unroll
                    for (int j = 0; j < VPW; ++j) buf[(k + 1) & 1][j] = ld_row(again ? spare : rn + off[j]);
                }
                const float wk = readlane_f(wt, min(k, a.K - 1));
                const bool uk = (um >> k) & 1;
#if EP_CMB_DUP
                const bool from_keep = (kept >> k) & 1;
                if (k == k1) {
#pragma unroll
                    for (int j = 0; j < VPW; ++j) keep[j] = buf[k & 1][j];
                }
#endif
#pragma unroll
                for (int j = 0; j < VPW; ++j) {
#if EP_CMB_DUP
                    const u32x4 v = from_keep ? keep[j] : buf[k & 1][j];
#else
                    const u32x4 v = buf[k & 1][j];
#endif
                    if (CHUNKED) {
                        const bool ok = v[0] == a.epoch && v[1] == a.epoch && v[2] == a.epoch && v[3] == a.epoch;
                        bad |= (flag[j] && uk && !ok) ? (1u << k) : 0u;
                    }
                    if (uk) fma8(acc[j], wk, v);
                }
            }
#pragma unroll
            for (int j = 0; j < VPW; ++j)
                if (valid[j]) st_out(out_row + (int64_t)p[j] * 16, pack8(acc[j]));
        }
        if (!CHUNKED || pass == 1) return;
        // The rows whose flags failed in this slice's blocks, then in any
        // slice of the token.
        uint64_t drop = 0;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (((um >> k) & 1) && __ballot((bad >> k) & 1)) drop |= 1ull << k;
        if (lane == 0) {
            drop_lds[2 * wave] = (uint32_t)drop;
            drop_lds[2 * wave + 1] = (uint32_t)(drop >> 32);
        }
        __syncthreads();
        const int w0 = wave - part;  // first wave of this token in the workgroup
        for (int q = 0; q < slices; ++q)
            drop |= ((uint64_t)drop_lds[2 * (w0 + q) + 1] << 32) | drop_lds[2 * (w0 + q)];
        if (!drop || !live) return;
        if (lane == 0 && part == 0) report(a.err, EP_DEVERR_FLAG);
        // Every lane reading a dropped row drops with it.
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if ((drop >> k) & 1) drop |= __ballot(use && s == readlane(s, min(k, a.K - 1)));
        um &= ~drop;
    }
}

// Narrow plain rows (at most 32 vectors: H <= 256) with K <= 8: one token
// per wave would leave most lanes idle, so a wave holds TPW tokens, one per
// group of G = 64 / TPW lanes (the row's vectors padded to a power of two).
// Each lane loads its token's K rows' vector (clamped to a usable row,
// issued together), then sums them in ascending k with fmaf from +0.0f and
// rounds once to bf16: the same arithmetic as the kernels above.
template <int TPW>
__global__ __launch_bounds__(kCmbThreads) void combine_narrow_kernel(CombineArgs a) {
    constexpr int G = kWave / TPW;
    const int lane = lane_id();
    const int gw = blockIdx.x * kCmbWaves + wave_in_block();
    const int t = gw * TPW + lane / G;
    const int v = lane % G;
    if (t >= a.T) return;
    int s[8];
    float wk[8];
    int any = -1;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        s[k] = -1;
        wk[k] = 0.f;
        if (k < a.K) {
            s[k] = a.slot[(int64_t)t * a.K + k];
            wk[k] = a.w[(int64_t)t * a.K + k];
        }
    }
    bool over = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (s[k] >= a.y_rows) {
            over = true;
            s[k] = -1;
        }
        if (any < 0 && s[k] >= 0) any = s[k];
    }
    if (over && v == 0) report(a.err, EP_DEVERR_CAPACITY);
    const int nvh = a.H / 8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (any >= 0) {
        const int64_t off = (int64_t)min(v, nvh - 1) * 16;
        u32x4 y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = ld_row(a.y + (int64_t)(s[k] >= 0 ? s[k] : any) * a.stride + off);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (s[k] >= 0) fma8(acc, wk[k], y[k]);
    }
    if (v < nvh) st_out(reinterpret_cast<uint8_t*>(a.out) + ((int64_t)t * nvh + v) * 16, pack8(acc));
}

template <bool CHUNKED>
hipError_t launch_k(const CombineArgs& a, hipStream_t st) {
    const dim3 block(kCmbThreads);
    const int nvh = a.H / 8;
    if (!CHUNKED && a.K <= 8 && nvh <= kWave / 2) {
        int g = 1;
        while (g < nvh) g *= 2;
        const int tpw = kWave / g;
        const int64_t waves = ((int64_t)a.T + tpw - 1) / tpw;
        const dim3 grid((unsigned)((waves + kCmbWaves - 1) / kCmbWaves));
        switch (tpw) {
            case 2: hipLaunchKernelGGL(combine_narrow_kernel<2>, grid, block, 0, st, a); break;
            case 4: hipLaunchKernelGGL(combine_narrow_kernel<4>, grid, block, 0, st, a); break;
            case 8: hipLaunchKernelGGL(combine_narrow_kernel<8>, grid, block, 0, st, a); break;
            case 16: hipLaunchKernelGGL(combine_narrow_kernel<16>, grid, block, 0, st, a); break;
            case 32: hipLaunchKernelGGL(combine_narrow_kernel<32>, grid, block, 0, st, a); break;
            default: hipLaunchKernelGGL(combine_narrow_kernel<64>, grid, block, 0, st, a); break;
        }
        return hipGetLastError();
    }
#if EP_CMB_ROWS
    if (a.K <= 8) {
        const int nch = (2 * a.H + kChunkPayload - 1) / kChunkPayload;
        const int iters = CHUNKED ? (nch + 1) / 2 : (a.H / 8 + kWave - 1) / kWave;
        const int vpw = iters > 8 && (CHUNKED ? EP_CMB_VPWMAX_CH : EP_CMB_VPWMAX) >= 8 ? 8 : 4;
        const int slices = (iters + vpw - 1) / vpw;
        // Chunked rows need the slices of a token inside one workgroup.
        if (!CHUNKED || (EP_CMB_ROWS >= 2 && kCmbWaves % slices == 0)) {
            const dim3 grid((unsigned)(((int64_t)a.T * slices + kCmbWaves - 1) / kCmbWaves));
            if (vpw == 8)
                hipLaunchKernelGGL((combine_rows_kernel<8, 8, CHUNKED>), grid, block, 0, st, a, slices);
            else
                hipLaunchKernelGGL((combine_rows_kernel<8, 4, CHUNKED>), grid, block, 0, st, a, slices);
            return hipGetLastError();
        }
    }
#endif
    const dim3 grid((a.T + kCmbWaves - 1) / kCmbWaves);
    if (a.K <= 2)
        hipLaunchKernelGGL((combine_kernel<2, 8, CHUNKED>), grid, block, 0, st, a);
    else if (a.K <= 4)
        hipLaunchKernelGGL((combine_kernel<4, 4, CHUNKED>), grid, block, 0, st, a);
    else if (a.K <= 8)
        hipLaunchKernelGGL((combine_kernel<8, EP_CMB_NB8, CHUNKED>), grid, block, 0, st, a);
    else if (a.K <= 16)
        hipLaunchKernelGGL((combine_kernel<16, 1, CHUNKED>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((combine_kernel<0, 1, CHUNKED>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const ep_shape& s, const ep_layout& L, const void* y, int64_t y_rows,
                          int64_t y_stride, int fmt, uint32_t epoch, const float* w,
                          uint16_t* out, char* ws, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const WsLayout W = ws_layout(s);
    CombineArgs a;
    a.T = s.T; a.H = s.H; a.K = s.K;
    a.slot = L.slot;
    a.w = w;
    a.y = reinterpret_cast<const uint8_t*>(y);
    a.y_rows = y_rows;
    a.stride = y_stride;
    a.epoch = epoch;
    a.out = out;
    a.err = reinterpret_cast<uint32_t*>(ws + W.err);
    return fmt == EP_FMT_CHUNKED ? launch_k<true>(a, st) : launch_k<false>(a, st);
}

}  // namespace ep
