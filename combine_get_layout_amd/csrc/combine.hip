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
// CDNA4 mapping: one wave64 per output token. A lane owns 16-byte vectors (8
// bf16) of the hidden row. All distinct source rows of a group of NB vectors
// are loaded before any arithmetic (K x NB loads in flight per lane), a row
// shared by two lanes k is loaded once, and the fp32 accumulation runs in
// ascending k with v_fma_f32. Chunked rows (512 B blocks, 480 B payload) are
// read in place: wave iteration i covers blocks 2i and 2i+1, lane L holds
// payload vector 30 * (2i + L/32) + L%32 when L%32 < 30; every block that
// carries hidden bytes must have its 32-byte flag equal to epoch.
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
#define EP_CMB_WPB 4        // waves (tokens) per workgroup
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

// KMAX > 0: up to KMAX lanes unrolled with per-lane registers; KMAX == 0:
// any K, one lane at a time (repeated rows are simply re-read).
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
    const int nvh = a.H / 8;
    if (CHUNKED) {
        // Flag check of every distinct usable row over its hidden-carrying blocks.
        const int nch = (2 * a.H + kChunkPayload - 1) / kChunkPayload;
        const uint64_t um = __ballot(use);
        for (uint64_t m = um; m; m &= m - 1) {
            const int k = __ffsll((unsigned long long)m) - 1;
            const int sk = readlane(s, k);
            bool dup = false;
            for (uint64_t q = um & ((1ull << k) - 1); q; q &= q - 1)
                dup |= readlane(s, __ffsll((unsigned long long)q) - 1) == sk;
            if (dup) continue;
            const uint8_t* row = a.y + (int64_t)sk * a.stride;
            bool ok = true;
            for (int i = lane; i < 2 * nch; i += kWave) {
                const u32x4 f = ld16(row + (int64_t)(i >> 1) * kChunkBytes + kChunkPayload + (i & 1) * 16);
                ok &= f[0] == a.epoch && f[1] == a.epoch && f[2] == a.epoch && f[3] == a.epoch;
            }
            if (__ballot(!ok)) {
                if (lane == 0) report(a.err, EP_DEVERR_FLAG);
                if (s == sk) use = false;
            }
        }
    }
    const uint64_t um = __ballot(use);
    const int iters = CHUNKED ? ((2 * a.H + kChunkPayload - 1) / kChunkPayload + 1) / 2
                              : (nvh + kWave - 1) / kWave;
    uint8_t* out_row = reinterpret_cast<uint8_t*>(a.out) + (int64_t)t * a.H * 2;

    if constexpr (KMAX == 0) {
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
            if (valid) st16_stream(out_row + (int64_t)p * 16, pack8(acc));
        }
    } else {
        int sk[KMAX], src[KMAX];
        float wk[KMAX];
        bool uk[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            uk[k] = k < a.K && ((um >> k) & 1);
            sk[k] = k < a.K ? readlane(s, k) : -1;
            wk[k] = k < a.K ? readlane_f(wt, k) : 0.f;
            src[k] = k;
#pragma unroll
            for (int j = KMAX - 1; j >= 0; --j)
                if (j < k && uk[j] && uk[k] && sk[j] == sk[k]) src[k] = j;
        }
        for (int it0 = 0; it0 < iters; it0 += NB) {
            u32x4 v[KMAX][NB];
            int p[NB];
            int64_t off[NB];
            bool valid[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) valid[j] = it0 + j < iters && lane_vector<CHUNKED>(it0 + j, lane, nvh, p[j], off[j]);
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (!uk[k] || src[k] != k) continue;
                const uint8_t* row = a.y + (int64_t)sk[k] * a.stride;
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    if (valid[j]) v[k][j] = ld_row(row + off[j]);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < KMAX; ++k) {
                    if (!uk[k]) continue;
                    u32x4 val;
                    if (src[k] == k) {
                        val = v[k][j];
                    } else {
#pragma unroll
                        for (int m = 0; m < KMAX; ++m)
                            if (m < k && src[k] == m) val = v[m][j];
                    }
                    fma8(acc, wk[k], val);
                }
                if (valid[j]) st16_stream(out_row + (int64_t)p[j] * 16, pack8(acc));
            }
        }
    }
}

template <bool CHUNKED>
hipError_t launch_k(const CombineArgs& a, hipStream_t st) {
    const dim3 grid((a.T + kCmbWaves - 1) / kCmbWaves), block(kCmbThreads);
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
