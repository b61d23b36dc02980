// layout.hip -- ep_get_layout on gfx950: counts, offsets, masks and slots.
//
// What is computed follows "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK
// 复制机制", §3.3 阶段1 (notify warps: per-lane expert counts, per-token rank
// deduplication, prefix sums) and the slot hand-out of §3.3 阶段2, with slots
// made deterministic: the row of (token t, rank r) is
//     rank_offsets[r] + #{t' < t : token t' sends to r}.
//
// Three stream-ordered launches, all integer work:
//   1. count  : one thread per token, 256 tokens per workgroup. Each token ORs
//               its bit into an LDS bit matrix bits[r][t/32] (a repeated rank
//               sets the same bit, which is the deduplication) and bumps an
//               LDS expert histogram. Per-workgroup counts are popcounts of
//               the bit rows; the is-token-in-rank mask is expanded from the
//               same bits with 16-byte stores.
//   2. reduce : one thread per column (rank, group, expert); turns the
//               per-workgroup counts into workgroup-exclusive prefixes and
//               totals.
//   3. assign : rebuilds the bit matrix, scans the totals in LDS, and gives
//               every lane its slot = region start + workgroup prefix +
//               popcount of the bits of earlier tokens in the workgroup.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kWords = kLayoutTokens / 32;  // bit-matrix words per rank per workgroup

struct LayoutArgs {
    int T, K, E, R, G, epr, P, nb;
    const int64_t* topk;
    uint32_t* err;
    int32_t* part_rank;
    int32_t* part_group;
    int32_t* part_expert;
    int32_t* tot_rank;
    int32_t* tot_group;
    int32_t* tot_expert;
    ep_layout out;
};

// Set this token's bit for every rank (and group) its valid lanes reach.
// Returns whether any lane held an invalid id (< -1 or >= E).
__device__ __forceinline__ bool mark_token(const LayoutArgs& a, int t, uint32_t* bits_r,
                                           uint32_t* bits_g, int32_t* cnt_e) {
    const int64_t* row = a.topk + (int64_t)t * a.K;
    const int w = threadIdx.x / 32;
    const uint32_t bit = 1u << (threadIdx.x & 31);
    bool bad = false;
#pragma unroll 8
    for (int k = 0; k < a.K; ++k) {
        const int64_t e = row[k];
        bad |= expert_bad(e, a.E);
        if (!expert_ok(e, a.E)) continue;
        const int r = (int)e / a.epr;
        atomicOr(&bits_r[r * kWords + w], bit);
        if (bits_g) atomicOr(&bits_g[(r / a.P) * kWords + w], bit);
        if (cnt_e) atomicAdd(&cnt_e[(int)e], 1);
    }
    return bad;
}

// Expand bits[c][t/32] of this workgroup's nt tokens into mask bytes
// [t0*C, (t0+nt)*C) of a [T, C] uint8 mask. 16-byte stores; the span starts
// at a multiple of 256*C bytes, so it is 16-byte aligned for an aligned base.
__device__ void write_mask(const uint32_t* bits, int C, int t0, int nt, uint8_t* mask) {
    const int64_t begin = (int64_t)t0 * C;
    const int64_t nbytes = (int64_t)nt * C;
    const int64_t nvec = nbytes / 16;
    for (int64_t v = threadIdx.x; v < nvec; v += kBlockThreads) {
        int64_t idx = v * 16;
        int lt = (int)(idx / C);
        int c = (int)(idx - (int64_t)lt * C);
        uint32_t word[4] = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            uint32_t b = (bits[c * kWords + (lt >> 5)] >> (lt & 31)) & 1u;
            word[j >> 2] |= b << (8 * (j & 3));
            if (++c == C) { c = 0; ++lt; }
        }
        u32x4 out = {word[0], word[1], word[2], word[3]};
        st16(mask + begin + idx, out);
    }
    for (int64_t i = nvec * 16 + threadIdx.x; i < nbytes; i += kBlockThreads) {
        int lt = (int)(i / C), c = (int)(i - (int64_t)lt * C);
        mask[begin + i] = (uint8_t)((bits[c * kWords + (lt >> 5)] >> (lt & 31)) & 1u);
    }
}

__device__ __forceinline__ int popc_row(const uint32_t* bits, int c) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) s += __popc(bits[c * kWords + w]);
    return s;
}

__global__ __launch_bounds__(kBlockThreads) void layout_count_kernel(LayoutArgs a) {
    extern __shared__ uint32_t lds[];
    uint32_t* bits_r = lds;
    uint32_t* bits_g = bits_r + a.R * kWords;
    int32_t* cnt_e = reinterpret_cast<int32_t*>(bits_g + a.G * kWords);
    const int b = blockIdx.x;
    if (b == 0 && threadIdx.x == 0) *a.err = 0u;  // a pass of calls starts with a clean word
    const int n_lds = (a.R + a.G) * kWords + a.E;
    for (int i = threadIdx.x; i < n_lds; i += kBlockThreads) lds[i] = 0u;
    __syncthreads();

    const int t0 = b * kLayoutTokens;
    const int t = t0 + threadIdx.x;
    if (t < a.T) mark_token(a, t, bits_r, bits_g, cnt_e);
    __syncthreads();

    for (int c = threadIdx.x; c < a.R; c += kBlockThreads)
        a.part_rank[(int64_t)b * a.R + c] = popc_row(bits_r, c);
    for (int c = threadIdx.x; c < a.G; c += kBlockThreads)
        a.part_group[(int64_t)b * a.G + c] = popc_row(bits_g, c);
    for (int c = threadIdx.x; c < a.E; c += kBlockThreads)
        a.part_expert[(int64_t)b * a.E + c] = cnt_e[c];

    const int nt = min(kLayoutTokens, a.T - t0);
    if (nt > 0 && a.out.is_token_in_rank) write_mask(bits_r, a.R, t0, nt, a.out.is_token_in_rank);
    if (nt > 0 && a.out.is_token_in_group) write_mask(bits_g, a.G, t0, nt, a.out.is_token_in_group);
}

// One thread per column of the [nb][C] per-workgroup count tables: replace the
// column by its exclusive prefix over workgroups and record the total.
__device__ __forceinline__ void reduce_column(int32_t* part, int C, int c, int nb, int32_t* tot,
                                              int32_t* out_count) {
    constexpr int kBatch = 16;
    int32_t run = 0;
    for (int b0 = 0; b0 < nb; b0 += kBatch) {
        int32_t v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) v[j] = (b0 + j < nb) ? part[(int64_t)(b0 + j) * C + c] : 0;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (b0 + j < nb) part[(int64_t)(b0 + j) * C + c] = run;
            run += v[j];
        }
    }
    tot[c] = run;
    if (out_count) out_count[c] = run;
}

__global__ __launch_bounds__(kBlockThreads) void layout_reduce_kernel(LayoutArgs a) {
    int c = blockIdx.x * kBlockThreads + threadIdx.x;
    if (c < a.R) { reduce_column(a.part_rank, a.R, c, a.nb, a.tot_rank, a.out.tokens_per_rank); return; }
    c -= a.R;
    if (c < a.G) { reduce_column(a.part_group, a.G, c, a.nb, a.tot_group, a.out.tokens_per_group); return; }
    c -= a.G;
    if (c < a.E) reduce_column(a.part_expert, a.E, c, a.nb, a.tot_expert, a.out.tokens_per_expert);
}

// Workgroup-wide exclusive scan of in[0, n) (n <= 16 * 256). Writes the
// exclusive prefix to lds_out[i] (if non-null) and to gl_out[i] (if non-null),
// gl_out[n] = total. scratch: 256 ints of LDS.
__device__ void block_exclusive_scan(const int32_t* in, int n, int32_t* lds_out, int32_t* gl_out,
                                     int32_t* scratch) {
    const int tid = threadIdx.x;
    const int per = (n + kBlockThreads - 1) / kBlockThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int32_t s = 0;
    for (int i = lo; i < hi; ++i) s += in[i];
    scratch[tid] = s;
    __syncthreads();
    for (int off = 1; off < kBlockThreads; off <<= 1) {
        int32_t v = tid >= off ? scratch[tid - off] : 0;
        __syncthreads();
        scratch[tid] += v;
        __syncthreads();
    }
    int32_t run = tid ? scratch[tid - 1] : 0;
    for (int i = lo; i < hi; ++i) {
        if (lds_out) lds_out[i] = run;
        if (gl_out) gl_out[i] = run;
        run += in[i];
    }
    if (gl_out && tid == kBlockThreads - 1) gl_out[n] = scratch[kBlockThreads - 1];
    __syncthreads();
}

__global__ __launch_bounds__(kBlockThreads) void layout_assign_kernel(LayoutArgs a) {
    extern __shared__ uint32_t lds[];
    uint32_t* bits_r = lds;
    uint32_t* bits_g = bits_r + a.R * kWords;
    int32_t* base_r = reinterpret_cast<int32_t*>(bits_g + a.G * kWords);
    int32_t* base_g = base_r + a.R;
    int32_t* scratch = base_g + a.G;
    const int b = blockIdx.x;
    const bool groups = a.out.group_slot != nullptr;
    for (int i = threadIdx.x; i < (a.R + a.G) * kWords; i += kBlockThreads) lds[i] = 0u;
    __syncthreads();

    const int t0 = b * kLayoutTokens;
    const int t = t0 + threadIdx.x;
    bool bad = false;
    if (t < a.T) bad = mark_token(a, t, bits_r, groups ? bits_g : nullptr, nullptr);

    // Region starts: exclusive scan of the totals; workgroup 0 also publishes
    // the offset arrays.
    block_exclusive_scan(a.tot_rank, a.R, base_r, b == 0 ? a.out.rank_offsets : nullptr, scratch);
    block_exclusive_scan(a.tot_group, a.G, base_g, b == 0 ? a.out.group_offsets : nullptr, scratch);
    if (b == 0 && a.out.expert_offsets)
        block_exclusive_scan(a.tot_expert, a.E, nullptr, a.out.expert_offsets, scratch);
    for (int c = threadIdx.x; c < a.R; c += kBlockThreads) base_r[c] += a.part_rank[(int64_t)b * a.R + c];
    for (int c = threadIdx.x; c < a.G; c += kBlockThreads) base_g[c] += a.part_group[(int64_t)b * a.G + c];
    __syncthreads();

    if (bad) report(a.err, EP_DEVERR_EXPERT_ID);
    if (t >= a.T) return;
    const int w = threadIdx.x / 32;
    const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
    const int64_t* row = a.topk + (int64_t)t * a.K;
#pragma unroll 8
    for (int k = 0; k < a.K; ++k) {
        const int64_t e = row[k];
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
    a.tot_rank = reinterpret_cast<int32_t*>(ws + W.tot_rank);
    a.tot_group = reinterpret_cast<int32_t*>(ws + W.tot_group);
    a.tot_expert = reinterpret_cast<int32_t*>(ws + W.tot_expert);
    a.out = L;

    const size_t lds_count = sizeof(uint32_t) * ((size_t)(s.R + s.G) * kWords + s.E);
    hipLaunchKernelGGL(layout_count_kernel, dim3(W.nb), dim3(kBlockThreads), lds_count, st, a);
    const int cols = s.R + s.G + s.E;
    hipLaunchKernelGGL(layout_reduce_kernel, dim3((cols + kBlockThreads - 1) / kBlockThreads),
                       dim3(kBlockThreads), 0, st, a);
    const size_t lds_assign =
        sizeof(uint32_t) * ((size_t)(s.R + s.G) * kWords + s.R + s.G + kBlockThreads);
    hipLaunchKernelGGL(layout_assign_kernel, dim3(W.nb), dim3(kBlockThreads), lds_assign, st, a);
    return hipGetLastError();
}

}  // namespace ep
