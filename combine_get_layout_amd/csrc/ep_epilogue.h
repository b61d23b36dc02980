// ep_epilogue.h -- the copy epilogue's unpacking of one chunked record into a
// row of the receive arrays, shared by the copy epilogue launch and the fused
// send-and-epilogue launch.
//
// What is computed follows "DeepEP V2 深度深潜：统一接口、SM 估算本质与 TopK
// 复制机制", §3.3 阶段3 (the copy epilogue copies each received row out of its
// source's region into the dense receive rows) on the chunked records of
// "Ascend Send Ordering", 导言 (512 B blocks: 480 B payload + 32 B flag).
#pragma once

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kEpiloguePieceIters = 16;  // wave iterations (2 blocks each) held in VGPRs

struct EpilogueArgs {
    int H, K, RS;
    int64_t cap;
    RecordGeom geom;
    const int32_t* offs;
    const uint8_t* staging;
    uint8_t* rx;
    uint8_t* rfp8;
    float* rscales;
    int32_t* rsrc;
    int32_t* ridx;
    float* rw;
    int64_t rcap;
    uint32_t epoch;
    uint32_t* err;
};

// Record vector q of a row, to the receive arrays' row `row`.
__device__ __forceinline__ void put_vector(const EpilogueArgs& a, int64_t row, int q, u32x4 v) {
    const RecordGeom& g = a.geom;
    if (q < g.q_fp8) {
        if (a.rx) st16_stream(a.rx + row * 2 * a.H + (int64_t)q * 16, v);
    } else if (q < g.q_scales) {
        if (a.rfp8) st16_stream(a.rfp8 + row * a.H + (int64_t)(q - g.q_fp8) * 16, v);
    } else if (q < g.q_idx) {
        const int ns = a.H / 128, i0 = (q - g.q_scales) * 4;
        if (a.rscales)
            for (int m = 0; m < 4; ++m)
                if (i0 + m < ns) a.rscales[row * ns + i0 + m] = __uint_as_float(v[m]);
    } else if (q < g.q_w) {
        const int k0 = (q - g.q_idx) * 4;
        if (a.ridx)
            for (int m = 0; m < 4; ++m)
                if (k0 + m < a.K) a.ridx[row * a.K + k0 + m] = (int32_t)v[m];
    } else if (q < g.q_src) {
        const int k0 = (q - g.q_w) * 4;
        if (a.rw)
            for (int m = 0; m < 4; ++m)
                if (k0 + m < a.K) a.rw[row * a.K + k0 + m] = __uint_as_float(v[m]);
    } else if (q == g.q_src) {
        if (a.rsrc) a.rsrc[row] = (int32_t)v[0];
    }
}

__device__ __forceinline__ bool epilogue_flag_ok(u32x4 f, uint32_t epoch) {
    return f[0] == epoch && f[1] == epoch && f[2] == epoch && f[3] == epoch;
}

// 16-byte vector at byte `off` of a staging row of `stride` bytes. DEV: with
// device scope (cache-policy 16, sc1), for rows written by other workgroups
// of the same launch; otherwise non-temporal (rows written by an earlier
// launch and read once).
template <bool DEV, bool NT = true>
__device__ __forceinline__ u32x4 epilogue_load(const uint8_t* row, int64_t stride, int64_t off) {
    if constexpr (DEV)
        return __builtin_amdgcn_raw_buffer_load_b128(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(row), 0, (int)stride, 0x00020000), (int)off, 0, 16);
    else if constexpr (NT)
        return ld16_stream(row + off);
    else
        return ld16(row + off);
}

// Unpack the chunked record at src_row into row i of the receive arrays (one
// wave): the record's flags must all equal epoch, else nothing is written and
// EP_DEVERR_FLAG is set.
template <bool DEV>
__device__ __forceinline__ void epilogue_row(const EpilogueArgs& a, int64_t i, const uint8_t* src_row) {
    const int lane = lane_id();
    const int nchunks = a.geom.nchunks;
    const int iters = (nchunks + 1) / 2;
    const int64_t stride = a.geom.stride;
    const int c_half = lane >> 5, wv = lane & 31;
    const bool one_piece = iters <= kEpiloguePieceIters;
    u32x4 v[kEpiloguePieceIters];
    bool ok = true;
    if (one_piece) {
        // The whole row at once; lanes past the last block reload it.
#pragma unroll
        for (int it = 0; it < kEpiloguePieceIters; ++it) {
            const int c = min(2 * it + c_half, nchunks - 1);
            v[it] = epilogue_load<DEV>(src_row, stride, (int64_t)c * kChunkBytes + (int64_t)wv * 16);
        }
#pragma unroll
        for (int it = 0; it < kEpiloguePieceIters; ++it) ok &= wv < kChunkPayloadVecs || epilogue_flag_ok(v[it], a.epoch);
    } else {
        for (int f = lane; f < 2 * nchunks; f += kWave)
            ok &= epilogue_flag_ok(  // flags first (plain loads: the blocks are read again below)
                epilogue_load<DEV, false>(src_row, stride, (int64_t)(f >> 1) * kChunkBytes + kChunkPayload + (f & 1) * 16),
                a.epoch);
    }
    if (__ballot(!ok)) {
        if (lane == 0) report(a.err, EP_DEVERR_FLAG);
        return;
    }
    for (int it0 = 0; it0 < iters; it0 += kEpiloguePieceIters) {
        if (!one_piece) {
#pragma unroll
            for (int jj = 0; jj < kEpiloguePieceIters; ++jj) {
                const int c = min(2 * (it0 + jj) + c_half, nchunks - 1);
                v[jj] = epilogue_load<DEV>(src_row, stride, (int64_t)c * kChunkBytes + (int64_t)wv * 16);
            }
        }
#pragma unroll
        for (int jj = 0; jj < kEpiloguePieceIters; ++jj) {
            const int c = 2 * (it0 + jj) + c_half;
            if (it0 + jj < iters && c < nchunks && wv < kChunkPayloadVecs)
                put_vector(a, i, c * kChunkPayloadVecs + wv, v[jj]);
        }
    }
}

}  // namespace
}  // namespace ep
