"""CPU oracle for the expert-parallel MoE dispatch / combine path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the HIP implementation in ``combine_get_layout_amd`` and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, single thread, built with gcc);
this module only builds it, loads it and marshals numpy arrays. Every function
here mirrors one C function; see ``oracle.c`` for the page and section each
follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ERR_EXPERT = 1
ERR_CAPACITY = 2
ERR_FLAG = 4

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fused multiply-add
    contraction other than the explicit fmaf calls)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, u32 = ctypes.c_int, ctypes.c_int64, ctypes.c_uint32
        lib.oracle_layout.argtypes = [i32, i32, i32, i32, i32, P] + [P] * 10 + [P]
        lib.oracle_layout.restype = i32
        lib.oracle_dispatch.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, i64,
                                        P, P, P, P, P, P, P]
        lib.oracle_dispatch.restype = None
        lib.oracle_record_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.oracle_record_bytes.restype = i64
        lib.oracle_chunked_bytes.argtypes = [i64]
        lib.oracle_chunked_bytes.restype = i64
        lib.oracle_pack_record.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P]
        lib.oracle_pack_record.restype = None
        lib.oracle_chunk.argtypes = [P, i64, u32, P]
        lib.oracle_chunk.restype = None
        lib.oracle_unchunk.argtypes = [P, i64, u32, P]
        lib.oracle_unchunk.restype = i32
        lib.oracle_hier_dispatch.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                             P, u32, P, i64, P, i64, i32, P]
        lib.oracle_hier_dispatch.restype = i32
        lib.oracle_unpack_rows.argtypes = [P, i64, i32, i32, i32, i32, i32, u32,
                                           P, P, P, P, P, P]
        lib.oracle_unpack_rows.restype = i64
        lib.oracle_combine.argtypes = [i32, i32, i32, P, P, P, i64, i64, i32, u32, P, P]
        lib.oracle_combine.restype = None
        lib.oracle_partial_row_bytes.argtypes = [i32]
        lib.oracle_partial_row_bytes.restype = i64
        lib.oracle_combine_two_level.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, i64, i64,
                                                 i32, u32, P, i64, i32, P, P]
        lib.oracle_combine_two_level.restype = None
        lib.oracle_source_counts.argtypes = [i32, i32, i32, i32, i32, P, P, P]
        lib.oracle_source_counts.restype = i32
        lib.oracle_source_slots.argtypes = [i32, i32, i32, i32, i32, P, i64, P, P]
        lib.oracle_source_slots.restype = i32
        lib.oracle_source_dispatch.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P,
                                               u32, P, i64, P]
        lib.oracle_source_dispatch.restype = i32
        lib.oracle_copy_epilogue.argtypes = [i32, i32, i32, i32, P, P, i64, i32, i32, i32, u32,
                                             i64, P, P, P, P, P, P, P]
        lib.oracle_copy_epilogue.restype = i32
        lib.oracle_expert_slots.argtypes = [i32, i32, i32, P, P, P]
        lib.oracle_expert_slots.restype = i32
        lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        _lib = lib
    return _lib


def _p(a):
    """Pointer to a C-contiguous numpy array, or NULL for None."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# Layout
# --------------------------------------------------------------------------

def layout(topk_idx: np.ndarray, E: int, R: int, G: int = 1) -> dict:
    """Counts, offsets, masks and slots of [T, K] int64 expert choices."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    out = dict(
        tokens_per_expert=np.zeros(E, np.int32),
        tokens_per_rank=np.zeros(R, np.int32),
        tokens_per_group=np.zeros(G, np.int32),
        expert_offsets=np.zeros(E + 1, np.int32),
        rank_offsets=np.zeros(R + 1, np.int32),
        group_offsets=np.zeros(G + 1, np.int32),
        is_token_in_rank=np.zeros((T, R), np.uint8),
        is_token_in_group=np.zeros((T, G), np.uint8),
        slot=np.zeros((T, K), np.int32),
        group_slot=np.zeros((T, K), np.int32),
    )
    err = np.zeros(1, np.uint32)
    rc = _load().oracle_layout(
        T, K, E, R, G, _p(topk_idx),
        _p(out["tokens_per_expert"]), _p(out["tokens_per_rank"]), _p(out["tokens_per_group"]),
        _p(out["expert_offsets"]), _p(out["rank_offsets"]), _p(out["group_offsets"]),
        _p(out["is_token_in_rank"]), _p(out["is_token_in_group"]),
        _p(out["slot"]), _p(out["group_slot"]), _p(err))
    if rc != 0:
        raise ValueError("oracle_layout: bad shape")
    out["err"] = int(err[0])
    return out


def source_counts(topk_idx, E, R, S) -> dict:
    """Counts exchange of S source ranks: counts [S, R] and the rank-major
    receive offsets [R * S + 1]."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    counts = np.zeros((S, R), np.int32)
    offs = np.zeros(R * S + 1, np.int32)
    if _load().oracle_source_counts(T, K, E, R, S, _p(topk_idx), _p(counts), _p(offs)) != 0:
        raise ValueError("oracle_source_counts: bad arguments")
    return dict(counts=counts, recv_offsets=offs)


def expert_slots(topk_idx, E, expert_offsets) -> np.ndarray:
    """Expand-mode row of every (token, lane): [T, K] int32, -1 if skipped."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    expert_offsets = _c(expert_offsets, np.int32)
    out = np.zeros((T, K), np.int32)
    if _load().oracle_expert_slots(T, K, E, _p(topk_idx), _p(expert_offsets), _p(out)) != 0:
        raise MemoryError("oracle_expert_slots")
    return out


def dispatch_rows(topk_idx, E, rows, n_rows, x=None, x_fp8=None, x_scales=None, topk_w=None):
    """Receive buffers when the token of each (t, k) with rows[t, k] >= 0 is
    written to row rows[t, k] (expand mode: one row per lane). Written from
    the definition with numpy indexing, as the record is the same as in
    direct dispatch."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    rows = np.asarray(rows)
    tt, kk = np.nonzero(rows >= 0)
    dst = rows[tt, kk]
    clean = np.where((topk_idx >= 0) & (topk_idx < E), topk_idx, -1).astype(np.int32)
    out = {}
    if x is not None:
        out["recv_x"] = np.zeros((n_rows, x.shape[1]), np.uint16)
        out["recv_x"][dst] = x[tt]
    if x_fp8 is not None:
        out["recv_fp8"] = np.zeros((n_rows, x_fp8.shape[1]), np.uint8)
        out["recv_fp8"][dst] = x_fp8[tt]
    if x_scales is not None:
        out["recv_scales"] = np.zeros((n_rows, x_scales.shape[1]), np.float32)
        out["recv_scales"][dst] = x_scales[tt]
    out["recv_src"] = np.full(n_rows, -7, np.int32)
    out["recv_src"][dst] = tt
    out["recv_topk_idx"] = np.full((n_rows, K), -7, np.int32)
    out["recv_topk_idx"][dst] = clean[tt]
    if topk_w is not None:
        out["recv_topk_w"] = np.zeros((n_rows, K), np.float32)
        out["recv_topk_w"][dst] = topk_w[tt]
    return out


# --------------------------------------------------------------------------
# Direct dispatch
# --------------------------------------------------------------------------

def dispatch(topk_idx, E, R, rank_offsets, x=None, x_fp8=None, x_scales=None,
             topk_w=None, capacity=None, with_meta=True) -> dict:
    """Receive buffers of the direct dispatch; rows = capacity (default N)."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    x = _c(x, np.uint16)
    x_fp8 = _c(x_fp8, np.uint8)
    x_scales = _c(x_scales, np.float32)
    topk_w = _c(topk_w, np.float32)
    rank_offsets = _c(rank_offsets, np.int32)
    H = x.shape[1] if x is not None else (x_fp8.shape[1] if x_fp8 is not None else
                                           (x_scales.shape[1] * 128 if x_scales is not None else 0))
    N = int(rank_offsets[R])
    cap = N if capacity is None else int(capacity)
    out = dict(
        recv_x=np.zeros((cap, H), np.uint16) if x is not None else None,
        recv_fp8=np.zeros((cap, H), np.uint8) if x_fp8 is not None else None,
        recv_scales=np.zeros((cap, H // 128), np.float32) if x_scales is not None else None,
        recv_src=np.full(cap, -7, np.int32) if with_meta else None,
        recv_topk_idx=np.full((cap, K), -7, np.int32) if with_meta else None,
        recv_topk_w=np.zeros((cap, K), np.float32) if (with_meta and topk_w is not None) else None,
    )
    err = np.zeros(1, np.uint32)
    _load().oracle_dispatch(T, H, K, E, R, _p(topk_idx), _p(topk_w), _p(x), _p(x_fp8),
                            _p(x_scales), _p(rank_offsets), cap,
                            _p(out["recv_x"]), _p(out["recv_fp8"]), _p(out["recv_scales"]),
                            _p(out["recv_src"]), _p(out["recv_topk_idx"]),
                            _p(out["recv_topk_w"]), _p(err))
    out["err"] = int(err[0])
    return out


# --------------------------------------------------------------------------
# Record / chunk codec
# --------------------------------------------------------------------------

def record_bytes(H, K, with_bf16=True, with_fp8=False, with_scales=False) -> int:
    return int(_load().oracle_record_bytes(H, K, int(with_bf16), int(with_fp8), int(with_scales)))


def chunked_bytes(payload_bytes: int) -> int:
    return int(_load().oracle_chunked_bytes(int(payload_bytes)))


def pack_record(t, topk_idx, E, x=None, x_fp8=None, x_scales=None, topk_w=None) -> np.ndarray:
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    x = _c(x, np.uint16)
    x_fp8 = _c(x_fp8, np.uint8)
    x_scales = _c(x_scales, np.float32)
    topk_w = _c(topk_w, np.float32)
    H = x.shape[1] if x is not None else (x_fp8.shape[1] if x_fp8 is not None else 0)
    P = record_bytes(H, K, x is not None, x_fp8 is not None, x_scales is not None)
    rec = np.zeros(P, np.uint8)
    _load().oracle_pack_record(int(t), H, K, E, _p(topk_idx), _p(topk_w), _p(x), _p(x_fp8),
                               _p(x_scales), _p(rec))
    return rec


def chunk(rec: np.ndarray, epoch: int) -> np.ndarray:
    rec = _c(rec, np.uint8)
    out = np.zeros(chunked_bytes(rec.size), np.uint8)
    _load().oracle_chunk(_p(rec), rec.size, int(epoch), _p(out))
    return out


def unchunk(blocks: np.ndarray, payload_bytes: int, epoch: int):
    """Returns (record bytes, flags_ok)."""
    blocks = _c(blocks, np.uint8)
    rec = np.zeros(int(payload_bytes), np.uint8)
    bad = _load().oracle_unchunk(_p(blocks), int(payload_bytes), int(epoch), _p(rec))
    return rec, bad == 0


# --------------------------------------------------------------------------
# Two-level dispatch
# --------------------------------------------------------------------------

def hier_dispatch(topk_idx, E, R, G, slot, group_offsets, epoch, x=None, x_fp8=None,
                  x_scales=None, topk_w=None, group_cap=None, peer_cap=None, steps=3,
                  group_buf=None, peer_buf=None) -> dict:
    """Chunked group-region and scale-up-region buffers of the two-level
    dispatch (uint8 arrays [rows, stride]). steps: 1 = scale-out write only,
    2 = forward only (from the given group_buf), 3 = both."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    x = _c(x, np.uint16)
    x_fp8 = _c(x_fp8, np.uint8)
    x_scales = _c(x_scales, np.float32)
    topk_w = _c(topk_w, np.float32)
    slot = _c(slot, np.int32)
    group_offsets = _c(group_offsets, np.int32)
    H = x.shape[1] if x is not None else (x_fp8.shape[1] if x_fp8 is not None else 0)
    P = record_bytes(H, K, x is not None, x_fp8 is not None, x_scales is not None)
    stride = chunked_bytes(P)
    gcap = int(group_offsets[G]) if group_cap is None else int(group_cap)
    pcap = (int(slot.max()) + 1 if slot.size else 0) if peer_cap is None else int(peer_cap)
    if group_buf is None:
        group_buf = np.zeros((gcap, stride), np.uint8)
    if peer_buf is None:
        peer_buf = np.zeros((pcap, stride), np.uint8)
    assert group_buf.shape == (gcap, stride) and peer_buf.shape == (pcap, stride)
    assert group_buf.flags["C_CONTIGUOUS"] and peer_buf.flags["C_CONTIGUOUS"]
    err = np.zeros(1, np.uint32)
    rc = _load().oracle_hier_dispatch(T, H, K, E, R, G, _p(topk_idx), _p(topk_w), _p(x),
                                      _p(x_fp8), _p(x_scales), _p(slot),
                                      _p(group_offsets), int(epoch), _p(group_buf), gcap,
                                      _p(peer_buf), pcap, int(steps), _p(err))
    if rc != 0:
        raise MemoryError("oracle_hier_dispatch")
    return dict(group_buf=group_buf, peer_buf=peer_buf, record_bytes=P, stride=stride,
                err=int(err[0]))


def unpack_rows(buf, H, K, epoch, with_bf16=True, with_fp8=False, with_scales=False) -> dict:
    buf = _c(buf, np.uint8)
    rows = buf.shape[0]
    out = dict(
        recv_x=np.zeros((rows, H), np.uint16) if with_bf16 else None,
        recv_fp8=np.zeros((rows, H), np.uint8) if with_fp8 else None,
        recv_scales=np.zeros((rows, H // 128), np.float32) if with_scales else None,
        recv_src=np.zeros(rows, np.int32),
        recv_topk_idx=np.zeros((rows, K), np.int32),
        recv_topk_w=np.zeros((rows, K), np.float32),
    )
    bad = _load().oracle_unpack_rows(_p(buf), rows, H, K, int(with_bf16), int(with_fp8),
                                     int(with_scales), int(epoch), _p(out["recv_x"]),
                                     _p(out["recv_fp8"]), _p(out["recv_scales"]),
                                     _p(out["recv_src"]), _p(out["recv_topk_idx"]),
                                     _p(out["recv_topk_w"]))
    out["bad_rows"] = int(bad)
    return out


# --------------------------------------------------------------------------
# Several source ranks: send into per-source regions, copy epilogue
# --------------------------------------------------------------------------

def source_slots(topk_idx, E, R, S, cap) -> dict:
    """Staging row [T, K] of every lane (-1 if skipped) and the error bits."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    out = np.zeros((T, K), np.int32)
    err = np.zeros(1, np.uint32)
    if _load().oracle_source_slots(T, K, E, R, S, _p(topk_idx), int(cap), _p(out), _p(err)) != 0:
        raise ValueError("oracle_source_slots: bad arguments")
    return dict(src_slot=out, err=int(err[0]))


def source_dispatch(topk_idx, E, R, S, cap, epoch, x=None, x_fp8=None, x_scales=None,
                    topk_w=None) -> dict:
    """Staging buffer [R * S * cap, stride] (uint8, zero where not written)
    after every source rank sent its tokens into its regions."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    x = _c(x, np.uint16)
    x_fp8 = _c(x_fp8, np.uint8)
    x_scales = _c(x_scales, np.float32)
    topk_w = _c(topk_w, np.float32)
    H = x.shape[1] if x is not None else x_fp8.shape[1]
    P = record_bytes(H, K, x is not None, x_fp8 is not None, x_scales is not None)
    stride = chunked_bytes(P)
    staging = np.zeros((R * S * cap, stride), np.uint8)
    err = np.zeros(1, np.uint32)
    rc = _load().oracle_source_dispatch(T, H, K, E, R, S, _p(topk_idx), _p(topk_w), _p(x),
                                        _p(x_fp8), _p(x_scales), int(epoch), _p(staging),
                                        int(cap), _p(err))
    if rc != 0:
        raise ValueError("oracle_source_dispatch: bad arguments")
    return dict(staging=staging, stride=stride, err=int(err[0]))


def copy_epilogue(recv_offsets, staging, H, K, R, S, cap, epoch, with_bf16=True,
                  with_fp8=False, with_scales=False, recv_cap=None) -> dict:
    """Dense receive arrays (rows = recv_cap, default N) filled from the
    staging regions; rows not written keep -7 (ids, src) or 0."""
    recv_offsets = _c(recv_offsets, np.int32)
    staging = _c(staging, np.uint8)
    N = int(recv_offsets[R * S])
    rows = N if recv_cap is None else int(recv_cap)
    out = dict(
        recv_x=np.zeros((rows, H), np.uint16) if with_bf16 else None,
        recv_fp8=np.zeros((rows, H), np.uint8) if with_fp8 else None,
        recv_scales=np.zeros((rows, H // 128), np.float32) if with_scales else None,
        recv_src=np.full(rows, -7, np.int32),
        recv_topk_idx=np.full((rows, K), -7, np.int32),
        recv_topk_w=np.zeros((rows, K), np.float32),
    )
    err = np.zeros(1, np.uint32)
    rc = _load().oracle_copy_epilogue(H, K, R, S, _p(recv_offsets), _p(staging), int(cap),
                                      int(with_bf16), int(with_fp8), int(with_scales), int(epoch),
                                      rows, _p(out["recv_x"]), _p(out["recv_fp8"]),
                                      _p(out["recv_scales"]), _p(out["recv_src"]),
                                      _p(out["recv_topk_idx"]), _p(out["recv_topk_w"]), _p(err))
    if rc != 0:
        raise ValueError("oracle_copy_epilogue: bad arguments")
    out["err"] = int(err[0])
    return out


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------

def combine(slot, topk_w, y, H, chunked=False, epoch=0, row_stride=None) -> dict:
    """Weighted combine of rows of y (uint16 [rows, H] plain, or uint8
    [rows, stride] chunked) back into token order: returns out [T, H] bf16
    bits and the error bits."""
    slot = _c(slot, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, K = slot.shape
    y = np.ascontiguousarray(y)
    rows = y.shape[0]
    stride = int(row_stride) if row_stride is not None else (y.nbytes // rows if rows else 2 * H)
    out = np.zeros((T, H), np.uint16)
    err = np.zeros(1, np.uint32)
    _load().oracle_combine(T, H, K, _p(slot), _p(topk_w), _p(y), rows, stride, int(bool(chunked)),
                           int(epoch), _p(out), _p(err))
    return dict(out=out, err=int(err[0]))


def partial_row_bytes(H: int) -> int:
    return int(_load().oracle_partial_row_bytes(int(H)))


def combine_two_level(topk_idx, E, R, G, slot, group_slot, topk_w, y, H, group_cap, epoch,
                      chunked=False, row_stride=None, steps=3, group_buf=None) -> dict:
    """Two-level combine: partial rows per (token, group) in group_buf (uint8
    [group_cap, partial stride]) and the final out [T, H] bf16 bits."""
    topk_idx = _c(topk_idx, np.int64)
    slot = _c(slot, np.int32)
    group_slot = _c(group_slot, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, K = slot.shape
    y = np.ascontiguousarray(y)
    rows = y.shape[0]
    stride = int(row_stride) if row_stride is not None else (y.nbytes // rows if rows else 2 * H)
    pstride = partial_row_bytes(H)
    if group_buf is None:
        group_buf = np.zeros((int(group_cap), pstride), np.uint8)
    assert group_buf.shape == (int(group_cap), pstride) and group_buf.flags["C_CONTIGUOUS"]
    out = np.zeros((T, H), np.uint16)
    err = np.zeros(1, np.uint32)
    _load().oracle_combine_two_level(T, H, K, E, R, G, _p(topk_idx), _p(slot), _p(group_slot),
                                     _p(topk_w), _p(y), rows, stride, int(bool(chunked)), int(epoch),
                                     _p(group_buf), int(group_cap), int(steps), _p(out), _p(err))
    return dict(out=out, group_buf=group_buf, err=int(err[0]))


def f32_to_bf16(f: float) -> int:
    return int(_load().oracle_f32_to_bf16(float(f)))


def bf16_to_f32(h: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(h)))
