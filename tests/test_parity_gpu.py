"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Bar: layout, masks, offsets, slots and every permuted / chunked byte are
bit-exact; combine outputs are within max |diff| <= 1e-2 and relative L2
<= 4e-3 of the oracle (and, because both sides use one fp32 fused
multiply-add per top-k lane in ascending order, are checked bit-exact too).
All five workloads run at full size; the edge cases cover empty and ragged
inputs, invalid ids, duplicates, capacity overflow, stale and corrupted flags.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_get_layout_amd import ep

pytestmark = pytest.mark.gpu

ATOL, RTOL_L2 = 1e-2, 4e-3


@pytest.fixture(scope="module", autouse=True)
def _ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()
    oracle.build(force=False)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # move 16-bit patterns as int16, keep the uint16 view
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.uint16)
    return torch.from_numpy(a).cuda()


def host(t):
    if t.dtype == torch.uint16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def poison(t, byte=0xAB):
    t.view(torch.uint8).fill_(byte)
    return t


def run_layout(w, topk, masks=True, groups=True):
    shape = ep.make_shape(topk.shape[0], w.H, topk.shape[1], w.E, w.R, w.G)
    L = ep.alloc_layout(shape, masks=masks, groups=groups)
    for t in L.values():
        poison(t)
    ws = ep.alloc_workspace(shape)
    tk = dev(topk)
    ep.ep_get_layout(shape, tk, L, ws)
    torch.cuda.synchronize()
    return shape, L, ws, tk


def check_layout(L, O, T):
    for k in ("tokens_per_expert", "tokens_per_rank", "tokens_per_group", "expert_offsets",
              "rank_offsets", "group_offsets", "is_token_in_rank", "is_token_in_group",
              "slot", "group_slot"):
        if k in L:
            np.testing.assert_array_equal(host(L[k]).reshape(O[k].shape), O[k], err_msg=k)


def combine_close(out_bits, ref_bits):
    o = synth.bf16_to_float(out_bits).astype(np.float64)
    r = synth.bf16_to_float(ref_bits).astype(np.float64)
    d = np.abs(o - r)
    assert d.max(initial=0.0) <= ATOL
    nr = np.linalg.norm(r)
    assert np.linalg.norm(o - r) <= RTOL_L2 * max(nr, 1e-30)


WORKLOADS = ["tiny", "ep32", "ep256", "zipf", "hier8x8"]


# --------------------------------------------------------------------------
# Layout
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", WORKLOADS)
def test_layout_full_size(name):
    w = synth.workload(name)
    inp = synth.make_inputs(w, with_x=False)
    shape, L, ws, _ = run_layout(w, inp["topk_idx"])
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    check_layout(L, O, w.T)
    assert ep.ep_check_errors(ws) == 0


LAYOUT_EDGES = [
    # (T, K, E, R, G, kind)
    (0, 8, 256, 32, 4, "uniform"),
    (1, 8, 256, 32, 4, "uniform"),
    (257, 3, 12, 6, 3, "random"),      # ragged block, K not a power of two
    (1001, 20, 64, 16, 4, "random"),   # K above 16, duplicates and -1
    (300, 1, 16, 16, 1, "random"),     # top-1
    (513, 4, 16, 1, 1, "random"),      # one rank
    (640, 8, 4096, 1024, 256, "uniform"),  # largest supported R, G, E
    (200, 4, 16, 4, 2, "one_rank"),    # all tokens to one rank, empty ranks
    (700, 64, 128, 16, 4, "random"),   # largest supported K
    (70000, 2, 64, 8, 2, "uniform"),   # 274 layout workgroups (many row batches)
]


def _edge_topk(T, K, E, R, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        return synth.topk_uniform(rng, T, E, K)
    if kind == "one_rank":
        epr = E // R
        return rng.integers(epr, 2 * epr, size=(T, K)).astype(np.int64)
    return rng.integers(-1, E, size=(T, K)).astype(np.int64)


@pytest.mark.parametrize("case", LAYOUT_EDGES, ids=[f"T{c[0]}K{c[1]}E{c[2]}R{c[3]}G{c[4]}{c[5]}"
                                                    for c in LAYOUT_EDGES])
def test_layout_edges(case):
    T, K, E, R, G, kind = case
    w = synth.Workload("edge", T, 128, E, R, G, K, "uniform")
    topk = _edge_topk(T, K, E, R, kind, seed=T + K)
    shape, L, ws, _ = run_layout(w, topk)
    O = oracle.layout(topk, E, R, G)
    check_layout(L, O, T)
    assert ep.ep_check_errors(ws) == 0


def test_layout_invalid_ids_flagged():
    w = synth.Workload("bad", 300, 128, 32, 8, 2, 4, "uniform")
    rng = np.random.default_rng(5)
    topk = rng.integers(-1, 32, size=(300, 4)).astype(np.int64)
    topk[3, 1], topk[70, 0], topk[299, 3] = 32, -2, 1 << 40
    shape, L, ws, _ = run_layout(w, topk)
    O = oracle.layout(topk, w.E, w.R, w.G)
    assert O["err"] == oracle.ERR_EXPERT
    check_layout(L, O, w.T)
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_EXPERT_ID
    # the next pass starts with a clean error word
    ep.ep_get_layout(shape, dev(np.maximum(topk % 32, 0)), L, ws)
    assert ep.ep_check_errors(ws) == 0


# --------------------------------------------------------------------------
# Dispatch
# --------------------------------------------------------------------------

def run_dispatch(w, inp, shape, L, ws, tk, capacity=None, fp8=False, meta=True):
    N = int(host(L["rank_offsets"])[-1])
    cap = N if capacity is None else capacity
    tokens = dict(x=dev(inp["x"]), topk_idx=tk, topk_weights=dev(inp["topk_w"]))
    if fp8:
        tokens["x_fp8"] = dev(inp["x_fp8"])
        tokens["x_scales"] = dev(inp["x_scales"])
    recv = ep.alloc_recv(shape, max(cap, 1), fp8=fp8, scales=fp8, meta=meta)
    for t in recv.values():
        poison(t)
    ep.ep_dispatch(shape, L, tokens, recv, cap, ws)
    torch.cuda.synchronize()
    return recv, N, cap


def check_dispatch(recv, D, rows):
    pairs = [("x", "recv_x"), ("x_fp8", "recv_fp8"), ("x_scales", "recv_scales"),
             ("src_idx", "recv_src"), ("topk_idx", "recv_topk_idx"),
             ("topk_weights", "recv_topk_w")]
    for g, o in pairs:
        if g in recv and D.get(o) is not None:
            a = host(recv[g])[:rows]
            b = D[o][:rows]
            np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8), err_msg=g)


@pytest.mark.parametrize("name,fp8", [("tiny", False), ("ep32", False), ("ep32", True),
                                      ("ep256", False), ("zipf", False), ("hier8x8", False)])
def test_dispatch_full_size(name, fp8):
    w = synth.workload(name)
    inp = synth.make_inputs(w, with_fp8=fp8)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    recv, N, _ = run_dispatch(w, inp, shape, L, ws, tk, fp8=fp8)
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    D = oracle.dispatch(inp["topk_idx"], w.E, w.R, O["rank_offsets"], x=inp["x"],
                        x_fp8=inp.get("x_fp8"), x_scales=inp.get("x_scales"),
                        topk_w=inp["topk_w"])
    assert D["recv_x"].shape[0] == N
    check_dispatch(recv, D, N)
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("T,H,K,E,R", [(1, 8, 1, 4, 2), (3, 1032, 3, 12, 6), (1001, 4096, 20, 64, 16),
                                       (257, 16, 8, 64, 64), (500, 384, 4, 16, 1),
                                       (300, 256, 64, 256, 64),
                                       # column slices rounded to 128 B: the last one is shorter
                                       (200, 7232, 8, 64, 16), (130, 4104, 5, 40, 8),
                                       # long rows: 8 and 16 vectors per lane, two passes per slice
                                       (40, 16384, 8, 64, 16), (12, 65536, 4, 32, 8)])
def test_dispatch_edges(T, H, K, E, R):
    w = synth.Workload("edge", T, H, E, R, 1, K, "uniform")
    rng = np.random.default_rng(T * 7 + H)
    inp = dict(x=rng.integers(0, 65536, size=(T, H)).astype(np.uint16),
               topk_idx=rng.integers(-1, E, size=(T, K)).astype(np.int64),
               topk_w=rng.standard_normal((T, K)).astype(np.float32))
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    recv, N, _ = run_dispatch(w, inp, shape, L, ws, tk)
    O = oracle.layout(inp["topk_idx"], E, R, 1)
    D = oracle.dispatch(inp["topk_idx"], E, R, O["rank_offsets"], x=inp["x"], topk_w=inp["topk_w"])
    check_dispatch(recv, D, N)


@pytest.mark.parametrize("T,H,K,E,R,segs", [
    # rows of at most 32 vectors and K <= 8: 2, 4 or 8 tokens per wave
    (1000, 128, 8, 64, 16, "x+fp8+scales"), (77, 256, 3, 24, 6, "x+fp8+scales"),
    (999, 64, 6, 32, 32, "x"), (5, 32, 8, 8, 8, "x"), (130, 8, 1, 4, 4, "x"),
    (333, 512, 5, 40, 10, "fp8"), (257, 256, 8, 16, 2, "scales")])
def test_dispatch_narrow_rows(T, H, K, E, R, segs):
    """The several-tokens-per-wave dispatch: skipped (-1) and repeated lanes,
    every payload piece on its own, rows compared byte for byte."""
    w = synth.Workload("narrow", T, H, E, R, 1, K, "uniform")
    rng = np.random.default_rng(T * 31 + H * 7 + K)
    x = rng.integers(0, 65536, size=(T, H)).astype(np.uint16)
    topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    topk[::5, -1] = topk[::5, 0]  # repeated experts in some tokens
    inp = dict(x=x, topk_idx=topk, topk_w=rng.standard_normal((T, K)).astype(np.float32))
    want_x, want_fp8, want_sc = "x" in segs.split("+"), "fp8" in segs, "scales" in segs
    if want_fp8 or want_sc:
        inp["x_fp8"] = rng.integers(0, 256, size=(T, H)).astype(np.uint8)
        inp["x_scales"] = rng.standard_normal((T, max(H // 128, 1))).astype(np.float32)[:, :H // 128]
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    N = int(host(L["rank_offsets"])[-1])
    tokens = dict(topk_idx=tk, topk_weights=dev(inp["topk_w"]))
    if want_x:
        tokens["x"] = dev(inp["x"])
    if want_fp8:
        tokens["x_fp8"] = dev(inp["x_fp8"])
    if want_sc:
        tokens["x_scales"] = dev(np.ascontiguousarray(inp["x_scales"]))
    recv = ep.alloc_recv(shape, N, x=want_x, fp8=want_fp8, scales=want_sc, meta=True)
    for t in recv.values():
        poison(t)
    ep.ep_dispatch(shape, L, tokens, recv, N, ws)
    torch.cuda.synchronize()
    O = oracle.layout(inp["topk_idx"], E, R, 1)
    D = oracle.dispatch(inp["topk_idx"], E, R, O["rank_offsets"], x=inp["x"] if want_x else None,
                        x_fp8=inp["x_fp8"] if want_fp8 else None,
                        x_scales=np.ascontiguousarray(inp["x_scales"]) if want_sc else None,
                        topk_w=inp["topk_w"])
    check_dispatch(recv, D, N)
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("segs", ["fp8+scales", "x", "scales", "meta", "fp8"])
def test_dispatch_segment_subsets(segs):
    """Every payload piece is optional on its own; the metadata too."""
    w = synth.Workload("segs", 700, 1024, 48, 12, 1, 6, "uniform")
    inp = synth.make_inputs(w, with_fp8=True)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    N = int(host(L["rank_offsets"])[-1])
    want_x, want_fp8 = segs == "x", "fp8" in segs
    want_sc, meta = "scales" in segs, segs in ("fp8+scales", "scales", "meta")
    tokens = dict(topk_idx=tk, topk_weights=dev(inp["topk_w"]))
    if want_x:
        tokens["x"] = dev(inp["x"])
    if want_fp8:
        tokens["x_fp8"] = dev(inp["x_fp8"])
    if want_sc:
        tokens["x_scales"] = dev(inp["x_scales"])
    recv = ep.alloc_recv(shape, N, x=want_x, fp8=want_fp8, scales=want_sc, meta=meta)
    for t in recv.values():
        poison(t)
    ep.ep_dispatch(shape, L, tokens, recv, N, ws)
    O = oracle.layout(inp["topk_idx"], w.E, w.R, 1)
    D = oracle.dispatch(inp["topk_idx"], w.E, w.R, O["rank_offsets"],
                        x=inp["x"] if want_x else None, x_fp8=inp["x_fp8"] if want_fp8 else None,
                        x_scales=inp["x_scales"] if want_sc else None, topk_w=inp["topk_w"],
                        with_meta=meta)
    assert set(recv) == {k for k, o in [("x", "recv_x"), ("x_fp8", "recv_fp8"), ("x_scales", "recv_scales"),
                                         ("src_idx", "recv_src"), ("topk_idx", "recv_topk_idx"),
                                         ("topk_weights", "recv_topk_w")] if D.get(o) is not None}
    check_dispatch(recv, D, N)
    assert ep.ep_check_errors(ws) == 0


def test_dispatch_capacity_overflow():
    w = synth.workload("tiny")
    inp = synth.make_inputs(w)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    N = int(host(L["rank_offsets"])[-1])
    recv, _, cap = run_dispatch(w, inp, shape, L, ws, tk, capacity=N - 17)
    O = oracle.layout(inp["topk_idx"], w.E, w.R)
    D = oracle.dispatch(inp["topk_idx"], w.E, w.R, O["rank_offsets"], x=inp["x"],
                        topk_w=inp["topk_w"], capacity=N - 17)
    assert D["err"] == oracle.ERR_CAPACITY
    check_dispatch(recv, D, cap)
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_CAPACITY


def test_dispatch_zero_tokens():
    w = synth.Workload("empty", 0, 256, 16, 4, 1, 2, "uniform")
    topk = np.zeros((0, 2), np.int64)
    shape, L, ws, tk = run_layout(w, topk)
    assert (host(L["rank_offsets"]) == 0).all()
    recv = ep.alloc_recv(shape, 1, meta=False)
    ep.ep_dispatch(shape, L, dict(x=torch.empty((0, 256), dtype=torch.uint16, device="cuda"),
                                  topk_idx=tk), recv, 0, ws)
    out = torch.empty((0, 256), dtype=torch.uint16, device="cuda")
    ep.ep_combine(shape, L, recv["x"], 0, 512, ep.EP_FMT_PLAIN, 0,
                  torch.empty((0, 2), device="cuda"), out, ws)
    assert ep.ep_check_errors(ws) == 0


def test_zero_tokens_every_other_path():
    """No tokens through the two-level dispatch (two launches and fused), the
    chunked and two-level combines and the expand rows: every call succeeds,
    the offsets are all zero, no error bit is set and one-row sentinel
    buffers handed in with zero capacity are left as they were."""
    T, H, K, E, R, G = 0, 512, 4, 32, 8, 4
    shape = ep.make_shape(T, H, K, E, R, G)
    L = ep.alloc_layout(shape, masks=True, groups=True, expand=True)
    ws = ep.alloc_workspace(shape)
    tk = dict(x=torch.empty((0, H), dtype=torch.uint16, device="cuda"),
              topk_idx=torch.empty((0, K), dtype=torch.int64, device="cuda"),
              topk_weights=torch.empty((0, K), dtype=torch.float32, device="cuda"))
    ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
    torch.cuda.synchronize()
    for k in ("rank_offsets", "group_offsets", "expert_offsets", "tokens_per_rank",
              "tokens_per_group", "tokens_per_expert"):
        assert (host(L[k]) == 0).all(), k
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    gb = poison(torch.empty((1, stride), dtype=torch.uint8, device="cuda"), 0xA5)
    pb = poison(torch.empty((1, stride), dtype=torch.uint8, device="cuda"), 0xA5)
    ep.ep_hierarchical_dispatch(shape, L, tk, 3, 3, gb, 0, pb, 0, ws)
    ep.ep_hierarchical_dispatch_fused(shape, L, tk, 4, gb, 0, pb, 0, ws)
    out = poison(torch.empty((1, H), dtype=torch.uint16, device="cuda"), 0xA5)
    ep.ep_combine(shape, L, pb, 0, stride, ep.EP_FMT_CHUNKED, 4, tk["topk_weights"], out, ws)
    part = poison(torch.empty((1, ep.ep_partial_row_bytes(shape)), dtype=torch.uint8, device="cuda"), 0xA5)
    ep.ep_combine_two_level(shape, L, tk["topk_idx"], pb, 0, stride, ep.EP_FMT_CHUNKED, 4,
                            tk["topk_weights"], part, 0, 3, out, ws)
    recv = ep.alloc_recv(shape, 1)
    for t in recv.values():
        poison(t, 0xA5)
    ep.ep_dispatch_expand(shape, L, tk, recv, 0, ws)
    ep.ep_combine_expand(shape, L, recv["x"], 0, 2 * H, ep.EP_FMT_PLAIN, 0, tk["topk_weights"], out, ws)
    torch.cuda.synchronize()
    for name, t in [("group_buf", gb), ("peer_buf", pb), ("out", out), ("partials", part)] + \
            [("recv " + k, v) for k, v in recv.items()]:
        assert (t.view(torch.uint8) == 0xA5).all(), name
    assert ep.ep_check_errors(ws) == 0


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ep32", "ep256", "zipf"])
def test_combine_full_size(name):
    """Combine of stand-in expert outputs (random bf16 rows) and, for the
    identity expert, of the dispatched rows (round trip back to x)."""
    w = synth.workload(name)
    inp = synth.make_inputs(w)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    N = int(host(L["rank_offsets"])[-1])
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    y = synth.random_bf16_rows(N, w.H, seed=99)
    yd = dev(y)
    wd = dev(inp["topk_w"])
    out = poison(torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda"))
    ep.ep_combine(shape, L, yd, N, 2 * w.H, ep.EP_FMT_PLAIN, 0, wd, out, ws)
    C = oracle.combine(O["slot"], inp["topk_w"], y, w.H)
    got = host(out)
    combine_close(got, C["out"])
    np.testing.assert_array_equal(got, C["out"])
    assert ep.ep_check_errors(ws) == 0
    # round trip: dispatch -> identity expert -> combine reproduces x
    recv, _, _ = run_dispatch(w, inp, shape, L, ws, tk, meta=False)
    ep.ep_combine(shape, L, recv["x"], N, 2 * w.H, ep.EP_FMT_PLAIN, 0, wd, out, ws)
    combine_close(host(out), inp["x"])


@pytest.mark.parametrize("T,H,K", [(1, 8, 1), (77, 1032, 3), (300, 264, 2), (129, 512, 5),
                                   (64, 2048, 16), (33, 128, 24), (40, 512, 64),
                                   (40, 16384, 8), (12, 65536, 4),
                                   # narrow rows, several tokens per wave
                                   (77, 128, 8), (1001, 64, 3), (5, 8, 8), (333, 256, 8), (65, 24, 7)])
def test_combine_edges(T, H, K):
    rng = np.random.default_rng(T + H + K)
    rows = 3 * T + 1
    slot = rng.integers(-1, rows, size=(T, K)).astype(np.int32)
    if K > 1:
        slot[::3, 1] = slot[::3, 0]          # repeated rows
    slot[0] = -1                              # no usable lane -> zeros
    w = rng.standard_normal((T, K)).astype(np.float32)
    y = synth.random_bf16_rows(rows, H, seed=T)
    shape = ep.make_shape(T, H, K, 4, 2, 1)
    ws = ep.alloc_workspace(shape)
    L = dict(slot=dev(slot))
    out = poison(torch.empty((T, H), dtype=torch.uint16, device="cuda"))
    ep.ep_clear_errors(ws)
    ep.ep_combine(shape, L, dev(y), rows, 2 * H, ep.EP_FMT_PLAIN, 0, dev(w), out, ws)
    C = oracle.combine(slot, w, y, H)
    np.testing.assert_array_equal(host(out), C["out"])
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("H", [264, 256, 40])
def test_combine_special_values(H):
    """bf16 rows and fp32 weights holding +-0, +-Inf, NaN with several
    payloads, subnormals, the largest finite values and products that
    overflow: the GPU's fused multiply-adds (subnormals kept, no flush to
    zero) and its bf16 rounding (NaN -> 0x7FC0) match the oracle bit for bit
    (H = 256 and 40: the narrow-row kernel, several tokens per wave)."""
    rng = np.random.default_rng(8)
    T, K, rows = 96, 6, 200
    specials16 = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x0001, 0x8001,
                           0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80], np.uint16)
    y = synth.random_bf16_rows(rows, H, seed=9)
    pick = rng.random((rows, H)) < 0.05
    y[pick] = rng.choice(specials16, size=int(pick.sum()))
    # rows 0-49: bf16 subnormals only (sums of them stay subnormal or become
    # the smallest normals)
    y[:50] = rng.integers(1, 0x80, size=(50, H)).astype(np.uint16) | \
        (rng.integers(0, 2, size=(50, H)).astype(np.uint16) << 15)
    specials32 = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1e-40, 3.0e38, -3.0e38,
                           1.0, 0.5], np.float32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    pickw = rng.random((T, K)) < 0.1
    w[pickw] = rng.choice(specials32, size=int(pickw.sum()))
    slot = rng.integers(-1, rows, size=(T, K)).astype(np.int32)
    slot[: T // 2] = rng.integers(0, 50, size=(T // 2, K))  # half the tokens read only subnormal rows
    shape = ep.make_shape(T, H, K, 4, 2, 1)
    ws = ep.alloc_workspace(shape)
    out = poison(torch.empty((T, H), dtype=torch.uint16, device="cuda"))
    ep.ep_clear_errors(ws)
    ep.ep_combine(shape, dict(slot=dev(slot)), dev(y), rows, 2 * H, ep.EP_FMT_PLAIN, 0, dev(w), out, ws)
    C = oracle.combine(slot, w, y, H)
    np.testing.assert_array_equal(host(out), C["out"])
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("pad", [8, 64, 1000])
def test_combine_padded_row_stride(pad):
    """Expert outputs in rows wider than the hidden size (stride > 2H bytes)."""
    T, H, K = 333, 2048, 8
    rng = np.random.default_rng(pad)
    rows = 2 * T
    slot = rng.integers(-1, rows, size=(T, K)).astype(np.int32)
    slot[::5, 3] = slot[::5, 1]
    w = rng.standard_normal((T, K)).astype(np.float32)
    y_wide = synth.random_bf16_rows(rows, H + pad, seed=pad)
    shape = ep.make_shape(T, H, K, 4, 2, 1)
    ws = ep.alloc_workspace(shape)
    out = poison(torch.empty((T, H), dtype=torch.uint16, device="cuda"))
    ep.ep_clear_errors(ws)
    ep.ep_combine(shape, dict(slot=dev(slot)), dev(y_wide), rows, 2 * (H + pad), ep.EP_FMT_PLAIN, 0,
                  dev(w), out, ws)
    C = oracle.combine(slot, w, np.ascontiguousarray(y_wide[:, :H]), H)
    np.testing.assert_array_equal(host(out), C["out"])
    assert ep.ep_check_errors(ws) == 0


def test_combine_rows_out_of_range():
    T, H, K, rows = 50, 256, 4, 40
    rng = np.random.default_rng(8)
    slot = rng.integers(-1, 60, size=(T, K)).astype(np.int32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    y = synth.random_bf16_rows(64, H, seed=3)
    shape = ep.make_shape(T, H, K, 4, 2, 1)
    ws = ep.alloc_workspace(shape)
    out = torch.empty((T, H), dtype=torch.uint16, device="cuda")
    ep.ep_clear_errors(ws)
    ep.ep_combine(shape, dict(slot=dev(slot)), dev(y), rows, 2 * H, ep.EP_FMT_PLAIN, 0, dev(w), out, ws)
    C = oracle.combine(slot, w, y[:rows], H)
    assert C["err"] == oracle.ERR_CAPACITY
    np.testing.assert_array_equal(host(out), C["out"])
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_CAPACITY


# --------------------------------------------------------------------------
# Two-level dispatch with 512 B data-as-flag chunks
# --------------------------------------------------------------------------

def run_hier(w, inp, shape, L, ws, tk, epoch, steps=3, group_buf=None, peer_buf=None, fp8=False):
    seg = ep.EP_SEG_BF16 | ((ep.EP_SEG_FP8 | ep.EP_SEG_SCALES) if fp8 else 0)
    stride = ep.ep_chunked_record_bytes(shape, seg)
    G_rows = int(host(L["group_offsets"])[-1])
    N = int(host(L["rank_offsets"])[-1])
    if group_buf is None:
        group_buf = torch.zeros((max(G_rows, 1), stride), dtype=torch.uint8, device="cuda")
    if peer_buf is None:
        peer_buf = torch.zeros((max(N, 1), stride), dtype=torch.uint8, device="cuda")
    tokens = dict(x=dev(inp["x"]), topk_idx=tk, topk_weights=dev(inp["topk_w"]))
    if fp8:
        tokens["x_fp8"] = dev(inp["x_fp8"])
        tokens["x_scales"] = dev(inp["x_scales"])
    ep.ep_hierarchical_dispatch(shape, L, tokens, epoch, steps, group_buf, G_rows, peer_buf, N, ws)
    torch.cuda.synchronize()
    return group_buf, peer_buf, G_rows, N, stride


@pytest.mark.parametrize("name,fp8", [("hier8x8", False), ("small", True), ("small", False),
                                      ("big", True)])
def test_hierarchical_full(name, fp8):
    """("big", True): a 21.8 KB record of 46 blocks, more than one piece of
    wave-iterations in both steps."""
    if name == "small":
        w = synth.Workload("small", 1500, 1024, 64, 16, 4, 6, "uniform")
    elif name == "big":
        w = synth.Workload("big", 300, 7168, 64, 16, 4, 8, "uniform")
    else:
        w = synth.workload(name)
    inp = synth.make_inputs(w, with_fp8=fp8)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    epoch = 5
    gb, pb, G_rows, N, stride = run_hier(w, inp, shape, L, ws, tk, epoch, fp8=fp8)
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    Hd = oracle.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], epoch,
                              x=inp["x"], x_fp8=inp.get("x_fp8"), x_scales=inp.get("x_scales"),
                              topk_w=inp["topk_w"])
    assert Hd["stride"] == stride and Hd["err"] == 0
    np.testing.assert_array_equal(host(gb)[:G_rows], Hd["group_buf"])
    np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])
    assert ep.ep_check_errors(ws) == 0
    # combine straight from the chunked scale-up rows
    out = poison(torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda"))
    ep.ep_combine(shape, L, pb, N, stride, ep.EP_FMT_CHUNKED, epoch, dev(inp["topk_w"]), out, ws)
    C = oracle.combine(O["slot"], inp["topk_w"], Hd["peer_buf"], w.H, chunked=True, epoch=epoch)
    assert C["err"] == 0
    got = host(out)
    np.testing.assert_array_equal(got, C["out"])
    combine_close(got, inp["x"])
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("T,H,K,E,R,G,ids", [
    (257, 264, 3, 24, 8, 8, "uniform"),     # one peer per group (G = R)
    (300, 512, 4, 32, 8, 1, "uniform"),     # one group holding every rank
    (129, 1032, 12, 48, 16, 4, "uniform"),  # K > 8, hidden row not a whole number of blocks
    (1, 8, 1, 4, 2, 2, "uniform"),          # one token, one lane
    (400, 256, 5, 20, 10, 5, "random"),     # skipped lanes and repeated experts
    (300, 4608, 6, 24, 8, 4, "uniform"),    # 20 hidden blocks: slices that do not fill a workgroup
    (40, 16384, 8, 64, 16, 4, "uniform"),   # records of several 32-block pieces
    (12, 65536, 4, 32, 8, 2, "random"),     # 275-block records
    (150, 1024, 64, 1024, 512, 256, "random")])  # largest K and G
def test_hierarchical_edges(T, H, K, E, R, G, ids):
    w = synth.Workload("edge", T, H, E, R, G, K, "uniform")
    inp = synth.make_inputs(w)
    if ids == "random":
        inp["topk_idx"] = np.random.default_rng(T + H).integers(-1, E, size=(T, K)).astype(np.int64)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    epoch = 9
    gb, pb, G_rows, N, stride = run_hier(w, inp, shape, L, ws, tk, epoch)
    O = oracle.layout(inp["topk_idx"], E, R, G)
    np.testing.assert_array_equal(host(L["group_slot"]), O["group_slot"])
    Hd = oracle.hier_dispatch(inp["topk_idx"], E, R, G, O["slot"], O["group_offsets"], epoch,
                              x=inp["x"], topk_w=inp["topk_w"])
    assert Hd["stride"] == stride and Hd["err"] == 0
    np.testing.assert_array_equal(host(gb)[:G_rows], Hd["group_buf"])
    np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])
    out = poison(torch.empty((T, H), dtype=torch.uint16, device="cuda"))
    ep.ep_combine(shape, L, pb, N, stride, ep.EP_FMT_CHUNKED, epoch, dev(inp["topk_w"]), out, ws)
    C = oracle.combine(O["slot"], inp["topk_w"], Hd["peer_buf"], H, chunked=True, epoch=epoch)
    np.testing.assert_array_equal(host(out), C["out"])
    assert ep.ep_check_errors(ws) == 0


def test_hierarchical_corrupted_flag_and_stale_epoch():
    w = synth.Workload("small", 400, 512, 32, 8, 4, 4, "uniform")
    inp = synth.make_inputs(w, seed=31)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    epoch = 11
    gb, pb, G_rows, N, stride = run_hier(w, inp, shape, L, ws, tk, epoch, steps=ep.EP_HIER_SCALEOUT)
    row, byte = 37, 2 * 512 + 480 + 9
    gb[row, byte] ^= 0x10
    run_hier(w, inp, shape, L, ws, tk, epoch, steps=ep.EP_HIER_FORWARD, group_buf=gb, peer_buf=pb)
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_FLAG
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    kw = dict(x=inp["x"], topk_w=inp["topk_w"])
    s1 = oracle.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], epoch,
                              steps=1, **kw)
    g = s1["group_buf"].copy()
    g[row, byte] ^= 0x10
    s2 = oracle.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], epoch,
                              steps=2, group_buf=g, **kw)
    assert s2["err"] == oracle.ERR_FLAG
    np.testing.assert_array_equal(host(pb)[:N], s2["peer_buf"])
    # combine with a stale epoch: every row rejected, zeros out
    ep.ep_clear_errors(ws)
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")
    ep.ep_combine(shape, L, pb, N, stride, ep.EP_FMT_CHUNKED, epoch + 1, dev(inp["topk_w"]), out, ws)
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_FLAG
    assert (host(out) == 0).all()
    # combine with the right epoch: the holes left by the dropped row are skipped
    ep.ep_clear_errors(ws)
    ep.ep_combine(shape, L, pb, N, stride, ep.EP_FMT_CHUNKED, epoch, dev(inp["topk_w"]), out, ws)
    C = oracle.combine(O["slot"], inp["topk_w"], s2["peer_buf"], w.H, chunked=True, epoch=epoch)
    assert C["err"] == oracle.ERR_FLAG
    np.testing.assert_array_equal(host(out), C["out"])
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_FLAG


def test_repeat_calls_identical():
    """Same inputs, two dispatch passes into fresh buffers: identical bytes (a
    race or ordering bug would show as a difference)."""
    w = synth.workload("ep32").scaled(2048)
    inp = synth.make_inputs(w)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    r1, N, _ = run_dispatch(w, inp, shape, L, ws, tk)
    r2, _, _ = run_dispatch(w, inp, shape, L, ws, tk)
    for k in r1:
        assert torch.equal(r1[k][:N].view(torch.uint8), r2[k][:N].view(torch.uint8)), k


# --------------------------------------------------------------------------
# Expand mode (one row per token and lane, grouped by expert)
# --------------------------------------------------------------------------

def run_expand(w, inp, fp8=False):
    topk = inp["topk_idx"]
    shape = ep.make_shape(topk.shape[0], w.H, topk.shape[1], w.E, w.R, w.G)
    L = ep.alloc_layout(shape, groups=w.G > 1, expand=True)
    for t in L.values():
        poison(t)
    ws = ep.alloc_workspace(shape)
    tk = dev(topk)
    ep.ep_get_layout(shape, tk, L, ws)
    torch.cuda.synchronize()
    return shape, L, ws, tk


@pytest.mark.parametrize("name", ["tiny", "ep32", "ep256", "zipf", "hier8x8"])
def test_expand_layout_full_size(name):
    w = synth.workload(name)
    inp = synth.make_inputs(w, with_x=False)
    shape, L, ws, _ = run_expand(w, inp)
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    check_layout(L, O, w.T)
    es = oracle.expert_slots(inp["topk_idx"], w.E, O["expert_offsets"])
    np.testing.assert_array_equal(host(L["expert_slot"]), es)
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("T,K,E,R", [(0, 8, 64, 8), (1, 1, 4, 2), (300, 3, 12, 6), (777, 16, 64, 16),
                                     (513, 8, 4096, 1024), (1000, 6, 16, 1),
                                     # K > 16: sorted passes of 4096 entries per workgroup
                                     (1100, 17, 64, 16), (600, 64, 128, 16), (300, 40, 4096, 512),
                                     (513, 64, 2048, 256), (70, 24, 24, 8)])
def test_expand_layout_edges(T, K, E, R):
    w = synth.Workload("edge", T, 128, E, R, 1, K, "uniform")
    rng = np.random.default_rng(T + K + E)
    topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    if T > 5:
        topk[5, :] = topk[5, 0]        # the same expert on every lane
        topk[2, 0] = E + 3             # invalid id
    shape, L, ws, _ = run_expand(w, dict(topk_idx=topk))
    O = oracle.layout(topk, E, R, 1)
    np.testing.assert_array_equal(host(L["expert_slot"]).reshape(T, K),
                                  oracle.expert_slots(topk, E, O["expert_offsets"]))
    np.testing.assert_array_equal(host(L["expert_offsets"]), O["expert_offsets"])
    assert ep.ep_check_errors(ws) == (ep.EP_DEVERR_EXPERT_ID if T > 5 else 0)


@pytest.mark.parametrize("T,K,E,R", [(1100, 8, 256, 32), (700, 4, 2048, 256), (600, 8, 4096, 512)])
def test_expand_layout_mixed_paths(T, K, E, R):
    """Workgroups of distinct top-k (the LDS bit-matrix rows) next to one whose
    token repeats an expert (the sorted rows), plus skipped lanes."""
    w = synth.Workload("edge", T, 128, E, R, 1, K, "uniform")
    topk = synth.topk_uniform(np.random.default_rng(T + E), T, E, K)
    topk[300, K - 1] = topk[300, 0]   # workgroup 1: a repeated expert
    topk[520, 1] = -1                 # workgroup 2: a skipped lane
    topk[T - 3, :] = -1               # a token with no expert
    shape, L, ws, _ = run_expand(w, dict(topk_idx=topk))
    O = oracle.layout(topk, E, R, 1)
    np.testing.assert_array_equal(host(L["expert_offsets"]), O["expert_offsets"])
    np.testing.assert_array_equal(host(L["expert_slot"]).reshape(T, K),
                                  oracle.expert_slots(topk, E, O["expert_offsets"]))
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("name,fp8", [("ep32", False), ("ep32", True), ("zipf", False), ("wide", False)])
def test_expand_dispatch_and_combine(name, fp8):
    """"wide": top-32 of 256 experts, so expand rows take the sorted passes."""
    w = synth.Workload("wide", 1000, 2048, 256, 32, 1, 32, "uniform") if name == "wide" else synth.workload(name)
    inp = synth.make_inputs(w, with_fp8=fp8)
    shape, L, ws, tk = run_expand(w, inp)
    n_rows = int(host(L["expert_offsets"])[-1])
    assert n_rows == w.T * w.K
    tokens = dict(x=dev(inp["x"]), topk_idx=tk, topk_weights=dev(inp["topk_w"]))
    if fp8:
        tokens["x_fp8"] = dev(inp["x_fp8"])
        tokens["x_scales"] = dev(inp["x_scales"])
    recv = ep.alloc_recv(shape, n_rows, fp8=fp8, scales=fp8)
    for t in recv.values():
        poison(t)
    ep.ep_dispatch_expand(shape, L, tokens, recv, n_rows, ws)
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    es = oracle.expert_slots(inp["topk_idx"], w.E, O["expert_offsets"])
    D = oracle.dispatch_rows(inp["topk_idx"], w.E, es, n_rows, x=inp["x"], x_fp8=inp.get("x_fp8"),
                             x_scales=inp.get("x_scales"), topk_w=inp["topk_w"])
    check_dispatch(recv, D, n_rows)
    # combine of stand-in expert outputs over the expand rows
    y = synth.random_bf16_rows(n_rows, w.H, seed=77)
    out = poison(torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda"))
    ep.ep_combine_expand(shape, L, dev(y), n_rows, 2 * w.H, ep.EP_FMT_PLAIN, 0,
                         tokens["topk_weights"], out, ws)
    C = oracle.combine(es, inp["topk_w"], y, w.H)
    got = host(out)
    combine_close(got, C["out"])
    np.testing.assert_array_equal(got, C["out"])
    # identity expert: round trip back to x
    ep.ep_combine_expand(shape, L, recv["x"], n_rows, 2 * w.H, ep.EP_FMT_PLAIN, 0,
                         tokens["topk_weights"], out, ws)
    combine_close(host(out), inp["x"])
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("T,H,K,E,R,G,expand", [
    (140000, 64, 8, 256, 64, 8, True),      # 547 workgroups: the scanned count tables, groups, expand rows
    (1048576, 8, 4, 64, 16, 4, False),      # 4,096 workgroups
])
def test_layout_many_workgroups_scanned(T, H, K, E, R, G, expand):
    """From 512 layout workgroups up, a scan launch turns the count tables into
    per-workgroup prefixes and each assign workgroup reads two rows: every
    layout output must still be the oracle's."""
    w = synth.Workload("scan", T, H, E, R, G, K, "uniform")
    print(f"scanned layout: T={T} K={K} E={E} R={R} G={G} expand={expand}", flush=True)
    topk = np.random.default_rng(T).integers(-1, E, size=(T, K)).astype(np.int64)
    topk[::97, 0] = E + 3  # some invalid ids
    shape = ep.make_shape(T, H, K, E, R, G)
    L = ep.alloc_layout(shape, masks=True, groups=True, expand=expand)
    for t in L.values():
        poison(t)
    ws = ep.alloc_workspace(shape)
    ep.ep_get_layout(shape, dev(topk), L, ws)
    torch.cuda.synchronize()
    O = oracle.layout(topk, E, R, G)
    for k in ("tokens_per_expert", "tokens_per_rank", "tokens_per_group", "expert_offsets", "rank_offsets",
              "group_offsets", "is_token_in_rank", "is_token_in_group", "slot", "group_slot"):
        np.testing.assert_array_equal(host(L[k]).reshape(O[k].shape), O[k], err_msg=k)
    if expand:
        es = oracle.expert_slots(topk, E, O["expert_offsets"])
        np.testing.assert_array_equal(host(L["expert_slot"]).reshape(T, K), es, err_msg="expert_slot")
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_EXPERT_ID


def test_many_tokens_end_to_end():
    """262,144 tokens: 1,024 layout workgroups, so every assign workgroup
    sums 1,024 rows of the count tables (spread over 15 thread groups); then
    dispatch and combine over about 1.9 M receive rows of a 256-wide hidden."""
    w = synth.Workload("many", 262144, 256, 256, 32, 1, 8, "uniform")
    inp = synth.make_inputs(w, seed=5)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    check_layout(L, O, w.T)
    recv, N, _ = run_dispatch(w, inp, shape, L, ws, tk)
    D = oracle.dispatch(inp["topk_idx"], w.E, w.R, O["rank_offsets"], x=inp["x"], topk_w=inp["topk_w"])
    check_dispatch(recv, D, N)
    out = poison(torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda"))
    ep.ep_combine(shape, L, recv["x"], N, 2 * w.H, ep.EP_FMT_PLAIN, 0, dev(inp["topk_w"]), out, ws)
    np.testing.assert_array_equal(host(out), oracle.combine(O["slot"], inp["topk_w"], D["recv_x"], w.H)["out"])
    assert ep.ep_check_errors(ws) == 0


# --------------------------------------------------------------------------
# Two-level combine (partials per token and group, then the cross-group sum)
# --------------------------------------------------------------------------

# Shapes beyond the five workloads, at full size: an expert count that is not
# a power of two (384 over 48 ranks), a 4096-wide hidden row, a hidden size
# that is not a multiple of 128 (2880: bf16 only; its 360 16-byte vectors are
# not a multiple of the 64 lanes of a wave) and six experts per token over 160
# experts in 4 groups.
OTHER_SHAPES = [
    ("E384", synth.Workload("E384", 4096, 7168, 384, 48, 1, 8, "uniform"), True),
    ("H4096", synth.Workload("H4096", 4096, 4096, 128, 16, 1, 8, "uniform"), True),
    ("H2880", synth.Workload("H2880", 3000, 2880, 128, 32, 4, 4, "uniform"), False),
    ("E160", synth.Workload("E160", 2048, 5120, 160, 20, 4, 6, "uniform"), True),
]


@pytest.mark.parametrize("name,w,fp8", OTHER_SHAPES, ids=[o[0] for o in OTHER_SHAPES])
def test_other_shapes_end_to_end(name, w, fp8):
    inp = synth.make_inputs(w, with_fp8=fp8)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    L["_ws"] = ws
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    check_layout(L, O, w.T)
    recv, N, _ = run_dispatch(w, inp, shape, L, ws, tk, fp8=fp8)
    D = oracle.dispatch(inp["topk_idx"], w.E, w.R, O["rank_offsets"], x=inp["x"],
                        x_fp8=inp.get("x_fp8"), x_scales=inp.get("x_scales"), topk_w=inp["topk_w"])
    check_dispatch(recv, D, N)
    wd = dev(inp["topk_w"])
    out = poison(torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda"))
    ep.ep_combine(shape, L, recv["x"], N, 2 * w.H, ep.EP_FMT_PLAIN, 0, wd, out, ws)
    combine_close(host(out), inp["x"])  # identity expert: back to x
    y = synth.random_bf16_rows(N, w.H, seed=5)
    ep.ep_combine(shape, L, dev(y), N, 2 * w.H, ep.EP_FMT_PLAIN, 0, wd, out, ws)
    np.testing.assert_array_equal(host(out), oracle.combine(O["slot"], inp["topk_w"], y, w.H)["out"])
    if w.G > 1:
        epoch = 21
        gb, pb, G_rows, _, stride = run_hier(w, inp, shape, L, ws, tk, epoch, fp8=fp8)
        Hd = oracle.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], epoch,
                                  x=inp["x"], x_fp8=inp.get("x_fp8"), x_scales=inp.get("x_scales"),
                                  topk_w=inp["topk_w"])
        np.testing.assert_array_equal(host(gb)[:G_rows], Hd["group_buf"])
        np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])
        gbuf, out2, gcap = run_two_level(shape, L, tk, pb, N, stride, ep.EP_FMT_CHUNKED, epoch, wd)
        C2 = oracle.combine_two_level(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_slot"],
                                      inp["topk_w"], Hd["peer_buf"], w.H, gcap, epoch, chunked=True)
        np.testing.assert_array_equal(host(gbuf)[:gcap], C2["group_buf"])
        np.testing.assert_array_equal(host(out2), C2["out"])
    assert ep.ep_check_errors(ws) == 0


def run_two_level(shape, L, tk, y, y_rows, y_stride, fmt, epoch, w_dev, steps=3, group_buf=None,
                  min_buf_bytes=0):
    """min_buf_bytes: pass a partial-row buffer (and capacity) of at least this
    many bytes; from 512 MB the library runs both steps as one launch."""
    gcap = int(host(L["group_offsets"])[-1])
    pstride = ep.ep_partial_row_bytes(shape)
    cap = max(gcap, -(-min_buf_bytes // pstride))
    if group_buf is None:
        group_buf = torch.zeros((max(cap, 1), pstride), dtype=torch.uint8, device="cuda")
    out = poison(torch.empty((shape.T, shape.H), dtype=torch.uint16, device="cuda"))
    ep.ep_combine_two_level(shape, L, tk, y, y_rows, y_stride, fmt, epoch, w_dev, group_buf, cap,
                            steps, out, ws=L["_ws"])
    torch.cuda.synchronize()
    return group_buf, out, gcap


@pytest.mark.parametrize("name", ["hier8x8", "small", "mid", "wide"])
def test_two_level_combine_chunked(name):
    """"mid": 20 hidden blocks per row, whose 3 slices do not fill a
    workgroup, so both steps take the one-wave-per-token kernels. "wide":
    top-24 over 16 groups, so both steps take the any-K kernels."""
    if name == "wide":
        w = synth.Workload("wide", 600, 2048, 256, 64, 16, 24, "uniform")
    elif name == "small":
        w = synth.Workload("small", 900, 1024, 64, 16, 4, 6, "uniform")
    elif name == "mid":
        w = synth.Workload("mid", 500, 4608, 64, 16, 4, 8, "uniform")
    else:
        w = synth.workload(name)
    inp = synth.make_inputs(w)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    L["_ws"] = ws
    epoch = 6
    gb, pb, G_rows, N, stride = run_hier(w, inp, shape, L, ws, tk, epoch)
    wd = dev(inp["topk_w"])
    gbuf, out, gcap = run_two_level(shape, L, tk, pb, N, stride, ep.EP_FMT_CHUNKED, epoch, wd)
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    Hd = oracle.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], epoch,
                              x=inp["x"], topk_w=inp["topk_w"])
    C = oracle.combine_two_level(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_slot"],
                                 inp["topk_w"], Hd["peer_buf"], w.H, gcap, epoch, chunked=True)
    assert C["err"] == 0
    np.testing.assert_array_equal(host(gbuf)[:gcap], C["group_buf"])
    got = host(out)
    np.testing.assert_array_equal(got, C["out"])
    # round trip to x: the bf16 partials add one more rounding, so the max
    # error bound is one bf16 half-ulp looser than the flat combine's
    o = synth.bf16_to_float(got).astype(np.float64)
    x = synth.bf16_to_float(inp["x"]).astype(np.float64)
    assert np.abs(o - x).max() <= 2e-2 and np.linalg.norm(o - x) <= RTOL_L2 * np.linalg.norm(x)
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("T,H,K,E,R,G", [(300, 512, 3, 24, 8, 4), (257, 264, 12, 64, 16, 2),
                                         (64, 7168, 8, 256, 64, 8), (128, 256, 2, 16, 4, 1),
                                         (300, 1032, 24, 64, 16, 4), (150, 264, 40, 128, 64, 64),
                                         (77, 4608, 64, 128, 32, 8), (50, 520, 17, 34, 17, 1),
                                         (40, 16384, 8, 64, 16, 4), (30, 16384, 24, 64, 16, 4),
                                         (100, 1024, 64, 1024, 512, 256),
                                         (200, 2048, 8, 64, 16, 4), (96, 3840, 5, 40, 8, 2),
                                         (60, 5768, 8, 64, 16, 4)])
def test_two_level_combine_plain(T, H, K, E, R, G):
    w = synth.Workload("edge", T, H, E, R, G, K, "uniform")
    rng = np.random.default_rng(T + H + K)
    topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    wts = rng.standard_normal((T, K)).astype(np.float32)
    shape, L, ws, tk = run_layout(w, topk)
    L["_ws"] = ws
    N = int(host(L["rank_offsets"])[-1])
    y = synth.random_bf16_rows(max(N, 1), H, seed=T)
    gbuf, out, gcap = run_two_level(shape, L, tk, dev(y), N, 2 * H, ep.EP_FMT_PLAIN, 9, dev(wts))
    O = oracle.layout(topk, E, R, G)
    C = oracle.combine_two_level(topk, E, R, G, O["slot"], O["group_slot"], wts, y[:N], H, gcap, 9)
    np.testing.assert_array_equal(host(gbuf)[:gcap], C["group_buf"])
    np.testing.assert_array_equal(host(out), C["out"])
    if G == 1:  # one group: identical to the flat combine
        flat = poison(torch.empty((T, H), dtype=torch.uint16, device="cuda"))
        ep.ep_combine(shape, L, dev(y), N, 2 * H, ep.EP_FMT_PLAIN, 0, dev(wts), flat, ws)
        np.testing.assert_array_equal(host(flat), host(out))
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("T,H,K,E,R,G", [(300, 512, 3, 24, 8, 4), (500, 2048, 8, 64, 16, 4),
                                         (257, 3840, 5, 40, 8, 2), (120, 7168, 8, 256, 64, 8),
                                         (64, 5768, 8, 64, 16, 4)])
def test_two_level_combine_one_launch(T, H, K, E, R, G):
    """Small shapes through the one-launch two-level combine (a partial-row
    capacity of 512 MB selects it), rows of 1, 2 and 4 slices: partial rows and
    outputs against the oracle and against the two launches (steps 1, then 2)."""
    w = synth.Workload("edge", T, H, E, R, G, K, "uniform")
    rng = np.random.default_rng(T + 7 * H + K)
    topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    wts = rng.standard_normal((T, K)).astype(np.float32)
    shape, L, ws, tk = run_layout(w, topk)
    L["_ws"] = ws
    N = int(host(L["rank_offsets"])[-1])
    y = synth.random_bf16_rows(max(N, 1), H, seed=T + H)
    gbuf, out, gcap = run_two_level(shape, L, tk, dev(y), N, 2 * H, ep.EP_FMT_PLAIN, 9, dev(wts),
                                    min_buf_bytes=512 << 20)
    O = oracle.layout(topk, E, R, G)
    C = oracle.combine_two_level(topk, E, R, G, O["slot"], O["group_slot"], wts, y[:N], H, gcap, 9)
    np.testing.assert_array_equal(host(gbuf[:gcap]), C["group_buf"])
    np.testing.assert_array_equal(host(out), C["out"])
    g1, _, _ = run_two_level(shape, L, tk, dev(y), N, 2 * H, ep.EP_FMT_PLAIN, 9, dev(wts), steps=1)
    _, out2, _ = run_two_level(shape, L, tk, dev(y), N, 2 * H, ep.EP_FMT_PLAIN, 9, dev(wts), steps=2,
                               group_buf=g1)
    np.testing.assert_array_equal(host(out2), host(out))
    assert ep.ep_check_errors(ws) == 0


def test_two_level_combine_special_values():
    """The two-level combine on rows and weights holding signed zeros,
    infinities, NaN, subnormals and overflowing products: the bf16 partials
    and the fp32 cross-group sums match the oracle bit for bit."""
    T, H, K, E, R, G = 200, 264, 6, 48, 12, 4
    w = synth.Workload("edge", T, H, E, R, G, K, "uniform")
    rng = np.random.default_rng(12)
    topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    shape, L, ws, tk = run_layout(w, topk)
    L["_ws"] = ws
    N = int(host(L["rank_offsets"])[-1])
    specials16 = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x8001, 0x007F, 0x7F7F,
                           0xFF7F], np.uint16)
    y = synth.random_bf16_rows(N, H, seed=13)
    pick = rng.random((N, H)) < 0.05
    y[pick] = rng.choice(specials16, size=int(pick.sum()))
    y[: N // 3] = rng.integers(1, 0x80, size=(N // 3, H)).astype(np.uint16)  # subnormal rows
    wts = rng.standard_normal((T, K)).astype(np.float32)
    pickw = rng.random((T, K)) < 0.1
    wts[pickw] = rng.choice(np.array([0.0, -0.0, np.inf, np.nan, 1e-40, 3.0e38], np.float32),
                            size=int(pickw.sum()))
    gbuf, out, gcap = run_two_level(shape, L, tk, dev(y), N, 2 * H, ep.EP_FMT_PLAIN, 5, dev(wts))
    O = oracle.layout(topk, E, R, G)
    C = oracle.combine_two_level(topk, E, R, G, O["slot"], O["group_slot"], wts, y, H, gcap, 5)
    np.testing.assert_array_equal(host(gbuf)[:gcap], C["group_buf"])
    np.testing.assert_array_equal(host(out), C["out"])
    assert ep.ep_check_errors(ws) == 0


@pytest.mark.parametrize("K", [6, 24])
def test_two_level_combine_corrupted_input_rows(K):
    """A chunked expert-output row with a bad flag in its first or last hidden
    block is dropped by the group step, for every lane that reads it (K = 24:
    the any-K kernels, which check the flags before the sums)."""
    w = synth.Workload("small", 700, 1024, 64, 16, 4, K, "uniform")
    inp = synth.make_inputs(w, seed=43)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    L["_ws"] = ws
    epoch = 11
    gb, pb, G_rows, N, stride = run_hier(w, inp, shape, L, ws, tk, epoch)
    nblk = (2 * w.H + 479) // 480
    bad = {5: 0, 211: nblk - 1, 1000: 2}  # row -> block whose flag is hit
    for row, blk in bad.items():
        pb[row, blk * 512 + 480 + 5] ^= 0x40
    wd = dev(inp["topk_w"])
    gbuf, out, gcap = run_two_level(shape, L, tk, pb, N, stride, ep.EP_FMT_CHUNKED, epoch, wd)
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_FLAG
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    Hd = oracle.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], epoch,
                              x=inp["x"], topk_w=inp["topk_w"])
    y = Hd["peer_buf"].copy()
    for row, blk in bad.items():
        y[row, blk * 512 + 480 + 5] ^= 0x40
    C = oracle.combine_two_level(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_slot"],
                                 inp["topk_w"], y, w.H, gcap, epoch, chunked=True)
    assert C["err"] == oracle.ERR_FLAG
    np.testing.assert_array_equal(host(gbuf)[:gcap], C["group_buf"])
    np.testing.assert_array_equal(host(out), C["out"])


@pytest.mark.parametrize("K", [4, 20])
def test_two_level_combine_corrupted_partial(K):
    w = synth.Workload("small", 300, 512, 32, 8, 4, K, "uniform")
    inp = synth.make_inputs(w, seed=41)
    shape, L, ws, tk = run_layout(w, inp["topk_idx"])
    L["_ws"] = ws
    N = int(host(L["rank_offsets"])[-1])
    y = synth.random_bf16_rows(N, w.H, seed=2)
    wd = dev(inp["topk_w"])
    gbuf, out, gcap = run_two_level(shape, L, tk, dev(y), N, 2 * w.H, ep.EP_FMT_PLAIN, 3, wd, steps=1)
    gbuf[7, 512 + 480 + 1] ^= 0x20
    _, out2, _ = run_two_level(shape, L, tk, dev(y), N, 2 * w.H, ep.EP_FMT_PLAIN, 3, wd, steps=2,
                               group_buf=gbuf)
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_FLAG
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    C1 = oracle.combine_two_level(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_slot"],
                                  inp["topk_w"], y, w.H, gcap, 3, steps=1)
    g = C1["group_buf"].copy()
    g[7, 512 + 480 + 1] ^= 0x20
    C2 = oracle.combine_two_level(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_slot"],
                                  inp["topk_w"], y, w.H, gcap, 3, steps=2, group_buf=g)
    assert C2["err"] == oracle.ERR_FLAG
    np.testing.assert_array_equal(host(out2), C2["out"])


# --------------------------------------------------------------------------
# Several source ranks: per-source regions, counts exchange, copy epilogue
# --------------------------------------------------------------------------

def expected_src_slot(topk, E, R, S, cap):
    return oracle.source_slots(topk, E, R, S, cap)["src_slot"]


def run_sources(w, inp, S, cap=None, fp8=False, epoch=9, steps=("layout", "send", "epilogue")):
    topk = inp["topk_idx"]
    T = topk.shape[0]
    shape = ep.make_shape(T, w.H, topk.shape[1], w.E, w.R, 1)
    X = oracle.source_counts(topk, w.E, w.R, S)
    cap = max(int(X["counts"].max(initial=0)), 1) if cap is None else cap
    src = ep.alloc_sources(shape, S, cap)
    for k in ("counts", "recv_offsets", "src_slot"):
        poison(src[k])
    ws = ep.alloc_source_workspace(shape, S)
    tk = dev(topk)
    ep.ep_source_layout(shape, tk, src, ws)
    seg = ep.EP_SEG_BF16 | ((ep.EP_SEG_FP8 | ep.EP_SEG_SCALES) if fp8 else 0)
    stride = ep.ep_chunked_record_bytes(shape, seg)
    staging = torch.zeros((max(w.R * S * cap, 1), stride), dtype=torch.uint8, device="cuda")
    tokens = dict(x=dev(inp["x"]), topk_idx=tk, topk_weights=dev(inp["topk_w"]))
    if fp8:
        tokens["x_fp8"] = dev(inp["x_fp8"])
        tokens["x_scales"] = dev(inp["x_scales"])
    if "send" in steps:
        ep.ep_source_dispatch(shape, src, tokens, epoch, staging, ws)
    torch.cuda.synchronize()
    return dict(shape=shape, src=src, ws=ws, staging=staging, stride=stride, seg=seg, cap=cap,
                X=X, epoch=epoch, tokens=tokens)


def run_epilogue(ctx, fp8=False, capacity=None):
    N = int(host(ctx["src"]["recv_offsets"])[-1])
    rows = N if capacity is None else capacity
    recv = ep.alloc_recv(ctx["shape"], max(rows, 1), fp8=fp8, scales=fp8)
    for t in recv.values():
        poison(t)
    ep.ep_copy_epilogue(ctx["shape"], ctx["src"], ctx["staging"], ctx["epoch"], ctx["seg"], recv,
                        rows, ctx["ws"])
    torch.cuda.synchronize()
    return recv, N


def check_sources_layout(ctx, topk, w, S):
    X = ctx["X"]
    O = oracle.layout(topk, w.E, w.R, 1)
    np.testing.assert_array_equal(host(ctx["src"]["counts"]), X["counts"])
    np.testing.assert_array_equal(host(ctx["src"]["recv_offsets"]), X["recv_offsets"])
    np.testing.assert_array_equal(host(ctx["src"]["src_slot"]).reshape(topk.shape),
                                  expected_src_slot(topk, w.E, w.R, S, ctx["cap"]))
    return O


@pytest.mark.parametrize("name,S", [("tiny", 1), ("tiny", 3), ("tiny", 4), ("ep32", 32),
                                    ("ep256", 256), ("zipf", 256), ("hier8x8", 64)])
def test_source_layout_full_size(name, S):
    w = synth.workload(name)
    inp = synth.make_inputs(w, with_x=False)
    inp["x"] = np.zeros((w.T, w.H), np.uint16)
    ctx = run_sources(w, inp, S, steps=("layout",))
    check_sources_layout(ctx, inp["topk_idx"], w, S)
    assert ep.ep_check_errors(ctx["ws"]) == 0


@pytest.mark.parametrize("name,S,fp8", [("tiny", 1, False), ("tiny", 3, True), ("ep32", 32, False),
                                        ("small", 5, True)])
def test_source_dispatch_and_epilogue(name, S, fp8):
    """Staging buffer byte for byte against the oracle's send step, dense
    rows against the oracle's copy epilogue and its direct dispatch, and the
    combine over the staging rows against the oracle's combine."""
    w = synth.workload(name) if name != "small" else synth.Workload("small", 1500, 1024, 64, 16, 1, 6, "uniform")
    inp = synth.make_inputs(w, with_fp8=fp8)
    topk = inp["topk_idx"]
    ctx = run_sources(w, inp, S, fp8=fp8)
    O = check_sources_layout(ctx, topk, w, S)
    extra = dict(x_fp8=inp["x_fp8"], x_scales=inp["x_scales"]) if fp8 else {}
    Sd = oracle.source_dispatch(topk, w.E, w.R, S, ctx["cap"], ctx["epoch"], x=inp["x"],
                                topk_w=inp["topk_w"], **extra)
    assert Sd["err"] == 0 and Sd["stride"] == ctx["stride"]
    np.testing.assert_array_equal(host(ctx["staging"]), Sd["staging"])
    recv, N = run_epilogue(ctx, fp8=fp8)
    Ce = oracle.copy_epilogue(ctx["X"]["recv_offsets"], Sd["staging"], w.H, w.K, w.R, S, ctx["cap"],
                              ctx["epoch"], with_fp8=fp8, with_scales=fp8)
    assert Ce["err"] == 0
    check_dispatch(recv, Ce, N)
    D = oracle.dispatch(topk, w.E, w.R, O["rank_offsets"], x=inp["x"], topk_w=inp["topk_w"], **extra)
    check_dispatch(recv, D, N)
    assert ep.ep_check_errors(ctx["ws"]) == 0
    # combine over the staging rows, addressed by src_slot
    out = poison(torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda"))
    L = dict(slot=ctx["src"]["src_slot"])
    ep.ep_combine(ctx["shape"], L, ctx["staging"], ctx["staging"].shape[0], ctx["stride"],
                  ep.EP_FMT_CHUNKED, ctx["epoch"], ctx["tokens"]["topk_weights"], out, ctx["ws"])
    slot = expected_src_slot(topk, w.E, w.R, S, ctx["cap"])
    C = oracle.combine(slot, inp["topk_w"], Sd["staging"], w.H, chunked=True, epoch=ctx["epoch"])
    assert C["err"] == 0
    np.testing.assert_array_equal(host(out), C["out"])
    assert ep.ep_check_errors(ctx["ws"]) == 0


@pytest.mark.parametrize("name,S", [("ep256", 256), ("zipf", 16), ("hier8x8", 64)])
def test_source_epilogue_full_size(name, S):
    """Full-size workloads whose staging buffers are too large for the oracle's
    send step: the dense rows are compared with the oracle's direct dispatch
    (equal to its copy epilogue, a pinned identity), and sampled staging rows
    with the oracle's chunked record of their token."""
    w = synth.workload(name)
    inp = synth.make_inputs(w)
    topk = inp["topk_idx"]
    ctx = run_sources(w, inp, S)
    O = check_sources_layout(ctx, topk, w, S)
    recv, N = run_epilogue(ctx)
    D = oracle.dispatch(topk, w.E, w.R, O["rank_offsets"], x=inp["x"], topk_w=inp["topk_w"])
    check_dispatch(recv, D, N)
    assert ep.ep_check_errors(ctx["ws"]) == 0
    slot = expected_src_slot(topk, w.E, w.R, S, ctx["cap"])
    rng = np.random.default_rng(5)
    for t in rng.choice(w.T, size=24, replace=False):
        k = int(np.argmax(slot[t] >= 0))
        if slot[t, k] < 0:
            continue
        rec = oracle.pack_record(int(t), topk, w.E, x=inp["x"], topk_w=inp["topk_w"])
        want = oracle.chunk(rec, ctx["epoch"])
        np.testing.assert_array_equal(host(ctx["staging"][int(slot[t, k])]), want)


@pytest.mark.parametrize("T,K,E,R,S", [(0, 8, 64, 8, 4), (5, 2, 16, 4, 8), (300, 3, 12, 6, 7),
                                       (1001, 20, 64, 16, 3), (513, 4, 16, 1, 2)])
def test_source_edges(T, K, E, R, S):
    """Empty input, more sources than tokens (empty sources), ragged sources,
    K above 16 with duplicates and -1, one rank."""
    w = synth.Workload("edge", T, 264, E, R, 1, K, "uniform")
    rng = np.random.default_rng(T + 13 * S)
    inp = dict(x=rng.integers(0, 65536, size=(T, 264)).astype(np.uint16),
               topk_idx=rng.integers(-1, E, size=(T, K)).astype(np.int64),
               topk_w=rng.standard_normal((T, K)).astype(np.float32))
    ctx = run_sources(w, inp, S)
    O = check_sources_layout(ctx, inp["topk_idx"], w, S)
    recv, N = run_epilogue(ctx)
    Sd = oracle.source_dispatch(inp["topk_idx"], E, R, S, ctx["cap"], ctx["epoch"], x=inp["x"],
                                topk_w=inp["topk_w"])
    if T:
        np.testing.assert_array_equal(host(ctx["staging"]), Sd["staging"])
    D = oracle.dispatch(inp["topk_idx"], E, R, O["rank_offsets"], x=inp["x"], topk_w=inp["topk_w"])
    check_dispatch(recv, D, N)
    assert ep.ep_check_errors(ctx["ws"]) == 0


@pytest.mark.parametrize("T,H,K,E,R,S", [(64, 16384, 8, 64, 16, 4), (20, 65536, 4, 32, 8, 2)])
def test_source_long_records(T, H, K, E, R, S):
    """Records longer than the 32 blocks the copy epilogue holds at once."""
    w = synth.Workload("edge", T, H, E, R, 1, K, "uniform")
    inp = synth.make_inputs(w, seed=T + S)
    ctx = run_sources(w, inp, S)
    O = check_sources_layout(ctx, inp["topk_idx"], w, S)
    recv, N = run_epilogue(ctx)
    Sd = oracle.source_dispatch(inp["topk_idx"], E, R, S, ctx["cap"], ctx["epoch"], x=inp["x"],
                                topk_w=inp["topk_w"])
    np.testing.assert_array_equal(host(ctx["staging"]), Sd["staging"])
    D = oracle.dispatch(inp["topk_idx"], E, R, O["rank_offsets"], x=inp["x"], topk_w=inp["topk_w"])
    check_dispatch(recv, D, N)
    assert ep.ep_check_errors(ctx["ws"]) == 0


def test_source_capacity_and_corrupted_flag():
    w = synth.workload("tiny")
    inp = synth.make_inputs(w, seed=77)
    topk = inp["topk_idx"]
    S = 2
    X = oracle.source_counts(topk, w.E, w.R, S)
    cap = int(X["counts"].max()) - 3
    ctx = run_sources(w, inp, S, cap=cap)
    check_sources_layout(ctx, topk, w, S)
    assert ep.ep_check_errors(ctx["ws"]) == ep.EP_DEVERR_CAPACITY
    Sd = oracle.source_dispatch(topk, w.E, w.R, S, cap, ctx["epoch"], x=inp["x"], topk_w=inp["topk_w"])
    assert Sd["err"] == oracle.ERR_CAPACITY
    np.testing.assert_array_equal(host(ctx["staging"]), Sd["staging"])
    # one stale flag word in a region row; a receive capacity below N
    victim = (1 * S + 1) * cap + 2
    ctx["staging"][victim, 512 + 480 + 4] ^= 1
    st = Sd["staging"].copy()
    st[victim, 512 + 480 + 4] ^= 1
    N = int(X["recv_offsets"][-1])
    ep.ep_clear_errors(ctx["ws"])
    recv, _ = run_epilogue(ctx, capacity=N - 5)
    Ce = oracle.copy_epilogue(X["recv_offsets"], st, w.H, w.K, w.R, S, cap, ctx["epoch"],
                              recv_cap=N - 5)
    assert Ce["err"] == oracle.ERR_CAPACITY | oracle.ERR_FLAG
    assert ep.ep_check_errors(ctx["ws"]) == ep.EP_DEVERR_CAPACITY | ep.EP_DEVERR_FLAG
    written = Ce["recv_src"] != -7
    assert written.sum() < N - 5
    # rows the epilogue skipped keep their poison
    assert (host(recv["src_idx"])[~written].view(np.uint32) == 0xABABABAB).all()
    for g, o in [("x", "recv_x"), ("src_idx", "recv_src"), ("topk_idx", "recv_topk_idx"),
                 ("topk_weights", "recv_topk_w")]:
        np.testing.assert_array_equal(host(recv[g])[written].view(np.uint8),
                                      Ce[o][written].view(np.uint8), err_msg=g)
