"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here runs on a GPU. Each test checks the oracle against something
other than itself: the closed form for the expected number of distinct
destinations (DeepEP V2 deep-dive page, 1.3 关键因子 1) and its worked
example, the chunk arithmetic of the Ascend Send Ordering page (能省多少),
count and offset invariants, brute force on tiny inputs through an
independent sort-based formulation, special cases that reduce to a library
routine (numpy's stable argsort, torch's bfloat16 cast), and exact rational
arithmetic for the combine's fused multiply-adds.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# Independent formulations used as pins
# --------------------------------------------------------------------------

def expected_distinct(E, G, k):
    """Closed form of the DeepEP V2 deep-dive page (get_expected_topk) plus the
    exact variance of the number of distinct groups hit by one token, from
    pairwise inclusion: Var = G q1 (1 - q1) + G (G - 1) (q2 - q1^2), where q1
    (q2) is the probability that a given group (pair of groups) is missed."""
    m = E // G
    c = math.comb(E, k)
    q1 = math.comb(E - m, k) / c
    q2 = math.comb(E - 2 * m, k) / c if E - 2 * m >= 0 else 0.0
    mean = G * (1 - q1)
    var = G * q1 * (1 - q1) + G * (G - 1) * (q2 - q1 * q1)
    return mean, max(var, 0.0)


def brute_layout(topk, E, R, G):
    """Sort-based formulation: receive rows are the positions of the distinct
    (rank, token) pairs in lexicographic order, so each rank's region is
    contiguous, regions follow rank order and rows follow token order."""
    epr, P = E // R, R // G
    T, K = topk.shape
    ok = lambda e: 0 <= e < E
    pairs = sorted({(int(e) // epr, t) for t in range(T) for e in topk[t] if ok(e)})
    gpairs = sorted({((int(e) // epr) // P, t) for t in range(T) for e in topk[t] if ok(e)})
    row = {p: i for i, p in enumerate(pairs)}
    grow = {p: i for i, p in enumerate(gpairs)}
    slot = np.full((T, K), -1, np.int64)
    gslot = np.full((T, K), -1, np.int64)
    for t in range(T):
        for k in range(K):
            e = int(topk[t, k])
            if ok(e):
                slot[t, k] = row[(e // epr, t)]
                gslot[t, k] = grow[((e // epr) // P, t)]
    tpe = np.bincount([int(e) for e in topk.ravel() if ok(e)], minlength=E)
    tpr = np.bincount([p[0] for p in pairs], minlength=R)
    tpg = np.bincount([p[0] for p in gpairs], minlength=G)
    mask = np.zeros((T, R), np.uint8)
    gmask = np.zeros((T, G), np.uint8)
    for r, t in pairs:
        mask[t, r] = 1
    for g, t in gpairs:
        gmask[t, g] = 1
    return dict(pairs=pairs, gpairs=gpairs, slot=slot, group_slot=gslot,
                tokens_per_expert=tpe, tokens_per_rank=tpr, tokens_per_group=tpg,
                is_token_in_rank=mask, is_token_in_group=gmask)


def check_layout_against_brute(L, B):
    for key in ("slot", "group_slot", "tokens_per_expert", "tokens_per_rank",
                "tokens_per_group", "is_token_in_rank", "is_token_in_group"):
        np.testing.assert_array_equal(np.asarray(L[key], np.int64), np.asarray(B[key], np.int64),
                                      err_msg=key)
    for cnt, off in (("tokens_per_expert", "expert_offsets"), ("tokens_per_rank", "rank_offsets"),
                     ("tokens_per_group", "group_offsets")):
        np.testing.assert_array_equal(L[off], np.concatenate([[0], np.cumsum(B[cnt])]), err_msg=off)


def round_to_f32(q: Fraction) -> float:
    """Correctly rounded (nearest, ties to even) binary32 of an exact rational."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def key(c):
        lsb = int(np.array(c, np.float32).view(np.uint32)) & 1
        return (abs(Fraction(float(c)) - q), lsb)

    return float(min(cands, key=key))


def torch_bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# Golden values printed on the pages
# --------------------------------------------------------------------------

def test_golden_expected_distinct_examples():
    g = json.load(open(os.path.join(GOLDEN, "expected_distinct.json")))
    ex1, ex2 = g["examples"]
    mean, var = expected_distinct(ex1["E"], ex1["G"], ex1["k"])
    assert mean == pytest.approx(ex1["page_value"], abs=1e-12) and var == pytest.approx(0, abs=1e-9)
    mean2, _ = expected_distinct(ex2["E"], ex2["G"], ex2["k"])
    assert round(mean2, 3) == ex2["formula_value"]
    m = ex2["E"] // ex2["G"]
    p_hit = 1 - math.comb(ex2["E"] - m, ex2["k"]) / math.comb(ex2["E"], ex2["k"])
    assert round(p_hit, 3) == ex2["per_group_hit_probability"]


def test_golden_chunk_overhead(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "chunk_overhead.json")))
    ex = g["worked_example"]
    P = ex["payload_bytes"]
    assert oracle_lib.chunked_bytes(P) == ex["chunked_bytes"]
    blocks = oracle_lib.chunked_bytes(P) // g["block_bytes"]
    assert blocks == ex["blocks"]
    assert blocks * g["flag_bytes_per_block"] == ex["flag_bytes"]
    assert g["flag_bytes_per_block"] / g["block_bytes"] == ex["flag_share_of_line"]
    assert round(g["flag_bytes_per_block"] / g["payload_per_block"], 4) == ex["flag_overhead_vs_payload"]
    # block-boundary sizes: 479 / 480 / 481 bytes -> 1 / 1 / 2 blocks
    assert [oracle_lib.chunked_bytes(p) for p in (0, 1, 479, 480, 481, 960, 961)] == \
        [0, 512, 512, 512, 1024, 1024, 1536]


# --------------------------------------------------------------------------
# Closed form, statistically
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ep32", "ep256", "hier8x8"])
def test_mean_distinct_ranks_matches_closed_form(oracle_lib, name):
    w = synth.workload(name)
    inp = synth.make_inputs(w, with_x=False)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R, w.G)
    per_tok = L["is_token_in_rank"].sum(axis=1)
    mean, var = expected_distinct(w.E, w.R, w.K)
    se = math.sqrt(var / w.T)
    assert abs(per_tok.mean() - mean) <= 5 * se + 1e-12, (per_tok.mean(), mean, se)
    if w.G > 1:
        per_tok_g = L["is_token_in_group"].sum(axis=1)
        mg, vg = expected_distinct(w.E, w.G, w.K)
        assert abs(per_tok_g.mean() - mg) <= 5 * math.sqrt(vg / w.T) + 1e-12
    if w.E == w.R:  # worked example of the page: one expert per rank -> exactly K ranks
        assert (per_tok == w.K).all()


def test_expert_marginal_uniform(oracle_lib):
    w = synth.workload("ep32")
    inp = synth.make_inputs(w, with_x=False)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R, w.G)
    c = L["tokens_per_expert"].astype(np.float64)
    exp = w.T * w.K / w.E
    chi2 = ((c - exp) ** 2 / exp).sum()
    dof = w.E - 1
    assert chi2 < dof + 6 * math.sqrt(2 * dof)


# --------------------------------------------------------------------------
# Invariants on every workload
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ep32", "ep256", "zipf", "hier8x8"])
def test_count_offset_invariants(oracle_lib, name):
    w = synth.workload(name)
    inp = synth.make_inputs(w, with_x=False)
    topk = inp["topk_idx"]
    L = oracle_lib.layout(topk, w.E, w.R, w.G)
    assert L["err"] == 0
    mask, gmask = L["is_token_in_rank"], L["is_token_in_group"]
    N = int(mask.sum())
    assert L["tokens_per_rank"].sum() == N == L["rank_offsets"][-1]
    assert L["tokens_per_expert"].sum() == (topk >= 0).sum() == w.T * w.K
    for cnt, off in (("tokens_per_expert", "expert_offsets"), ("tokens_per_rank", "rank_offsets"),
                     ("tokens_per_group", "group_offsets")):
        assert L[off][0] == 0
        np.testing.assert_array_equal(np.diff(L[off]), L[cnt])
    per_tok = mask.sum(axis=1)
    assert per_tok.min() >= 1 and per_tok.max() <= min(w.K, w.R)
    epr, P = w.E // w.R, w.R // w.G
    per_rank_expert = L["tokens_per_expert"].reshape(w.R, epr).sum(axis=1)
    assert (L["tokens_per_rank"] <= per_rank_expert).all()
    tpr_by_group = L["tokens_per_rank"].reshape(w.G, P)
    assert (L["tokens_per_group"] <= tpr_by_group.sum(axis=1)).all()
    assert (L["tokens_per_group"] >= tpr_by_group.max(axis=1)).all()
    np.testing.assert_array_equal(gmask, mask.reshape(w.T, w.G, P).max(axis=2))
    # slots: every (t, r) pair in the mask owns exactly one row of r's region,
    # rows within a region ascend with t, repeated ranks share the row
    slot = L["slot"]
    rank = np.where(topk >= 0, topk // epr, -1)
    assert ((slot >= 0) == (topk >= 0)).all()
    for r in np.unique(rank[rank >= 0])[:64]:
        rows = np.unique(slot[rank == r])
        lo, hi = L["rank_offsets"][r], L["rank_offsets"][r + 1]
        np.testing.assert_array_equal(rows, np.arange(lo, hi))
        toks = np.nonzero(mask[:, r])[0]
        t_of_row = np.full(hi - lo, -1)
        tt, kk = np.nonzero(rank == r)
        t_of_row[slot[tt, kk] - lo] = tt
        np.testing.assert_array_equal(t_of_row, toks)
    if name == "zipf":  # skew the workload is meant to stress
        assert L["tokens_per_rank"].max() > 10 * L["tokens_per_rank"].mean()


# --------------------------------------------------------------------------
# Brute force on tiny inputs
# --------------------------------------------------------------------------

def _tiny_cases():
    rng = np.random.default_rng(7)
    cases = []
    # every single-token choice with K = 3 over E = 6 experts, including -1 and
    # repeated experts, stacked as one batch (so slots also see token order)
    vals = list(range(-1, 6))
    allrows = np.array(list(itertools.product(vals, repeat=3)), np.int64)
    for R, G in ((1, 1), (2, 1), (2, 2), (3, 1), (3, 3), (6, 2), (6, 3)):
        cases.append((allrows, 6, R, G))
    # every pair of tokens with K = 2 over E = 4
    vals = list(range(-1, 4))
    rows2 = np.array(list(itertools.product(vals, repeat=2)), np.int64)
    for a, b in itertools.product(range(len(rows2)), repeat=2):
        if (a * 31 + b) % 7 == 0:
            cases.append((np.stack([rows2[a], rows2[b]]), 4, 2, 2))
    # random small batches
    for i in range(40):
        E = int(rng.choice([2, 4, 6, 8, 12]))
        R = int(rng.choice([r for r in (1, 2, 3, 4, 6) if E % r == 0]))
        G = int(rng.choice([g for g in (1, 2, 3) if R % g == 0]))
        T, K = int(rng.integers(0, 6)), int(rng.integers(1, 5))
        cases.append((rng.integers(-1, E, size=(T, K)).astype(np.int64), E, R, G))
    return cases


def test_layout_brute_force(oracle_lib):
    for topk, E, R, G in _tiny_cases():
        L = oracle_lib.layout(topk, E, R, G)
        B = brute_layout(topk, E, R, G)
        check_layout_against_brute(L, B)
        assert L["err"] == 0


def test_dispatch_brute_force(oracle_lib):
    rng = np.random.default_rng(11)
    for topk, E, R, G in _tiny_cases():
        T, K = topk.shape
        H = 128
        x = rng.integers(0, 65536, size=(T, H)).astype(np.uint16)
        fp8 = rng.integers(0, 256, size=(T, H)).astype(np.uint8)
        sc = rng.standard_normal((T, 1)).astype(np.float32)
        w = rng.standard_normal((T, K)).astype(np.float32)
        L = oracle_lib.layout(topk, E, R, G)
        D = oracle_lib.dispatch(topk, E, R, L["rank_offsets"], x=x, x_fp8=fp8, x_scales=sc, topk_w=w)
        B = brute_layout(topk, E, R, G)
        srcs = np.array([t for (_, t) in B["pairs"]], np.int64)
        assert D["recv_x"].shape[0] == len(srcs)
        if len(srcs):
            np.testing.assert_array_equal(D["recv_src"], srcs)
            np.testing.assert_array_equal(D["recv_x"], x[srcs])
            np.testing.assert_array_equal(D["recv_fp8"], fp8[srcs])
            np.testing.assert_array_equal(D["recv_scales"].view(np.uint32), sc[srcs].view(np.uint32))
            np.testing.assert_array_equal(D["recv_topk_idx"], topk[srcs])
            np.testing.assert_array_equal(D["recv_topk_w"].view(np.uint32), w[srcs].view(np.uint32))


# --------------------------------------------------------------------------
# Special cases that reduce to library routines
# --------------------------------------------------------------------------

def test_single_rank_is_identity(oracle_lib):
    w = synth.Workload("r1", 300, 256, 16, 1, 1, 4, "uniform")
    inp = synth.make_inputs(w, seed=5)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R, w.G)
    D = oracle_lib.dispatch(inp["topk_idx"], w.E, w.R, L["rank_offsets"], x=inp["x"])
    np.testing.assert_array_equal(D["recv_x"], inp["x"])
    np.testing.assert_array_equal(D["recv_src"], np.arange(w.T))


def test_top1_one_expert_per_rank_is_stable_counting_sort(oracle_lib):
    rng = np.random.default_rng(3)
    T, E = 1000, 16
    topk = rng.integers(0, E, size=(T, 1)).astype(np.int64)
    L = oracle_lib.layout(topk, E, E, 1)
    D = oracle_lib.dispatch(topk, E, E, L["rank_offsets"])
    np.testing.assert_array_equal(D["recv_src"], np.argsort(topk[:, 0], kind="stable"))
    np.testing.assert_array_equal(L["slot"][:, 0], np.argsort(np.argsort(topk[:, 0], kind="stable")))


# --------------------------------------------------------------------------
# Edge cases and errors
# --------------------------------------------------------------------------

def test_zero_tokens(oracle_lib):
    topk = np.zeros((0, 8), np.int64)
    L = oracle_lib.layout(topk, 256, 32, 4)
    assert L["rank_offsets"].sum() == 0 and L["tokens_per_expert"].sum() == 0
    D = oracle_lib.dispatch(topk, 256, 32, L["rank_offsets"], x=np.zeros((0, 128), np.uint16))
    assert D["recv_x"].shape == (0, 128)
    C = oracle_lib.combine(L["slot"], np.zeros((0, 8), np.float32), np.zeros((0, 128), np.uint16), 128)
    assert C["out"].shape == (0, 128) and C["err"] == 0


def test_all_tokens_one_rank_and_empty_ranks(oracle_lib):
    T, K, E, R = 50, 4, 16, 4
    topk = np.tile(np.array([5, 4, 6, 7], np.int64), (T, 1))  # all on rank 1
    L = oracle_lib.layout(topk, E, R, 1)
    np.testing.assert_array_equal(L["tokens_per_rank"], [0, T, 0, 0])
    np.testing.assert_array_equal(L["rank_offsets"], [0, 0, T, T, T])
    assert (L["slot"] == np.arange(T)[:, None]).all()


def test_invalid_expert_ids_flagged_and_skipped(oracle_lib):
    topk = np.array([[0, 16], [-2, 3], [-1, 5]], np.int64)
    L = oracle_lib.layout(topk, 16, 4, 1)
    assert L["err"] & oracle_lib.ERR_EXPERT
    clean = np.where((topk >= 0) & (topk < 16), topk, -1)
    Lc = oracle_lib.layout(clean, 16, 4, 1)
    assert Lc["err"] == 0
    for key in ("slot", "tokens_per_rank", "tokens_per_expert", "rank_offsets"):
        np.testing.assert_array_equal(L[key], Lc[key])
    x = np.arange(3 * 128, dtype=np.uint16).reshape(3, 128)
    D = oracle_lib.dispatch(topk, 16, 4, L["rank_offsets"], x=x)
    assert D["err"] & oracle_lib.ERR_EXPERT
    assert (D["recv_topk_idx"] == clean[D["recv_src"]]).all()


def test_capacity_overflow(oracle_lib):
    w = synth.workload("tiny")
    inp = synth.make_inputs(w)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R)
    N = int(L["rank_offsets"][-1])
    full = oracle_lib.dispatch(inp["topk_idx"], w.E, w.R, L["rank_offsets"], x=inp["x"])
    part = oracle_lib.dispatch(inp["topk_idx"], w.E, w.R, L["rank_offsets"], x=inp["x"],
                               capacity=N - 10)
    assert full["err"] == 0 and part["err"] == oracle_lib.ERR_CAPACITY
    np.testing.assert_array_equal(part["recv_x"], full["recv_x"][:N - 10])


# --------------------------------------------------------------------------
# Number helpers against torch's cast
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch(oracle_lib):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x00008000, 0x00018000, 0x807FFFFF,
                        0x7F7FFFFF, 0x7F7F8000, 0xFF7F8000, 0x7F800000, 0x00000000, 0x80000000,
                        0x00000001, 0x3F7FFFFF], np.uint32)
    bits = np.concatenate([special, bits])
    vals = bits.view(np.float32)
    finite = np.isfinite(vals) | np.isinf(vals)
    ours = np.array([oracle_lib.f32_to_bf16(v) for v in vals], np.uint16)
    ref = torch_bf16_bits(vals)
    np.testing.assert_array_equal(ours[finite & ~np.isnan(vals)], ref[finite & ~np.isnan(vals)])
    nan = np.float32(np.nan)
    assert oracle_lib.f32_to_bf16(nan) == 0x7FC0
    for h in (0x0000, 0x8000, 0x3F80, 0xC2F7, 0x0001, 0x7F80):
        assert np.float32(oracle_lib.bf16_to_f32(h)) == synth.bf16_to_float(np.array([h]))[0]


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------

def test_combine_exact_rational_fma_order(oracle_lib):
    """Sequential single-rounding FMAs in ascending k from +0, then one
    bfloat16 rounding, recomputed with exact rationals."""
    rng = np.random.default_rng(2)
    T, H, K, rows = 12, 48, 5, 20
    y = synth.bf16_bits(rng.standard_normal((rows, H)).astype(np.float32) * 3)
    slot = rng.integers(-1, rows, size=(T, K)).astype(np.int32)
    slot[0] = -1                 # no usable lane -> zeros
    slot[1, 3] = slot[1, 1]      # repeated row
    w = rng.standard_normal((T, K)).astype(np.float32)
    C = oracle_lib.combine(slot, w, y, H)
    yf = synth.bf16_to_float(y)
    exp = np.zeros((T, H), np.float32)
    for t in range(T):
        for h in range(H):
            acc = 0.0
            for k in range(K):
                if slot[t, k] < 0:
                    continue
                acc = round_to_f32(Fraction(float(w[t, k])) * Fraction(float(yf[slot[t, k], h]))
                                   + Fraction(acc))
            exp[t, h] = acc
    np.testing.assert_array_equal(C["out"], torch_bf16_bits(exp))
    assert (C["out"][0] == 0).all()


def test_combine_round_trip_identity_expert(oracle_lib):
    """dispatch -> identity expert -> combine with weights summing to 1 gives x
    back within the bf16 tolerance (max abs 1e-2, relative L2 4e-3)."""
    for name in ("tiny", "ep32"):
        w = synth.workload(name)
        if name == "ep32":
            w = w.scaled(512)
        inp = synth.make_inputs(w)
        L = oracle_lib.layout(inp["topk_idx"], w.E, w.R)
        D = oracle_lib.dispatch(inp["topk_idx"], w.E, w.R, L["rank_offsets"], x=inp["x"])
        C = oracle_lib.combine(L["slot"], inp["topk_w"], D["recv_x"], w.H)
        x = synth.bf16_to_float(inp["x"]).astype(np.float64)
        o = synth.bf16_to_float(C["out"]).astype(np.float64)
        assert np.abs(o - x).max() <= 1e-2
        assert np.linalg.norm(o - x) / np.linalg.norm(x) <= 4e-3


def test_combine_one_hot_is_exact_gather(oracle_lib):
    rng = np.random.default_rng(4)
    T, H, K, rows = 40, 256, 4, 60
    y = synth.bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    slot = rng.integers(0, rows, size=(T, K)).astype(np.int32)
    hot = rng.integers(0, K, size=T)
    w = np.zeros((T, K), np.float32)
    w[np.arange(T), hot] = 1.0
    C = oracle_lib.combine(slot, w, y, H)
    np.testing.assert_array_equal(C["out"], y[slot[np.arange(T), hot]])


def test_combine_out_of_range_rows(oracle_lib):
    y = np.ones((4, 128), np.uint16)
    slot = np.array([[0, 7], [3, -1]], np.int32)
    w = np.ones((2, 2), np.float32)
    C = oracle_lib.combine(slot, w, y, 128)
    assert C["err"] == oracle_lib.ERR_CAPACITY
    C2 = oracle_lib.combine(np.array([[0, -1], [3, -1]], np.int32), w, y, 128)
    np.testing.assert_array_equal(C["out"], C2["out"])


# --------------------------------------------------------------------------
# Record, chunk codec and the two-level dispatch
# --------------------------------------------------------------------------

def test_record_layout_pieces(oracle_lib):
    """Token record: bf16 hidden | fp8 hidden | fp32 scales | topk_idx (i32) |
    topk_w (f32) | src (i32), each piece padded to 16 B (TokenLayout of the
    DeepEP V2 deep-dive page, 3.4)."""
    rng = np.random.default_rng(9)
    T, H, K, E = 3, 384, 3, 12
    x = rng.integers(0, 65536, size=(T, H)).astype(np.uint16)
    fp8 = rng.integers(0, 256, size=(T, H)).astype(np.uint8)
    sc = rng.standard_normal((T, H // 128)).astype(np.float32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    topk = np.array([[1, 13, 5], [0, 1, 2], [-1, 4, 4]], np.int64)
    rec = oracle_lib.pack_record(0, topk, E, x=x, x_fp8=fp8, x_scales=sc, topk_w=w)
    assert rec.size == oracle_lib.record_bytes(H, K, True, True, True) == 768 + 384 + 16 + 16 + 16 + 16
    np.testing.assert_array_equal(rec[:768].view(np.uint16), x[0])
    np.testing.assert_array_equal(rec[768:1152], fp8[0])
    np.testing.assert_array_equal(rec[1152:1164].view(np.float32), sc[0])
    assert (rec[1164:1168] == 0).all()
    np.testing.assert_array_equal(rec[1168:1180].view(np.int32), [1, -1, 5])
    np.testing.assert_array_equal(rec[1184:1196].view(np.float32), w[0])
    assert rec[1200:1204].view(np.int32)[0] == 0 and (rec[1204:] == 0).all()
    assert oracle_lib.record_bytes(7168, 8) == 14416
    assert oracle_lib.chunked_bytes(14416) == 31 * 512 == 15872


def test_chunk_round_trip_and_flags(oracle_lib):
    rng = np.random.default_rng(10)
    for P in (16, 464, 480, 496, 14416):
        rec = rng.integers(0, 256, size=P).astype(np.uint8)
        blk = oracle_lib.chunk(rec, epoch=77)
        nb = blk.size // 512
        assert nb == -(-P // 480)
        b = blk.reshape(nb, 512)
        assert (b[:, 480:].copy().view(np.uint32) == 77).all()
        np.testing.assert_array_equal(b[:, :480].ravel()[:P], rec)
        assert (b[:, :480].ravel()[P:] == 0).all()
        back, ok = oracle_lib.unchunk(blk, P, 77)
        assert ok and (back == rec).all()
        _, ok_stale = oracle_lib.unchunk(blk, P, 76)
        assert not ok_stale
        bad = blk.copy()
        bad[(nb - 1) * 512 + 480 + 31] ^= 1
        _, ok_bad = oracle_lib.unchunk(bad, P, 77)
        assert not ok_bad


@pytest.mark.parametrize("with_fp8", [False, True])
def test_hierarchical_equals_direct(oracle_lib, with_fp8):
    w = synth.Workload("hier_small", 700, 512, 64, 16, 4, 6, "uniform")
    inp = synth.make_inputs(w, seed=12, with_fp8=with_fp8)
    topk = inp["topk_idx"].copy()
    topk[5, 2] = -1
    topk[9, 1] = topk[9, 0]
    L = oracle_lib.layout(topk, w.E, w.R, w.G)
    kw = dict(x=inp["x"], x_fp8=inp.get("x_fp8"), x_scales=inp.get("x_scales"),
              topk_w=inp["topk_w"])
    D = oracle_lib.dispatch(topk, w.E, w.R, L["rank_offsets"], **kw)
    Hd = oracle_lib.hier_dispatch(topk, w.E, w.R, w.G, L["slot"], L["group_offsets"], 3, **kw)
    assert Hd["err"] == 0
    assert Hd["group_buf"].shape[0] == L["tokens_per_group"].sum()
    U = oracle_lib.unpack_rows(Hd["peer_buf"], w.H, w.K, 3, True, with_fp8, with_fp8)
    assert U["bad_rows"] == 0
    for key in ("recv_x", "recv_fp8", "recv_scales", "recv_src", "recv_topk_idx", "recv_topk_w"):
        if D[key] is None:
            continue
        np.testing.assert_array_equal(U[key].view(np.uint8), D[key].view(np.uint8), err_msg=key)
    # group rows: one per (token, group) pair, ascending tokens in each region
    G = oracle_lib.unpack_rows(Hd["group_buf"], w.H, w.K, 3, True, with_fp8, with_fp8)
    assert G["bad_rows"] == 0
    B = brute_layout(topk, w.E, w.R, w.G)
    np.testing.assert_array_equal(G["recv_src"], [t for (_, t) in B["gpairs"]])
    np.testing.assert_array_equal(G["recv_x"], inp["x"][G["recv_src"]])
    # combine straight from the chunked rows == combine from plain rows
    Cp = oracle_lib.combine(L["slot"], inp["topk_w"], D["recv_x"], w.H)
    Cc = oracle_lib.combine(L["slot"], inp["topk_w"], Hd["peer_buf"], w.H, chunked=True, epoch=3)
    assert Cc["err"] == 0
    np.testing.assert_array_equal(Cc["out"], Cp["out"])


def test_hierarchical_corrupt_flag_drops_row(oracle_lib):
    w = synth.Workload("hier_small", 200, 256, 32, 8, 4, 4, "uniform")
    inp = synth.make_inputs(w, seed=13)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R, w.G)
    kw = dict(x=inp["x"], topk_w=inp["topk_w"])
    s1 = oracle_lib.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, L["slot"],
                                  L["group_offsets"], 9, steps=1, **kw)
    gb = s1["group_buf"].copy()
    gb[17, 512 + 480 + 5] ^= 0x40          # one flag byte of row 17
    s2 = oracle_lib.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, L["slot"],
                                  L["group_offsets"], 9, steps=2, group_buf=gb, **kw)
    assert s2["err"] == oracle_lib.ERR_FLAG
    good = oracle_lib.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, L["slot"],
                                    L["group_offsets"], 9, **kw)
    src17 = oracle_lib.unpack_rows(s1["group_buf"][17:18], w.H, w.K, 9)["recv_src"][0]
    U = oracle_lib.unpack_rows(s2["peer_buf"], w.H, w.K, 9)
    Ug = oracle_lib.unpack_rows(good["peer_buf"], w.H, w.K, 9)
    # the dropped record leaves holes (never-written rows, flags 0) exactly at
    # the rows of that token's ranks inside the corrupted row's group; every
    # other row is identical to the run without corruption
    diff = np.nonzero((s2["peer_buf"] != good["peer_buf"]).any(axis=1))[0]
    assert U["bad_rows"] == len(diff) >= 1
    assert (Ug["recv_src"][diff] == src17).all()
    assert (s2["peer_buf"][diff] == 0).all()
    epr, P = w.E // w.R, w.R // w.G
    g17 = int(np.searchsorted(L["group_offsets"], 17, side="right") - 1)
    ranks = {int(e) // epr for e in inp["topk_idx"][src17] if (int(e) // epr) // P == g17}
    assert len(diff) == len(ranks)


def test_stale_epoch_rejected_by_combine(oracle_lib):
    w = synth.Workload("hier_small", 64, 256, 16, 4, 2, 2, "uniform")
    inp = synth.make_inputs(w, seed=14)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R, w.G)
    Hd = oracle_lib.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, L["slot"],
                                  L["group_offsets"], 5, x=inp["x"], topk_w=inp["topk_w"])
    C = oracle_lib.combine(L["slot"], inp["topk_w"], Hd["peer_buf"], w.H, chunked=True, epoch=6)
    assert C["err"] == oracle_lib.ERR_FLAG and (C["out"] == 0).all()


# --------------------------------------------------------------------------
# Expand mode: one row per (token, lane), grouped by expert
# --------------------------------------------------------------------------

def brute_expert_slots(topk, E):
    """Rows are the positions of the sorted valid (expert, token, lane) triples."""
    T, K = topk.shape
    trip = sorted((int(topk[t, k]), t, k) for t in range(T) for k in range(K) if 0 <= topk[t, k] < E)
    out = np.full((T, K), -1, np.int64)
    for i, (_, t, k) in enumerate(trip):
        out[t, k] = i
    return out


def test_expert_slots_brute_force(oracle_lib):
    for topk, E, R, G in _tiny_cases():
        L = oracle_lib.layout(topk, E, R, G)
        es = oracle_lib.expert_slots(topk, E, L["expert_offsets"])
        np.testing.assert_array_equal(es, brute_expert_slots(topk, E))


@pytest.mark.parametrize("name", ["ep32", "zipf"])
def test_expert_slots_regions(oracle_lib, name):
    w = synth.workload(name)
    inp = synth.make_inputs(w, with_x=False)
    topk = inp["topk_idx"]
    L = oracle_lib.layout(topk, w.E, w.R, w.G)
    es = oracle_lib.expert_slots(topk, w.E, L["expert_offsets"])
    assert (es >= 0).all() and len(np.unique(es)) == w.T * w.K
    order = np.argsort(es.ravel())
    # rows are expert-major, then token, then lane
    e_sorted = topk.ravel()[order]
    assert (np.diff(e_sorted) >= 0).all()
    np.testing.assert_array_equal(np.bincount(e_sorted, minlength=w.E), L["tokens_per_expert"])
    tk = np.arange(w.T * w.K)[order]
    same = np.diff(e_sorted) == 0
    assert (np.diff(tk)[same] > 0).all()


def test_expert_slots_equal_rank_slots_with_one_expert_per_rank(oracle_lib):
    """With one expert per rank and distinct experts per token, a lane's rank
    row and its expert row coincide."""
    w = synth.Workload("e_eq_r", 500, 128, 64, 64, 1, 4, "uniform")
    inp = synth.make_inputs(w, with_x=False)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R)
    es = oracle_lib.expert_slots(inp["topk_idx"], w.E, L["expert_offsets"])
    np.testing.assert_array_equal(es, L["slot"])


def brute_expand_receive(topk, E, x, fp8, sc, w):
    """Receive arrays of expand mode built by enumeration: the i-th valid
    (expert, token, lane) triple in sorted order is row i, and it holds its
    token's record: hidden, FP8, scales and weights copied from token t, the
    source index t, and the token's ids with every id outside [0, E) shown
    as -1."""
    T, K = topk.shape
    trip = sorted((int(topk[t, k]), t, k) for t in range(T) for k in range(K) if 0 <= topk[t, k] < E)
    n = len(trip)
    out = dict(recv_x=np.zeros((n, x.shape[1]), np.uint16), recv_fp8=np.zeros((n, fp8.shape[1]), np.uint8),
               recv_scales=np.zeros((n, sc.shape[1]), np.float32), recv_src=np.zeros(n, np.int32),
               recv_topk_idx=np.zeros((n, K), np.int32), recv_topk_w=np.zeros((n, K), np.float32))
    for i, (_, t, _) in enumerate(trip):
        out["recv_x"][i] = x[t]
        out["recv_fp8"][i] = fp8[t]
        out["recv_scales"][i] = sc[t]
        out["recv_src"][i] = t
        for k in range(K):
            e = int(topk[t, k])
            out["recv_topk_idx"][i, k] = e if 0 <= e < E else -1
        out["recv_topk_w"][i] = w[t]
    return out


def _assert_receive_equal(got, want, fields):
    for f in fields:
        a, b = np.asarray(got[f]), np.asarray(want[f])
        assert a.shape == b.shape, f
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        np.testing.assert_array_equal(a, b, err_msg=f)


EXPAND_FIELDS = ("recv_x", "recv_fp8", "recv_scales", "recv_src", "recv_topk_idx", "recv_topk_w")


def test_expand_receive_arrays_brute_force(oracle_lib):
    """Every field of the expand-mode receive rows (DeepEP V2 page, 3.3 阶段3:
    the copy epilogue's per-expert rows) against the sorted-triple
    enumeration, on the tiny cases plus ids below -1 and at or above E (they
    are skipped and show as -1 in the copied ids)."""
    rng = np.random.default_rng(29)
    cases = list(_tiny_cases())
    for i in range(30):  # invalid ids other than -1
        E = int(rng.choice([4, 6, 8]))
        T, K = int(rng.integers(1, 6)), int(rng.integers(1, 5))
        topk = rng.integers(-3, E + 3, size=(T, K)).astype(np.int64)
        cases.append((topk, E, 1, 1))
    for topk, E, R, G in cases:
        T, K = topk.shape
        H = 256
        x = rng.integers(0, 65536, size=(T, H)).astype(np.uint16)
        fp8 = rng.integers(0, 256, size=(T, H)).astype(np.uint8)
        sc = rng.standard_normal((T, H // 128)).astype(np.float32)
        w = rng.standard_normal((T, K)).astype(np.float32)
        L = oracle_lib.layout(topk, E, R, G)
        es = oracle_lib.expert_slots(topk, E, L["expert_offsets"])
        n_rows = int(L["expert_offsets"][-1])
        D = oracle_lib.dispatch_rows(topk, E, es, n_rows, x=x, x_fp8=fp8, x_scales=sc, topk_w=w)
        _assert_receive_equal(D, brute_expand_receive(topk, E, x, fp8, sc, w), EXPAND_FIELDS)


def test_expand_receive_equals_direct_with_one_expert_per_rank(oracle_lib):
    """With one expert per rank (E = R) and distinct experts per token, each
    lane's expert row is its rank row, so the expand-mode receive arrays are
    the direct dispatch's, byte for byte, in every field."""
    w = synth.Workload("e_eq_r", 700, 256, 64, 64, 1, 6, "uniform")
    inp = synth.make_inputs(w, seed=31, with_fp8=True)
    topk = inp["topk_idx"]
    L = oracle_lib.layout(topk, w.E, w.R)
    es = oracle_lib.expert_slots(topk, w.E, L["expert_offsets"])
    n_rows = int(L["expert_offsets"][-1])
    assert n_rows == int(L["rank_offsets"][-1]) == w.T * w.K
    kw = dict(x=inp["x"], x_fp8=inp["x_fp8"], x_scales=inp["x_scales"], topk_w=inp["topk_w"])
    Dx = oracle_lib.dispatch_rows(topk, w.E, es, n_rows, **kw)
    D = oracle_lib.dispatch(topk, w.E, w.R, L["rank_offsets"], **kw)
    _assert_receive_equal(Dx, D, EXPAND_FIELDS)


def test_expand_round_trip_equals_rank_combine(oracle_lib):
    """Identity expert: combining the per-lane rows gives bit for bit what
    combining the deduplicated per-rank rows gives (same values, same order)."""
    w = synth.workload("ep32").scaled(300)
    inp = synth.make_inputs(w)
    topk = inp["topk_idx"].copy()
    topk[3, 5] = topk[3, 1]   # repeated expert
    topk[7, 2] = -1
    L = oracle_lib.layout(topk, w.E, w.R)
    es = oracle_lib.expert_slots(topk, w.E, L["expert_offsets"])
    n_rows = int(L["expert_offsets"][-1])
    Dx = oracle_lib.dispatch_rows(topk, w.E, es, n_rows, x=inp["x"], topk_w=inp["topk_w"])
    assert (Dx["recv_src"] >= 0).all()
    D = oracle_lib.dispatch(topk, w.E, w.R, L["rank_offsets"], x=inp["x"])
    C1 = oracle_lib.combine(es, inp["topk_w"], Dx["recv_x"], w.H)
    C2 = oracle_lib.combine(L["slot"], inp["topk_w"], D["recv_x"], w.H)
    np.testing.assert_array_equal(C1["out"], C2["out"])


# --------------------------------------------------------------------------
# Two-level combine (intra-group partials, then the cross-group sum)
# --------------------------------------------------------------------------

def test_two_level_combine_one_group_is_flat_combine(oracle_lib):
    w = synth.Workload("g1", 200, 256, 32, 8, 1, 4, "uniform")
    inp = synth.make_inputs(w, seed=21)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R, w.G)
    N = int(L["rank_offsets"][-1])
    y = synth.random_bf16_rows(N, w.H, seed=5)
    C2 = oracle_lib.combine_two_level(inp["topk_idx"], w.E, w.R, w.G, L["slot"], L["group_slot"],
                                      inp["topk_w"], y, w.H, int(L["group_offsets"][-1]), 3)
    C1 = oracle_lib.combine(L["slot"], inp["topk_w"], y, w.H)
    assert C2["err"] == 0
    np.testing.assert_array_equal(C2["out"], C1["out"])


def test_two_level_combine_exact_rational(oracle_lib):
    """partial[t,g] = bf16(sequential fmas of the group's lanes), out =
    bf16(sum of the partials in ascending group, fp32 adds), recomputed with
    exact rationals and torch's bf16 cast."""
    w = synth.Workload("g4", 12, 40, 16, 8, 4, 5, "uniform")
    rng = np.random.default_rng(8)
    topk = rng.integers(-1, w.E, size=(w.T, w.K)).astype(np.int64)
    topk[0] = -1
    wts = rng.standard_normal((w.T, w.K)).astype(np.float32)
    L = oracle_lib.layout(topk, w.E, w.R, w.G)
    N = int(L["rank_offsets"][-1])
    y = synth.bf16_bits(rng.standard_normal((max(N, 1), w.H)).astype(np.float32) * 2)
    C = oracle_lib.combine_two_level(topk, w.E, w.R, w.G, L["slot"], L["group_slot"], wts, y, w.H,
                                     int(L["group_offsets"][-1]), 7)
    yf = synth.bf16_to_float(y)
    epr, P = w.E // w.R, w.R // w.G
    exp = np.zeros((w.T, w.H), np.float32)
    for t in range(w.T):
        groups = sorted({(int(e) // epr) // P for e in topk[t] if e >= 0})
        for h in range(w.H):
            total = 0.0
            for g in groups:
                acc = 0.0
                for k in range(w.K):
                    e = int(topk[t, k])
                    if e < 0 or (e // epr) // P != g:
                        continue
                    acc = round_to_f32(Fraction(float(wts[t, k])) * Fraction(float(yf[L["slot"][t, k], h]))
                                       + Fraction(acc))
                part = synth.bf16_to_float(torch_bf16_bits([acc]))[0]
                total = round_to_f32(Fraction(total) + Fraction(float(part)))
            exp[t, h] = total
    np.testing.assert_array_equal(C["out"], torch_bf16_bits(exp))
    assert (C["out"][0] == 0).all()


def test_two_level_combine_round_trip_and_corruption(oracle_lib):
    w = synth.Workload("hier_small", 400, 512, 64, 16, 4, 6, "uniform")
    inp = synth.make_inputs(w, seed=22)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R, w.G)
    Hd = oracle_lib.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, L["slot"], L["group_offsets"], 4,
                                  x=inp["x"], topk_w=inp["topk_w"])
    gcap = int(L["group_offsets"][-1])
    C = oracle_lib.combine_two_level(inp["topk_idx"], w.E, w.R, w.G, L["slot"], L["group_slot"],
                                     inp["topk_w"], Hd["peer_buf"], w.H, gcap, 4, chunked=True)
    assert C["err"] == 0
    x = synth.bf16_to_float(inp["x"]).astype(np.float64)
    o = synth.bf16_to_float(C["out"]).astype(np.float64)
    assert np.abs(o - x).max() <= 2e-2 and np.linalg.norm(o - x) / np.linalg.norm(x) <= 4e-3
    flat = oracle_lib.combine(L["slot"], inp["topk_w"], Hd["peer_buf"], w.H, chunked=True, epoch=4)
    f = synth.bf16_to_float(flat["out"]).astype(np.float64)
    assert np.linalg.norm(o - f) / np.linalg.norm(f) <= 4e-3
    # a corrupted partial flag drops that (token, group) from the sum
    gb = C["group_buf"].copy()
    gb[11, 480 + 3] ^= 1
    C2 = oracle_lib.combine_two_level(inp["topk_idx"], w.E, w.R, w.G, L["slot"], L["group_slot"],
                                      inp["topk_w"], Hd["peer_buf"], w.H, gcap, 4, chunked=True,
                                      steps=2, group_buf=gb)
    assert C2["err"] == oracle_lib.ERR_FLAG
    t_bad = int(np.nonzero((L["group_slot"] == 11).any(axis=1))[0][0])
    diff = np.nonzero((C2["out"] != C["out"]).any(axis=1))[0]
    assert set(diff.tolist()) <= {t_bad}


# --------------------------------------------------------------------------
# Several source ranks: the counts exchange
# --------------------------------------------------------------------------

@pytest.mark.parametrize("S", [1, 2, 7, 32])
def test_source_counts_invariants(oracle_lib, S):
    w = synth.workload("ep32").scaled(1000)
    inp = synth.make_inputs(w, with_x=False)
    topk = inp["topk_idx"]
    L = oracle_lib.layout(topk, w.E, w.R)
    X = oracle_lib.source_counts(topk, w.E, w.R, S)
    c, off = X["counts"], X["recv_offsets"]
    np.testing.assert_array_equal(c.sum(axis=0), L["tokens_per_rank"])
    np.testing.assert_array_equal(off.reshape(-1)[:-1].reshape(w.R, S)[:, 0], L["rank_offsets"][:-1])
    assert off[-1] == L["rank_offsets"][-1]
    np.testing.assert_array_equal(np.diff(off), c.T.reshape(-1))
    # brute force: source s's rows in rank r are exactly its tokens, in order
    Ts = -(-w.T // S)
    epr = w.E // w.R
    for r in (0, 5, w.R - 1):
        toks = [t for t in range(w.T) if any(0 <= e < w.E and e // epr == r for e in topk[t])]
        for s in range(S):
            mine = [t for t in toks if t // Ts == s]
            assert c[s, r] == len(mine)
            rows = [L["slot"][t][[k for k in range(w.K) if topk[t, k] // epr == r][0]] for t in mine]
            np.testing.assert_array_equal(rows, off[r * S + s] + np.arange(len(mine)))


def _multi_source(oracle_lib, w, S, cap=None, fp8=False, corrupt=None):
    inp = synth.make_inputs(w, with_fp8=fp8)
    topk = inp["topk_idx"]
    X = oracle_lib.source_counts(topk, w.E, w.R, S)
    cap = int(X["counts"].max()) if cap is None else cap
    extra = dict(x_fp8=inp["x_fp8"], x_scales=inp["x_scales"]) if fp8 else {}
    sd = oracle_lib.source_dispatch(topk, w.E, w.R, S, cap, 5, x=inp["x"], topk_w=inp["topk_w"], **extra)
    if corrupt is not None:
        corrupt(sd["staging"])
    ce = oracle_lib.copy_epilogue(X["recv_offsets"], sd["staging"], w.H, w.K, w.R, S, cap, 5,
                                  with_fp8=fp8, with_scales=fp8)
    return inp, X, sd, ce


@pytest.mark.parametrize("S", [1, 3, 4, 32])
def test_multi_source_equals_direct(oracle_lib, S):
    """Per-source regions then the copy epilogue give exactly the direct
    dispatch's receive rows: the sources are ascending token ranges, so the
    concatenation of their regions in each rank is ascending token order."""
    w = synth.workload("tiny")
    inp, X, sd, ce = _multi_source(oracle_lib, w, S, fp8=True)
    L = oracle_lib.layout(inp["topk_idx"], w.E, w.R)
    D = oracle_lib.dispatch(inp["topk_idx"], w.E, w.R, L["rank_offsets"], x=inp["x"],
                            x_fp8=inp["x_fp8"], x_scales=inp["x_scales"], topk_w=inp["topk_w"])
    assert sd["err"] == 0 and ce["err"] == 0
    for f in ("recv_x", "recv_fp8", "recv_scales", "recv_src", "recv_topk_idx", "recv_topk_w"):
        np.testing.assert_array_equal(ce[f], D[f], err_msg=f)


def test_multi_source_staging_brute_force(oracle_lib):
    """Row j of region (r, s) holds the j-th token of source s that sends to r."""
    w = synth.workload("tiny")
    S = 3
    inp, X, sd, _ = _multi_source(oracle_lib, w, S)
    topk = inp["topk_idx"]
    Ts = -(-w.T // S)
    epr = w.E // w.R
    cap = int(X["counts"].max())
    rows = oracle_lib.unpack_rows(sd["staging"], w.H, w.K, 5)
    for s in range(S):
        for r in range(w.R):
            toks = [t for t in range(s * Ts, min((s + 1) * Ts, w.T))
                    if any(0 <= e < w.E and e // epr == r for e in topk[t])]
            base = (r * S + s) * cap
            np.testing.assert_array_equal(rows["recv_src"][base:base + len(toks)], toks)
            np.testing.assert_array_equal(rows["recv_x"][base:base + len(toks)], inp["x"][toks])
            assert not sd["staging"][base + len(toks):base + cap].any()


def test_multi_source_capacity_and_flags(oracle_lib):
    w = synth.workload("tiny")
    S = 2
    inp, X, sd, ce = _multi_source(oracle_lib, w, S)
    full_cap = int(X["counts"].max())
    # A smaller region capacity: rows j >= cap are neither sent nor copied.
    cap = full_cap - 3
    _, _, sd2, ce2 = _multi_source(oracle_lib, w, S, cap=cap)
    assert sd2["err"] == 2 and ce2["err"] == 2  # capacity
    off = X["recv_offsets"]
    for reg in range(w.R * S):
        for i in range(off[reg], off[reg + 1]):
            if i - off[reg] < cap:
                assert ce2["recv_src"][i] == ce["recv_src"][i]
            else:
                assert ce2["recv_src"][i] == -7
    # A staging row with one stale flag word is dropped and reported.
    stride = sd["stride"]
    reg = 1 * S + 1  # rank 1, source 1
    victim = reg * full_cap + 2

    def corrupt(st):
        st[victim, 512 + 480 + 4] ^= 1  # second block's flag

    _, _, _, ce3 = _multi_source(oracle_lib, w, S, corrupt=corrupt)
    i = off[reg] + 2
    assert ce3["err"] == 4 and ce3["recv_src"][i] == -7  # stale flag
    keep = np.arange(len(ce["recv_src"])) != i
    np.testing.assert_array_equal(ce3["recv_src"][keep], ce["recv_src"][keep])
    assert stride >= 1024


@pytest.mark.parametrize("S", [1, 3, 32])
def test_source_slots_against_layout_and_staging(oracle_lib, S):
    """src_slot is pinned two ways: its in-region index j equals the layout
    slot minus the region's dense start (both count earlier tokens of the same
    rank, the sources being ascending token ranges), and the staging row it
    names holds that token's record."""
    w = synth.workload("tiny")
    inp = synth.make_inputs(w)
    topk = inp["topk_idx"].copy()
    topk[5, 1] = topk[5, 0]          # a repeated expert
    topk[9, 0] = -1                  # an empty lane
    L = oracle_lib.layout(topk, w.E, w.R)
    X = oracle_lib.source_counts(topk, w.E, w.R, S)
    cap = int(X["counts"].max())
    ss = oracle_lib.source_slots(topk, w.E, w.R, S, cap)
    assert ss["err"] == 0
    Ts = -(-w.T // S)
    epr = w.E // w.R
    for t in range(w.T):
        for k in range(w.K):
            e = topk[t, k]
            if not 0 <= e < w.E:
                assert ss["src_slot"][t, k] == -1
                continue
            reg = (e // epr) * S + t // Ts
            assert ss["src_slot"][t, k] == reg * cap + L["slot"][t, k] - X["recv_offsets"][reg]
    sd = oracle_lib.source_dispatch(topk, w.E, w.R, S, cap, 3, x=inp["x"], topk_w=inp["topk_w"])
    rows = oracle_lib.unpack_rows(sd["staging"], w.H, w.K, 3)
    valid = ss["src_slot"] >= 0
    tt = np.nonzero(valid)[0]
    np.testing.assert_array_equal(rows["recv_src"][ss["src_slot"][valid]], tt)
    # capacity: lanes beyond it get -1 and the error bit
    small = oracle_lib.source_slots(topk, w.E, w.R, S, cap - 1)
    assert small["err"] == 2
    assert ((small["src_slot"] == -1) | (small["src_slot"] % (cap - 1) < cap - 1)).all()
    assert (small["src_slot"] == -1).sum() > (~valid).sum()
