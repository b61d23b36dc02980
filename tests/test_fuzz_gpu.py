"""Seeded random shapes through every entry point, each compared with the CPU
oracle: layout (all outputs, groups and expand rows; also through the
allocation-free entry point), dispatch with a random subset of payload
pieces, combine, the two-level chunked dispatch (two launches, and the fused
one-launch form with a random batch size, also with its group rows through a
ring of a random number of batches) with the flat and the two-level
combine, expand-mode dispatch and combine, and the several-source send and
copy epilogue in one launch with a random source count.

The shapes are drawn from a fixed seed list (200 seeds; EP_FUZZ_SEEDS sets
another count), so a failure names a case that
reproduces exactly. Sizes stay small (the oracle runs each in milliseconds)
but ragged: T, H, K, E, R and G take values that are not powers of two, and
the routing mixes distinct top-k with skipped lanes and repeated experts.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from combine_get_layout_amd import ep

pytestmark = pytest.mark.gpu

SEEDS = list(range(1, 1 + int(os.environ.get("EP_FUZZ_SEEDS", "200"))))


@pytest.fixture(scope="module", autouse=True)
def _ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()
    oracle.build(force=False)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.uint16)
    return torch.from_numpy(a).cuda()


def host(t):
    if t.dtype == torch.uint16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def poison(t):
    t.view(torch.uint8).fill_(0xAB)
    return t


def draw_case(seed):
    """A random shape and routing within the library's limits."""
    rng = np.random.default_rng(10_000 + seed)
    R = int(rng.choice([1, 2, 3, 5, 6, 8, 12, 16, 24, 40, 64]))
    G = int(rng.choice([g for g in range(1, R + 1) if R % g == 0]))
    epr = int(rng.choice([1, 2, 3, 4, 8]))
    E = R * epr
    r = rng.random()
    if r < 0.15:
        K = int(rng.integers(17, 65))
    elif r < 0.4:
        K = int(rng.integers(1, min(16, E + 1) + 1))
    else:
        K = int(rng.integers(1, min(8, E) + 1))
    T = int(rng.integers(1, 900))
    fp8 = bool(rng.random() < 0.5)
    H = int(rng.choice([128, 256, 384, 1024, 1536])) if fp8 else int(8 * rng.integers(1, 200))
    if rng.random() < 0.5 and K <= E:
        topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
        holes = rng.random((T, K)) < 0.05
        topk[holes] = -1
    else:
        topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    x = synth.random_bf16_rows(T, H, seed=seed)
    w = rng.standard_normal((T, K)).astype(np.float32)
    case = dict(T=T, H=H, K=K, E=E, R=R, G=G, topk=topk, x=x, w=w, fp8=fp8, seed=seed)
    if fp8:
        case["x_fp8"] = rng.integers(0, 256, size=(T, H)).astype(np.uint8)
        case["x_scales"] = rng.standard_normal((T, H // 128)).astype(np.float32)
    return case


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_all_entry_points(seed):
    c = draw_case(seed)
    T, H, K, E, R, G = c["T"], c["H"], c["K"], c["E"], c["R"], c["G"]
    topk, x, w = c["topk"], c["x"], c["w"]
    print(f"case seed={seed} T={T} H={H} K={K} E={E} R={R} G={G} fp8={c['fp8']}", flush=True)
    shape = ep.make_shape(T, H, K, E, R, G)
    ws = ep.alloc_workspace(shape)
    tk = dev(topk)
    wd = dev(w)

    # layout, every output (groups, masks, expand rows)
    L = ep.alloc_layout(shape, masks=True, groups=True, expand=True)
    for t in L.values():
        poison(t)
    ep.ep_get_layout(shape, tk, L, ws)
    O = oracle.layout(topk, E, R, G)
    for k in ("tokens_per_expert", "tokens_per_rank", "tokens_per_group", "expert_offsets",
              "rank_offsets", "group_offsets", "is_token_in_rank", "is_token_in_group",
              "slot", "group_slot"):
        np.testing.assert_array_equal(host(L[k]).reshape(O[k].shape), O[k], err_msg=k)
    es = oracle.expert_slots(topk, E, O["expert_offsets"])
    np.testing.assert_array_equal(host(L["expert_slot"]).reshape(T, K), es, err_msg="expert_slot")
    assert ep.ep_check_errors(ws) == 0
    # the allocation-free layout gives the same outputs
    L2 = ep.alloc_layout(shape, masks=True, groups=True, expand=True)
    for t in L2.values():
        poison(t)
    ep.ep_get_layout_noalloc(shape, tk, L2, ws)
    for k in L:
        assert torch.equal(L2[k].view(torch.uint8), L[k].view(torch.uint8)), "noalloc " + k
    assert ep.ep_check_errors(ws) == 0
    N = int(O["rank_offsets"][R])
    G_rows = int(O["group_offsets"][G])

    # dispatch with a random subset of the payload pieces
    rng = np.random.default_rng(seed)
    want_x = bool(rng.random() < 0.8) or not c["fp8"]
    want_fp8 = c["fp8"] and bool(rng.random() < 0.7)
    want_sc = c["fp8"] and bool(rng.random() < 0.7)
    meta = bool(rng.random() < 0.8)
    tokens = dict(topk_idx=tk, topk_weights=wd)
    if want_x:
        tokens["x"] = dev(x)
    if want_fp8:
        tokens["x_fp8"] = dev(c["x_fp8"])
    if want_sc:
        tokens["x_scales"] = dev(c["x_scales"])
    recv = ep.alloc_recv(shape, max(N, 1), x=want_x, fp8=want_fp8, scales=want_sc, meta=meta)
    for t in recv.values():
        poison(t)
    ep.ep_dispatch(shape, L, tokens, recv, N, ws)
    D = oracle.dispatch(topk, E, R, O["rank_offsets"], x=x if want_x else None,
                        x_fp8=c["x_fp8"] if want_fp8 else None,
                        x_scales=c["x_scales"] if want_sc else None, topk_w=w, with_meta=meta)
    for g, o in [("x", "recv_x"), ("x_fp8", "recv_fp8"), ("x_scales", "recv_scales"),
                 ("src_idx", "recv_src"), ("topk_idx", "recv_topk_idx"), ("topk_weights", "recv_topk_w")]:
        if g in recv:
            np.testing.assert_array_equal(host(recv[g])[:N].view(np.uint8), D[o][:N].view(np.uint8),
                                          err_msg=g)

    # combine of stand-in expert outputs
    y = synth.random_bf16_rows(max(N, 1), H, seed=seed + 7)
    out = poison(torch.empty((T, H), dtype=torch.uint16, device="cuda"))
    ep.ep_combine(shape, L, dev(y), N, 2 * H, ep.EP_FMT_PLAIN, 0, wd, out, ws)
    np.testing.assert_array_equal(host(out), oracle.combine(O["slot"], w, y[:N], H)["out"])
    assert ep.ep_check_errors(ws) == 0

    # two-level chunked dispatch, flat combine on its rows, two-level combine
    epoch = 100 + seed
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    gb = poison(torch.empty((max(G_rows, 1), stride), dtype=torch.uint8, device="cuda"))
    pb = poison(torch.empty((max(N, 1), stride), dtype=torch.uint8, device="cuda"))
    htok = dict(x=dev(x), topk_idx=tk, topk_weights=wd)
    ep.ep_hierarchical_dispatch(shape, L, htok, epoch, ep.EP_HIER_SCALEOUT | ep.EP_HIER_FORWARD,
                                gb, G_rows, pb, N, ws)
    Hd = oracle.hier_dispatch(topk, E, R, G, O["slot"], O["group_offsets"], epoch, x=x, topk_w=w)
    np.testing.assert_array_equal(host(gb)[:G_rows], Hd["group_buf"])
    np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])
    # the fused one-launch form, a random batch size, a new epoch
    tile = int(rng.choice([4, 7, 16, 33, 64]))
    gbf = poison(torch.empty_like(gb))
    pbf = poison(torch.empty_like(pb))
    ep.ep_hierarchical_dispatch_fused(shape, L, htok, epoch + 1000, gbf, G_rows, pbf, N, ws, tile=tile)
    Hf = oracle.hier_dispatch(topk, E, R, G, O["slot"], O["group_offsets"], epoch + 1000, x=x, topk_w=w)
    np.testing.assert_array_equal(host(gbf)[:G_rows], Hf["group_buf"], err_msg=f"fused tile {tile}")
    np.testing.assert_array_equal(host(pbf)[:N], Hf["peer_buf"], err_msg=f"fused tile {tile}")
    assert ep.ep_check_errors(ws) == 0
    # ring mode (its own generator, so the draws above and below stay those of the seed)
    rr = np.random.default_rng(20_000 + seed)
    rtile, ring = int(rr.choice([1, 2, 3])), int(rr.choice([65, 80, 129]))
    ring_rows = ring * rtile * min(K, G)
    gbr = torch.empty((ring_rows, stride), dtype=torch.uint8, device="cuda")
    pbr = poison(torch.empty_like(pb))
    ep.ep_hierarchical_dispatch_fused(shape, L, htok, epoch + 1000, gbr, ring_rows, pbr, N, ws, tile=rtile,
                                      ring=ring)
    np.testing.assert_array_equal(host(pbr)[:N], Hf["peer_buf"], err_msg=f"ring {ring} tile {rtile}")
    assert ep.ep_check_errors(ws) == 0
    del gbr, pbr
    ep.ep_combine(shape, L, pb, N, stride, ep.EP_FMT_CHUNKED, epoch, wd, out, ws)
    C = oracle.combine(O["slot"], w, Hd["peer_buf"], H, chunked=True, epoch=epoch)
    np.testing.assert_array_equal(host(out), C["out"])
    pstride = ep.ep_partial_row_bytes(shape)
    part = poison(torch.empty((max(G_rows, 1), pstride), dtype=torch.uint8, device="cuda"))
    ep.ep_combine_two_level(shape, L, tk, pb, N, stride, ep.EP_FMT_CHUNKED, epoch, wd, part, G_rows, 3,
                            out, ws)
    C2 = oracle.combine_two_level(topk, E, R, G, O["slot"], O["group_slot"], w, Hd["peer_buf"], H,
                                  G_rows, epoch, chunked=True)
    np.testing.assert_array_equal(host(part)[:G_rows], C2["group_buf"])
    np.testing.assert_array_equal(host(out), C2["out"])
    assert ep.ep_check_errors(ws) == 0

    # expand rows: dispatch and combine
    n_rows = int(O["expert_offsets"][E])
    rx = ep.alloc_recv(shape, max(n_rows, 1), meta=True)
    for t in rx.values():
        poison(t)
    ep.ep_dispatch_expand(shape, L, htok, rx, n_rows, ws)
    Dx = oracle.dispatch_rows(topk, E, es, n_rows, x=x, topk_w=w)
    for g, o in [("x", "recv_x"), ("src_idx", "recv_src"), ("topk_idx", "recv_topk_idx"),
                 ("topk_weights", "recv_topk_w")]:
        np.testing.assert_array_equal(host(rx[g])[:n_rows].view(np.uint8), Dx[o][:n_rows].view(np.uint8),
                                      err_msg="expand " + g)
    yx = synth.random_bf16_rows(max(n_rows, 1), H, seed=seed + 11)
    ep.ep_combine_expand(shape, L, dev(yx), n_rows, 2 * H, ep.EP_FMT_PLAIN, 0, wd, out, ws)
    np.testing.assert_array_equal(host(out), oracle.combine(es, w, yx[:n_rows], H)["out"])
    assert ep.ep_check_errors(ws) == 0

    # several sources: send and copy epilogue in one launch
    S = int(rng.choice([1, 2, 3, 5, 8]))
    s1 = ep.make_shape(T, H, K, E, R, 1)
    X = oracle.source_counts(topk, E, R, S)
    cap = max(int(X["counts"].max(initial=0)), 1)
    src = ep.alloc_sources(s1, S, cap)
    wss = ep.alloc_source_workspace(s1, S)
    ep.ep_source_layout(s1, tk, src, wss)
    staging = torch.zeros((R * S * cap, ep.ep_chunked_record_bytes(s1, ep.EP_SEG_BF16)), dtype=torch.uint8,
                          device="cuda")
    n_src = int(X["recv_offsets"][-1])
    rs = ep.alloc_recv(s1, max(n_src, 1), meta=True)
    for t in rs.values():
        poison(t)
    ep.ep_source_dispatch_fused(s1, src, htok, epoch + 2000, staging, rs, n_src, wss)
    Sd = oracle.source_dispatch(topk, E, R, S, cap, epoch + 2000, x=x, topk_w=w)
    np.testing.assert_array_equal(host(staging), Sd["staging"], err_msg=f"sources {S}")
    Ds = oracle.dispatch(topk, E, R, O["rank_offsets"], x=x, topk_w=w)
    for g, o in [("x", "recv_x"), ("src_idx", "recv_src"), ("topk_idx", "recv_topk_idx"),
                 ("topk_weights", "recv_topk_w")]:
        np.testing.assert_array_equal(host(rs[g])[:n_src].view(np.uint8), Ds[o][:n_src].view(np.uint8),
                                      err_msg=f"sources {S} " + g)
    assert ep.ep_check_errors(wss) == 0
