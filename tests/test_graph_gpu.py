"""The path captured into a HIP graph (torch.cuda.CUDAGraph over the C ABI
calls) and replayed several times, with eager work and synchronisations
between the replays: every replay must equal the eager result bit for bit.
The graph holds kernel launches only (the per-pass error word is cleared by
the layout kernel, not by a memset)."""
import numpy as np
import pytest
import torch

import synth
from combine_get_layout_amd import ep

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.uint16)
    return torch.from_numpy(a).cuda()


def replay_and_compare(run, outputs, replays=3):
    """run() enqueues the path; outputs are the tensors it writes."""
    run()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(replays):
        for o in outputs:  # eager work between replays: clobber every output
            o.view(torch.uint8).fill_(0x5A + r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outputs, want)):
            assert torch.equal(o.view(torch.uint8), w.view(torch.uint8)), (r, i)


def test_graph_flat_step():
    w = synth.workload("ep32").scaled(1024)
    inp = synth.make_inputs(w)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, 1)
    L = ep.alloc_layout(shape, masks=True, groups=False, expand=True)
    ws = ep.alloc_workspace(shape)
    tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
    ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
    torch.cuda.synchronize()
    N = int(L["rank_offsets"][-1].item())
    NE = int(L["expert_offsets"][-1].item())
    recv = ep.alloc_recv(shape, N)
    recv_e = ep.alloc_recv(shape, NE)
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")
    out_e = torch.empty_like(out)

    def run():
        ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
        ep.ep_dispatch(shape, L, tk, recv, N, ws)
        ep.ep_combine(shape, L, recv["x"], N, 2 * w.H, ep.EP_FMT_PLAIN, 0, tk["topk_weights"], out, ws)
        ep.ep_dispatch_expand(shape, L, tk, recv_e, NE, ws)
        ep.ep_combine_expand(shape, L, recv_e["x"], NE, 2 * w.H, ep.EP_FMT_PLAIN, 0,
                             tk["topk_weights"], out_e, ws)

    outputs = [L["slot"], L["rank_offsets"], L["is_token_in_rank"], L["expert_slot"], out, out_e] + \
        [recv[k][:N] for k in recv] + [recv_e[k][:NE] for k in recv_e]
    replay_and_compare(run, outputs)
    assert ep.ep_check_errors(ws) == 0


def test_graph_two_level_step():
    w = synth.workload("hier8x8").scaled(2048)
    inp = synth.make_inputs(w)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    L = ep.alloc_layout(shape, masks=False, groups=True)
    ws = ep.alloc_workspace(shape)
    tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
    ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
    torch.cuda.synchronize()
    N = int(L["rank_offsets"][-1].item())
    GR = int(L["group_offsets"][-1].item())
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    gbuf = torch.zeros((GR, stride), dtype=torch.uint8, device="cuda")
    pbuf = torch.zeros((N, stride), dtype=torch.uint8, device="cuda")
    part = torch.zeros((GR, ep.ep_partial_row_bytes(shape)), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")
    out2 = torch.empty_like(out)

    def run():
        ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
        ep.ep_hierarchical_dispatch(shape, L, tk, 7, 3, gbuf, GR, pbuf, N, ws)
        ep.ep_combine(shape, L, pbuf, N, stride, ep.EP_FMT_CHUNKED, 7, tk["topk_weights"], out, ws)
        ep.ep_combine_two_level(shape, L, tk["topk_idx"], pbuf, N, stride, ep.EP_FMT_CHUNKED, 7,
                                tk["topk_weights"], part, GR, 3, out2, ws)

    replay_and_compare(run, [L["slot"], L["group_slot"], gbuf, pbuf, part, out, out2])
    assert ep.ep_check_errors(ws) == 0


def test_graph_fused_two_level_step():
    """The fused two-level dispatch in a graph: its flag-and-counter reset is a
    kernel node, so every replay (same epoch) starts from zeroed flags."""
    w = synth.workload("hier8x8").scaled(2048)
    inp = synth.make_inputs(w, seed=3)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    L = ep.alloc_layout(shape, masks=False, groups=True)
    ws = ep.alloc_workspace(shape)
    tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
    ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
    torch.cuda.synchronize()
    N = int(L["rank_offsets"][-1].item())
    GR = int(L["group_offsets"][-1].item())
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    gbuf = torch.zeros((GR, stride), dtype=torch.uint8, device="cuda")
    pbuf = torch.zeros((N, stride), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")

    def run():
        ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
        ep.ep_hierarchical_dispatch_fused(shape, L, tk, 9, gbuf, GR, pbuf, N, ws, tile=16)
        ep.ep_combine(shape, L, pbuf, N, stride, ep.EP_FMT_CHUNKED, 9, tk["topk_weights"], out, ws)

    replay_and_compare(run, [L["slot"], L["group_slot"], gbuf, pbuf, out])
    assert ep.ep_check_errors(ws) == 0
    assert ep.ep_check_sticky_errors(ws) == 0


def test_graph_sources_step():
    w = synth.workload("ep32").scaled(1024)
    inp = synth.make_inputs(w)
    S = 8
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, 1)
    ws = ep.alloc_source_workspace(shape, S)
    tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
    src = ep.alloc_sources(shape, S, -(-w.T // S))
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    staging = torch.zeros((w.R * S * src["capacity"], stride), dtype=torch.uint8, device="cuda")
    ep.ep_source_layout(shape, tk["topk_idx"], src, ws)
    torch.cuda.synchronize()
    N = int(src["recv_offsets"][-1].item())
    recv = ep.alloc_recv(shape, N)
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")

    def run():
        ep.ep_source_layout(shape, tk["topk_idx"], src, ws)
        ep.ep_source_dispatch(shape, src, tk, 3, staging, ws)
        ep.ep_copy_epilogue(shape, src, staging, 3, ep.EP_SEG_BF16, recv, N, ws)
        ep.ep_combine(shape, dict(slot=src["src_slot"]), staging, staging.shape[0], stride,
                      ep.EP_FMT_CHUNKED, 3, tk["topk_weights"], out, ws)

    outputs = [src["counts"], src["recv_offsets"], src["src_slot"], out] + [recv[k][:N] for k in recv]
    replay_and_compare(run, outputs)
    assert ep.ep_check_errors(ws) == 0


def test_graph_cycle_of_steps():
    """Several steps, one per input batch, captured in one graph (how the
    benchmark amortises graph launches): the steps share the workspace and the
    receive buffer, and each step's combine output must equal its eager run."""
    w = synth.workload("ep32").scaled(1024)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, 1)
    ws = ep.alloc_workspace(shape)
    batches = []
    for i in range(3):
        inp = synth.make_inputs(w, seed=100 + i)
        batches.append(dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"])))
    Ls = [ep.alloc_layout(shape, masks=True, groups=False) for _ in batches]
    cap = w.T * min(w.K, w.R)
    recv = ep.alloc_recv(shape, cap)
    outs = [torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda") for _ in batches]

    def step(i):
        tk, L = batches[i], Ls[i]
        ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
        ep.ep_dispatch(shape, L, tk, recv, cap, ws)
        ep.ep_combine(shape, L, recv["x"], cap, 2 * w.H, ep.EP_FMT_PLAIN, 0, tk["topk_weights"], outs[i], ws)

    def run():
        for i in range(len(batches)):
            step(i)

    replay_and_compare(run, outs + [L["slot"] for L in Ls])
    assert ep.ep_check_errors(ws) == 0
    assert ep.ep_check_sticky_errors(ws) == 0


def test_graph_cycle_error_in_an_earlier_step_is_kept():
    """An invalid expert id in the first batch of a two-step cycle graph:
    the second step's layout clears the per-pass error word, so only the
    word kept since ep_clear_errors still shows the error after the replay."""
    w = synth.workload("ep32").scaled(1024)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, 1)
    ws = ep.alloc_workspace(shape)
    batches = []
    for i in range(2):
        inp = synth.make_inputs(w, seed=200 + i)
        ids = inp["topk_idx"].copy()
        if i == 0:
            ids[17, 3] = w.E + 5
        batches.append(dict(x=dev(inp["x"]), topk_idx=dev(ids), topk_weights=dev(inp["topk_w"])))
    Ls = [ep.alloc_layout(shape, masks=False, groups=False) for _ in batches]
    cap = w.T * min(w.K, w.R)
    recv = ep.alloc_recv(shape, cap)
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")

    def run():
        for tk, L in zip(batches, Ls):
            ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
            ep.ep_dispatch(shape, L, tk, recv, cap, ws)
            ep.ep_combine(shape, L, recv["x"], cap, 2 * w.H, ep.EP_FMT_PLAIN, 0, tk["topk_weights"], out, ws)

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    ep.ep_clear_errors(ws)
    assert ep.ep_check_sticky_errors(ws) == 0
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    assert ep.ep_check_errors(ws) == 0  # the last step's pass is clean
    assert ep.ep_check_sticky_errors(ws) == ep.EP_DEVERR_EXPERT_ID
    ep.ep_clear_errors(ws)
    assert ep.ep_check_sticky_errors(ws) == 0


@pytest.mark.parametrize("name,fp8", [("ep32", False), ("ep32", True), ("ep256", False), ("zipf", False)])
def test_graph_cycle_full_size_against_oracle(name, fp8):
    """The full-size workload in the launch configuration the benchmark times:
    the steps of two input batches captured in one graph (shared workspace
    and receive buffer, per-batch layouts), replayed, and every output of the
    last replay compared with the CPU oracle."""
    import oracle

    oracle.build(force=False)
    w = synth.workload(name)
    print(f"graph cycle: {name} fp8={fp8}", flush=True)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, 1)
    ws = ep.alloc_workspace(shape)
    inps = [synth.make_inputs(w, seed=synth.seed_of(w) + 1000 * i, with_fp8=fp8) for i in range(2)]
    batches = [dict(x=dev(b["x"]), topk_idx=dev(b["topk_idx"]), topk_weights=dev(b["topk_w"])) for b in inps]
    if fp8:
        for tk, b in zip(batches, inps):
            tk["x_fp8"] = dev(b["x_fp8"])
            tk["x_scales"] = dev(b["x_scales"])
    Ls = [ep.alloc_layout(shape, masks=True, groups=False) for _ in batches]
    cap = w.T * min(w.K, w.R)
    recv = ep.alloc_recv(shape, cap, fp8=fp8, scales=fp8)
    outs = [torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda") for _ in batches]

    def run():
        for i, tk in enumerate(batches):
            ep.ep_get_layout(shape, tk["topk_idx"], Ls[i], ws)
            ep.ep_dispatch(shape, Ls[i], tk, recv, cap, ws)
            ep.ep_combine(shape, Ls[i], recv["x"], cap, 2 * w.H, ep.EP_FMT_PLAIN, 0, tk["topk_weights"],
                          outs[i], ws)

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for o in outs:
        o.view(torch.uint8).fill_(0xA5)
    recv["x"].view(torch.uint8).fill_(0xA5)
    torch.cuda.synchronize()
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    assert ep.ep_check_errors(ws) == 0
    assert ep.ep_check_sticky_errors(ws) == 0
    for i, b in enumerate(inps):
        O = oracle.layout(b["topk_idx"], w.E, w.R, 1)
        np.testing.assert_array_equal(Ls[i]["slot"].cpu().numpy().reshape(w.T, w.K), O["slot"])
        D = oracle.dispatch(b["topk_idx"], w.E, w.R, O["rank_offsets"], x=b["x"], topk_w=b["topk_w"],
                            x_fp8=b.get("x_fp8"), x_scales=b.get("x_scales"))
        C = oracle.combine(O["slot"], b["topk_w"], D["recv_x"], w.H)
        got = outs[i].view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, C["out"], err_msg=f"batch {i}")
        if i == len(inps) - 1:  # the receive rows hold the last batch's dispatch
            N = int(O["rank_offsets"][-1])
            rx = recv["x"].view(torch.int16).cpu().numpy().view(np.uint16)[:N]
            np.testing.assert_array_equal(rx, D["recv_x"])
            np.testing.assert_array_equal(recv["src_idx"].cpu().numpy()[:N], D["recv_src"])
            np.testing.assert_array_equal(recv["topk_idx"].cpu().numpy()[:N], D["recv_topk_idx"])
            if fp8:
                np.testing.assert_array_equal(recv["x_fp8"].cpu().numpy()[:N], D["recv_fp8"])
                np.testing.assert_array_equal(recv["x_scales"].cpu().numpy()[:N].view(np.uint32),
                                              D["recv_scales"].view(np.uint32))


@pytest.mark.parametrize("fused,ring", [pytest.param(False, 0, id="False"), pytest.param(True, 0, id="True"),
                                        pytest.param(True, 1024, id="ring1024")])
def test_graph_cycle_full_size_hier8x8_against_oracle(fused, ring):
    """hier8x8 at full size as the benchmark times it: the steps of two input
    batches (layout, two-level dispatch (two launches, or the fused one, or
    the fused one with its group rows through a ring of 1,024 batches),
    combine on the chunked scale-up rows) in one graph, replayed twice, and
    the last replay's group rows (not in ring mode), scale-up rows and
    combine outputs compared with the CPU oracle."""
    import oracle

    oracle.build(force=False)
    w = synth.workload("hier8x8")
    print(f"graph cycle: hier8x8 fused={fused} ring={ring}", flush=True)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    ws = ep.alloc_workspace(shape)
    inps = [synth.make_inputs(w, seed=synth.seed_of(w) + 1000 * i) for i in range(2)]
    batches = [dict(x=dev(b["x"]), topk_idx=dev(b["topk_idx"]), topk_weights=dev(b["topk_w"])) for b in inps]
    Ls = [ep.alloc_layout(shape, masks=False, groups=True) for _ in batches]
    Os = [oracle.layout(b["topk_idx"], w.E, w.R, w.G) for b in inps]
    Ns = [int(O["rank_offsets"][-1]) for O in Os]
    Gs = [int(O["group_offsets"][-1]) for O in Os]
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    ring_rows = ring * 2 * min(w.K, w.G)  # the default batch is 2 tokens
    if ring:
        Gs = [ring_rows] * len(Gs)
    gbuf = torch.zeros((max(Gs), stride), dtype=torch.uint8, device="cuda")
    pbuf = torch.zeros((max(Ns), stride), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda") for _ in batches]

    def run():
        for i, tk in enumerate(batches):
            e = 40 + i
            ep.ep_get_layout(shape, tk["topk_idx"], Ls[i], ws)
            if fused:
                ep.ep_hierarchical_dispatch_fused(shape, Ls[i], tk, e, gbuf, Gs[i], pbuf, Ns[i], ws, ring=ring)
            else:
                ep.ep_hierarchical_dispatch(shape, Ls[i], tk, e, 3, gbuf, Gs[i], pbuf, Ns[i], ws)
            ep.ep_combine(shape, Ls[i], pbuf, Ns[i], stride, ep.EP_FMT_CHUNKED, e, tk["topk_weights"], outs[i], ws)

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for o in outs:
        o.view(torch.uint8).fill_(0xA5)
    pbuf.fill_(0)
    torch.cuda.synchronize()
    ep.ep_clear_errors(ws)
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    assert ep.ep_check_sticky_errors(ws) == 0
    for i, b in enumerate(inps):
        O = Os[i]
        Hd = oracle.hier_dispatch(b["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], 40 + i,
                                  x=b["x"], topk_w=b["topk_w"])
        C = oracle.combine(O["slot"], b["topk_w"], Hd["peer_buf"], w.H, chunked=True, epoch=40 + i)
        got = outs[i].view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, C["out"], err_msg=f"batch {i}")
        if i == len(inps) - 1:  # the buffers hold the last batch's dispatch
            if not ring:
                np.testing.assert_array_equal(gbuf.cpu().numpy()[:Gs[i]], Hd["group_buf"])
            np.testing.assert_array_equal(pbuf.cpu().numpy()[:Ns[i]], Hd["peer_buf"])


def _capture_twice(run):
    """Run once eagerly, capture, replay twice; returns nothing (the outputs of
    the last replay are in the caller's buffers)."""
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    return g


def test_graph_cycle_full_size_ep32_expand_against_oracle():
    """ep32 with expand rows (one receive row per (token, lane), grouped by
    expert) at full size, as `bench.py --workload ep32 --expand` times it: the
    steps of two input batches in one graph, replayed twice, and every output
    of the last replay compared with the CPU oracle."""
    import oracle

    oracle.build(force=False)
    w = synth.workload("ep32")
    print("graph cycle: ep32 expand", flush=True)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, 1)
    ws = ep.alloc_workspace(shape)
    inps = [synth.make_inputs(w, seed=synth.seed_of(w) + 1000 * i) for i in range(2)]
    batches = [dict(x=dev(b["x"]), topk_idx=dev(b["topk_idx"]), topk_weights=dev(b["topk_w"])) for b in inps]
    Ls = [ep.alloc_layout(shape, masks=True, groups=False, expand=True) for _ in batches]
    cap = w.T * w.K
    recv = ep.alloc_recv(shape, cap)
    outs = [torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda") for _ in batches]

    def run():
        for i, tk in enumerate(batches):
            ep.ep_get_layout(shape, tk["topk_idx"], Ls[i], ws)
            ep.ep_dispatch_expand(shape, Ls[i], tk, recv, cap, ws)
            ep.ep_combine_expand(shape, Ls[i], recv["x"], cap, 2 * w.H, ep.EP_FMT_PLAIN, 0,
                                 tk["topk_weights"], outs[i], ws)

    ep.ep_clear_errors(ws)
    _capture_twice(run)
    assert ep.ep_check_sticky_errors(ws) == 0
    for i, b in enumerate(inps):
        O = oracle.layout(b["topk_idx"], w.E, w.R, 1)
        es = oracle.expert_slots(b["topk_idx"], w.E, O["expert_offsets"])
        np.testing.assert_array_equal(Ls[i]["expert_slot"].cpu().numpy().reshape(w.T, w.K), es)
        n_rows = int(O["expert_offsets"][-1])
        D = oracle.dispatch_rows(b["topk_idx"], w.E, es, n_rows, x=b["x"], topk_w=b["topk_w"])
        C = oracle.combine(es, b["topk_w"], D["recv_x"], w.H)
        got = outs[i].view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, C["out"], err_msg=f"batch {i}")
        if i == len(inps) - 1:
            rx = recv["x"].view(torch.int16).cpu().numpy().view(np.uint16)[:n_rows]
            np.testing.assert_array_equal(rx, D["recv_x"])
            np.testing.assert_array_equal(recv["src_idx"].cpu().numpy()[:n_rows], D["recv_src"])
            np.testing.assert_array_equal(recv["topk_idx"].cpu().numpy()[:n_rows], D["recv_topk_idx"])
            np.testing.assert_array_equal(recv["topk_weights"].cpu().numpy()[:n_rows].view(np.uint32),
                                          D["recv_topk_w"].view(np.uint32))


def test_graph_cycle_full_size_hier8x8_two_level_combine_against_oracle():
    """hier8x8 with the two-level combine at full size, as `bench.py
    --workload hier8x8 --two-level-combine` times it: two batches in one graph,
    replayed twice; the last replay's partial rows and outputs against the
    oracle."""
    import oracle

    oracle.build(force=False)
    w = synth.workload("hier8x8")
    print("graph cycle: hier8x8 two-level combine", flush=True)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    ws = ep.alloc_workspace(shape)
    inps = [synth.make_inputs(w, seed=synth.seed_of(w) + 1000 * i) for i in range(2)]
    batches = [dict(x=dev(b["x"]), topk_idx=dev(b["topk_idx"]), topk_weights=dev(b["topk_w"])) for b in inps]
    Ls = [ep.alloc_layout(shape, masks=False, groups=True) for _ in batches]
    Os = [oracle.layout(b["topk_idx"], w.E, w.R, w.G) for b in inps]
    Ns = [int(O["rank_offsets"][-1]) for O in Os]
    Gs = [int(O["group_offsets"][-1]) for O in Os]
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    gbuf = torch.zeros((max(Gs), stride), dtype=torch.uint8, device="cuda")
    pbuf = torch.zeros((max(Ns), stride), dtype=torch.uint8, device="cuda")
    part = torch.zeros((max(Gs), ep.ep_partial_row_bytes(shape)), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda") for _ in batches]

    def run():
        for i, tk in enumerate(batches):
            e = 60 + i
            ep.ep_get_layout(shape, tk["topk_idx"], Ls[i], ws)
            ep.ep_hierarchical_dispatch(shape, Ls[i], tk, e, 3, gbuf, Gs[i], pbuf, Ns[i], ws)
            ep.ep_combine_two_level(shape, Ls[i], tk["topk_idx"], pbuf, Ns[i], stride, ep.EP_FMT_CHUNKED, e,
                                    tk["topk_weights"], part, Gs[i], 3, outs[i], ws)

    ep.ep_clear_errors(ws)
    _capture_twice(run)
    assert ep.ep_check_sticky_errors(ws) == 0
    for i, b in enumerate(inps):
        O = Os[i]
        Hd = oracle.hier_dispatch(b["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], 60 + i,
                                  x=b["x"], topk_w=b["topk_w"])
        C2 = oracle.combine_two_level(b["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_slot"], b["topk_w"],
                                      Hd["peer_buf"], w.H, Gs[i], 60 + i, chunked=True)
        assert C2["err"] == 0
        got = outs[i].view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, C2["out"], err_msg=f"batch {i}")
        if i == len(inps) - 1:
            np.testing.assert_array_equal(part.cpu().numpy()[:Gs[i]], C2["group_buf"])


def test_graph_cycle_full_size_ep32_sources_against_oracle():
    """ep32 as 32 source ranks of 128 tokens at full size, as `bench.py
    --workload ep32 --sources 32` times it: source layout, send into the
    per-(rank, source) staging regions, copy epilogue and combine over the
    staging rows, for two batches in one graph replayed twice; the last
    replay's outputs against the oracle."""
    import oracle

    oracle.build(force=False)
    w = synth.workload("ep32")
    S = 32
    print("graph cycle: ep32 32 sources", flush=True)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, 1)
    ws = ep.alloc_source_workspace(shape, S)
    inps = [synth.make_inputs(w, seed=synth.seed_of(w) + 1000 * i) for i in range(2)]
    batches = [dict(x=dev(b["x"]), topk_idx=dev(b["topk_idx"]), topk_weights=dev(b["topk_w"])) for b in inps]
    srcs = [ep.alloc_sources(shape, S, -(-w.T // S)) for _ in batches]
    Xs = [oracle.source_counts(b["topk_idx"], w.E, w.R, S) for b in inps]
    cap = max(int(X["counts"].max()) for X in Xs)
    for src in srcs:
        src["capacity"] = cap
    Ns = [int(X["recv_offsets"][-1]) for X in Xs]
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    staging = torch.zeros((w.R * S * cap, stride), dtype=torch.uint8, device="cuda")
    recv = ep.alloc_recv(shape, max(Ns))
    outs = [torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda") for _ in batches]

    def run():
        for i, tk in enumerate(batches):
            e = 80 + i
            ep.ep_source_layout(shape, tk["topk_idx"], srcs[i], ws)
            ep.ep_source_dispatch(shape, srcs[i], tk, e, staging, ws)
            ep.ep_copy_epilogue(shape, srcs[i], staging, e, ep.EP_SEG_BF16, recv, Ns[i], ws)
            ep.ep_combine(shape, dict(slot=srcs[i]["src_slot"]), staging, staging.shape[0], stride,
                          ep.EP_FMT_CHUNKED, e, tk["topk_weights"], outs[i], ws)

    ep.ep_clear_errors(ws)
    _capture_twice(run)
    assert ep.ep_check_sticky_errors(ws) == 0
    for i, b in enumerate(inps):
        X = Xs[i]
        np.testing.assert_array_equal(srcs[i]["counts"].cpu().numpy(), X["counts"])
        np.testing.assert_array_equal(srcs[i]["recv_offsets"].cpu().numpy(), X["recv_offsets"])
        sl = oracle.source_slots(b["topk_idx"], w.E, w.R, S, cap)["src_slot"]
        np.testing.assert_array_equal(srcs[i]["src_slot"].cpu().numpy().reshape(w.T, w.K), sl)
        Sd = oracle.source_dispatch(b["topk_idx"], w.E, w.R, S, cap, 80 + i, x=b["x"], topk_w=b["topk_w"])
        C = oracle.combine(sl, b["topk_w"], Sd["staging"], w.H, chunked=True, epoch=80 + i)
        got = outs[i].view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, C["out"], err_msg=f"batch {i}")
        if i == len(inps) - 1:
            Ep = oracle.copy_epilogue(X["recv_offsets"], Sd["staging"], w.H, w.K, w.R, S, cap, 80 + i)
            n = Ns[i]
            rx = recv["x"].view(torch.int16).cpu().numpy().view(np.uint16)[:n]
            np.testing.assert_array_equal(rx, Ep["recv_x"])
            np.testing.assert_array_equal(recv["src_idx"].cpu().numpy()[:n], Ep["recv_src"])
            np.testing.assert_array_equal(recv["topk_idx"].cpu().numpy()[:n], Ep["recv_topk_idx"])
