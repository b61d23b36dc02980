"""Send and copy epilogue of several source ranks in one launch
(ep_source_dispatch_fused), against the CPU oracle: the staging rows byte for
byte against the oracle's send step, the dense receive rows against its copy
epilogue and its direct dispatch, and equality with the two-call path."""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_get_layout_amd import ep

pytestmark = pytest.mark.gpu


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


def poison(t, byte=0xAB):
    t.view(torch.uint8).fill_(byte)
    return t


def run(w, inp, S, fp8=False, cap=None, recv_rows=None, epoch=11, fused=True):
    """Source layout, then the fused call (or the send and the epilogue)."""
    topk = inp["topk_idx"]
    T, K = topk.shape
    print(f"source fused={fused}: T={T} H={w.H} K={K} E={w.E} R={w.R} S={S} fp8={fp8}", flush=True)
    shape = ep.make_shape(T, w.H, K, w.E, w.R, 1)
    X = oracle.source_counts(topk, w.E, w.R, S)
    cap = max(int(X["counts"].max(initial=0)), 1) if cap is None else cap
    src = ep.alloc_sources(shape, S, cap)
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
    N = int(X["recv_offsets"][-1])
    rows = N if recv_rows is None else recv_rows
    recv = ep.alloc_recv(shape, max(rows, 1), fp8=fp8, scales=fp8)
    for t in recv.values():
        poison(t)
    if fused:
        ep.ep_source_dispatch_fused(shape, src, tokens, epoch, staging, recv, rows, ws)
    else:
        ep.ep_source_dispatch(shape, src, tokens, epoch, staging, ws)
        ep.ep_copy_epilogue(shape, src, staging, epoch, seg, recv, rows, ws)
    torch.cuda.synchronize()
    return dict(shape=shape, src=src, ws=ws, staging=staging, recv=recv, N=N, rows=rows, cap=cap,
                X=X, epoch=epoch)


def check_recv(recv, D, rows):
    pairs = [("x", "recv_x"), ("x_fp8", "recv_fp8"), ("x_scales", "recv_scales"),
             ("src_idx", "recv_src"), ("topk_idx", "recv_topk_idx"), ("topk_weights", "recv_topk_w")]
    for g, o in pairs:
        if g in recv and D.get(o) is not None:
            np.testing.assert_array_equal(host(recv[g])[:rows].view(np.uint8), D[o][:rows].view(np.uint8),
                                          err_msg=g)


def check_against_oracle(w, inp, S, c, fp8=False, staging=True):
    topk = inp["topk_idx"]
    extra = dict(x_fp8=inp["x_fp8"], x_scales=inp["x_scales"]) if fp8 else {}
    if staging:
        Sd = oracle.source_dispatch(topk, w.E, w.R, S, c["cap"], c["epoch"], x=inp["x"],
                                    topk_w=inp["topk_w"], **extra)
        np.testing.assert_array_equal(host(c["staging"]), Sd["staging"])
    O = oracle.layout(topk, w.E, w.R, 1)
    D = oracle.dispatch(topk, w.E, w.R, O["rank_offsets"], x=inp["x"], topk_w=inp["topk_w"], **extra)
    check_recv(c["recv"], D, c["N"])


def test_source_fused_small_first():
    w = synth.workload("tiny")
    inp = synth.make_inputs(w, with_fp8=True)
    c = run(w, inp, 3, fp8=True)
    check_against_oracle(w, inp, 3, c, fp8=True)
    assert ep.ep_check_errors(c["ws"]) == 0


@pytest.mark.parametrize("T,H,K,E,R,S", [
    (0, 264, 8, 64, 8, 4),           # no tokens
    (5, 264, 2, 16, 4, 8),           # more sources than tokens (empty sources)
    (300, 264, 3, 12, 6, 7),         # ragged sources
    (1001, 264, 20, 64, 16, 3),      # K above 16, duplicates and -1
    (513, 264, 4, 16, 1, 2),         # one rank
    (64, 16384, 8, 64, 16, 4),       # records longer than the 32 blocks held at once
    (700, 2048, 8, 128, 32, 32),     # many batches, far more than the lag
])
def test_source_fused_edges(T, H, K, E, R, S):
    w = synth.Workload("edge", T, H, E, R, 1, K, "uniform")
    rng = np.random.default_rng(T + 13 * S)
    inp = dict(x=rng.integers(0, 65536, size=(T, H)).astype(np.uint16),
               topk_idx=rng.integers(-1, E, size=(T, K)).astype(np.int64),
               topk_w=rng.standard_normal((T, K)).astype(np.float32))
    c = run(w, inp, S)
    check_against_oracle(w, inp, S, c, staging=T > 0)
    assert ep.ep_check_errors(c["ws"]) == 0


@pytest.mark.parametrize("name,S", [("ep32", 32), ("zipf", 16)])
def test_source_fused_full_size(name, S):
    """Full size: the dense rows against the oracle's direct dispatch (equal to
    its copy epilogue, a pinned identity) and sampled staging rows against the
    oracle's chunked record of their token."""
    w = synth.workload(name)
    inp = synth.make_inputs(w)
    topk = inp["topk_idx"]
    c = run(w, inp, S)
    check_against_oracle(w, inp, S, c, staging=False)
    assert ep.ep_check_errors(c["ws"]) == 0
    slot = oracle.source_slots(topk, w.E, w.R, S, c["cap"])["src_slot"]
    np.testing.assert_array_equal(host(c["src"]["src_slot"]).reshape(topk.shape), slot)
    rng = np.random.default_rng(9)
    for t in rng.choice(w.T, size=24, replace=False):
        k = int(np.argmax(slot[t] >= 0))
        if slot[t, k] < 0:
            continue
        want = oracle.chunk(oracle.pack_record(int(t), topk, w.E, x=inp["x"], topk_w=inp["topk_w"]), c["epoch"])
        np.testing.assert_array_equal(host(c["staging"][int(slot[t, k])]), want)


def test_source_fused_equals_two_calls():
    w = synth.Workload("eq", 1500, 1024, 64, 16, 1, 6, "uniform")
    inp = synth.make_inputs(w, seed=21, with_fp8=True)
    a = run(w, inp, 5, fp8=True, fused=True)
    b = run(w, inp, 5, fp8=True, fused=False)
    np.testing.assert_array_equal(host(a["staging"]), host(b["staging"]))
    for k in a["recv"]:
        np.testing.assert_array_equal(host(a["recv"][k]).view(np.uint8), host(b["recv"][k]).view(np.uint8),
                                      err_msg=k)
    assert ep.ep_check_errors(a["ws"]) == 0


def test_source_fused_capacities():
    """A source capacity below the counts (the layout reports it; the rows of
    those lanes are neither sent nor unpacked) and a receive capacity below N
    (rows past it skipped with EP_DEVERR_CAPACITY, the others written)."""
    w = synth.workload("tiny")
    inp = synth.make_inputs(w, seed=77)
    topk = inp["topk_idx"]
    S = 2
    X = oracle.source_counts(topk, w.E, w.R, S)
    cap = int(X["counts"].max()) - 3
    N = int(X["recv_offsets"][-1])
    c = run(w, inp, S, cap=cap, recv_rows=N - 5)
    assert ep.ep_check_errors(c["ws"]) == ep.EP_DEVERR_CAPACITY
    Sd = oracle.source_dispatch(topk, w.E, w.R, S, cap, c["epoch"], x=inp["x"], topk_w=inp["topk_w"])
    np.testing.assert_array_equal(host(c["staging"]), Sd["staging"])
    Ce = oracle.copy_epilogue(X["recv_offsets"], Sd["staging"], w.H, w.K, w.R, S, cap, c["epoch"],
                              recv_cap=N - 5)
    written = Ce["recv_src"] != -7
    got_src = host(c["recv"]["src_idx"])[:N - 5]
    np.testing.assert_array_equal(got_src[written[:N - 5]], Ce["recv_src"][:N - 5][written[:N - 5]])
    assert (got_src[~written[:N - 5]].view(np.uint32) == 0xABABABAB).all()
    np.testing.assert_array_equal(host(c["recv"]["x"])[:N - 5][written[:N - 5]],
                                  Ce["recv_x"][:N - 5][written[:N - 5]])


def test_source_fused_graph_replays():
    """Source layout, the fused call and the combine over the staging rows in
    a graph, replayed three times with eager work between: every replay
    equals the eager result."""
    w = synth.workload("ep32").scaled(1024)
    inp = synth.make_inputs(w, seed=4)
    S = 8
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, 1)
    X = oracle.source_counts(inp["topk_idx"], w.E, w.R, S)
    cap = int(X["counts"].max())
    src = ep.alloc_sources(shape, S, cap)
    ws = ep.alloc_source_workspace(shape, S)
    tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    staging = torch.zeros((w.R * S * cap, stride), dtype=torch.uint8, device="cuda")
    N = int(X["recv_offsets"][-1])
    recv = ep.alloc_recv(shape, N)
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")

    def step():
        ep.ep_source_layout(shape, tk["topk_idx"], src, ws)
        ep.ep_source_dispatch_fused(shape, src, tk, 5, staging, recv, N, ws)
        ep.ep_combine(shape, dict(slot=src["src_slot"]), staging, staging.shape[0], stride,
                      ep.EP_FMT_CHUNKED, 5, tk["topk_weights"], out, ws)

    outs = [staging, out] + [recv[k] for k in recv]
    step()
    torch.cuda.synchronize()
    want = [host(t).copy() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs[1:]:  # every receive row and output is rewritten (staging rows past the counts are not)
            poison(t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            np.testing.assert_array_equal(host(a).view(np.uint8), b.view(np.uint8), err_msg=f"replay {rep}")
        torch.zeros(1 << 20, device="cuda").sum().item()  # eager work between replays
    assert ep.ep_check_sticky_errors(ws) == 0
