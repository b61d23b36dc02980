"""The persistent one-launch kernels while another stream keeps the GPU busy.

Their workgroups wait only for batches that earlier-claimed workgroups
produce, so they need no co-residency: with a memory-bound kernel of another
stream holding the CUs, their workgroups start a few at a time, and every
call must still end with the oracle's rows and no error bit (a wait that
gave up would set EP_DEVERR_TIMEOUT). Covered: the fused two-level dispatch,
also in ring mode, the several-source send with its copy epilogue, and the
one-launch two-level combine.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_get_layout_amd import ep

pytestmark = pytest.mark.gpu

BUSY_ELEMS = 128 << 20  # fp32 elements of the side stream's buffer (512 MB)
BUSY_PASSES = 6         # in-place multiplies queued on the side stream


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


def keep_busy(buf):
    """Queue memory-bound kernels on a side stream (default priority); they
    start before the calls that follow on the current stream. Returns the
    stream and an event recorded after them."""
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(BUSY_PASSES):
            buf.mul_(1.0000001)
        end = torch.cuda.Event(enable_timing=True)
        end.record(side)
    return side, end


def report_overlap(start, done, side_end):
    """Print how the call's time span sits against the side stream's end
    (overlap is up to the scheduler, so it is reported, not asserted)."""
    print(f"call ended {side_end.elapsed_time(done):+.3f} ms after the side stream's end, took "
          f"{start.elapsed_time(done):.3f} ms", flush=True)


@pytest.mark.parametrize("ring", [0, 80])
def test_fused_two_level_beside_a_busy_stream(ring):
    w = synth.Workload("busy", 4000, 2048, 128, 32, 8, 8, "uniform")
    inp = synth.make_inputs(w, seed=31)
    print(f"fused beside a busy stream: ring={ring}", flush=True)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    L = ep.alloc_layout(shape, masks=False, groups=True)
    ws = ep.alloc_workspace(shape)
    tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
    ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
    torch.cuda.synchronize()
    N = int(L["rank_offsets"][-1].item())
    GR = int(L["group_offsets"][-1].item())
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    g_rows = ring * 2 * min(w.K, w.G) if ring else GR  # the default batch is 2 tokens
    gb = torch.zeros((g_rows, stride), dtype=torch.uint8, device="cuda")
    pb = torch.zeros((N, stride), dtype=torch.uint8, device="cuda")
    busy = torch.ones(BUSY_ELEMS, dtype=torch.float32, device="cuda")
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    for call, epoch in enumerate((21, 22)):
        pb.fill_(0xA5)
        side, side_end = keep_busy(busy)
        start, done = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        ep.ep_hierarchical_dispatch_fused(shape, L, tk, epoch, gb, g_rows, pb, N, ws, ring=ring)
        done.record()
        torch.cuda.synchronize()
        side.synchronize()
        report_overlap(start, done, side_end)
        assert ep.ep_check_errors(ws) == 0, f"call {call}"
        Hd = oracle.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], epoch,
                                  x=inp["x"], topk_w=inp["topk_w"])
        np.testing.assert_array_equal(host(pb), Hd["peer_buf"], err_msg=f"call {call}")
        if not ring:
            np.testing.assert_array_equal(host(gb), Hd["group_buf"], err_msg=f"call {call}")


def test_source_fused_beside_a_busy_stream():
    w = synth.Workload("busy_src", 3000, 2048, 64, 16, 1, 6, "uniform")
    inp = synth.make_inputs(w, seed=32)
    S = 8
    print(f"source fused beside a busy stream: S={S}", flush=True)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, 1)
    X = oracle.source_counts(inp["topk_idx"], w.E, w.R, S)
    cap = int(X["counts"].max())
    src = ep.alloc_sources(shape, S, cap)
    ws = ep.alloc_source_workspace(shape, S)
    tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
    ep.ep_source_layout(shape, tk["topk_idx"], src, ws)
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    staging = torch.zeros((w.R * S * cap, stride), dtype=torch.uint8, device="cuda")
    N = int(X["recv_offsets"][-1])
    recv = ep.alloc_recv(shape, N)
    busy = torch.ones(BUSY_ELEMS, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    side, side_end = keep_busy(busy)
    start, done = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    ep.ep_source_dispatch_fused(shape, src, tk, 9, staging, recv, N, ws)
    done.record()
    torch.cuda.synchronize()
    side.synchronize()
    report_overlap(start, done, side_end)
    assert ep.ep_check_errors(ws) == 0
    Sd = oracle.source_dispatch(inp["topk_idx"], w.E, w.R, S, cap, 9, x=inp["x"], topk_w=inp["topk_w"])
    np.testing.assert_array_equal(host(staging), Sd["staging"])
    O = oracle.layout(inp["topk_idx"], w.E, w.R, 1)
    D = oracle.dispatch(inp["topk_idx"], w.E, w.R, O["rank_offsets"], x=inp["x"], topk_w=inp["topk_w"])
    np.testing.assert_array_equal(host(recv["x"])[:N], D["recv_x"][:N])
    np.testing.assert_array_equal(host(recv["src_idx"])[:N], D["recv_src"][:N])


def test_two_level_combine_one_launch_beside_a_busy_stream():
    """The one-launch two-level combine (a partial-row capacity of 512 MB
    selects it) while the side stream holds the CUs: partial rows and outputs
    against the oracle."""
    w = synth.Workload("busy_c2", 3000, 2048, 128, 32, 8, 8, "uniform")
    inp = synth.make_inputs(w, seed=33)
    print("two-level combine beside a busy stream", flush=True)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    L = ep.alloc_layout(shape, masks=False, groups=True)
    ws = ep.alloc_workspace(shape)
    tk = dev(inp["topk_idx"])
    wd = dev(inp["topk_w"])
    ep.ep_get_layout(shape, tk, L, ws)
    torch.cuda.synchronize()
    N = int(L["rank_offsets"][-1].item())
    GR = int(L["group_offsets"][-1].item())
    y = synth.random_bf16_rows(N, w.H, seed=34)
    pstride = ep.ep_partial_row_bytes(shape)
    gcap = max(GR, -(-(512 << 20) // pstride))
    part = torch.empty((gcap, pstride), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")
    busy = torch.ones(BUSY_ELEMS, dtype=torch.float32, device="cuda")
    yd = dev(y)
    torch.cuda.synchronize()
    side, side_end = keep_busy(busy)
    start, done = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    ep.ep_combine_two_level(shape, L, tk, yd, N, 2 * w.H, ep.EP_FMT_PLAIN, 9, wd, part, gcap, 3, out, ws)
    done.record()
    torch.cuda.synchronize()
    side.synchronize()
    report_overlap(start, done, side_end)
    assert ep.ep_check_errors(ws) == 0
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    C = oracle.combine_two_level(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_slot"], inp["topk_w"], y,
                                 w.H, gcap, 9)
    np.testing.assert_array_equal(host(part)[:GR], C["group_buf"][:GR])
    np.testing.assert_array_equal(host(out), C["out"])
