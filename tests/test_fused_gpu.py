"""The fused two-level dispatch (ep_hierarchical_dispatch_fused: both steps in
one persistent launch, forwarders taking each batch of records as soon as
its flag is published) against the CPU oracle's two-level dispatch: group
rows and scale-up rows byte for byte. Also: ragged batches and several batch
sizes, the FP8 + scales payload, repeated calls on the same buffers with new
epochs, the full hier8x8 workload, and the bounded wait: with one batch's
flag withheld by the host the wait gives up, the error bit is set, every
other row is still right and the launch ends. Ring mode (group rows through
a ring of batches that the forwarders free): the scale-up rows byte for byte,
at several ring sizes, with a withheld flag, and at full size."""
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
    return t.cpu().numpy()


def setup(w, inp, fp8=False):
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    L = ep.alloc_layout(shape, masks=False, groups=True)
    ws = ep.alloc_workspace(shape)
    tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
    if fp8:
        tk["x_fp8"] = dev(inp["x_fp8"])
        tk["x_scales"] = dev(inp["x_scales"])
    ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
    torch.cuda.synchronize()
    N = int(L["rank_offsets"][-1].item())
    GR = int(L["group_offsets"][-1].item())
    seg = ep.EP_SEG_BF16 | ((ep.EP_SEG_FP8 | ep.EP_SEG_SCALES) if fp8 else 0)
    stride = ep.ep_chunked_record_bytes(shape, seg)
    gb = torch.full((max(GR, 1), stride), 0xA5, dtype=torch.uint8, device="cuda")
    pb = torch.full((max(N, 1), stride), 0xA5, dtype=torch.uint8, device="cuda")
    return shape, L, ws, tk, gb, pb, GR, N


def expected(w, inp, epoch, fp8=False):
    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    Hd = oracle.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, O["slot"], O["group_offsets"], epoch,
                              x=inp["x"], x_fp8=inp.get("x_fp8") if fp8 else None,
                              x_scales=inp.get("x_scales") if fp8 else None, topk_w=inp["topk_w"])
    assert Hd["err"] == 0
    return O, Hd


def run_case(w, tile, fp8=False, seed=None, epoch=5, ids=None):
    inp = synth.make_inputs(w, seed=seed, with_fp8=fp8)
    if ids is not None:
        inp["topk_idx"] = ids
    print(f"fused: T={w.T} H={w.H} K={w.K} E={w.E} R={w.R} G={w.G} tile={tile} fp8={fp8}", flush=True)
    shape, L, ws, tk, gb, pb, GR, N = setup(w, inp, fp8)
    ep.ep_hierarchical_dispatch_fused(shape, L, tk, epoch, gb, GR, pb, N, ws, tile=tile)
    torch.cuda.synchronize()
    O, Hd = expected(w, inp, epoch, fp8)
    np.testing.assert_array_equal(host(gb)[:GR], Hd["group_buf"])
    np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])
    assert ep.ep_check_errors(ws) == 0


def test_fused_small_first():
    """A small shape first: 13 batches of 16 tokens, 4 groups of 2 ranks."""
    run_case(synth.Workload("fz_small", 200, 256, 32, 8, 4, 4, "uniform"), tile=16)


@pytest.mark.parametrize("T,H,K,E,R,G,tile,fp8", [
    (1000, 512, 6, 64, 16, 4, 64, False),     # ragged last batch
    (1000, 512, 6, 64, 16, 4, 4, False),      # small batches
    (1000, 512, 6, 64, 16, 4, 2, False),      # the default batch: 500 batches, many more than the lag
    (300, 256, 4, 32, 8, 4, 1, False),        # one token per batch
    (50, 512, 6, 64, 16, 4, 64, False),       # one batch holds every token
    (777, 1024, 8, 128, 32, 8, 16, True),     # FP8 + scales, many small batches
    (300, 512, 4, 32, 8, 1, 32, False),       # one group holding every rank
    (257, 264, 3, 24, 8, 8, 16, False),       # one peer per group
    (129, 1032, 12, 48, 16, 4, 64, False),    # K > 8, row not a whole number of blocks
    (200, 256, 64, 1024, 256, 256, 64, False),  # K = 64, 256 groups of one rank
    (40, 16384, 8, 64, 16, 4, 16, False),     # records of several 32-block pieces
    (1, 8, 1, 4, 2, 2, 16, False),            # one token, one lane
])
def test_fused_shapes(T, H, K, E, R, G, tile, fp8):
    run_case(synth.Workload("fz", T, H, E, R, G, K, "uniform"), tile=tile, fp8=fp8)


def test_fused_skipped_and_repeated_lanes():
    w = synth.Workload("fz_rand", 400, 256, 20, 10, 5, 5, "uniform")
    ids = np.random.default_rng(5).integers(-1, w.E, size=(w.T, w.K)).astype(np.int64)
    run_case(w, tile=32, ids=ids)


def test_fused_repeated_calls_new_epochs():
    """Same buffers and workspace, three calls with new epochs and new
    tokens: the flags and counters of one call never satisfy the next."""
    w = synth.Workload("fz_rep", 900, 512, 64, 16, 4, 6, "uniform")
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    ws = ep.alloc_workspace(shape)
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    cap = w.T * min(w.K, w.R)
    gb = torch.zeros((cap, stride), dtype=torch.uint8, device="cuda")
    pb = torch.zeros((cap, stride), dtype=torch.uint8, device="cuda")
    L = ep.alloc_layout(shape, masks=False, groups=True)
    for call, epoch in enumerate((3, 4, 5)):
        inp = synth.make_inputs(w, seed=40 + call)
        tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
        ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
        ep.ep_hierarchical_dispatch_fused(shape, L, tk, epoch, gb, cap, pb, cap, ws, tile=32)
        torch.cuda.synchronize()
        O, Hd = expected(w, inp, epoch)
        GR, N = Hd["group_buf"].shape[0], Hd["peer_buf"].shape[0]
        np.testing.assert_array_equal(host(gb)[:GR], Hd["group_buf"], err_msg=f"call {call}")
        np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"], err_msg=f"call {call}")
        assert ep.ep_check_errors(ws) == 0


def test_fused_same_epoch_twice():
    """Two calls with the same epoch on one workspace and new tokens: the
    call's reset kernel clears the previous call's flags, so no batch of the
    second call is forwarded before it is written."""
    w = synth.Workload("fz_same", 1200, 512, 64, 16, 4, 6, "uniform")
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    ws = ep.alloc_workspace(shape)
    stride = ep.ep_chunked_record_bytes(shape, ep.EP_SEG_BF16)
    cap = w.T * min(w.K, w.R)
    gb = torch.zeros((cap, stride), dtype=torch.uint8, device="cuda")
    pb = torch.zeros((cap, stride), dtype=torch.uint8, device="cuda")
    L = ep.alloc_layout(shape, masks=False, groups=True)
    for call in range(2):
        inp = synth.make_inputs(w, seed=60 + call)
        tk = dict(x=dev(inp["x"]), topk_idx=dev(inp["topk_idx"]), topk_weights=dev(inp["topk_w"]))
        ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
        ep.ep_hierarchical_dispatch_fused(shape, L, tk, 7, gb, cap, pb, cap, ws)
        torch.cuda.synchronize()
        O, Hd = expected(w, inp, 7)
        GR, N = Hd["group_buf"].shape[0], Hd["peer_buf"].shape[0]
        np.testing.assert_array_equal(host(gb)[:GR], Hd["group_buf"], err_msg=f"call {call}")
        np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"], err_msg=f"call {call}")
        assert ep.ep_check_errors(ws) == 0


def test_fused_equals_two_launch_path():
    w = synth.Workload("fz_eq", 2000, 2048, 128, 32, 8, 8, "uniform")
    inp = synth.make_inputs(w, seed=77)
    shape, L, ws, tk, gb, pb, GR, N = setup(w, inp)
    ep.ep_hierarchical_dispatch_fused(shape, L, tk, 21, gb, GR, pb, N, ws)
    gb2, pb2 = torch.full_like(gb, 0x11), torch.full_like(pb, 0x11)
    ep.ep_hierarchical_dispatch(shape, L, tk, 21, 3, gb2, GR, pb2, N, ws)
    torch.cuda.synchronize()
    assert torch.equal(gb[:GR], gb2[:GR]) and torch.equal(pb[:N], pb2[:N])
    assert ep.ep_check_errors(ws) == 0


def test_fused_withheld_flag_times_out():
    """The host withholds batch 3's flag: the forwarder's bounded wait gives
    up after 2 ms, EP_DEVERR_TIMEOUT is set, batch 3's scale-up rows are
    left unwritten, and every other row is the oracle's."""
    w = synth.Workload("fz_hold", 1000, 512, 64, 16, 4, 6, "uniform")
    inp = synth.make_inputs(w, seed=8)
    tile, held, epoch = 64, 3, 12
    shape, L, ws, tk, gb, pb, GR, N = setup(w, inp)
    ep.ep_hierarchical_dispatch_fused(shape, L, tk, epoch, gb, GR, pb, N, ws, tile=tile,
                                      timeout_us=2000, withhold=held)
    torch.cuda.synchronize()
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_TIMEOUT
    O, Hd = expected(w, inp, epoch)
    np.testing.assert_array_equal(host(gb)[:GR], Hd["group_buf"])  # production is complete
    sl = O["slot"][held * tile:(held + 1) * tile]
    held_rows = np.unique(sl[sl >= 0])
    keep = np.setdiff1d(np.arange(N), held_rows)
    got = host(pb)[:N]
    np.testing.assert_array_equal(got[keep], Hd["peer_buf"][keep])
    assert (got[held_rows] == 0xA5).all()  # never forwarded
    # the next call (new epoch, nothing withheld) is whole again
    ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
    ep.ep_hierarchical_dispatch_fused(shape, L, tk, epoch + 1, gb, GR, pb, N, ws, tile=tile)
    torch.cuda.synchronize()
    assert ep.ep_check_errors(ws) == 0
    O, Hd = expected(w, inp, epoch + 1)
    np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])


def test_fused_full_hier8x8():
    w = synth.workload("hier8x8")
    inp = synth.make_inputs(w)
    print("fused: full hier8x8", flush=True)
    shape, L, ws, tk, gb, pb, GR, N = setup(w, inp)
    ep.ep_hierarchical_dispatch_fused(shape, L, tk, 7, gb, GR, pb, N, ws)
    torch.cuda.synchronize()
    assert ep.ep_check_errors(ws) == 0
    O, Hd = expected(w, inp, 7)
    np.testing.assert_array_equal(host(gb)[:GR], Hd["group_buf"])
    np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])


def run_ring(w, inp, tile, ring, epoch=9, fp8=False, withhold=None, timeout_us=0, calls=1):
    """Fused call(s) in ring mode; group_buf holds only the ring."""
    print(f"fused ring: T={w.T} H={w.H} K={w.K} E={w.E} R={w.R} G={w.G} tile={tile} ring={ring} "
          f"fp8={fp8} withhold={withhold}", flush=True)
    shape, L, ws, tk, _, pb, GR, N = setup(w, inp, fp8)
    stride = pb.shape[1]
    ring_rows = ring * tile * min(w.K, w.G)
    gb = torch.full((ring_rows, stride), 0xA5, dtype=torch.uint8, device="cuda")
    for _ in range(calls):
        pb.fill_(0xA5)
        ep.ep_hierarchical_dispatch_fused(shape, L, tk, epoch, gb, ring_rows, pb, N, ws, tile=tile, ring=ring,
                                          withhold=withhold, timeout_us=timeout_us)
        torch.cuda.synchronize()
    return ws, pb, N


@pytest.mark.parametrize("T,H,K,E,R,G,tile,ring,fp8", [
    (1000, 512, 6, 64, 16, 4, 2, 65, False),      # smallest ring: 500 batches through 65
    (1000, 512, 6, 64, 16, 4, 2, 100, False),
    (1000, 512, 6, 64, 16, 4, 4, 300, False),     # ring longer than the batch count
    (777, 1024, 8, 128, 32, 8, 16, 70, True),     # FP8 + scales
    (129, 1032, 12, 48, 16, 4, 1, 65, False),     # K > G: min(K, G) rows per token
    (200, 256, 64, 1024, 256, 256, 1, 65, False),  # 64 groups per token at most
    (40, 16384, 8, 64, 16, 4, 1, 65, False),      # records of several 32-block pieces
])
def test_fused_ring_shapes(T, H, K, E, R, G, tile, ring, fp8):
    w = synth.Workload("fz_ring", T, H, E, R, G, K, "uniform")
    inp = synth.make_inputs(w, seed=T + ring, with_fp8=fp8)
    ws, pb, N = run_ring(w, inp, tile, ring, fp8=fp8)
    assert ep.ep_check_errors(ws) == 0
    _, Hd = expected(w, inp, 9, fp8)
    np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])


def test_fused_ring_skipped_lanes_and_repeats():
    """-1 and repeated experts, and two calls on one workspace with the same
    epoch (the freed words of the first call are cleared for the second)."""
    w = synth.Workload("fz_ring_rand", 600, 256, 20, 10, 5, 5, "uniform")
    inp = synth.make_inputs(w, seed=3)
    inp["topk_idx"] = np.random.default_rng(6).integers(-1, w.E, size=(w.T, w.K)).astype(np.int64)
    ws, pb, N = run_ring(w, inp, 1, 80, calls=2)
    assert ep.ep_check_errors(ws) == 0
    _, Hd = expected(w, inp, 9)
    np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])


@pytest.mark.parametrize("held", [5, 150])
def test_fused_ring_withheld_flag(held):
    """One batch's flag withheld in ring mode (in the ring's first pass, and
    in its third): its forwarder gives up and still frees the batch's ring
    rows; the producer that reuses them and every later wait of that slot
    have longer limits, so only the withheld batch is lost: every other
    scale-up row is the oracle's."""
    w = synth.Workload("fz_ring_hold", 1000, 512, 64, 16, 4, 6, "uniform")
    inp = synth.make_inputs(w, seed=18)
    tile = 2
    ws, pb, N = run_ring(w, inp, tile, 70, withhold=held, timeout_us=2000)
    assert ep.ep_check_errors(ws) == ep.EP_DEVERR_TIMEOUT
    O, Hd = expected(w, inp, 9)
    sl = O["slot"][held * tile:(held + 1) * tile]
    held_rows = np.unique(sl[sl >= 0])
    keep = np.setdiff1d(np.arange(N), held_rows)
    got = host(pb)[:N]
    np.testing.assert_array_equal(got[keep], Hd["peer_buf"][keep])
    assert (got[held_rows] == 0xA5).all()


@pytest.mark.parametrize("ring", [128, 512])
def test_fused_ring_full_hier8x8(ring):
    w = synth.workload("hier8x8")
    inp = synth.make_inputs(w)
    ws, pb, N = run_ring(w, inp, 2, ring)
    assert ep.ep_check_errors(ws) == 0
    _, Hd = expected(w, inp, 9)
    np.testing.assert_array_equal(host(pb)[:N], Hd["peer_buf"])
