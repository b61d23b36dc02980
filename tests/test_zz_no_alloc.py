"""The allocation-free layout (ep_get_layout_noalloc: count tables in the
library's static per-GPU scratch array instead of a workspace) against
ep_get_layout on the same inputs: every output bit for bit, on two calls in a
row, the second with a smaller input, so that what the first call left in the
shared scratch cannot leak into the second. Also the size limit (a shape
whose tables exceed the array is refused before any launch) and the error
words."""
import numpy as np
import pytest
import torch

import synth
from combine_get_layout_amd import ep

pytestmark = pytest.mark.gpu

OUTS = ("tokens_per_expert", "tokens_per_rank", "tokens_per_group", "expert_offsets", "rank_offsets",
        "group_offsets", "is_token_in_rank", "is_token_in_group", "slot", "group_slot", "expert_slot")


@pytest.fixture(scope="module", autouse=True)
def _ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def both_layouts(w, seed, bad_id=False):
    """Outputs of ep_get_layout and of ep_get_layout_noalloc for one input,
    with their error words."""
    inp = synth.make_inputs(w, seed=seed, with_x=False)
    ids = inp["topk_idx"].copy()
    if bad_id:
        ids[w.T // 2, 0] = w.E + 7
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    topk = dev(ids)
    ref = ep.alloc_layout(shape, masks=True, groups=True, expand=True)
    got = ep.alloc_layout(shape, masks=True, groups=True, expand=True)
    for L in (ref, got):  # poison: every output must be written
        for t in L.values():
            t.view(torch.uint8).fill_(0xA7)
    ws = ep.alloc_workspace(shape)
    errs = torch.zeros(64, dtype=torch.uint8, device="cuda")
    errs[:8].fill_(0xFF)  # word 0 must be cleared by the call
    ep.ep_get_layout(shape, topk, ref, ws)
    ep.ep_get_layout_noalloc(shape, topk, got, errs)
    torch.cuda.synchronize()
    return ref, got, ep.ep_check_errors(ws), errs[:8].view(torch.int32).cpu().numpy().view(np.uint32)


def assert_same(ref, got, what):
    for n in OUTS:
        a = ref[n].view(torch.uint8).cpu().numpy()
        b = got[n].view(torch.uint8).cpu().numpy()
        np.testing.assert_array_equal(b, a, err_msg=f"{what}: {n}")


def test_noalloc_layout_equals_layout_on_two_calls():
    # first call: the largest table of the sequence (zipf: 2048 experts, 256 ranks)
    w1 = synth.workload("zipf")
    ref, got, bits, words = both_layouts(w1, seed=11)
    print(f"call 1: T={w1.T} E={w1.E} R={w1.R} G={w1.G}", flush=True)
    assert_same(ref, got, "call 1")
    assert bits == 0 and words[0] == 0
    # second call, smaller and with groups: the scratch still holds call 1's tables
    w2 = synth.Workload("small_hier", 1000, 256, 96, 24, 6, 8, "uniform")  # T H E R G K
    ref, got, bits, words = both_layouts(w2, seed=12)
    print(f"call 2: T={w2.T} E={w2.E} R={w2.R} G={w2.G}", flush=True)
    assert_same(ref, got, "call 2")
    assert bits == 0 and words[0] == 0


def test_noalloc_layout_reports_invalid_ids():
    w = synth.Workload("bad_ids", 700, 256, 64, 16, 4, 4, "uniform")  # T H E R G K
    ref, got, bits, words = both_layouts(w, seed=13, bad_id=True)
    assert_same(ref, got, "invalid id")
    assert bits == ep.EP_DEVERR_EXPERT_ID
    assert words[0] == ep.EP_DEVERR_EXPERT_ID and words[1] & ep.EP_DEVERR_EXPERT_ID


def test_noalloc_layout_full_ep32_then_tiny():
    for w, seed in ((synth.workload("ep32"), 14), (synth.workload("tiny"), 15)):
        ref, got, bits, words = both_layouts(w, seed=seed)
        print(f"{w.name}: T={w.T}", flush=True)
        assert_same(ref, got, w.name)
        assert bits == 0 and words[0] == 0


def test_noalloc_layout_refuses_shapes_beyond_the_scratch():
    s = ep.make_shape(1 << 20, 7168, 8, 256, 64, 1)
    assert ep.ep_workspace_bytes(s) > ep.EP_LAYOUT_SCRATCH_BYTES
    L = ep.ep_layout()
    rc = ep.lib().ep_get_layout_noalloc(ctypes_ref(s), 0x1000, ctypes_ref(L), 0x2000, None)
    assert rc == ep.EP_ERR_SCRATCH
    assert "scratch" in ep.ep_status_string(rc)


def ctypes_ref(x):
    import ctypes
    return ctypes.byref(x)
