"""The calls run on the caller's stream.

Work is enqueued on a side stream behind a spin kernel (torch.cuda._sleep, a
bounded busy wait) and a copy of the inputs made on that stream, so the calls
only see their inputs if they are ordered after them on the same stream. The
stream is passed both ways the binding allows: as torch's current stream and
as an explicit argument. Results are compared with the CPU oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_get_layout_amd import ep

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 20_000_000  # about 10 ms of busy wait at the chip's clock


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


@pytest.mark.parametrize("how", ["current", "explicit"])
def test_calls_run_on_the_callers_stream(how):
    w = synth.Workload("stream", 2048, 2048, 64, 16, 4, 6, "uniform")
    inp = synth.make_inputs(w, seed=3)
    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    x0, tk0, w0 = dev(inp["x"]), dev(inp["topk_idx"]), dev(inp["topk_w"])
    L = ep.alloc_layout(shape)
    ws = ep.alloc_workspace(shape)
    cap = w.T * min(w.K, w.R)
    recv = ep.alloc_recv(shape, cap)
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    if how == "current":
        with torch.cuda.stream(s):
            torch.cuda._sleep(SPIN_CYCLES)
            x, tk, wt = x0.clone(), tk0.clone(), w0.clone()
            ep.ep_get_layout(shape, tk, L, ws)
            tokens = dict(x=x, topk_idx=tk, topk_weights=wt)
            ep.ep_dispatch(shape, L, tokens, recv, cap, ws)
            ep.ep_combine(shape, L, recv["x"], cap, 2 * w.H, ep.EP_FMT_PLAIN, 0, wt, out, ws)
            done = torch.cuda.Event()
            done.record(s)
    else:
        with torch.cuda.stream(s):
            torch.cuda._sleep(SPIN_CYCLES)
            x, tk, wt = x0.clone(), tk0.clone(), w0.clone()
        # the current stream is the default one again; the calls name s
        ep.ep_get_layout(shape, tk, L, ws, stream=s)
        tokens = dict(x=x, topk_idx=tk, topk_weights=wt)
        ep.ep_dispatch(shape, L, tokens, recv, cap, ws, stream=s)
        ep.ep_combine(shape, L, recv["x"], cap, 2 * w.H, ep.EP_FMT_PLAIN, 0, wt, out, ws, stream=s)
        done = torch.cuda.Event()
        done.record(s)
    done.synchronize()

    O = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
    N = int(O["rank_offsets"][-1])
    np.testing.assert_array_equal(host(L["slot"]).reshape(w.T, w.K), O["slot"])
    D = oracle.dispatch(inp["topk_idx"], w.E, w.R, O["rank_offsets"], x=inp["x"], topk_w=inp["topk_w"])
    np.testing.assert_array_equal(host(recv["x"])[:N], D["recv_x"])
    C = oracle.combine(O["slot"], inp["topk_w"], D["recv_x"], w.H)
    np.testing.assert_array_equal(host(out), C["out"])
    assert ep.ep_check_errors(ws, stream=s) == 0
