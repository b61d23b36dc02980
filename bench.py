#!/usr/bin/env python3
"""Throughput of the MoE dispatch / combine hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic tokens:
  flat workloads   : ep_get_layout -> ep_dispatch -> ep_combine (identity expert:
                     the combine gathers the dispatched rows back)
  two-level (hier) : ep_get_layout -> ep_hierarchical_dispatch_fused (both
                     steps in one launch; --two-launch: ep_hierarchical_dispatch,
                     the two steps as two launches) -> ep_combine on the
                     chunked scale-up rows
  --sources S      : S source ranks (default R) on the flat workloads:
                     ep_source_layout -> ep_source_dispatch_fused (send into
                     per-(rank, source) staging regions and copy epilogue into
                     dense receive rows in one launch; --two-launch:
                     ep_source_dispatch, then ep_copy_epilogue) -> ep_combine
                     over the staging rows
With no --workload the run times every target configuration in turn (ep32,
ep32 with the FP8 + scales payload, ep256, zipf, hier8x8); the headline
fields are ep32's and `per_config` holds one entry per configuration. With
--workload only that one is timed.

Inputs are seeded and already resident in HBM when the timed region starts.
Per configuration: W untimed warm-up steps; then K eager steps whose launches
(the first 20) are bracketed by events on the launch stream (the per-kernel
durations); then, unless --eager, the K steps are captured into one HIP graph
(for K <= 512; above that one graph per cycle of input batches, replayed,
plus single-step graphs for the remainder) and replayed between two device
synchronisations: that is `value` and `ms_per_step`. Prints one JSON line.

Also reported per configuration: per-kernel average durations from HIP events
recorded on the stream the kernels run on, the roofline of the dominant kernel
(algorithmic bytes per launch / average duration, against 8 TB/s HBM), HBM
traffic from the committed rocprofv3 counter summary when it matches the
current kernel sources, and the CPU oracle timed on the host cores on a
bounded sample.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MALL_EVICT_BYTES = 320 << 20  # more than the 256 MB MALL
METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=None,
                   choices=["tiny", "ep32", "ep256", "zipf", "hier8x8", "many"],
                   help="time only this workload (default: every target configuration, ep32 first)")
    p.add_argument("--hidden", type=int, default=0,
                   help="with --workload: this hidden size instead of the workload's (labelled _h<H>)")
    p.add_argument("--fp8", action="store_true", help="also move the FP8 payload + scales")
    p.add_argument("--fused", action="store_true",
                   help="two-level workloads and --sources: the one-launch forms with per-batch flags "
                        "(ep_hierarchical_dispatch_fused, ep_source_dispatch_fused; the default)")
    p.add_argument("--two-launch", action="store_true",
                   help="two-level workloads: the two dispatch steps as two launches "
                        "(ep_hierarchical_dispatch); --sources: the send and the copy epilogue as "
                        "two calls")
    p.add_argument("--fused-tile", type=int, default=0,
                   help="tokens per batch of the fused two-level dispatch (0: default)")
    p.add_argument("--ring", type=int, default=0,
                   help="fused two-level dispatch: group rows through a ring of this many batches "
                        "(> 64; 0: at their group-region rows; labelled _ring<N>)")
    p.add_argument("--two-level-combine", action="store_true",
                   help="two-level workloads: combine through per-group partial rows")
    p.add_argument("--expand", action="store_true",
                   help="expand mode: one receive row per (token, lane), grouped by expert")
    p.add_argument("--sources", type=int, default=None, const=0, nargs="?",
                   help="several source ranks on one GPU (S; bare flag = one per rank)")
    p.add_argument("--eager", action="store_true",
                   help="time eager launches only (default: replay a HIP graph of the timed steps)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="time budget of the CPU-oracle baseline of the headline configuration "
                        f"(the others get at most {CPU_SECONDS_OTHER} s and at least one pass; 0 = skip)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain 1 GiB device copy (counter calibration under rocprofv3)")
    p.add_argument("--ceilings", action="store_true",
                   help="measure the chip's practical HBM rates with library kernels "
                        "(read, constant write, copy over 1 GiB buffers), print one JSON line and exit")
    return p.parse_args()


EVENT_STEPS = 20  # eager steps whose launches are bracketed by timing events


def ceilings(reps: int = 20) -> dict:
    """Practical HBM rates of library kernels on 1 GiB buffers (GB/s): a
    reduction (read only), a constant fill (write only), two ways of writing
    an 8 MiB random tile 128 times (a broadcast copy and a concatenation: the
    source stays cached, so HBM sees writes of varying data, the shape of a
    read-once, write-many fan-out) and a device copy (read + write). Context
    for the roofline fractions, not a target."""
    import torch

    n = 1 << 30
    a = torch.randn(n // 4, device="cuda")  # fp32, 1 GiB
    b = torch.empty_like(a)
    bi = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    tile = torch.randn(1, n // 4 // 128, device="cuda")  # 8 MiB of random values
    out = torch.empty((), device="cuda")
    ops = {
        "read (torch.sum, fp32)": (lambda: torch.sum(a, dim=(0,), out=out), n),
        "write (fill_, constant)": (lambda: b.fill_(1.5), n),
        "write (fill_, int32 constant)": (lambda: bi.fill_(7), n),
        "broadcast copy (8 MiB random tile x 128)": (lambda: b.view(128, -1).copy_(tile), n),
        "cat (8 MiB random tile x 128)": (lambda: torch.cat([tile.view(-1)] * 128, out=b), n),
        "copy (copy_, device to device)": (lambda: b.copy_(a), 2 * n),
    }
    res = {}
    for name, (fn, nbytes) in ops.items():
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"GB/s": nbytes / (ms * 1e-3) / 1e9, "us": ms * 1e3, "bytes": nbytes}
    return res


# Source files behind each kernel whose traffic bench.py reports. A counter
# summary stays valid while these files (and the shared headers and launch
# code) are unchanged.
KERNEL_FILES = {
    "layout_*": ["layout.hip"],
    "dispatch_kernel": ["dispatch.hip"],
    "combine_kernel": ["combine.hip"],
    "scaleout_kernel+forward_kernel": ["hier.hip"],
    "fused_hier_kernel": ["hier.hip"],
    "scaleout_kernel": ["hier.hip"],
    "copy_epilogue_kernel": ["source.hip", "ep_epilogue.h"],
    "source_fused_kernel": ["hier.hip", "ep_epilogue.h"],
    "combine_group_kernel+combine_cross_kernel": ["combine2.hip"],
    "combine_two_level_fused_kernel": ["combine2.hip"],
}
COMMON_FILES = ["ep_device.h", "ep_internal.h", "api.hip"]


def kernel_source_hash(kernel: str) -> str:
    """sha256 prefix of the sources `kernel` is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_get_layout_amd", "csrc")
    for f in COMMON_FILES + KERNEL_FILES[kernel]:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "ep.h"), "rb").read())
    return h.hexdigest()[:16]


def two_level_combine_kernel(H: int, K: int, group_cap: int) -> str:
    """The launch ep_combine_two_level makes with both steps: one fused kernel
    when K <= 8, a token's slices of 4 wave-iterations fill a 4-wave
    workgroup evenly and the partial rows (group_cap of them) take at least
    512 MB, else the group and cross kernels."""
    blocks = (2 * H + 479) // 480
    slices = ((blocks + 1) // 2 + 3) // 4
    big = group_cap * 512 * blocks >= 512 << 20
    return "combine_two_level_fused_kernel" if K <= 8 and 4 % slices == 0 and big else \
        "combine_group_kernel+combine_cross_kernel"


def committed_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None if there is none or it was taken from other sources of that kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    k = d.get("kernels", {}).get(kernel)
    if k is None or k.get("source_sha") != kernel_source_hash(kernel):
        return None
    return k.get("hbm_bytes_per_launch")


# The configurations the default run times: the headline first.
TARGET_CONFIGS = [
    ("ep32", dict(fp8=False)),
    ("ep32_fp8", dict(fp8=True)),
    ("ep256", dict(fp8=False)),
    ("zipf", dict(fp8=False)),
    ("hier8x8", dict(fp8=False)),
]
GRAPH_MAX_STEPS = 512  # up to this many timed steps go into one graph
CPU_SECONDS_OTHER = 3.0  # CPU-oracle budget of the non-headline configurations


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the path has no "
              "cross-GPU step; several GPUs are not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    from combine_get_layout_amd import ep

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.ceilings:
        torch.cuda.set_device(0)
        print(json.dumps({"ceilings": ceilings(), "peak_GB/s": HBM_PEAK_GBS,
                          "device": torch.cuda.get_device_name(0)}), flush=True)
        return
    ep.lib()
    torch.cuda.set_device(0)
    variants = (args.fp8 or args.expand or args.two_level_combine or args.fused or args.two_launch or
                args.fused_tile or args.hidden or args.ring or args.sources is not None)
    if args.workload is None and not variants:
        runs = [(label, "ep32" if label.startswith("ep32") else label, kw) for label, kw in TARGET_CONFIGS]
    else:
        w = args.workload or "ep32"
        runs = [(w, w, dict(fp8=bool(args.fp8)))]
    per = {}
    for n, (label, wname, kw) in enumerate(runs):
        print(f"[bench] {label}: {args.warmup} warm-up + {args.steps} timed steps", file=sys.stderr,
              flush=True)
        cpu_s = args.cpu_seconds if n == 0 else min(args.cpu_seconds, CPU_SECONDS_OTHER)
        per[label] = run_config(args, wname, kw["fp8"], cpu_s)
        print(f"[bench] {label}: {per[label]['ms_per_step'] * 1e3:.1f} us per step, "
              f"{100 * per[label]['hbm_frac_step']:.1f}% of HBM peak", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    head = per[runs[0][0]]
    rec = {"metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup}
    rec.update({k: v for k, v in head.items() if k not in ("value",)})
    if len(per) > 1:
        rec["per_config"] = {label: {k: r[k] for k in PER_CONFIG_KEYS} for label, r in per.items()}
    print(json.dumps(rec), flush=True)


PER_CONFIG_KEYS = ("value", "unit", "ms_per_step", "hbm_gbs_step", "hbm_frac_step", "launch", "config",
                   "kernel_ms", "roofline", "cpu_baseline")


def run_config(args, wname: str, fp8: bool, cpu_seconds: float) -> dict:
    """Time one configuration; returns its record (without the run-wide fields)."""
    import numpy as np
    import torch

    import synth
    from combine_get_layout_amd import ep

    w = synth.workload(wname)
    if args.hidden:
        if args.hidden % 8 or (fp8 and args.hidden % 128):
            print("--hidden must be a multiple of 8 (of 128 with --fp8)", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, name=f"{w.name}_h{args.hidden}", H=args.hidden)
    hier = w.G > 1
    expand = bool(args.expand)
    two_level = bool(args.two_level_combine)
    if args.fused and args.two_launch:
        print("--fused and --two-launch exclude each other", file=sys.stderr)
        sys.exit(2)
    multi = args.sources is not None
    if (args.fused or args.two_launch) and not (hier or multi):
        print("--fused and --two-launch apply to the two-level workloads and to --sources", file=sys.stderr)
        sys.exit(2)
    if (args.fused_tile or args.ring) and not hier:
        print("--fused-tile and --ring apply to the two-level workloads", file=sys.stderr)
        sys.exit(2)
    fused = (hier or multi) and not args.two_launch
    if args.ring and not fused:
        print("--ring applies to the fused two-level dispatch", file=sys.stderr)
        sys.exit(2)
    if two_level and not hier:
        print("--two-level-combine applies to the two-level workloads", file=sys.stderr)
        sys.exit(2)
    if expand and hier:
        print("--expand applies to the flat workloads", file=sys.stderr)
        sys.exit(2)
    S = (args.sources or w.R) if multi else 1
    if multi and (hier or expand or two_level):
        print("--sources applies to the flat workloads without --expand", file=sys.stderr)
        sys.exit(2)
    # Independent input batches, rotated step by step, so that the x rows a
    # step reads were not left in the 256 MB MALL by an earlier step: the
    # other batches' x alone exceed it.
    x_bytes = w.T * w.H * 2
    n_batches = max(2, 1 + -(-MALL_EVICT_BYTES // x_bytes))
    seeds = [synth.seed_of(w) + 1000 * i for i in range(n_batches)]
    inputs = [synth.make_inputs(w, seed=sd, with_fp8=fp8) for sd in seeds]
    inp = inputs[0]

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.uint16)
        return torch.from_numpy(a).cuda()

    shape = ep.make_shape(w.T, w.H, w.K, w.E, w.R, w.G)
    batches = []
    for b_in in inputs:
        tk = dict(x=dev(b_in["x"]), topk_idx=dev(b_in["topk_idx"]), topk_weights=dev(b_in["topk_w"]))
        if fp8:
            tk["x_fp8"] = dev(b_in["x_fp8"])
            tk["x_scales"] = dev(b_in["x_scales"])
        batches.append(tk)
    if n_batches > 64:  # (tiny) keep the host copies of only the batch the CPU leg uses
        inputs = [inp]
    L = ep.alloc_layout(shape, masks=True, groups=hier, expand=expand)
    ws = ep.alloc_workspace(shape)
    Ns, Gs = [], []
    if multi:
        # Region capacity: the largest per-(source, rank) count over the
        # batches (a first pass with capacity = tokens per source cannot
        # overflow).
        ws = ep.alloc_source_workspace(shape, S)
        Ts = -(-w.T // S)
        src = ep.alloc_sources(shape, S, Ts)
        cap = 1
        for tk in batches:
            ep.ep_source_layout(shape, tk["topk_idx"], src, ws)
            torch.cuda.synchronize()
            cap = max(cap, int(src["counts"].max().item()))
            Ns.append(int(src["recv_offsets"][-1].item()))
            Gs.append(0)
        src["capacity"] = cap
    else:
        for tk in batches:
            ep.ep_get_layout(shape, tk["topk_idx"], L, ws)
            torch.cuda.synchronize()
            Ns.append(int((L["expert_offsets"] if expand else L["rank_offsets"])[-1].item()))
            Gs.append(int(L["group_offsets"][-1].item()) if hier else 0)
    N_cap, G_cap = max(Ns), max(Gs)
    out = torch.empty((w.T, w.H), dtype=torch.uint16, device="cuda")
    seg = ep.EP_SEG_BF16 | ((ep.EP_SEG_FP8 | ep.EP_SEG_SCALES) if fp8 else 0)
    if hier:
        stride = ep.ep_chunked_record_bytes(shape, seg)
        group_buf = torch.empty((G_cap, stride), dtype=torch.uint8, device="cuda")
        peer_buf = torch.empty((N_cap, stride), dtype=torch.uint8, device="cuda")
        if two_level:
            pstride = ep.ep_partial_row_bytes(shape)
            part_buf = torch.empty((G_cap, pstride), dtype=torch.uint8, device="cuda")
    else:
        recv = ep.alloc_recv(shape, N_cap, fp8=fp8, scales=fp8, meta=True)
    if multi:
        stride = ep.ep_chunked_record_bytes(shape, seg)
        staging = torch.empty((w.R * S * cap, stride), dtype=torch.uint8, device="cuda")
        y_src = dict(slot=src["src_slot"])

    epoch = [0]
    stream = torch.cuda.current_stream()
    names = ((["layout", "send+epilogue", "combine"] if fused else ["layout", "send", "epilogue", "combine"])
             if multi else ["layout", "hier" if hier else "dispatch", "combine"])
    ev = {n: [] for n in names}
    used = []

    def timed(name, fn, record):
        if record:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev[name].append((a, b))
        else:
            fn()

    def run_step(i, e, record):
        """One pass of the path over batch i with flag epoch e."""
        tokens, N, G_rows = batches[i], Ns[i], Gs[i]
        if multi:
            timed("layout", lambda: ep.ep_source_layout(shape, tokens["topk_idx"], src, ws), record)
            if fused:
                timed("send+epilogue", lambda: ep.ep_source_dispatch_fused(shape, src, tokens, e, staging,
                                                                           recv, N, ws), record)
            else:
                timed("send", lambda: ep.ep_source_dispatch(shape, src, tokens, e, staging, ws), record)
                timed("epilogue", lambda: ep.ep_copy_epilogue(shape, src, staging, e, seg, recv, N, ws),
                      record)
            timed("combine", lambda: ep.ep_combine(shape, y_src, staging, staging.shape[0], stride,
                                                   ep.EP_FMT_CHUNKED, e, tokens["topk_weights"],
                                                   out, ws), record)
            return
        timed("layout", lambda: ep.ep_get_layout(shape, tokens["topk_idx"], L, ws), record)
        if hier and fused:
            timed("hier", lambda: ep.ep_hierarchical_dispatch_fused(
                shape, L, tokens, e, group_buf, G_rows, peer_buf, N, ws, tile=args.fused_tile, ring=args.ring),
                record)
        if hier and not fused:
            timed("hier", lambda: ep.ep_hierarchical_dispatch(
                shape, L, tokens, e, ep.EP_HIER_SCALEOUT | ep.EP_HIER_FORWARD,
                group_buf, G_rows, peer_buf, N, ws), record)
        if hier:
            if two_level:
                timed("combine", lambda: ep.ep_combine_two_level(
                    shape, L, tokens["topk_idx"], peer_buf, N, stride, ep.EP_FMT_CHUNKED, e,
                    tokens["topk_weights"], part_buf, G_rows, 3, out, ws), record)
            else:
                timed("combine", lambda: ep.ep_combine(shape, L, peer_buf, N, stride, ep.EP_FMT_CHUNKED,
                                                       e, tokens["topk_weights"], out, ws), record)
        elif expand:
            timed("dispatch", lambda: ep.ep_dispatch_expand(shape, L, tokens, recv, N, ws), record)
            timed("combine", lambda: ep.ep_combine_expand(shape, L, recv["x"], N, 2 * w.H,
                                                          ep.EP_FMT_PLAIN, 0, tokens["topk_weights"],
                                                          out, ws), record)
        else:
            timed("dispatch", lambda: ep.ep_dispatch(shape, L, tokens, recv, N, ws), record)
            timed("combine", lambda: ep.ep_combine(shape, L, recv["x"], N, 2 * w.H, ep.EP_FMT_PLAIN,
                                                   0, tokens["topk_weights"], out, ws), record)

    def step(record, events=None):
        """One step; `record` counts it as timed, `events` (default: record)
        brackets its launches with events."""
        i = epoch[0] % n_batches
        epoch[0] += 1
        if record:
            used.append(i)
        run_step(i, epoch[0], record if events is None else events)

    def check_errors(when):
        # the word kept since the last clear: an error in any step counts, not
        # only in the last step's pass
        bits = ep.ep_check_sticky_errors(ws)
        if bits != 0:
            raise RuntimeError(f"device error bits {bits} set during {when}")

    ep.ep_clear_errors(ws)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    check_errors("warm-up")

    def timed_region(body):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        a.record(stream)
        for k in range(args.steps):
            body(k)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b), time.perf_counter() - w0

    # Eager pass: every launch bracketed by events on the launch stream, for
    # the per-kernel durations.
    # Events only on the first EVENT_STEPS steps: every timing event holds a
    # runtime signal until it is read, and with hundreds of them outstanding
    # the runtime stalls between launches, which the events would then time.
    ms_eager, wall_eager = timed_region(lambda k: step(True, k < EVENT_STEPS))
    avg_ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / len(ev[n]) for n in names}
    check_errors("the eager steps")

    ms_total, wall = ms_eager, wall_eager
    graph_used = not args.eager
    launch = "eager"
    if graph_used and args.steps <= GRAPH_MAX_STEPS:
        # One graph holding exactly the K timed steps (their launches only:
        # no memset or host work), batches in rotation; step k writes flag
        # epoch 1000 + k, so consecutive steps never share an epoch.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(args.steps):
                run_step(k % n_batches, 1000 + k, False)
        g.replay()  # untimed: first replay
        torch.cuda.synchronize()
        used.clear()
        used.extend(k % n_batches for k in range(args.steps))
        ms_total, wall = timed_region(lambda k: g.replay() if k == 0 else None)
        launch = f"one hip graph holding the {args.steps} timed steps"
        check_errors("the graph replay")
    elif graph_used:
        # One graph per batch holding its whole step, and one holding a whole
        # cycle (the step of every batch in order), so that one graph launch
        # serves n_batches steps. The timed steps replay the cycle K //
        # n_batches times, then the single-step graphs of the first K %
        # n_batches batches. Batch i's graphs write flag epoch 1000 + i.
        graphs = []
        for i in range(n_batches):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(i, 1000 + i, False)
            graphs.append(g)
        use_cycle = n_batches <= 64 and args.steps >= n_batches
        if use_cycle:
            cycle = torch.cuda.CUDAGraph()
            with torch.cuda.graph(cycle):
                for i in range(n_batches):
                    run_step(i, 1000 + i, False)
        for g in graphs:
            g.replay()
        if use_cycle:
            cycle.replay()
        torch.cuda.synchronize()
        used.clear()
        full_until = (args.steps // n_batches) * n_batches if use_cycle else 0

        def replay(k):
            i = k % n_batches
            used.append(i)
            if k >= full_until:
                graphs[i].replay()
            elif i == 0:
                cycle.replay()

        ms_total, wall = timed_region(replay)
        launch = ("hip graphs: one per cycle of the input batches (one step per batch), single-step "
                  "graphs for the remainder" if use_cycle else "hip graph per step")
        check_errors("the graph replays")
    ms_step = ms_total / args.steps

    # Algorithmic bytes per launch: what the method must move, from the byte
    # model per token (read each row once, write each receive row once, plus
    # the routing metadata), averaged over the batches the timed steps used.
    T, H, K, R = w.T, w.H, w.K, w.R
    row = 2 * H + ((H + 4 * (H // 128)) if fp8 else 0)
    meta = 4 + 8 * K
    route = T * K * (8 + 4 + 4)  # topk_idx read, weights read, slots read
    bytes_layout = T * K * 8 + T * K * 4 + T * R + (T * K * 4 + T * w.G if hier else 0) + \
        (T * K * 8 + T * K * 4 if expand else 0)
    N = sum(Ns[i] for i in used) / len(used)
    G_rows = sum(Gs[i] for i in used) / len(used)
    if multi:
        rec_b = ep.ep_chunked_record_bytes(shape, seg)
        hid = 512 * ((2 * H + 479) // 480)
        bytes_layout = T * K * 8 + T * K * 4
        by = {"layout": bytes_layout,
              "send": T * row + route + N * rec_b,
              "epilogue": N * rec_b + N * (row + meta),
              "combine": N * hid + T * 2 * H + T * K * 8}
        if fused:
            by["send+epilogue"] = by.pop("send") + by.pop("epilogue")
    elif hier:
        rec_b = ep.ep_chunked_record_bytes(shape, seg)
        hid = 512 * ((2 * H + 479) // 480)
        bytes_main = T * row + route + T * K * 4 + 2 * G_rows * rec_b + N * rec_b
        bytes_combine = N * hid + T * 2 * H + T * K * 8
        if two_level:  # partial rows written, then read back
            bytes_combine += 2 * G_rows * hid + T * K * 8
    else:
        bytes_main = T * row + route + N * (row + meta)
        bytes_combine = N * 2 * H + T * 2 * H + T * K * 8
    if not multi:
        by = {"layout": bytes_layout, names[1]: bytes_main, "combine": bytes_combine}
    step_bytes = sum(by.values())
    kernel_of = {"layout": "layout_*", "dispatch": "dispatch_kernel", "send": "scaleout_kernel",
                 "epilogue": "copy_epilogue_kernel", "send+epilogue": "source_fused_kernel",
                 "hier": "fused_hier_kernel" if fused else "scaleout_kernel+forward_kernel",
                 "combine": (two_level_combine_kernel(w.H, w.K, int(G_rows)) if two_level else "combine_kernel")}
    dom = max(names[1:], key=lambda n: avg_ms[n])
    achieved = by[dom] / (avg_ms[dom] * 1e-3) / 1e9
    label = w.name + ("_fp8" if fp8 else "") + ("_expand" if expand else "") + \
        ("_2lc" if two_level else "") + (f"_s{S}" if multi else "") + ("_2launch" if (hier or multi) and not fused else "") + \
        (f"_ring{args.ring}" if args.ring else "")
    traffic = committed_traffic(label, kernel_of[dom])

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if cpu_seconds > 0:
        cpu = cpu_baseline(w, inp, fp8, hier, cpu_seconds, expand, S if multi else 0)

    return {
        "value": T * args.steps / (ms_total * 1e-3),
        "unit": "tokens/s",
        "ms_per_step": ms_step,
        "ms_per_step_eager": ms_eager / args.steps,
        "launch": launch,
        "wall_s": wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "payload_dtype": "bf16" + ("+fp8e4m3" if fp8 else ""),
        "data": "synthetic (seeded; see synth/__init__.py)",
        "config": {"workload": label, "tokens": T, "hidden": H, "experts": w.E,
                   "ranks": R, "groups": w.G, "topk": K, "routing": w.routing,
                   "receive_rows": N, "fp8_payload": fp8, "expand_rows": expand,
                   "two_level_combine": two_level, "fused_two_level_dispatch": fused,
                   "ring_batches": args.ring or None,
                   "sources": S if multi else None,
                   "region_capacity": cap if multi else None,
                   "input_batches": n_batches,
                   "parallelism": "single GPU"},
        "hbm_gbs_step": step_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac_step": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernel_ms": avg_ms,
        "kernel_algorithmic_bytes": by,
        "roofline": {"kernel": kernel_of[dom], "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }


def cpu_baseline(w, inp, fp8, hier, budget_s, expand=False, sources=0):
    """The oracle as it stands, single-threaded, on repeated full passes of the
    same batch until the time budget is spent (at least one pass)."""
    import oracle

    oracle.build(force=False)
    passes, t0 = 0, time.perf_counter()
    while True:
        if sources:
            X = oracle.source_counts(inp["topk_idx"], w.E, w.R, sources)
            cap = int(X["counts"].max())
            Sd = oracle.source_dispatch(inp["topk_idx"], w.E, w.R, sources, cap, 1, x=inp["x"],
                                        x_fp8=inp.get("x_fp8"), x_scales=inp.get("x_scales"),
                                        topk_w=inp["topk_w"])
            oracle.copy_epilogue(X["recv_offsets"], Sd["staging"], w.H, w.K, w.R, sources, cap, 1,
                                 with_fp8=fp8, with_scales=fp8)
            slot = oracle.source_slots(inp["topk_idx"], w.E, w.R, sources, cap)["src_slot"]
            oracle.combine(slot, inp["topk_w"], Sd["staging"], w.H, chunked=True, epoch=1)
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
            continue
        L = oracle.layout(inp["topk_idx"], w.E, w.R, w.G)
        if hier:
            Hd = oracle.hier_dispatch(inp["topk_idx"], w.E, w.R, w.G, L["slot"], L["group_offsets"],
                                      1, x=inp["x"], x_fp8=inp.get("x_fp8"),
                                      x_scales=inp.get("x_scales"), topk_w=inp["topk_w"])
            oracle.combine(L["slot"], inp["topk_w"], Hd["peer_buf"], w.H, chunked=True, epoch=1)
        elif expand:
            es = oracle.expert_slots(inp["topk_idx"], w.E, L["expert_offsets"])
            n_rows = int(L["expert_offsets"][-1])
            D = oracle.dispatch_rows(inp["topk_idx"], w.E, es, n_rows, x=inp["x"],
                                     x_fp8=inp.get("x_fp8"), x_scales=inp.get("x_scales"),
                                     topk_w=inp["topk_w"])
            oracle.combine(es, inp["topk_w"], D["recv_x"], w.H)
        else:
            D = oracle.dispatch(inp["topk_idx"], w.E, w.R, L["rank_offsets"], x=inp["x"],
                                x_fp8=inp.get("x_fp8"), x_scales=inp.get("x_scales"),
                                topk_w=inp["topk_w"])
            oracle.combine(L["slot"], inp["topk_w"], D["recv_x"], w.H)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": w.T * passes / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"{passes} full pass(es) of source counts+send+copy epilogue "
                       f"+combine ({sources} sources)" if sources else
                       f"{passes} full pass(es) of layout+{'two-level dispatch' if hier else 'dispatch'}"
                       "+combine") + f" over the same {w.T}-token batch, {el:.1f} s, single thread",
            "host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model}


if __name__ == "__main__":
    main()
