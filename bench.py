#!/usr/bin/env python3
"""Benchmark of MoE expert-parallel dispatch + combine on one MI355X.

A step is one pass of the whole path over one batch: routing layout, pack +
TransferCmd emission (with the CPU proxy threads draining the ring), and the
gate-weighted combine of the returned rows.  The returned rows are the packed
rows themselves (identity experts) for bf16, seeded N(0,1) bf16 rows for fp8.

Prints one JSON line: effective HBM GB/s over the algorithmic bytes of the
step, tokens/s, per-op times from HIP events recorded on the launch stream,
the roofline of the dominant kernel, and the CPU oracle timed on the host.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload train]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine effective HBM GB/s (% of peak) and tokens/s, EP32 top-8"
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, 8 TB/s


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def row_bytes(H: int, fmt: int) -> int:
    """Payload bytes of one send-buffer row: the fp8 row's zero pad up to a
    whole number of 128-byte lines is written but not counted."""
    return 2 * H if fmt == 0 else H + 4 * (H // 128)


def row_pitch(H: int, fmt: int) -> int:
    return row_bytes(H, fmt) if fmt == 0 else (row_bytes(H, fmt) + 127) // 128 * 128


def algorithmic_bytes(w, P: int) -> dict:
    """Bytes the method must move per step (each input read once, each output
    written once)."""
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    rb = row_bytes(H, w.fmt)
    layout_r = 4 * T * k
    layout_w = 4 * (2 * R + 2 * E + 2) + T * R + 4 * T * R
    pack_r = 2 * T * H + 8 * T * k + 4 * T * R + 4 * (R + 1)
    pack_w = P * rb + P * (4 + 8 * k)
    comb_r = 2 * P * H + 8 * T * k + 4 * T * R
    comb_w = 2 * T * H
    return {"layout": layout_r + layout_w, "dispatch": pack_r + pack_w,
            "combine": comb_r + comb_w,
            "total": layout_r + layout_w + pack_r + pack_w + comb_r + comb_w}


def algorithmic_bytes_ll(w, Q: int) -> dict:
    """Per-expert mode: one row per kept choice (Q rows), each input read
    once and each output written once."""
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    rb = row_bytes(H, w.fmt)
    base = algorithmic_bytes(w, 0)
    layout = base["layout"] + 4 * T * k + 4 * T * k    # + row table: read idx, write slots
    pack_r = 2 * T * H + 8 * T * k + 4 * T * k + 4 * (E + 1)
    pack_w = Q * rb + Q * 8
    comb_r = 2 * Q * H + 8 * T * k + 4 * T * k
    comb_w = 2 * T * H
    return {"layout": layout, "dispatch": pack_r + pack_w, "combine": comb_r + comb_w,
            "total": layout + pack_r + pack_w + comb_r + comb_w}


KERNEL_SOURCES = ["combine_topk_rank_amd/csrc/ep_dispatch.hip",
                  "combine_topk_rank_amd/csrc/ep_combine.hip",
                  "combine_topk_rank_amd/csrc/ep_layout.hip",
                  "combine_topk_rank_amd/csrc/ep_common.h"]


def measured_traffic(kernel_prefix: str, workload: str):
    """HBM bytes per launch of a kernel from the rocprofv3 counter summaries
    under profiles/, or None when none matches the current kernel sources."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    sha = h.hexdigest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        text = open(path).read()
        for m in re.finditer(r"```json\n(.*?)\n```", text, re.S):
            try:
                block = json.loads(m.group(1))
            except ValueError:
                continue
            if block.get("source_sha256") != sha:
                continue
            for c in block.get("counters", []):
                if kernel_prefix in c["kernel"] and c["workload"] == workload:
                    return int(c["traffic_bytes"]), os.path.relpath(path, ROOT)
    return None


def cpu_baseline(w, inp, budget_s: float, mode: str = "rank") -> dict:
    """The oracle as it stands, single thread, on whole passes of the same
    workload until about budget_s seconds of CPU work."""
    import numpy as np
    import oracle
    oracle.default()
    passes, t_total, P = 0, 0.0, 0
    while True:
        t0 = time.perf_counter()
        if mode == "ll":
            L = oracle.ll_layout(inp["topk_idx"], w.E)
            P = L["Q"]
            pk = oracle.ll_pack(inp["x"], inp["topk_w"], L["expert_slot"], w.fmt, capacity_rows=P)
            oracle.ll_descriptors(L["num_tokens_per_expert"], L["expert_offset"], w.R,
                                  row_pitch(w.H, w.fmt), w.channels)
        else:
            L = oracle.layout(inp["topk_idx"], w.E, w.R)
            P = L["P"]
            pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R,
                             w.fmt, capacity_rows=P)
            oracle.descriptors(L["num_tokens_per_rank"], L["rank_offset"],
                               row_pitch(w.H, w.fmt), w.channels)
        if w.fmt == 0:
            y = pk["send_buf"].view(np.uint16).reshape(P, w.H)
        else:
            y = np.zeros((P, w.H), np.uint16)
        if mode == "ll":
            oracle.ll_combine(y, inp["topk_idx"], inp["topk_w"], L["expert_slot"], H=w.H)
        else:
            oracle.combine(y, inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R)
        t_total += time.perf_counter() - t0
        passes += 1
        del pk, y
        if t_total >= budget_s:
            break
    per = t_total / passes
    ab = algorithmic_bytes_ll(w, P) if mode == "ll" else algorithmic_bytes(w, P)
    gbs = ab["total"] / per / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} whole pass(es) of the {w.name} workload"
                      f"{' (per-expert mode)' if mode == 'll' else ''} (layout, pack, "
                      f"descriptors, combine); {per:.3f} s per pass, "
                      f"{w.T / per:.0f} tokens/s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train")
    ap.add_argument("--loopback", action="store_true",
                    help="proxy threads execute every command against per-rank receive regions "
                         "and count words (copies on their own streams); the timed region then "
                         "ends when every command has completed")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (layout, dispatch, combine) in a HIP graph and time "
                         "its replays (per-op times are then not sampled)")
    ap.add_argument("--mode", choices=("rank", "ll"), default="rank",
                    help="rank: one row per (token, rank) pair; ll: the per-expert "
                         "(low-latency) mode, one row per kept choice")
    ap.add_argument("--fused", choices=("auto", "on", "off"), default="auto",
                    help="layout + dispatch in one call (ep_dispatch_fused, one kernel for "
                         "T <= 256; per-expert mode: ep_dispatch_ll_fused, T <= 256 and "
                         "E <= 1024); auto: for batches of at most 256 tokens")
    ap.add_argument("--proxy-threads", type=int, default=4)
    ap.add_argument("--op-events-every", type=int, default=5,
                    help="record per-op HIP events on every n-th timed step (events between "
                         "kernels cost a few us each)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0: skip)")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra steps with the 256 MB last-level cache flushed before each")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="only run 5 plain device-to-device copies of this many MiB (a known "
                         "byte count for scaling hardware traffic counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the EP ranks are "
              "simulated as regions of one GPU's HBM", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import combine_topk_rank_amd as ep
    import workloads as W

    w = W.WORKLOADS[args.workload]
    eprint(f"bench: workload {w.name} T={w.T} H={w.H} E={w.E} R={w.R} k={w.k} fmt={w.fmt}")
    inp = W.make_inputs(w, 0)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    d_x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    d_idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    d_w = torch.from_numpy(inp["topk_w"]).to(dev)
    s = ep.shape(w.T, w.H, w.E, w.R, w.k, w.fmt)
    ll = args.mode == "ll"
    # one-call layout + pack: rank mode any T (one kernel up to 256 tokens);
    # per-expert mode up to 256 tokens and 1024 experts
    if ll:
        fused = args.fused == "on" or (args.fused == "auto" and w.T <= 256 and w.E <= 1024)
    else:
        fused = args.fused == "on" or (args.fused == "auto" and w.T <= 256)
    b = ep.BuffersLL(s, device=dev) if ll else ep.Buffers(s, device=dev)
    cap = b.capacity_rows
    if w.fmt == 0:
        y = b.send_buf.view(torch.bfloat16).reshape(cap, w.H)
    else:
        g = torch.Generator(device=dev).manual_seed(0)
        y = torch.randn((cap, w.H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ring = ep.Ring(w.depth, w.channels, w.max_inflight, 10_000_000_000)
    lb_bufs = None
    if args.loopback:
        # receive regions sized from one layout pass: rank r gets its rows
        b.layout(d_idx)
        torch.cuda.synchronize()
        epr = w.E // w.R
        if ll:
            eo = b.expert_offset.cpu().numpy()
            nrows = [int(eo[(r + 1) * epr] - eo[r * epr]) for r in range(w.R)]
            nwords = epr
        else:
            ro = b.rank_offset.cpu().numpy()
            nrows = [int(ro[r + 1] - ro[r]) for r in range(w.R)]
            nwords = 1
        recv = [torch.empty(max(n, 1) * b.row_bytes, dtype=torch.uint8, device=dev) for n in nrows]
        cnt = [torch.zeros(nwords, dtype=torch.int32, device=dev) for _ in range(w.R)]
        lb_bufs = (recv, cnt)
        ring.set_loopback(b.send_buf, recv, cnt)
    ring.proxy_start(args.proxy_threads, 0)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if not fused:
            b.layout(d_idx, stream)
        if ev is not None:
            ev[1].record(stream)
        if fused:
            b.dispatch_fused(d_x, d_idx, d_w, ring=ring, stream=stream)
        else:
            b.dispatch(d_x, d_idx, d_w, ring=ring, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        b.combine(y, d_idx, d_w, stream)
        if ev is not None:
            ev[3].record(stream)

    graph = None
    if args.graph:
        # the library launches on torch's current stream, which is the capture
        # stream inside the capture
        def step_current():
            if fused:
                b.dispatch_fused(d_x, d_idx, d_w, ring=ring)
            else:
                b.layout(d_idx)
                b.dispatch(d_x, d_idx, d_w, ring=ring)
            b.combine(y, d_idx, d_w)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(max(2, args.warmup)):
                step_current()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_current()
        torch.cuda.synchronize()

        def step(ev=None):
            graph.replay()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = int(b.dev_status.item())
    if st != 0:
        eprint(f"device status after warmup: {ep.status_str(st)}")
        return 1
    if ll:
        P = int(b.expert_offset[-1].item())
        ab = algorithmic_bytes_ll(w, P)
    else:
        P = int(b.rank_offset[-1].item())
        ab = algorithmic_bytes(w, P)

    K = args.steps
    every = max(1, args.op_events_every)
    sampled = [] if graph is not None else [i for i in range(K) if i % every == 0]
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for i in sampled}
    drained0 = ring.proxy_drained()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evs.get(i))
    torch.cuda.synchronize()
    if lb_bufs is not None:
        ring.wait_complete(60_000_000_000)
    t1 = time.perf_counter()
    elapsed = t1 - t0
    st = int(b.dev_status.item())
    if st != 0:
        eprint(f"device status after the timed steps: {ep.status_str(st)}")
        return 1
    n_cmds = (ring.proxy_drained() - drained0) / K

    def avg_ms(a, z):
        return sum(e[a].elapsed_time(e[z]) for e in evs.values()) / len(evs)

    if graph is None:
        t_layout, t_disp, t_comb = avg_ms(0, 1), avg_ms(1, 2), avg_ms(2, 3)
    else:
        # no events inside a replay: split the step by the byte model instead
        ms = elapsed * 1e3 / K
        t_layout = ms * ab["layout"] / ab["total"]
        t_disp = ms * ab["dispatch"] / ab["total"]
        t_comb = ms * ab["combine"] / ab["total"]

    # cold: before each step, read 1 GiB so that the 256 MB memory-side
    # cache holds only clean lines of other data (a write flush would leave
    # dirty lines whose write-back then lands inside the timed step)
    cold = None
    if args.cold_steps > 0 and graph is None:
        scratch = torch.ones((1 << 30) // 4, dtype=torch.int32, device=dev)
        sink = torch.zeros((), dtype=torch.int64, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            sink += scratch.sum()
            step(cev[i])
        torch.cuda.synchronize()
        n = args.cold_steps
        c_l = sum(e[0].elapsed_time(e[1]) for e in cev) / n
        c_d = sum(e[1].elapsed_time(e[2]) for e in cev) / n
        c_c = sum(e[2].elapsed_time(e[3]) for e in cev) / n
        tot = c_l + c_d + c_c
        cold = {"layout_us": round(c_l * 1e3, 2), "dispatch_us": round(c_d * 1e3, 2),
                "combine_us": round(c_c * 1e3, 2),
                "GBps": round(ab["total"] / (tot * 1e-3) / 1e9, 1),
                "note": "1 GiB read before each step; kernel spans from HIP events"}
        del scratch, sink
    lb_stats = ring.loopback_stats() if lb_bufs is not None else None
    ring.proxy_stop(0)
    ring.destroy()

    # practical ceiling: a plain 1 GiB device-to-device copy (read + write)
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    value = ab["total"] * K / elapsed / 1e9
    tokens_s = w.T * K / elapsed
    # dominant kernel: the longer of pack (inside ep_dispatch) and combine
    if t_disp >= t_comb:
        if ll and fused:
            dom, prefix = "ll_fused_small_kernel (ep_dispatch_ll_fused)", "ll_fused_small_kernel"
        elif ll:
            dom, prefix = "ll_pack_kernel (ep_dispatch_ll)", "ll_pack_kernel"
        elif fused:
            dom, prefix = "fused_small_kernel (ep_dispatch_fused)", "fused_small_kernel"
        else:
            dom, prefix = "pack_kernel (ep_dispatch)", "pack_kernel"
        dom_ms, dom_bytes = t_disp, ab["dispatch"] + (ab["layout"] if fused else 0)
    else:
        dom = "combine_kernel (ep_combine_ll)" if ll else "combine_kernel (ep_combine)"
        dom_ms, dom_bytes, prefix = t_comb, ab["combine"], "combine_kernel"
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9 if graph is None else None
    traffic = measured_traffic(prefix, w.name + ("-ll" if ll else ""))

    cpu = None
    if args.cpu_budget > 0:
        eprint("bench: timing the CPU oracle")
        cpu = cpu_baseline(w, inp, args.cpu_budget, args.mode)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.fmt == 0 else "fp8-e4m3 pack, bf16 combine",
        "data": "synthetic (seeded routing and token rows)",
        "config": {"workload": f"{w.name}: T={w.T} H={w.H} E={w.E} ranks={w.R} top-{w.k}, "
                               f"{w.channels} ring channels, depth {w.depth}, "
                               f"{w.max_inflight} in flight",
                   "tokens": w.T, "hidden": w.H, "experts": w.E, "ranks": w.R, "top_k": w.k,
                   "mode": "per-expert (low-latency)" if ll else "per-rank",
                   ("rows_Q" if ll else "pairs_P"): P, "parallelism": "one GPU's share of EP"},
        "tokens_per_s": round(tokens_s, 1),
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "pct_of_copy_ceiling": round(100 * value / copy_gbs, 2),
        "algorithmic_bytes_per_step": ab,
        "fused_layout_dispatch": fused,
        "per_op_us": {"layout": round(t_layout * 1e3, 2), "dispatch": round(t_disp * 1e3, 2),
                      "combine": round(t_comb * 1e3, 2),
                      "note": (f"HIP events on the launch stream, every {every}th of the {K} timed "
                               f"steps ({len(evs)} samples)" + ("; layout and dispatch are "
                               "one call (" + ("ep_dispatch_ll_fused" if ll else
                                               "ep_dispatch_fused") +
                               "): its time is under dispatch" if fused else "")) if graph is None else
                              "graph replays: the step time split in proportion to the byte model, "
                              "not measured per op"},
        "graph": graph is not None,
        "descriptors_per_step": n_cmds,
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": round(achieved, 1) if achieved is not None else None,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4) if achieved is not None else None,
                     "algorithmic_bytes": dom_bytes,
                     "traffic": traffic[0] if traffic else None,
                     "traffic_source": traffic[1] if traffic else None},
        "cold": cold,
        "loopback": None if lb_stats is None else dict(
            lb_stats,
            note="commands executed by the proxy threads (row copies into per-rank receive "
                 "regions, count adds); latency = pop to completion; the timed region ends "
                 "when every command has completed"),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
