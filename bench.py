#!/usr/bin/env python3
"""Benchmark of MoE expert-parallel dispatch + combine on one MI355X.

A step is one pass of the whole path over one batch: routing layout, pack +
TransferCmd emission (with the CPU proxy threads draining the ring), and the
gate-weighted combine of the returned rows.  The returned rows (y) sit in a
buffer of their own, filled once before timing: the packed rows themselves
(identity experts) for bf16, seeded N(0,1) bf16 rows for fp8.  Dispatch never
writes y, so combine does not read what dispatch has just written.

Cold is the headline.  The timed steps rotate over several sets of buffers
(x, routing, send buffer, y, out, workspace), enough that each step's data was
last touched at least ~2x the 256 MB memory-side cache (MALL) of other traffic
earlier: no line of it is still cached and its page translations are not
warm.  Every workload in --workloads is measured the same way; the first one
(train, the metric's EP32 top-8 configuration) gives the top-level `value`.
Per workload:
  cold     K rotating steps timed by wall clock (the `value`), per-op HIP
           events on every n-th of them, and the step time's p10/p50/p90 over
           --pct-reps further rotating steps (one event per step boundary);
  flushed  --flush-reps steps on one buffer set, each after reading 1 GiB of
           other memory (events around the step only): a cross-check of cold;
  warm     K steps back to back on one buffer set (secondary).

Prints one JSON line.  The CPU oracle is timed on the headline workload on
one thread and on all host cores (OpenMP over tokens in pack and combine).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workloads train,fp8,...]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine effective HBM GB/s (% of peak) and tokens/s, EP32 top-8"
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
MALL_BYTES = 256 << 20  # MI355X memory-side cache (Infinity Cache)
DEFAULT_WORKLOADS = "train,fp8,skewed,decode,tiny"
BAR_FRAC = 0.60


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
    once and each output written once.  Its layout needs no rank outputs:
    read the ids, write the expert counts and offsets and the row table."""
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    rb = row_bytes(H, w.fmt)
    layout = 4 * T * k + 4 * (2 * E + 1) + 4 * T * k
    pack_r = 2 * T * H + 8 * T * k + 4 * T * k + 4 * (E + 1)
    pack_w = Q * rb + Q * 8
    comb_r = 2 * Q * H + 8 * T * k + 4 * T * k
    comb_w = 2 * T * H
    return {"layout": layout, "dispatch": pack_r + pack_w, "combine": comb_r + comb_w,
            "total": layout + pack_r + pack_w + comb_r + comb_w}


def rotation_sets(step_bytes: int) -> int:
    """Buffer sets the cold steps rotate over: enough that a set's data was
    last touched >= 2x the MALL of other traffic ago (2..16 sets)."""
    return max(2, min(16, math.ceil(2 * MALL_BYTES / max(step_bytes, 1)) + 1))


def quantiles(vals) -> dict:
    import numpy as np
    a = np.asarray(vals, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2),
            "p50": round(float(np.percentile(a, 50)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


KERNEL_SOURCES = ["combine_topk_rank_amd/csrc/ep_dispatch.hip",
                  "combine_topk_rank_amd/csrc/ep_combine.hip",
                  "combine_topk_rank_amd/csrc/ep_layout.hip",
                  "combine_topk_rank_amd/csrc/ep_common.h",
                  "combine_topk_rank_amd/csrc/ep_route.h",
                  "combine_topk_rank_amd/csrc/ep_ring_proto.h"]


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
            hits = [c for c in block.get("counters", [])
                    if kernel_prefix in c["kernel"] and c["workload"] == workload]
            # a pack kernel's last template argument is its publication mode:
            # prefer the one with a ring (the timed launches) over the
            # set-up launches without one ("..., 0>")
            hits.sort(key=lambda c: c["kernel"].endswith(", 0>"))
            if hits:
                return int(hits[0]["traffic_bytes"]), os.path.relpath(path, ROOT)
    return None


# ------------------------------------------------------------------ CPU oracle

def host_info() -> dict:
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for ln in out.splitlines():
            if ln.startswith("Model name:"):
                model = ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"nproc": usable, "cpu_count": os.cpu_count(), "model": model}


def cpu_threads_all(info: dict) -> int:
    """All host cores this process may use (OMP_NUM_THREADS caps it when set,
    as on machines that share their cores between jobs)."""
    n = info["nproc"]
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(w, inp, budget_s: float, threads: int, mode: str = "rank") -> dict:
    """The oracle as it stands on whole passes of the same workload until
    about budget_s seconds of wall clock; pack and combine split their token
    loops over `threads` OpenMP threads, layout and descriptors run on one."""
    import numpy as np
    import oracle
    oracle.default()
    used = oracle.set_threads(threads)
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
    oracle.set_threads(1)
    per = t_total / passes
    ab = algorithmic_bytes_ll(w, P) if mode == "ll" else algorithmic_bytes(w, P)
    gbs = ab["total"] / per / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": used, "kind": "oracle",
            "tokens_per_s": round(w.T / per, 1),
            "sample": f"{passes} whole pass(es) of the {w.name} workload"
                      f"{' (per-expert mode)' if mode == 'll' else ''} (layout, pack, "
                      f"descriptors, combine) on {used} thread(s); {per:.3f} s per pass"}


# ------------------------------------------------------------------ GPU runner

class Runner:
    """One workload on the GPU: `nsets` buffer sets (each with its own copy
    of the inputs), one ring whose proxy threads drain every dispatch, and a
    step on any set.  Plumbing only: every step is three calls of the C ABI."""

    def __init__(self, w, inp, args, nsets: int, dev):
        import numpy as np
        import torch

        import combine_topk_rank_amd as ep
        self.ep, self.torch, self.w, self.dev = ep, torch, w, dev
        self.ll = args.mode == "ll"
        if self.ll:
            self.fused = args.fused == "on" or (args.fused == "auto" and w.T <= 256 and w.E <= 1024)
        else:
            # the one call when it is one kernel (small batches; large bf16
            # batches, through a grid barrier), else the two calls, whose
            # per-op events then time the layout on its own
            self.fused = args.fused == "on" or (
                args.fused == "auto" and ep.ep_dispatch_fused_plan(
                    ep.shape(w.T, w.H, w.E, w.R, w.k, w.fmt)) != ep.EP_FUSED_TWO_CALLS)
        s = ep.shape(w.T, w.H, w.E, w.R, w.k, w.fmt)
        self.shape = s
        self.plan = ep.ep_dispatch_fused_plan(s) if (self.fused and not self.ll) else None
        # per-expert layout in one kernel (ep_dispatch_ll_layout) where it takes
        # the shape (E <= 1024, every tile resident); the first call finds out
        self.ll_one = self.ll and not self.fused and w.E <= 1024
        self.stream = torch.cuda.current_stream()
        x0 = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        i0 = torch.from_numpy(inp["topk_idx"]).to(dev)
        w0 = torch.from_numpy(inp["topk_w"]).to(dev)
        self.sets = []
        for j in range(nsets):
            b = ep.BuffersLL(s, device=dev) if self.ll else ep.Buffers(s, device=dev)
            st = {"b": b, "x": x0 if j == 0 else x0.clone(), "idx": i0 if j == 0 else i0.clone(),
                  "w": w0 if j == 0 else w0.clone()}
            # one pass without a ring fills the send buffer and the layout
            self._dispatch(st, ring=None)
            torch.cuda.synchronize()
            P = int((b.expert_offset if self.ll else b.rank_offset)[-1].item())
            if w.fmt == 0:
                y = b.send_buf[:P].clone().view(torch.bfloat16).reshape(P, w.H)
            else:
                g = torch.Generator(device=dev).manual_seed(0)
                y = torch.randn((max(P, 1), w.H), generator=g, device=dev,
                                dtype=torch.float32).to(torch.bfloat16)
            st["y"] = y
            self.sets.append(st)
        self.P = P
        self.ab = algorithmic_bytes_ll(w, P) if self.ll else algorithmic_bytes(w, P)
        self.ring = ep.Ring(w.depth, w.channels, w.max_inflight, 10_000_000_000)
        self.lb = None
        if args.loopback:
            self._set_loopback()
        self.ring.proxy_start(args.proxy_threads, 0)
        self.graphs = None
        if args.graph:
            self._capture(args.warmup)

    def _dispatch(self, st, ring, stream=None):
        b = st["b"]
        if self.fused:
            b.dispatch_fused(st["x"], st["idx"], st["w"], ring=ring, stream=stream)
        else:
            self._layout(st, stream)
            b.dispatch(st["x"], st["idx"], st["w"], ring=ring, stream=stream)

    def _layout(self, st, stream):
        if self.ll_one:
            try:
                st["b"].layout_one_call(st["idx"], stream)
                return
            except self.ep.EpError:
                self.ll_one = False   # rejected on the host, nothing enqueued
        st["b"].layout(st["idx"], stream)

    def _set_loopback(self):
        """Receive regions per rank for set 0 (loopback runs on one set)."""
        torch, w = self.torch, self.w
        b = self.sets[0]["b"]
        epr = w.E // w.R
        if self.ll:
            eo = b.expert_offset.cpu().numpy()
            nrows = [int(eo[(r + 1) * epr] - eo[r * epr]) for r in range(w.R)]
            nwords = epr
        else:
            ro = b.rank_offset.cpu().numpy()
            nrows = [int(ro[r + 1] - ro[r]) for r in range(w.R)]
            nwords = 1
        recv = [torch.empty(max(n, 1) * b.row_bytes, dtype=torch.uint8, device=self.dev)
                for n in nrows]
        cnt = [torch.zeros(nwords, dtype=torch.int32, device=self.dev) for _ in range(w.R)]
        self.lb = (recv, cnt)
        self.ring.set_loopback(b.send_buf, recv, cnt)

    def _capture(self, warmup):
        """One HIP graph per buffer set (layout, dispatch with the ring,
        combine), captured on a side stream after eager warm-up there."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(max(2, warmup)):
                for st in self.sets:
                    self._step_current(st)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graphs = []
        for st in self.sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._step_current(st)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def _step_current(self, st):
        # the library launches on torch's current stream (the capture stream
        # inside a capture)
        self._dispatch(st, self.ring)
        st["b"].combine(st["y"], st["idx"], st["w"])

    def step(self, j: int, ev=None):
        """One pass on buffer set j; ev: 4 events around layout, dispatch,
        combine (not with graphs)."""
        if self.graphs is not None:
            self.graphs[j % len(self.graphs)].replay()
            return
        st = self.sets[j % len(self.sets)]
        b, s = st["b"], self.stream
        if ev is not None:
            ev[0].record(s)
        if not self.fused:
            self._layout(st, s)
        if ev is not None:
            ev[1].record(s)
        if self.fused:
            b.dispatch_fused(st["x"], st["idx"], st["w"], ring=self.ring, stream=s)
        else:
            b.dispatch(st["x"], st["idx"], st["w"], ring=self.ring, stream=s)
        if ev is not None:
            ev[2].record(s)
        b.combine(st["y"], st["idx"], st["w"], s)
        if ev is not None:
            ev[3].record(s)
        if self.lb is not None:
            # loopback copies read the send buffer: the next dispatch may
            # rewrite it only once every command has completed
            self.torch.cuda.synchronize()
            self.ring.wait_complete(60_000_000_000)

    def status(self) -> int:
        for st in self.sets:
            v = int(st["b"].dev_status.item())
            if v:
                return v
        return 0

    def close(self):
        self.ring.proxy_stop(0)
        self.ring.destroy()
        self.sets = []
        self.graphs = None


def new_events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def per_op(evs: list, fused: bool, ll: bool, K: int) -> dict:
    n = len(evs)
    ms = lambda a, z: sum(e[a].elapsed_time(e[z]) for e in evs) / n
    d = {"layout": round(ms(0, 1) * 1e3, 2), "dispatch": round(ms(1, 2) * 1e3, 2),
         "combine": round(ms(2, 3) * 1e3, 2), "samples": n}
    if fused:
        d["note"] = ("layout and dispatch are one call (" +
                     ("ep_dispatch_ll_fused" if ll else "ep_dispatch_fused") +
                     "): its time is under dispatch; the layout column is the gap between two "
                     "events with no kernel between them")
    return d


def timed_steps(run: Runner, K: int, first: int, rotate: bool, every: int):
    """K steps (rotating over the buffer sets, or all on set 0) timed by
    wall clock between two device synchronisations; per-op events on every
    `every`-th step (none with graphs)."""
    torch = run.torch
    sampled = [] if run.graphs is not None else [i for i in range(K) if i % every == 0]
    evs = {i: new_events(4) for i in sampled}
    drained0 = run.ring.proxy_drained()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        run.step(first + i if rotate else 0, evs.get(i))
    torch.cuda.synchronize()
    if run.lb is not None:
        run.ring.wait_complete(60_000_000_000)
    elapsed = time.perf_counter() - t0
    cmds = (run.ring.proxy_drained() - drained0) / K
    return elapsed, (list(evs.values()) if evs else None), cmds


def step_percentiles(run: Runner, n: int, first: int) -> list:
    """Durations (ms) of n rotating steps, one event at each step boundary."""
    torch = run.torch
    ev = new_events(n + 1)
    torch.cuda.synchronize()
    for i in range(n):
        ev[i].record(run.stream)
        run.step(first + i)
    ev[n].record(run.stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def flushed_steps(run: Runner, n: int, scratch, sink):
    """n steps on set 0, each after reading `scratch` (1 GiB): step spans and
    per-op times from events."""
    torch = run.torch
    evs = [new_events(4) for _ in range(n)]
    for i in range(n):
        sink += scratch.sum()
        run.step(0, evs[i])
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[3]) for e in evs], evs


PRE_STEPS = ("none", "gpu_spin", "read64m", "read256m", "read1g", "write1g", "other_set")


def pre_step_times(run: Runner, names, reps: int, scratch, sink) -> dict:
    """Median layout / dispatch / combine times of a step on buffer set 0
    right after a given other piece of work (what the memory system holds
    when the step starts): nothing, a 1 ms GPU spin without memory traffic,
    a read of 64 MB / 256 MB / 1 GiB or a write of 1 GiB of other memory, or
    a step on buffer set 1."""
    import numpy as np
    torch = run.torch
    acts = {
        "none": lambda: None,
        "gpu_spin": lambda: torch.cuda._sleep(2_000_000),
        "read64m": lambda: sink.add_(scratch[: (64 << 20) // 4].sum()),
        "read256m": lambda: sink.add_(scratch[: (256 << 20) // 4].sum()),
        "read1g": lambda: sink.add_(scratch.sum()),
        "write1g": lambda: scratch.fill_(1),
        "other_set": lambda: run.step(1),
    }
    out = {}
    for n in names:
        if n == "other_set" and len(run.sets) < 2:
            continue
        evs = [new_events(4) for _ in range(reps)]
        for r in range(reps):
            acts[n]()
            run.step(0, evs[r])
        torch.cuda.synchronize()
        d = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                      for e in evs]) * 1e3
        med = np.median(d, axis=0)
        out[n] = {"layout": round(float(med[0]), 1), "dispatch": round(float(med[1]), 1),
                  "combine": round(float(med[2]), 1)}
        eprint(f"bench: {run.w.name} after {n}: layout/dispatch/combine us {out[n]}")
    return out


def dominant(run: Runner, ops: dict):
    """The longer of the pack (inside dispatch) and the combine kernel."""
    ab = run.ab
    if ops["dispatch"] >= ops["combine"]:
        if run.ll and run.fused:
            name, prefix = "ll_fused_small_kernel (ep_dispatch_ll_fused)", "ll_fused_small_kernel"
        elif run.ll:
            name, prefix = "ll_pack_kernel (ep_dispatch_ll)", "ll_pack_kernel"
        elif run.fused and run.plan == run.ep.EP_FUSED_ONE_KERNEL_SMALL:
            name, prefix = "fused_small_kernel (ep_dispatch_fused)", "fused_small_kernel"
        elif run.fused and run.plan == run.ep.EP_FUSED_ONE_KERNEL_LARGE:
            name, prefix = "fused_large_kernel (ep_dispatch_fused)", "fused_large_kernel"
        else:
            name, prefix = "pack_kernel (ep_dispatch)", "pack_kernel"
        # the one call's layout and pack are one kernel (or two back to back)
        return name, prefix, ops["dispatch"], ab["dispatch"] + (ab["layout"] if run.fused else 0)
    name = "combine_kernel (ep_combine_ll)" if run.ll else "combine_kernel (ep_combine)"
    return name, "combine_kernel", ops["combine"], ab["combine"]


def gbs(nbytes: float, ms: float) -> float:
    return nbytes / (ms * 1e-3) / 1e9


def bench_workload(w, args, scratch, sink, dev) -> dict:
    """All phases of one workload; returns its entry (headline fields for the
    top level included)."""
    import torch
    import workloads as W
    ll = args.mode == "ll"
    inp = W.make_inputs(w, 0)
    # per-step footprint from a first estimate of P (average fan-out 7.3)
    est = algorithmic_bytes(w, int(w.T * min(w.k, w.R)))["total"]
    nsets = 1 if (args.loopback or args.cold_sets == 1) else (
        args.cold_sets if args.cold_sets > 0 else rotation_sets(est))
    eprint(f"bench: {w.name} T={w.T} H={w.H} E={w.E} R={w.R} k={w.k} fmt={w.fmt} "
           f"mode={args.mode} buffer sets={nsets}")
    run = Runner(w, inp, args, nsets, dev)
    K, every = args.steps, max(1, args.op_events_every)
    ab, P = run.ab, run.P
    for i in range(args.warmup):
        run.step(i)
    torch.cuda.synchronize()
    st = run.status()
    if st:
        raise RuntimeError(f"{w.name}: device status after warmup: {run.ep.status_str(st)}")

    entry = {"workload": f"{w.name}: T={w.T} H={w.H} E={w.E} ranks={w.R} top-{w.k}, "
                         f"{'fp8 e4m3 rows' if w.fmt else 'bf16 rows'}, {w.channels} ring "
                         f"channel(s), depth {w.depth}, {w.max_inflight} in flight",
             ("rows_Q" if ll else "pairs_P"): P, "bytes_per_step": ab["total"],
             "algorithmic_bytes_per_step": ab, "buffer_sets": nsets,
             "fused_layout_dispatch": run.fused, "graph": run.graphs is not None}
    if run.plan is not None:
        entry["fused_plan"] = {run.ep.EP_FUSED_ONE_KERNEL_SMALL: "one kernel (small batch)",
                               run.ep.EP_FUSED_ONE_KERNEL_LARGE: "one kernel (grid barrier)",
                               run.ep.EP_FUSED_TWO_CALLS: "layout call, then dispatch call"}[run.plan]

    # cold (headline): K rotating steps by wall clock
    el, evs, cmds = timed_steps(run, K, args.warmup, rotate=nsets > 1, every=every)
    cold_ms = el * 1e3 / K
    cold = {"GBps": round(gbs(ab["total"], cold_ms), 1),
            "pct_of_peak": round(100 * gbs(ab["total"], cold_ms) / PEAK_HBM_GBS, 2),
            "us_per_step": round(cold_ms * 1e3, 2), "tokens_per_s": round(w.T / (cold_ms * 1e-3), 1),
            "steps": K}
    ops = per_op(evs, run.fused, ll, K) if evs else None
    if ops:
        cold["per_op_us"] = ops
    entry["descriptors_per_step"] = cmds
    entry["_elapsed"], entry["_cold_ms"] = el, cold_ms

    if run.graphs is None and args.pct_reps > 0:
        d = step_percentiles(run, args.pct_reps, args.warmup + K)
        q = quantiles([x * 1e3 for x in d])
        cold["step_us"] = q
        cold["reps"] = args.pct_reps
        cold["GBps_p50"] = round(gbs(ab["total"], q["p50"] * 1e-3), 1)
        cold["pct_of_peak_p50"] = round(100 * cold["GBps_p50"] / PEAK_HBM_GBS, 2)
        cold["GBps_p10_p90"] = [round(gbs(ab["total"], q["p90"] * 1e-3), 1),
                                round(gbs(ab["total"], q["p10"] * 1e-3), 1)]
    entry["cold"] = cold

    if ops:
        name, prefix, dom_us, dom_bytes = dominant(run, ops)
        achieved = gbs(dom_bytes, dom_us * 1e-3)
        traffic = measured_traffic(prefix, w.name + ("-ll" if ll else ""))
        entry["roofline"] = {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(achieved / PEAK_HBM_GBS, 4),
                             "traffic": traffic[0] if traffic else None,
                             "algorithmic_bytes": dom_bytes,
                             "duration_us": dom_us,
                             "traffic_source": traffic[1] if traffic else None,
                             "note": "algorithmic bytes of one launch / its mean duration from "
                                     "HIP events on the launch stream in the cold timed steps"}
        if run.plan == run.ep.EP_FUSED_ONE_KERNEL_LARGE and prefix == "fused_large_kernel":
            entry["roofline"]["note"] += (
                "; this kernel is the routing layout and the pack in one launch, so its time "
                "includes the layout's latency (id loads, ballots, a grid barrier and a table "
                "read before the first row store): algorithmic bytes are the layout's and the "
                "pack's")

    if run.graphs is None and args.flush_reps > 0:
        d, fevs = flushed_steps(run, args.flush_reps, scratch, sink)
        q = quantiles([x * 1e3 for x in d])
        entry["flushed"] = {"step_us": q, "reps": args.flush_reps,
                            "GBps_p50": round(gbs(ab["total"], q["p50"] * 1e-3), 1),
                            "per_op_us": per_op(fevs, run.fused, ll, args.flush_reps),
                            "note": "1 GiB of other memory read before each step; one buffer set"}

    if args.warm:
        el_w, evs_w, _ = timed_steps(run, K, 0, rotate=False, every=every)
        warm_ms = el_w * 1e3 / K
        entry["warm"] = {"GBps": round(gbs(ab["total"], warm_ms), 1),
                         "pct_of_peak": round(100 * gbs(ab["total"], warm_ms) / PEAK_HBM_GBS, 2),
                         "us_per_step": round(warm_ms * 1e3, 2)}
        if evs_w:
            entry["warm"]["per_op_us"] = per_op(evs_w, run.fused, ll, K)

    if args.pre_steps and run.graphs is None:
        entry["pre_steps"] = dict(
            pre_step_times(run, [n for n in args.pre_steps.split(",") if n], args.pre_reps,
                           scratch, sink),
            note="median per-op us (HIP events) of a step on one buffer set right after the "
                 "named work")

    st = run.status()
    if st:
        raise RuntimeError(f"{w.name}: device status after the timed steps: "
                           f"{run.ep.status_str(st)}")
    if run.lb is not None:
        entry["loopback"] = dict(run.ring.loopback_stats(),
                                 note="commands executed by the proxy threads (row copies into "
                                      "per-rank receive regions, count adds); latency = pop to "
                                      "completion; the timed region ends when every command "
                                      "has completed")
    p50 = cold.get("GBps_p50", cold["GBps"])
    entry["meets_60pct_of_peak"] = bool(p50 >= BAR_FRAC * PEAK_HBM_GBS)
    run.close()
    del run
    torch.cuda.empty_cache()
    entry["_inputs"] = inp
    return entry


def ceilings(dev) -> dict:
    """Read, write and copy rates of torch's own kernels over 1 GiB on this
    GPU: practical reference points next to the 8 TB/s peak.  The read rate
    is the best of a few whole-tensor reductions (torch has no plain read)."""
    import torch
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream()

    def rate(fn, nbytes, reps=5):
        fn()
        e0, e1 = new_events(2)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return round(reps * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)

    f = a.view(torch.float32)
    m = a.view(torch.bfloat16).view(-1, 8192)
    v = torch.ones(8192, dtype=torch.bfloat16, device=dev)
    reads = {"sum of int32": lambda: sink.add_(a.sum()),
             "amax of float32": lambda: sink.add_(f.amax()),
             "bf16 matrix-vector product": lambda: sink.add_(torch.mv(m, v)[0].float())}
    rr = {k: rate(fn, n) for k, fn in reads.items()}
    best = max(rr, key=rr.get)
    out = {"read_GBps": rr[best], "read_kernel": best, "reads_GBps": rr,
           "write_GBps": rate(lambda: b.fill_(3), n),
           "copy_GBps": rate(lambda: b.copy_(a), 2 * n),
           "note": "torch kernels over 1 GiB (read: the best of the reductions listed; fill for "
                   "write; copy counts read + write bytes)"}
    del a, b, f, m
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps per phase (K)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default=DEFAULT_WORKLOADS,
                    help="comma-separated workloads; the first gives the top-level value")
    ap.add_argument("--workload", default=None, help="a single workload (same as --workloads X)")
    ap.add_argument("--mode", choices=("rank", "ll"), default="rank",
                    help="rank: one row per (token, rank) pair; ll: the per-expert "
                         "(low-latency) mode, one row per kept choice")
    ap.add_argument("--fused", choices=("auto", "on", "off"), default="auto",
                    help="layout + dispatch in one call (ep_dispatch_fused: one kernel for "
                         "T <= 256 and for large bf16 batches whose rows take one wavefront; "
                         "per-expert mode: ep_dispatch_ll_fused, T <= 256 and E <= 1024); "
                         "auto: where the call is one kernel")
    ap.add_argument("--cold-sets", type=int, default=0,
                    help="buffer sets the cold steps rotate over (0: enough to exceed twice the "
                         "MALL; 1: no rotation)")
    ap.add_argument("--pct-reps", type=int, default=100,
                    help="rotating steps timed one by one for the p10/p50/p90 of the step time")
    ap.add_argument("--flush-reps", type=int, default=100,
                    help="steps each after a 1 GiB read (0: skip)")
    ap.add_argument("--no-warm", dest="warm", action="store_false",
                    help="skip the warm back-to-back phase")
    ap.add_argument("--pre-steps", default="",
                    help="comma-separated work to run right before each of --pre-reps steps, "
                         "timed per op: " + ",".join(PRE_STEPS) + " (empty: skip)")
    ap.add_argument("--pre-reps", type=int, default=12)
    ap.add_argument("--loopback", action="store_true",
                    help="proxy threads execute every command against per-rank receive regions "
                         "and count words (one buffer set); the timed region then ends when "
                         "every command has completed")
    ap.add_argument("--graph", action="store_true",
                    help="capture each buffer set's step (layout, dispatch, combine) in a HIP "
                         "graph and time replays (no per-op events)")
    ap.add_argument("--proxy-threads", type=int, default=4)
    ap.add_argument("--op-events-every", type=int, default=5,
                    help="record per-op HIP events on every n-th timed step (events between "
                         "kernels cost about a microsecond each)")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle wall clock per thread setting (0: skip)")
    ap.add_argument("--no-ceilings", dest="ceilings", action="store_false")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="only run 5 plain device-to-device copies of this many MiB (a known "
                         "byte count for scaling hardware traffic counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the EP ranks are "
              "simulated as regions of one GPU's HBM", file=sys.stderr)
        return 2
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

    import torch

    import workloads as W
    names = [args.workload] if args.workload else [n for n in args.workloads.split(",") if n]
    for n in names:
        if n not in W.WORKLOADS:
            print(f"unknown workload {n}; known: {', '.join(W.WORKLOADS)}", file=sys.stderr)
            return 2
    for n in [n for n in args.pre_steps.split(",") if n]:
        if n not in PRE_STEPS:
            print(f"unknown pre-step {n}; known: {', '.join(PRE_STEPS)}", file=sys.stderr)
            return 2
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    ceil = ceilings(dev) if args.ceilings else None
    need_scratch = args.flush_reps > 0 or bool(args.pre_steps)
    scratch = torch.ones((1 << 30) // 4, dtype=torch.int32, device=dev) if need_scratch else None
    sink = torch.zeros((), dtype=torch.int64, device=dev)

    entries = {}
    for n in names:
        entries[n] = bench_workload(W.WORKLOADS[n], args, scratch, sink, dev)
    del scratch
    head_name = names[0]
    head = entries[head_name]
    w = W.WORKLOADS[head_name]
    inp = head.pop("_inputs")
    elapsed, cold_ms = head.pop("_elapsed"), head.pop("_cold_ms")
    for e in entries.values():
        for key in ("_inputs", "_elapsed", "_cold_ms"):
            e.pop(key, None)

    cpu = None
    if args.cpu_budget > 0:
        info = host_info()
        nall = cpu_threads_all(info)
        eprint(f"bench: timing the CPU oracle on 1 and {nall} thread(s)")
        one = cpu_baseline(w, inp, args.cpu_budget, 1, args.mode)
        cpu = cpu_baseline(w, inp, args.cpu_budget, nall, args.mode) if nall > 1 else dict(one)
        cpu["single_thread"] = {k: one[k] for k in ("value", "cores", "tokens_per_s", "sample")}
        cpu["host"] = dict(info, threads_used=cpu["cores"])

    K = args.steps
    value = head["bytes_per_step"] / (cold_ms * 1e-3) / 1e9
    ll = args.mode == "ll"
    summary = {n: {"cold_GBps_p50": e["cold"].get("GBps_p50", e["cold"]["GBps"]),
                   "pct_of_peak_p50": e["cold"].get("pct_of_peak_p50", e["cold"]["pct_of_peak"]),
                   "meets_60pct_of_peak": e["meets_60pct_of_peak"]} for n, e in entries.items()}
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(cold_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.fmt == 0 else "fp8-e4m3 pack, bf16 combine",
        "data": "synthetic (seeded routing and token rows)",
        "config": {"workload": head["workload"], "tokens": w.T, "hidden": w.H, "experts": w.E,
                   "ranks": w.R, "top_k": w.k,
                   "mode": "per-expert (low-latency)" if ll else "per-rank",
                   ("rows_Q" if ll else "pairs_P"): head.get("rows_Q" if ll else "pairs_P"),
                   "parallelism": "one GPU's share of EP"},
        "tokens_per_s": round(w.T / (cold_ms * 1e-3), 1),
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "timing": "cold: the K timed steps rotate over buffer sets so that no step finds its "
                  "data in the 256 MB MALL; wall clock between two device synchronisations",
        "roofline": head.get("roofline"),
        "cpu_baseline": cpu,
        "ceilings": ceil,
        "summary": summary,
        "configs": entries,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
