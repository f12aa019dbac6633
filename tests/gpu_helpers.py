"""Helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the CPU oracle."""

from __future__ import annotations

import collections
import sys

import numpy as np

import oracle
import workloads as W

POISON = 0xA5


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev_bf16(bits: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    return t.cpu().numpy()


def run_hip(T, H, E, R, k, fmt, x, idx, w, capacity_rows=None, ring_cfg=None,
            proxy_threads=4, poison=POISON, log_capacity=1 << 20, repeat=1, fused=False):
    """layout + dispatch through the C ABI (fused: ep_dispatch_fused, one
    call).  ring_cfg = (depth, channels, max_inflight, timeout_ns) or None.
    Returns numpy outputs, the proxy log and the device status."""
    import combine_topk_rank_amd as ep
    torch = torch_mod()
    s = ep.shape(T, H, E, R, k, fmt)
    cap = T * min(k, R) if capacity_rows is None else capacity_rows
    buf = ep.Buffers(s, capacity_rows=cap)
    buf.send_buf.fill_(poison)
    buf.slot_src.fill_(-7)
    buf.slot_local_idx.fill_(-7)
    buf.slot_local_w.fill_(float("nan"))
    buf.send_slot.fill_(-99)
    buf.is_token_in_rank.fill_(7)
    d_x = dev_bf16(x)
    d_idx = dev(idx)
    d_w = dev(w)
    ring = None
    if ring_cfg is not None:
        ring = ep.Ring(*ring_cfg)
        if proxy_threads:
            ring.proxy_start(proxy_threads, log_capacity)
    logs = []
    for _ in range(repeat):
        if fused:
            buf.dispatch_fused(d_x, d_idx, d_w, ring=ring)
        else:
            buf.layout(d_idx)
            buf.dispatch(d_x, d_idx, d_w, ring=ring)
        torch.cuda.synchronize()
    if ring is not None and proxy_threads:
        lg, n_drained = ring.proxy_stop(log_capacity)
        logs.append((lg, n_drained))
    out = {
        "num_tokens_per_rank": host(buf.num_tokens_per_rank),
        "num_tokens_per_expert": host(buf.num_tokens_per_expert),
        "rank_offset": host(buf.rank_offset),
        "expert_offset": host(buf.expert_offset),
        "is_token_in_rank": host(buf.is_token_in_rank),
        "send_slot": host(buf.send_slot),
        "send_buf": host(buf.send_buf),
        "slot_src": host(buf.slot_src),
        "slot_local_idx": host(buf.slot_local_idx),
        "slot_local_w": host(buf.slot_local_w),
        "status": int(host(buf.dev_status)[0]),
        "logs": logs,
        "ring": ring,
        "buffers": buf,
        "d_idx": d_idx,
        "d_w": d_w,
    }
    return out


def run_hip_combine(buf, y_bits: np.ndarray, d_idx, d_w):
    import combine_topk_rank_amd as ep
    torch = torch_mod()
    y = dev_bf16(y_bits) if y_bits.shape[0] else torch.zeros((1, buf.shape.H), dtype=torch.bfloat16,
                                                              device="cuda")
    buf.dev_status.zero_()
    buf.out.fill_(float("nan"))
    ep.ep_combine(buf.shape, y, d_idx, d_w, buf.send_slot, buf.out, buf.dev_status)
    torch.cuda.synchronize()
    o = buf.out.view(torch.int16).cpu().numpy().view(np.uint16)
    return W.bf16_bits_to_f32(o).astype(np.float64), int(host(buf.dev_status)[0])


LAYOUT_KEYS = ("num_tokens_per_rank", "num_tokens_per_expert", "rank_offset", "expert_offset",
               "is_token_in_rank", "send_slot")


def assert_layout_equal(g, L):
    for key in LAYOUT_KEYS:
        a, b = g[key], L[key]
        assert a.shape == b.shape, key
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)[:5]
            raise AssertionError(f"{key} differs at {bad.tolist()}: gpu {a[tuple(bad[0])]} "
                                 f"oracle {b[tuple(bad[0])]}")


def assert_pack_equal(g, pk, P):
    cap = g["send_buf"].shape[0]
    a, b = g["send_buf"], pk["send_buf"]
    if not np.array_equal(a, b):
        rows = np.nonzero(np.any(a != b, axis=1))[0]
        raise AssertionError(f"send_buf differs in {rows.size} rows, first {rows[:5].tolist()}")
    n = min(P, cap)
    assert np.array_equal(g["slot_src"][:n], pk["slot_src"][:n])
    assert np.array_equal(g["slot_local_idx"][:n], pk["slot_local_idx"][:n])
    assert np.array_equal(g["slot_local_w"][:n].view(np.uint32), pk["slot_local_w"][:n].view(np.uint32))
    # untouched beyond P
    assert np.all(g["slot_src"][n:] == -7)


def cmd_key(d):
    return (int(d["type"]), int(d["op"]), int(d["num_tokens"]), int(d["dst_rank"]),
            int(d["size_or_value"]), int(d["src_offset"]), int(d["dst_offset"]))


def assert_descriptors(log_, want, channels, first_seq=None):
    """Same multiset of commands; per channel the seq numbers are consecutive
    tickets (none lost or repeated) and each rank's ATOMIC comes after its
    WRITEs."""
    got = sorted(cmd_key(d) for d in log_)
    exp = sorted(cmd_key(d) for d in want)
    if got != exp:
        cg, ce = collections.Counter(got), collections.Counter(exp)
        raise AssertionError(f"descriptor multisets differ: missing {list((ce - cg).items())[:4]} "
                             f"extra {list((cg - ce).items())[:4]} ({len(got)} vs {len(exp)})")
    by_ch = collections.defaultdict(list)
    for d in log_:
        by_ch[int(d["dst_rank"]) % channels].append(d)
    for c, ds in by_ch.items():
        seqs = np.sort(np.array([int(d["seq"]) for d in ds], np.int64))
        assert np.all(np.diff(seqs) == 1), f"channel {c}: tickets not consecutive"
        if first_seq is not None:
            assert seqs[0] == first_seq
        last_write = collections.defaultdict(lambda: -1)
        atomic_seq = {}
        for d in ds:
            r = int(d["dst_rank"])
            if d["type"] == 1:
                last_write[r] = max(last_write[r], int(d["seq"]))
            else:
                atomic_seq[r] = int(d["seq"])
        for r, sa in atomic_seq.items():
            assert sa > last_write[r], f"rank {r}: ATOMIC before a WRITE"


def pack_streams(T, H, fmt):
    """Whether a pack of T tokens publishes as messages complete (1024 or
    more whole-chunk wavefronts) rather than in closed form: the chunking of
    the pack kernels (vectors per lane by row size)."""
    nv = H // 8
    if nv <= 64:
        vpl = 1
    elif nv <= 128:
        vpl = 2
    elif nv <= 256:
        vpl = 4
    elif nv <= 512:
        vpl = 8
    elif fmt != 0:
        vpl = 14 if nv <= 896 else 8
    else:
        vpl = 14 if nv <= 896 else 16
    return T * -(-nv // (vpl * 64)) >= 1024


def assert_ll_descriptors(log_, want, channels, expert_offset, E, R, row_bytes_):
    """Per-expert streaming publication: the same multiset of commands; per
    channel consecutive tickets from 1; each expert's ATOMIC after all of
    its WRITEs."""
    got = sorted(cmd_key(d) for d in log_)
    exp = sorted(cmd_key(d) for d in want)
    if got != exp:
        cg, ce = collections.Counter(got), collections.Counter(exp)
        raise AssertionError(f"descriptor multisets differ: missing {list((ce - cg).items())[:4]} "
                             f"extra {list((cg - ce).items())[:4]} ({len(got)} vs {len(exp)})")
    epr = E // R
    eo = np.asarray(expert_offset, np.int64)
    by_ch = collections.defaultdict(list)
    for d in log_:
        by_ch[int(d["dst_rank"]) % channels].append(d)
    for c, ds in by_ch.items():
        seqs = np.sort(np.array([int(d["seq"]) for d in ds], np.int64))
        assert seqs[0] == 1 and np.all(np.diff(seqs) == 1), f"channel {c}: tickets not 1, 2, ..."
        last_write, atomic_seq = {}, {}
        for d in ds:
            r = int(d["dst_rank"])
            if d["type"] == 1:
                rel = int(d["dst_offset"]) // row_bytes_ + int(eo[r * epr])
                e = int(np.searchsorted(eo[r * epr:(r + 1) * epr + 1], rel, side="right")) - 1 + r * epr
                last_write[e] = max(last_write.get(e, -1), int(d["seq"]))
            else:
                atomic_seq[r * epr + int(d["dst_offset"]) // 4] = int(d["seq"])
        for e, sa in atomic_seq.items():
            assert sa > last_write.get(e, -1), f"expert {e}: ATOMIC before a WRITE"
        assert set(last_write) <= set(atomic_seq), "an expert's WRITEs without its ATOMIC"


def combine_tolerance_check(got, ref, what=""):
    """|gpu - ref| <= 1e-2 * max(1, |ref|) element by element."""
    err = np.abs(got - ref)
    lim = 1e-2 * np.maximum(1.0, np.abs(ref))
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond tolerance, first {i.tolist()} "
                             f"gpu {got[tuple(i)]} ref {ref[tuple(i)]}")
    return float(err.max()) if err.size else 0.0, float((err / lim).max()) if err.size else 0.0


def run_hip_ll(T, H, E, R, k, fmt, x, idx, w, capacity_rows=None, ring_cfg=None,
               proxy_threads=4, poison=POISON, log_capacity=1 << 20, repeat=1, fused=False,
               one_call_layout=False):
    """Per-expert mode through the C ABI: rank layout + per-expert row table +
    per-expert pack (and descriptors when ring_cfg is given); fused: the
    one-call ep_dispatch_ll_fused; one_call_layout: the layout by
    ep_dispatch_ll_layout, then the pack."""
    import combine_topk_rank_amd as ep
    torch = torch_mod()
    s = ep.shape(T, H, E, R, k, fmt)
    cap = T * k if capacity_rows is None else capacity_rows
    buf = ep.BuffersLL(s, capacity_rows=cap)
    buf.send_buf.fill_(poison)
    buf.slot_src.fill_(-7)
    buf.slot_w.fill_(float("nan"))
    buf.expert_slot.fill_(-99)
    d_x, d_idx, d_w = dev_bf16(x), dev(idx), dev(w)
    ring = None
    if ring_cfg is not None:
        ring = ep.Ring(*ring_cfg)
        if proxy_threads:
            ring.proxy_start(proxy_threads, log_capacity)
    logs = []
    buf.num_tokens_per_expert.fill_(-99)
    buf.expert_offset.fill_(-99)
    for _ in range(repeat):
        if fused:
            buf.dispatch_fused(d_x, d_idx, d_w, ring=ring)
        else:
            if one_call_layout:
                buf.layout_one_call(d_idx)
            else:
                buf.layout(d_idx)
            buf.dispatch(d_x, d_idx, d_w, ring=ring)
        torch.cuda.synchronize()
    if ring is not None and proxy_threads:
        logs.append(ring.proxy_stop(log_capacity))
    return {
        "num_tokens_per_expert": host(buf.num_tokens_per_expert),
        "expert_offset": host(buf.expert_offset),
        "expert_slot": host(buf.expert_slot),
        "send_buf": host(buf.send_buf),
        "slot_src": host(buf.slot_src),
        "slot_w": host(buf.slot_w),
        "status": int(host(buf.dev_status)[0]),
        "logs": logs,
        "ring": ring,
        "buffers": buf,
        "d_idx": d_idx,
        "d_w": d_w,
    }


def run_hip_combine_ll(buf, y_bits: np.ndarray, d_idx, d_w):
    import combine_topk_rank_amd as ep
    torch = torch_mod()
    y = dev_bf16(y_bits) if y_bits.shape[0] else torch.zeros((1, buf.shape.H), dtype=torch.bfloat16,
                                                              device="cuda")
    buf.dev_status.zero_()
    buf.out.fill_(float("nan"))
    ep.ep_combine_ll(buf.shape, y, d_idx, d_w, buf.expert_slot, buf.out, buf.dev_status)
    torch.cuda.synchronize()
    o = buf.out.view(torch.int16).cpu().numpy().view(np.uint16)
    return W.bf16_bits_to_f32(o).astype(np.float64), int(host(buf.dev_status)[0])


def assert_ll_equal(g, L, pk, Q):
    """Per-expert layout and pack against the oracle, element by element."""
    for key in ("num_tokens_per_expert", "expert_offset", "expert_slot"):
        a, b = g[key], L[key]
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)[:5]
            raise AssertionError(f"{key} differs at {bad.tolist()}")
    a, b = g["send_buf"], pk["send_buf"]
    if not np.array_equal(a, b):
        rows = np.nonzero(np.any(a != b, axis=1))[0]
        raise AssertionError(f"per-expert send_buf differs in {rows.size} rows, first {rows[:5].tolist()}")
    n = min(Q, g["slot_src"].shape[0])
    assert np.array_equal(g["slot_src"][:n], pk["slot_src"][:n])
    assert np.array_equal(g["slot_w"][:n].view(np.uint32), pk["slot_w"][:n].view(np.uint32))
    assert np.all(g["slot_src"][n:] == -7)


def assert_stream_in_order(log_, want, channels, calls=1):
    """Closed-form publication: per channel, the logged commands in ticket
    order are the oracle's channel stream, once per call; tickets run
    1, 2, ... without gaps."""
    by_ch = collections.defaultdict(list)
    for d in sorted(log_, key=lambda d: int(d["seq"])):
        by_ch[int(d["dst_rank"]) % channels].append(d)
    for c in range(channels):
        exp_c = [cmd_key(d) for d in want if int(d["dst_rank"]) % channels == c]
        got_c = by_ch.get(c, [])
        assert len(got_c) == calls * len(exp_c), f"channel {c}: {len(got_c)} vs {calls * len(exp_c)}"
        assert [int(d["seq"]) for d in got_c] == list(range(1, len(got_c) + 1))
        for i in range(calls):
            part = [cmd_key(d) for d in got_c[i * len(exp_c):(i + 1) * len(exp_c)]]
            assert part == exp_c, f"channel {c}, call {i}: stream differs"
