"""Per-expert (low-latency) mode on the GPU against the oracle, through the C
ABI: row table, packed rows and metadata bit-exact; the command stream
command for command where it is published in closed form (small batches),
else the same multiset with consecutive tickets per channel and each
expert's ATOMIC after its WRITEs (streaming publication); combine within
1e-2 * max(1, |ref|).  The same checks run on the one-call
ep_dispatch_ll_fused (T <= 256, E <= 1024)."""

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import (assert_ll_descriptors, assert_ll_equal, assert_stream_in_order,
                         combine_tolerance_check, log, pack_streams, run_hip_combine_ll, run_hip_ll)

pytestmark = pytest.mark.gpu

RING_TIMEOUT_NS = 5_000_000_000


def _check_case(T, H, E, R, k, fmt, inp, C, depth, mif, cap_extra=3, repeat=1, y_seed=7,
                fused=False, one_call_layout=False):
    idx, w, x = inp["topk_idx"], inp["topk_w"], inp["x"]
    L = oracle.ll_layout(idx, E)
    Q = L["Q"]
    pk = oracle.ll_pack(x, w, L["expert_slot"], fmt, capacity_rows=Q + cap_extra)
    want = oracle.ll_descriptors(L["num_tokens_per_expert"], L["expert_offset"], R,
                                 oracle.row_bytes(H, fmt), C)
    g = run_hip_ll(T, H, E, R, k, fmt, x, idx, w, capacity_rows=Q + cap_extra,
                   ring_cfg=(depth, C, mif, RING_TIMEOUT_NS), repeat=repeat, fused=fused,
                   one_call_layout=one_call_layout)
    assert g["status"] == 0, g["status"]
    assert_ll_equal(g, L, pk, Q)
    lg, nd = g["logs"][0]
    assert nd == repeat * len(want)
    if fused or not pack_streams(T, H, fmt):
        assert_stream_in_order(lg, want, C, calls=repeat)
    else:
        assert repeat == 1
        assert_ll_descriptors(lg, want, C, L["expert_offset"], E, R, oracle.row_bytes(H, fmt))
    if fmt == 0:
        y = W.make_expert_outputs(Q, H, y_seed)
        ref = oracle.ll_combine(y, idx, w, L["expert_slot"], H=H)
        got, st = run_hip_combine_ll(g["buffers"], y, g["d_idx"], g["d_w"])
        assert st == 0
        combine_tolerance_check(got, ref, f"per-expert combine T={T}")
        # identity experts: the packed rows come back, out = (sum_j w_j) * x
        yi = g["send_buf"][:Q].view(np.uint16).reshape(Q, H)
        got_i, st = run_hip_combine_ll(g["buffers"], yi, g["d_idx"], g["d_w"])
        ref_i = oracle.ll_combine(yi, idx, w, L["expert_slot"], H=H)
        combine_tolerance_check(got_i, ref_i, f"per-expert identity T={T}")
    return g


@pytest.mark.parametrize("name", ["tiny", "decode", "train", "fp8", "skewed"])
def test_ll_workload_parity(name):
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    log(f"[ll] workload {name}")
    _check_case(w.T, w.H, w.E, w.R, w.k, w.fmt, inp, w.channels, w.depth, w.max_inflight)


# (T, H, E, R, k, fmt, drop_prob, channels, depth, max_inflight)
LL_CASES = [
    (1, 8, 1, 1, 1, 0, 0.0, 1, 4, 1),
    (0, 64, 16, 4, 2, 0, 0.0, 2, 8, 4),
    (5, 16, 6, 3, 2, 0, 0.3, 2, 8, 2),
    (300, 200, 64, 8, 6, 0, 0.1, 3, 16, 4),
    (257, 512, 32, 16, 8, 1, 0.0, 4, 32, 8),
    (700, 1024, 64, 64, 4, 0, 0.0, 64, 32, 8),
    (600, 128, 4096, 64, 32, 0, 0.05, 8, 1024, 256),
    (3000, 136, 256, 32, 8, 0, 0.2, 5, 1024, 64),
    (2000, 384, 64, 16, 4, 1, 0.0, 4, 1024, 256),
]


@pytest.mark.parametrize("case", LL_CASES, ids=lambda c: "T%d_H%d_E%d_R%d_k%d_f%d" % c[:6])
def test_ll_random_case_parity(case):
    T, H, E, R, k, fmt, drop, C, depth, mif = case
    rng = np.random.default_rng(2000 + LL_CASES.index(case))
    inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=drop)
    log(f"[ll] case {case}")
    _check_case(T, H, E, R, k, fmt, inp, C, depth, mif)


@pytest.mark.parametrize("name", ["tiny", "decode", "train", "fp8", "skewed"])
def test_ll_one_call_layout_workloads(name):
    """ep_dispatch_ll_layout (counts, offsets and row table in one kernel),
    then the per-expert pack: the same checks as the three-call path."""
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    log(f"[ll] one-call layout, workload {name}")
    _check_case(w.T, w.H, w.E, w.R, w.k, w.fmt, inp, w.channels, w.depth, w.max_inflight,
                one_call_layout=True)


@pytest.mark.parametrize("case", [c for c in LL_CASES if c[2] <= 1024] +
                         [(600, 128, 1024, 64, 32, 0, 0.05, 8, 1024, 256),
                          (5000, 256, 512, 16, 8, 1, 0.1, 8, 1024, 256)],
                         ids=lambda c: "T%d_H%d_E%d_R%d_k%d_f%d" % c[:6])
def test_ll_one_call_layout_cases(case):
    T, H, E, R, k, fmt, drop, C, depth, mif = case
    rng = np.random.default_rng(3100 + T + E)
    inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=drop)
    if T > 0 and k > 1:
        idx = inp["topk_idx"].copy()
        idx[::5, 1] = idx[::5, 0]   # repeated experts: one row per choice
        inp = dict(inp, topk_idx=idx)
    log(f"[ll] one-call layout, case {case}")
    _check_case(T, H, E, R, k, fmt, inp, C, depth, mif, one_call_layout=True)


def test_ll_one_call_layout_uneven_rounds():
    """Wavefronts with different numbers of repeat rounds in one tile: ten
    tokens of one wavefront name a single expert k times (k rounds there),
    one token of another names it twice, the rest once."""
    rng = np.random.default_rng(41)
    T, H, E, R, k = 1000, 64, 64, 8, 6
    inp = W.make_random_case(rng, T, H, E, R, k)
    idx = inp["topk_idx"].copy()
    idx[100:110, :] = idx[100:110, :1]
    idx[200, 3] = idx[200, 2]
    inp = dict(inp, topk_idx=idx)
    log("[ll] one-call layout, uneven repeat rounds")
    _check_case(T, H, E, R, k, 0, inp, 2, 64, 16, one_call_layout=True)


def test_ll_one_call_layout_bad_expert():
    """A bad id is reported and treated as dropped; the rest of the table is
    the oracle's."""
    import combine_topk_rank_amd as ep
    import torch
    from gpu_helpers import dev, host
    rng = np.random.default_rng(9)
    T, H, E, R, k = 1500, 64, 96, 8, 6
    inp = W.make_random_case(rng, T, H, E, R, k)
    idx = inp["topk_idx"].copy()
    idx[3, 2] = E
    idx[1400, 0] = -4
    clean = idx.copy()
    clean[3, 2] = clean[1400, 0] = -1
    L = oracle.ll_layout(clean, E)
    b = ep.BuffersLL(ep.shape(T, H, E, R, k))
    b.expert_slot.fill_(-99)
    log("[ll] one-call layout with bad expert ids")
    b.layout_one_call(dev(idx))
    torch.cuda.synchronize()
    assert int(b.dev_status.item()) == ep.EP_ERR_BAD_EXPERT
    for key, got in (("num_tokens_per_expert", b.num_tokens_per_expert),
                     ("expert_offset", b.expert_offset), ("expert_slot", b.expert_slot)):
        assert np.array_equal(host(got), L[key]), key


def test_ll_repeated_experts_and_repeat_calls():
    """Tokens naming one expert several times send one row per choice; three
    calls on one ring keep tickets consecutive and each call's stream whole."""
    rng = np.random.default_rng(77)
    T, H, E, R, k = 200, 64, 32, 8, 4
    inp = W.make_random_case(rng, T, H, E, R, k)
    idx = inp["topk_idx"].copy()
    idx[::7, 1] = idx[::7, 0]
    idx[::11, :] = idx[::11, :1]
    inp = dict(inp, topk_idx=idx)
    log("[ll] repeated experts, three calls")
    _check_case(T, H, E, R, k, 0, inp, 3, 16, 4, repeat=3)


def test_ll_streaming_errors():
    """Large-batch per-expert pack (streaming publication): a bad expert id
    and a capacity shortfall publish nothing; expert_slot from another
    layout is reported and no WRITE escapes; after a reset the ring carries a
    correct dispatch."""
    import combine_topk_rank_amd as ep
    import torch
    from gpu_helpers import dev, dev_bf16
    rng = np.random.default_rng(41)
    T, H, E, R, k, C = 2048, 512, 64, 8, 4, 4
    assert pack_streams(T, H, 0)
    inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=0.1)
    idx = inp["topk_idx"].copy()
    idx[5, 0] = E
    clean = idx.copy()
    clean[5, 0] = -1
    L = oracle.ll_layout(clean, E)
    pk = oracle.ll_pack(inp["x"], inp["topk_w"], L["expert_slot"], 0, capacity_rows=T * k)
    log("[ll] streaming pack after a bad expert id")
    g = run_hip_ll(T, H, E, R, k, 0, inp["x"], idx, inp["topk_w"],
                   ring_cfg=(1024, C, 256, RING_TIMEOUT_NS))
    assert g["status"] == ep.EP_ERR_BAD_EXPERT
    assert g["logs"][0][1] == 0
    assert_ll_equal(g, L, pk, L["Q"])
    L = oracle.ll_layout(inp["topk_idx"], E)
    Q = L["Q"]
    log("[ll] streaming pack, capacity shortfall")
    g = run_hip_ll(T, H, E, R, k, 0, inp["x"], inp["topk_idx"], inp["topk_w"], capacity_rows=Q - 9,
                   ring_cfg=(1024, C, 256, RING_TIMEOUT_NS))
    assert g["status"] == ep.EP_ERR_CAPACITY
    assert g["logs"][0][1] == 0
    pk = oracle.ll_pack(inp["x"], inp["topk_w"], L["expert_slot"], 0, capacity_rows=Q - 9)
    assert np.array_equal(g["send_buf"], pk["send_buf"])
    log("[ll] streaming pack, expert_slot from another layout")
    s = ep.shape(T, H, E, R, k)
    b = ep.BuffersLL(s)
    d_idx, d_w, d_x = dev(inp["topk_idx"]), dev(inp["topk_w"]), dev_bf16(inp["x"])
    b.layout(d_idx)
    torch.cuda.synchronize()
    bad_slot = torch.flip(b.expert_slot, dims=[0]).contiguous()
    ring = ep.Ring(1024, C, 256, RING_TIMEOUT_NS)
    ring.proxy_start(2, 1 << 16)
    ep.ep_dispatch_ll(s, d_x, d_idx, d_w, b.expert_offset, bad_slot, b.send_buf, b.slot_src,
                      b.slot_w, ring, b.workspace, b.dev_status)
    torch.cuda.synchronize()
    lg, nd = ring.proxy_stop(1 << 16)
    assert int(b.dev_status.item()) == ep.EP_ERR_INVALID_ARG
    assert all(int(d["type"]) != 1 for d in lg)
    log("[ll] reset, then a clean streaming dispatch on the same ring")
    ring.reset()
    ring.proxy_start(2, 1 << 16)
    b.dev_status.zero_()
    ep.ep_dispatch_ll(s, d_x, d_idx, d_w, b.expert_offset, b.expert_slot, b.send_buf, b.slot_src,
                      b.slot_w, ring, b.workspace, b.dev_status)
    torch.cuda.synchronize()
    lg, nd = ring.proxy_stop(1 << 16)
    assert int(b.dev_status.item()) == 0
    want = oracle.ll_descriptors(L["num_tokens_per_expert"], L["expert_offset"], R,
                                 oracle.row_bytes(H, 0), C)
    assert nd == len(want)
    assert_ll_descriptors(lg, want, C, L["expert_offset"], E, R, oracle.row_bytes(H, 0))
    ring.destroy()


def test_ll_capacity_and_inconsistent_rows():
    import combine_topk_rank_amd as ep
    import torch
    from gpu_helpers import dev, dev_bf16
    rng = np.random.default_rng(5)
    T, H, E, R, k = 64, 64, 16, 4, 2
    inp = W.make_random_case(rng, T, H, E, R, k)
    L = oracle.ll_layout(inp["topk_idx"], E)
    Q = L["Q"]
    log("[ll] capacity shortfall")
    g = run_hip_ll(T, H, E, R, k, 0, inp["x"], inp["topk_idx"], inp["topk_w"], capacity_rows=Q - 1,
                   ring_cfg=(64, 1, 16, RING_TIMEOUT_NS))
    assert g["status"] == ep.EP_ERR_CAPACITY
    lg, nd = g["logs"][0]
    assert nd == 0
    pk = oracle.ll_pack(inp["x"], inp["topk_w"], L["expert_slot"], 0, capacity_rows=Q - 1)
    assert np.array_equal(g["send_buf"], pk["send_buf"])
    log("[ll] expert_slot from another layout")
    s = ep.shape(T, H, E, R, k)
    b = ep.BuffersLL(s)
    d_idx, d_w, d_x = dev(inp["topk_idx"]), dev(inp["topk_w"]), dev_bf16(inp["x"])
    b.layout(d_idx)
    torch.cuda.synchronize()
    bad_slot = torch.flip(b.expert_slot, dims=[0]).contiguous()
    ring = ep.Ring(64, 1, 16, RING_TIMEOUT_NS)
    ring.proxy_start(1, 1024)
    ep.ep_dispatch_ll(s, d_x, d_idx, d_w, b.expert_offset, bad_slot, b.send_buf, b.slot_src,
                      b.slot_w, ring, b.workspace, b.dev_status)
    torch.cuda.synchronize()
    lg, nd = ring.proxy_stop(1024)
    assert int(b.dev_status.item()) == ep.EP_ERR_INVALID_ARG
    assert nd == 0


# ------------------------------------------------- one-call per-expert dispatch
@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_ll_fused_workload_parity(name):
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    log(f"[ll-fused] workload {name}")
    _check_case(w.T, w.H, w.E, w.R, w.k, w.fmt, inp, w.channels, w.depth, w.max_inflight,
                fused=True)


LL_FUSED_CASES = [
    (0, 64, 16, 4, 2, 0, 0.0, 2, 8, 4),
    (1, 8, 1, 1, 1, 0, 0.0, 1, 4, 1),
    (5, 16, 6, 3, 2, 0, 0.3, 2, 8, 2),
    (63, 7168, 256, 32, 8, 0, 0.0, 1, 1024, 256),
    (64, 200, 64, 8, 6, 0, 0.1, 3, 16, 4),
    (65, 512, 32, 16, 8, 1, 0.0, 4, 32, 8),
    (128, 7168, 256, 32, 8, 1, 0.0, 1, 1024, 256),
    (200, 1024, 64, 64, 4, 0, 0.0, 64, 32, 8),
    (256, 128, 1024, 64, 32, 0, 0.05, 8, 1024, 256),
    (256, 136, 256, 32, 8, 0, 0.2, 5, 1024, 64),
    (100, 128, 64, 8, 4, 1, 0.1, 2, 64, 16),
]


@pytest.mark.parametrize("case", LL_FUSED_CASES, ids=lambda c: "T%d_H%d_E%d_R%d_k%d_f%d" % c[:6])
def test_ll_fused_random_case_parity(case):
    T, H, E, R, k, fmt, drop, C, depth, mif = case
    rng = np.random.default_rng(3000 + LL_FUSED_CASES.index(case))
    inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=drop)
    log(f"[ll-fused] case {case}")
    _check_case(T, H, E, R, k, fmt, inp, C, depth, mif, fused=True)


def test_ll_fused_repeated_experts_and_repeat_calls():
    """Repeats within a token (up to k occurrences) and three calls on one
    ring, through the one-call path."""
    rng = np.random.default_rng(78)
    T, H, E, R, k = 200, 64, 32, 8, 4
    inp = W.make_random_case(rng, T, H, E, R, k)
    idx = inp["topk_idx"].copy()
    idx[::7, 1] = idx[::7, 0]
    idx[::11, :] = idx[::11, :1]
    inp = dict(inp, topk_idx=idx)
    log("[ll-fused] repeated experts, three calls")
    _check_case(T, H, E, R, k, 0, inp, 3, 16, 4, repeat=3, fused=True)


def test_ll_fused_uneven_rounds():
    """One-call path, wavefronts with different numbers of repeat rounds:
    only wavefront 1's tokens 70..74 name one expert k times."""
    rng = np.random.default_rng(79)
    T, H, E, R, k = 200, 64, 32, 8, 4
    inp = W.make_random_case(rng, T, H, E, R, k)
    idx = inp["topk_idx"].copy()
    idx[70:75, :] = idx[70:75, :1]
    inp = dict(inp, topk_idx=idx)
    log("[ll-fused] uneven repeat rounds")
    _check_case(T, H, E, R, k, 0, inp, 3, 64, 16, fused=True)


def test_ll_fused_errors():
    """Capacity shortfall and a bad expert id: reported, no descriptor; rows
    below the capacity written.  Shapes beyond the one-kernel bounds are
    rejected on the host."""
    import combine_topk_rank_amd as ep
    rng = np.random.default_rng(6)
    T, H, E, R, k = 64, 64, 16, 4, 2
    inp = W.make_random_case(rng, T, H, E, R, k)
    L = oracle.ll_layout(inp["topk_idx"], E)
    Q = L["Q"]
    log("[ll-fused] capacity shortfall")
    g = run_hip_ll(T, H, E, R, k, 0, inp["x"], inp["topk_idx"], inp["topk_w"], capacity_rows=Q - 1,
                   ring_cfg=(64, 1, 16, RING_TIMEOUT_NS), fused=True)
    assert g["status"] == ep.EP_ERR_CAPACITY
    assert g["logs"][0][1] == 0
    pk = oracle.ll_pack(inp["x"], inp["topk_w"], L["expert_slot"], 0, capacity_rows=Q - 1)
    assert np.array_equal(g["send_buf"], pk["send_buf"])
    assert np.array_equal(g["expert_slot"], L["expert_slot"])
    log("[ll-fused] bad expert id")
    idx = inp["topk_idx"].copy()
    idx[3, 1] = E + 2
    g = run_hip_ll(T, H, E, R, k, 0, inp["x"], idx, inp["topk_w"],
                   ring_cfg=(64, 1, 16, RING_TIMEOUT_NS), fused=True)
    assert g["status"] == ep.EP_ERR_BAD_EXPERT
    assert g["logs"][0][1] == 0
    for T2, E2 in [(257, 16), (64, 2048)]:
        s = ep.shape(T2, H, E2, R, k)
        b = ep.BuffersLL(s)
        with pytest.raises(ep.EpError):
            b.dispatch_fused(b.out, b.expert_slot, b.slot_w)
