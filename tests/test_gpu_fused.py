"""GPU parity of ep_dispatch_fused (routing layout and pack in one call: one
kernel for T <= 256; one kernel with a grid barrier for larger bf16 batches
whose rows take one wavefront; else the two calls) against the CPU oracle,
through the C ABI.

Bit-exact: counts, offsets, membership, send slots, packed bytes (poisoned
buffers, rows past P untouched), metadata and fp8 codes.  The closed-form
command stream equals the oracle's command for command, per channel in ticket
order.  Combine on its outputs stays within 1e-2 * max(1, |ref|)."""

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import (assert_descriptors, assert_layout_equal, assert_pack_equal,
                         assert_stream_in_order, combine_tolerance_check, log, run_hip,
                         run_hip_combine)

pytestmark = pytest.mark.gpu

RING_TIMEOUT_NS = 5_000_000_000


def _check(g, L, pk, want, channels, calls=1):
    assert g["status"] == 0, g["status"]
    assert_layout_equal(g, L)
    assert_pack_equal(g, pk, L["P"])
    lg, nd = g["logs"][0]
    assert nd == calls * len(want) == len(lg)
    assert_stream_in_order(lg, want, channels, calls=calls)


def _check_stream(g, L, pk, want, channels):
    """streaming publication: the same multiset, tickets consecutive per
    channel, each rank's ATOMIC after its WRITEs"""
    assert g["status"] == 0, g["status"]
    assert_layout_equal(g, L)
    assert_pack_equal(g, pk, L["P"])
    lg, nd = g["logs"][0]
    assert nd == len(want) == len(lg)
    assert_descriptors(lg, want, channels, first_seq=1)


@pytest.mark.parametrize("name", ["tiny", "decode", "train", "fp8", "skewed"])
def test_fused_workload_parity(name):
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    L = oracle.layout(inp["topk_idx"], w.E, w.R)
    P = L["P"]
    pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R, w.fmt,
                     capacity_rows=P + 8)
    want = oracle.descriptors(L["num_tokens_per_rank"], L["rank_offset"],
                              oracle.row_bytes(w.H, w.fmt), w.channels)
    import combine_topk_rank_amd as ep
    plan = ep.ep_dispatch_fused_plan(ep.shape(w.T, w.H, w.E, w.R, w.k, w.fmt))
    # skewed's 16,384 tokens would make 4 passes of whole rows on the chip:
    # its rows go two wavefronts each, so it takes the two calls
    assert plan == {"tiny": ep.EP_FUSED_ONE_KERNEL_SMALL, "decode": ep.EP_FUSED_ONE_KERNEL_SMALL,
                    "train": ep.EP_FUSED_ONE_KERNEL_LARGE, "fp8": ep.EP_FUSED_TWO_CALLS,
                    "skewed": ep.EP_FUSED_TWO_CALLS}[name]
    log(f"[fused] workload {name}: T={w.T} H={w.H} R={w.R} k={w.k}, P={P}; one-kernel dispatch")
    g = run_hip(w.T, w.H, w.E, w.R, w.k, w.fmt, inp["x"], inp["topk_idx"], inp["topk_w"],
                capacity_rows=P + 8,
                ring_cfg=(w.depth, w.channels, w.max_inflight, RING_TIMEOUT_NS), fused=True)
    if w.T <= 256:
        _check(g, L, pk, want, w.channels)
    else:
        _check_stream(g, L, pk, want, w.channels)
    y = W.make_expert_outputs(P, w.H, 0)
    ref = oracle.combine(y, inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R)
    got, st = run_hip_combine(g["buffers"], y, g["d_idx"], g["d_w"])
    assert st == 0
    combine_tolerance_check(got, ref, f"{name} combine after the one-kernel dispatch")


# (T, H, E, R, k, fmt, drop_prob, channels, depth, max_inflight)
CASES = [
    (0, 64, 16, 4, 2, 0, 0.0, 2, 8, 4),
    (1, 8, 1, 1, 1, 0, 0.0, 1, 4, 1),
    (5, 16, 6, 3, 2, 0, 0.3, 2, 8, 2),
    (63, 7168, 256, 32, 8, 0, 0.0, 1, 1024, 256),
    (64, 200, 64, 8, 6, 0, 0.1, 3, 16, 4),
    (65, 1024, 64, 64, 4, 0, 0.0, 64, 32, 8),
    (200, 512, 4096, 64, 32, 0, 0.05, 8, 1024, 256),
    (256, 136, 32, 4, 3, 0, 0.5, 1, 1024, 256),
    (128, 512, 32, 16, 8, 1, 0.0, 4, 16, 4),
    (256, 4096, 128, 8, 4, 1, 0.2, 8, 1024, 256),
    (100, 384, 64, 16, 4, 1, 0.1, 4, 64, 16),
    (256, 640, 32, 4, 3, 1, 0.0, 1, 1024, 256),
    # above 256 tokens: layout, then pack (closed form or streaming publication)
    (300, 7168, 256, 32, 8, 0, 0.0, 8, 1024, 256),
    (1100, 7168, 64, 64, 8, 1, 0.1, 8, 64, 16),
    (2000, 2304, 6, 3, 2, 0, 0.3, 2, 1024, 256),
    # bf16: one kernel with a grid barrier (1024 tokens and more, one wavefront
    # a row); fp8: the two calls
    (1024, 7168, 256, 32, 8, 0, 0.0, 8, 1024, 256),
    (4099, 2048, 64, 16, 4, 0, 0.1, 4, 256, 64),
    (3000, 8192, 96, 48, 6, 0, 0.05, 8, 1024, 256),
    (2500, 2048, 128, 8, 8, 1, 0.0, 8, 1024, 256),
    (5000, 4096, 64, 64, 2, 1, 0.2, 8, 1024, 256),
    (20000, 4096, 32, 32, 1, 0, 0.0, 16, 2048, 256),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_E%d_R%d_k%d_f%d" % c[:6])
def test_fused_random_case_parity(case):
    T, H, E, R, k, fmt, drop, C, depth, mif = case
    rng = np.random.default_rng(2000 + CASES.index(case))
    inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=drop)
    L = oracle.layout(inp["topk_idx"], E, R)
    P = L["P"]
    cap = P + 5
    pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], E, R, fmt,
                     capacity_rows=cap)
    want = oracle.descriptors(L["num_tokens_per_rank"], L["rank_offset"],
                              oracle.row_bytes(H, fmt), C)
    log(f"[fused] case {case}: P={P}")
    g = run_hip(T, H, E, R, k, fmt, inp["x"], inp["topk_idx"], inp["topk_w"], capacity_rows=cap,
                ring_cfg=(depth, C, mif, RING_TIMEOUT_NS), fused=True)
    if T <= 256:
        _check(g, L, pk, want, C)
    else:
        _check_stream(g, L, pk, want, C)
    if T > 0:
        y = W.make_expert_outputs(P, H, 3)
        ref = oracle.combine(y, inp["topk_idx"], inp["topk_w"], L["send_slot"], E, R, H=H)
        got, st = run_hip_combine(g["buffers"], y, g["d_idx"], g["d_w"])
        assert st == 0
        combine_tolerance_check(got, ref, f"fused case {case}")


@pytest.mark.parametrize("name", ["decode", "train", "fp8"])
def test_fused_matches_two_calls_without_ring(name):
    """No ring: the one-kernel call and layout + dispatch give the same bytes."""
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    log(f"[fused] {name} without a ring: one call vs two calls")
    a = run_hip(w.T, w.H, w.E, w.R, w.k, w.fmt, inp["x"], inp["topk_idx"], inp["topk_w"],
                fused=True)
    b = run_hip(w.T, w.H, w.E, w.R, w.k, w.fmt, inp["x"], inp["topk_idx"], inp["topk_w"])
    assert a["status"] == b["status"] == 0
    for key in ("num_tokens_per_rank", "num_tokens_per_expert", "rank_offset", "expert_offset",
                "is_token_in_rank", "send_slot", "send_buf", "slot_src", "slot_local_idx"):
        assert np.array_equal(a[key], b[key]), key


def test_fused_repeated_calls_on_one_ring():
    """Three calls on one ring with a small in-flight window: every call's
    stream in closed-form order, tickets consecutive across the calls."""
    T, H, E, R, k, C = 100, 256, 64, 16, 4, 5
    rng = np.random.default_rng(77)
    inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=0.1)
    L = oracle.layout(inp["topk_idx"], E, R)
    pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], E, R, 0,
                     capacity_rows=L["P"])
    want = oracle.descriptors(L["num_tokens_per_rank"], L["rank_offset"], oracle.row_bytes(H, 0), C)
    log(f"[fused] three calls on one ring, T={T} R={R}, {len(want)} commands per call")
    g = run_hip(T, H, E, R, k, 0, inp["x"], inp["topk_idx"], inp["topk_w"],
                capacity_rows=L["P"], ring_cfg=(16, C, 4, RING_TIMEOUT_NS), repeat=3, fused=True)
    _check(g, L, pk, want, C, calls=3)


@pytest.mark.parametrize("name", ["decode", "train", "fp8"])
def test_fused_errors(name):
    """A bad expert id and a capacity shortfall are reported; no descriptor
    goes out, and the rows below the capacity are still written."""
    import combine_topk_rank_amd as ep
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    idx = inp["topk_idx"].copy()
    idx[7, 3] = w.E + 5
    log(f"[fused] {name}: bad expert id")
    g = run_hip(w.T, w.H, w.E, w.R, w.k, w.fmt, inp["x"], idx, inp["topk_w"],
                ring_cfg=(w.depth, w.channels, w.max_inflight, RING_TIMEOUT_NS), fused=True)
    assert g["status"] == ep.EP_ERR_BAD_EXPERT
    assert g["logs"][0][1] == 0
    L = oracle.layout(inp["topk_idx"], w.E, w.R)
    cap = L["P"] - 10
    pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R, w.fmt,
                     capacity_rows=cap)
    log(f"[fused] {name}: capacity {cap} < P = {L['P']}")
    g = run_hip(w.T, w.H, w.E, w.R, w.k, w.fmt, inp["x"], inp["topk_idx"], inp["topk_w"],
                capacity_rows=cap,
                ring_cfg=(w.depth, w.channels, w.max_inflight, RING_TIMEOUT_NS), fused=True)
    assert g["status"] == ep.EP_ERR_CAPACITY
    assert g["logs"][0][1] == 0
    assert_layout_equal(g, L)
    assert_pack_equal(g, pk, cap)


# one-kernel large path at its edges: (T, H, E, R, k, drop_prob, channels)
LARGE_EDGES = [
    (65536, 1032, 4, 2, 1, 0.0, 2),     # 4096 groups on 256 workgroups (all CUs): 16 passes, the maximum
    (32768, 1032, 4, 2, 1, 0.0, 2),     # 2048 groups on 256 workgroups: 8 passes
    (8192, 1032, 4032, 64, 8, 0.1, 8),  # the grid fills the chip: expert counts in the pack workgroups, E/64 ragged
    (4095, 4104, 7, 7, 3, 0.2, 3),      # one expert per rank, R not a power of two, ragged T
    (1025, 2048, 1, 1, 1, 0.5, 1),      # one rank, half the choices dropped, one token past 1024
    (6000, 7168, 64, 64, 1, 0.0, 8),    # k = 1, 64 ranks
    (4096, 2048, 256, 32, 12, 0.05, 4), # k = 12: the kernel built for k <= 32
]


@pytest.mark.parametrize("case", LARGE_EDGES, ids=lambda c: "T%d_H%d_E%d_R%d_k%d" % c[:5])
def test_fused_large_edges(case):
    import combine_topk_rank_amd as ep
    T, H, E, R, k, drop, C = case
    assert ep.ep_dispatch_fused_plan(ep.shape(T, H, E, R, k)) == ep.EP_FUSED_ONE_KERNEL_LARGE
    rng = np.random.default_rng(7000 + LARGE_EDGES.index(case))
    inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=drop)
    L = oracle.layout(inp["topk_idx"], E, R)
    P = L["P"]
    pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], E, R, 0,
                     capacity_rows=P + 3)
    want = oracle.descriptors(L["num_tokens_per_rank"], L["rank_offset"], oracle.row_bytes(H, 0), C)
    log(f"[fused] one-kernel large edge case {case}: P={P}")
    g = run_hip(T, H, E, R, k, 0, inp["x"], inp["topk_idx"], inp["topk_w"], capacity_rows=P + 3,
                ring_cfg=(1024, C, 256, RING_TIMEOUT_NS), fused=True)
    _check_stream(g, L, pk, want, C)
    y = W.make_expert_outputs(P, H, 5)
    ref = oracle.combine(y, inp["topk_idx"], inp["topk_w"], L["send_slot"], E, R, H=H)
    got, st = run_hip_combine(g["buffers"], y, g["d_idx"], g["d_w"])
    assert st == 0
    combine_tolerance_check(got, ref, f"one-kernel large edge {case}")


def test_fused_large_row_split_boundary():
    """bf16 rows of 7168 (one wavefront each) stay in the one-kernel path
    while whole rows make at most 3 passes over the chip's 256 workgroups;
    from 4 passes on, ep_dispatch gives each row two wavefronts and the fused
    call takes the two calls.  Without a ring nothing is split."""
    import combine_topk_rank_amd as ep
    for T, want in ((12288, ep.EP_FUSED_ONE_KERNEL_LARGE),    # 768 groups: 3 passes
                    (12352, ep.EP_FUSED_TWO_CALLS),           # 772 groups: 4 passes
                    (16384, ep.EP_FUSED_TWO_CALLS)):
        assert ep.ep_dispatch_fused_plan(ep.shape(T, 7168, 256, 64, 8)) == want, T
    assert ep.ep_dispatch_fused_plan(ep.shape(16384, 7168, 256, 64, 8), with_ring=False) == \
        ep.EP_FUSED_ONE_KERNEL_LARGE
    # fp8 rows always take the two calls
    assert ep.ep_dispatch_fused_plan(ep.shape(12288, 7168, 256, 64, 8, 1)) == ep.EP_FUSED_TWO_CALLS
