"""Device-side error reporting, forced from the host so that every kernel
still ends normally: a bad expert id, a send buffer below capacity, a ring
that nobody drains (a short timeout on the kernel's own bounded wait), and
inconsistent layout arguments."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_layout_equal, assert_pack_equal, log, run_hip

pytestmark = pytest.mark.gpu


def test_bad_expert_reported_and_skipped():
    rng = np.random.default_rng(31)
    inp = W.make_random_case(rng, 300, 64, 32, 8, 4)
    idx = inp["topk_idx"].copy()
    idx[7, 1] = 32          # == E
    idx[200, 3] = -5
    log("[errors] bad expert ids")
    g = run_hip(300, 64, 32, 8, 4, 0, inp["x"], idx, inp["topk_w"], ring_cfg=None)
    assert g["status"] == 2
    # the bad entries are skipped: same layout as with them dropped
    clean = idx.copy()
    clean[7, 1] = -1
    clean[200, 3] = -1
    L = oracle.layout(clean, 32, 8)
    assert_layout_equal(g, L)


def test_capacity_exceeded():
    rng = np.random.default_rng(32)
    T, H, E, R, k = 200, 128, 32, 8, 4
    inp = W.make_random_case(rng, T, H, E, R, k)
    L = oracle.layout(inp["topk_idx"], E, R)
    cap = L["P"] - 3
    pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], E, R, 0,
                     capacity_rows=cap)
    assert pk["status"] == 3
    log("[errors] capacity")
    g = run_hip(T, H, E, R, k, 0, inp["x"], inp["topk_idx"], inp["topk_w"], capacity_rows=cap,
                ring_cfg=(1024, 2, 256, 5_000_000_000))
    assert g["status"] == 3
    assert_pack_equal(g, pk, cap)
    lg, nd = g["logs"][0]
    assert nd == 0          # nothing is announced for a partial send


def test_ring_timeout_without_consumer():
    """No proxy runs and only 2 commands may be in flight: producers give up
    after the ring's 2 ms timeout and report it."""
    import combine_topk_rank_amd as ep
    w = W.WORKLOADS["tiny"]
    inp = W.make_inputs(w, 0)
    log("[errors] ring timeout (no consumer, 2 ms)")
    g = run_hip(w.T, w.H, w.E, w.R, w.k, w.fmt, inp["x"], inp["topk_idx"], inp["topk_w"],
                ring_cfg=(8, 1, 2, 2_000_000), proxy_threads=0)
    assert g["status"] == ep.EP_ERR_RING_TIMEOUT
    ring = g["ring"]
    first = ring.drain(0)
    assert len(first) == 2           # the two commands that fit
    ring.reset()
    assert len(ring.drain(0)) == 0


def test_manual_drain_api():
    """Without proxy threads, ep_ring_drain pops what fits in flight."""
    w = W.WORKLOADS["decode"]
    inp = W.make_inputs(w, 0)
    L = oracle.layout(inp["topk_idx"], w.E, w.R)
    want = oracle.descriptors(L["num_tokens_per_rank"], L["rank_offset"],
                              oracle.row_bytes(w.H, w.fmt), 1)
    assert len(want) <= 256
    log("[errors] manual drain, decode")
    g = run_hip(w.T, w.H, w.E, w.R, w.k, w.fmt, inp["x"], inp["topk_idx"], inp["topk_w"],
                ring_cfg=(1024, 1, 256, 5_000_000_000), proxy_threads=0)
    assert g["status"] == 0
    got = g["ring"].drain(0, 4096)
    from gpu_helpers import assert_descriptors
    assert_descriptors(got, want, 1, first_seq=1)
    assert np.all(np.diff(got["seq"].astype(np.int64)) == 1)   # FIFO order


def test_inconsistent_slots_rejected():
    """send_slot from one layout with rank_offset of another: reported, no
    descriptor escapes, nothing outside the buffers is touched."""
    import combine_topk_rank_amd as ep
    import torch
    from gpu_helpers import dev, dev_bf16
    rng = np.random.default_rng(33)
    T, H, E, R, k = 64, 64, 16, 4, 2
    inp = W.make_random_case(rng, T, H, E, R, k)
    s = ep.shape(T, H, E, R, k)
    b = ep.Buffers(s)
    d_idx, d_w, d_x = dev(inp["topk_idx"]), dev(inp["topk_w"]), dev_bf16(inp["x"])
    log("[errors] inconsistent rank_offset")
    b.layout(d_idx)
    torch.cuda.synchronize()
    bad_off = torch.zeros_like(b.rank_offset)
    bad_off[-1] = b.rank_offset[-1]           # every rank starts at 0
    ring = ep.Ring(64, 1, 16, 1_000_000_000)
    ring.proxy_start(1, 1024)
    ep.ep_dispatch(s, d_x, d_idx, d_w, bad_off, b.send_slot, b.send_buf, b.slot_src,
                   b.slot_local_idx, b.slot_local_w, ring, b.workspace, b.dev_status)
    torch.cuda.synchronize()
    lg, nd = ring.proxy_stop(1024)
    assert int(b.dev_status.item()) == ep.EP_ERR_INVALID_ARG
    assert all(d["type"] != 1 or d["dst_rank"] == 0 for d in lg)


def _streaming_case():
    # 2048 one-wavefront rows: the large-batch pack, which publishes as
    # messages complete
    rng = np.random.default_rng(34)
    T, H, E, R, k = 2048, 512, 64, 8, 4
    return (T, H, E, R, k), W.make_random_case(rng, T, H, E, R, k)


def _clean_dispatch_on(ring, shape, inp):
    """A correct dispatch on a ring that was reset: the exact stream again."""
    import combine_topk_rank_amd as ep
    import torch
    from gpu_helpers import assert_descriptors, dev, dev_bf16
    T, H, E, R, k = shape
    s = ep.shape(T, H, E, R, k)
    b = ep.Buffers(s)
    L = oracle.layout(inp["topk_idx"], E, R)
    want = oracle.descriptors(L["num_tokens_per_rank"], L["rank_offset"], oracle.row_bytes(H, 0),
                              ring.channels)
    ring.proxy_start(2, 1 << 16)
    d_idx = dev(inp["topk_idx"])
    b.layout(d_idx)
    b.dispatch(dev_bf16(inp["x"]), d_idx, dev(inp["topk_w"]), ring=ring)
    torch.cuda.synchronize()
    lg, nd = ring.proxy_stop(1 << 16)
    assert int(b.dev_status.item()) == 0
    assert nd == len(want)
    assert_descriptors(lg, want, ring.channels, first_seq=1)


def test_streaming_bad_expert_publishes_nothing():
    """A bad expert id found by the layout: the large-batch pack still packs
    every row (the bad choice skipped) but emits no command; after a reset
    the ring carries a correct dispatch."""
    import combine_topk_rank_amd as ep
    (T, H, E, R, k), inp = _streaming_case()
    idx = inp["topk_idx"].copy()
    idx[5, 0] = E
    idx[1700, 2] = -3
    clean = idx.copy()
    clean[5, 0] = clean[1700, 2] = -1
    L = oracle.layout(clean, E, R)
    pk = oracle.pack(inp["x"], clean, inp["topk_w"], L["send_slot"], E, R, 0,
                     capacity_rows=T * min(k, R))
    log("[errors] streaming pack after a bad expert id")
    g = run_hip(T, H, E, R, k, 0, inp["x"], idx, inp["topk_w"],
                ring_cfg=(1024, 4, 256, 5_000_000_000))
    assert g["status"] == ep.EP_ERR_BAD_EXPERT
    assert_layout_equal(g, L)
    assert_pack_equal(g, pk, L["P"])
    lg, nd = g["logs"][0]
    assert nd == 0
    ring = g["ring"]
    ring.reset()
    _clean_dispatch_on(ring, (T, H, E, R, k), inp)
    ring.destroy()


def test_streaming_inconsistent_slots():
    """send_slot with the rank_offset of another layout on the large-batch
    pack: reported, no WRITE escapes, and the ring works after a reset."""
    import combine_topk_rank_amd as ep
    import torch
    from gpu_helpers import dev, dev_bf16
    (T, H, E, R, k), inp = _streaming_case()
    s = ep.shape(T, H, E, R, k)
    b = ep.Buffers(s)
    d_idx, d_w, d_x = dev(inp["topk_idx"]), dev(inp["topk_w"]), dev_bf16(inp["x"])
    log("[errors] streaming pack, inconsistent rank_offset")
    b.layout(d_idx)
    torch.cuda.synchronize()
    bad_off = torch.zeros_like(b.rank_offset)
    bad_off[-1] = b.rank_offset[-1]           # every rank starts at 0
    ring = ep.Ring(1024, 4, 256, 5_000_000_000)
    ring.proxy_start(2, 1 << 16)
    ep.ep_dispatch(s, d_x, d_idx, d_w, bad_off, b.send_slot, b.send_buf, b.slot_src,
                   b.slot_local_idx, b.slot_local_w, ring, b.workspace, b.dev_status)
    torch.cuda.synchronize()
    lg, nd = ring.proxy_stop(1 << 16)
    assert int(b.dev_status.item()) == ep.EP_ERR_INVALID_ARG
    assert all(int(d["type"]) != 1 for d in lg)
    ring.reset()
    _clean_dispatch_on(ring, (T, H, E, R, k), inp)
    ring.destroy()


@pytest.mark.parametrize("mode", ["rank-one-kernel", "per-expert-streaming"])
def test_streaming_ring_timeout_without_consumer(mode):
    """Large batches publish as messages complete; with no proxy and 4
    commands in flight per channel, each channel takes exactly its first 4
    commands, the other producers give up after the 2 ms timeout and report
    it, and every row is still packed."""
    import combine_topk_rank_amd as ep
    from gpu_helpers import assert_ll_equal, pack_streams, run_hip_ll
    rng = np.random.default_rng(61)
    if mode == "rank-one-kernel":
        T, H, E, R, k = 2048, 2048, 64, 8, 4
        assert ep.ep_dispatch_fused_plan(ep.shape(T, H, E, R, k)) == ep.EP_FUSED_ONE_KERNEL_LARGE
    else:
        T, H, E, R, k = 2048, 512, 64, 8, 4
        assert pack_streams(T, H, 0)
    inp = W.make_random_case(rng, T, H, E, R, k)
    log(f"[errors] {mode}: ring timeout (no consumer, 2 ms)")
    if mode == "rank-one-kernel":
        L = oracle.layout(inp["topk_idx"], E, R)
        pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], E, R, 0,
                         capacity_rows=T * min(k, R))
        g = run_hip(T, H, E, R, k, 0, inp["x"], inp["topk_idx"], inp["topk_w"],
                    ring_cfg=(64, 2, 4, 2_000_000), proxy_threads=0, fused=True)
        assert_layout_equal(g, L)
        assert_pack_equal(g, pk, L["P"])
    else:
        L = oracle.ll_layout(inp["topk_idx"], E)
        pk = oracle.ll_pack(inp["x"], inp["topk_w"], L["expert_slot"], 0, capacity_rows=T * k)
        g = run_hip_ll(T, H, E, R, k, 0, inp["x"], inp["topk_idx"], inp["topk_w"],
                       ring_cfg=(64, 2, 4, 2_000_000), proxy_threads=0)
        assert_ll_equal(g, L, pk, L["Q"])
    assert g["status"] == ep.EP_ERR_RING_TIMEOUT
    ring = g["ring"]
    for c in range(2):
        got = ring.drain(c)
        assert len(got) == 4, (c, len(got))
        assert [int(d["seq"]) for d in got] == [1, 2, 3, 4]
    ring.reset()
    assert len(ring.drain(0)) == 0 and len(ring.drain(1)) == 0
    ring.destroy()
