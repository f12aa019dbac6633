"""End to end through the command stream: proxy threads execute every
command they pop against local memory (WRITE -> copy into the destination
rank's receive region, ATOMIC ADD -> add into its count word).  After two
dispatches, every receive region must hold exactly the rows the oracle packs
for that rank, byte for byte, its slack must be untouched, and every count
word must hold twice its count."""

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import dev, dev_bf16, log

pytestmark = pytest.mark.gpu

SLACK = 256
FILL = 0x5A


def _expected(w, inp, mode):
    """Per rank: the bytes its receive region must hold, and its count words."""
    rb = oracle.row_bytes(w.H, w.fmt)
    epr = w.E // w.R
    if mode == "ll":
        L = oracle.ll_layout(inp["topk_idx"], w.E)
        pk = oracle.ll_pack(inp["x"], inp["topk_w"], L["expert_slot"], w.fmt, capacity_rows=L["Q"])
        eo = L["expert_offset"]
        rows = [(int(eo[r * epr]), int(eo[(r + 1) * epr])) for r in range(w.R)]
        counts = [L["num_tokens_per_expert"][r * epr:(r + 1) * epr].astype(np.int32)
                  for r in range(w.R)]
    else:
        L = oracle.layout(inp["topk_idx"], w.E, w.R)
        pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R,
                         w.fmt, capacity_rows=L["P"])
        ro = L["rank_offset"]
        rows = [(int(ro[r]), int(ro[r + 1])) for r in range(w.R)]
        counts = [np.array([L["num_tokens_per_rank"][r]], np.int32) for r in range(w.R)]
    want = [pk["send_buf"][a:b].reshape(-1) for (a, b) in rows]
    return want, counts, rb


@pytest.mark.parametrize("name,mode", [("decode", "rank"), ("train", "rank"), ("fp8", "rank"),
                                       ("decode", "ll"), ("tiny", "ll")])
def test_loopback_receive_regions(name, mode):
    import combine_topk_rank_amd as ep
    import torch
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    want, counts, rb = _expected(w, inp, mode)
    s = ep.shape(w.T, w.H, w.E, w.R, w.k, w.fmt)
    b = ep.BuffersLL(s) if mode == "ll" else ep.Buffers(s)
    recv = [torch.full((want[r].size + SLACK,), FILL, dtype=torch.uint8, device="cuda")
            for r in range(w.R)]
    cnt = [torch.zeros(len(counts[r]), dtype=torch.int32, device="cuda") for r in range(w.R)]
    ring = ep.Ring(w.depth, w.channels, w.max_inflight, 5_000_000_000)
    ring.set_loopback(b.send_buf, recv, cnt)
    ring.proxy_start(4, 0)
    d_x, d_idx, d_w = dev_bf16(inp["x"]), dev(inp["topk_idx"]), dev(inp["topk_w"])
    for call in range(2):
        log(f"[loopback] {name} {mode}: dispatch {call}")
        b.layout(d_idx)
        b.dispatch(d_x, d_idx, d_w, ring=ring)
        torch.cuda.synchronize()
        assert int(b.dev_status.item()) == 0
        # the copies read the send buffer: it is rewritten only after they end
        ring.wait_complete(10_000_000_000)
    st = ring.loopback_stats()
    lg, nd = ring.proxy_stop(0)
    log(f"[loopback] {st}")
    assert st["errors"] == 0 and st["completed"] == nd
    assert sum(ring.completed(c) for c in range(w.channels)) == nd
    for r in range(w.R):
        got = recv[r].cpu().numpy()
        n = want[r].size
        if not np.array_equal(got[:n], want[r]):
            bad = int(np.argmax(got[:n] != want[r]))
            raise AssertionError(f"rank {r}: receive region differs at byte {bad} "
                                 f"(row {bad // rb})")
        assert np.all(got[n:] == FILL), f"rank {r}: slack written"
        assert np.array_equal(cnt[r].cpu().numpy(), 2 * counts[r]), f"rank {r}: count words"


def test_loopback_reports_commands_outside_the_regions():
    import combine_topk_rank_amd as ep
    import torch
    w = W.WORKLOADS["decode"]
    inp = pins.workload_inputs("decode")
    want, counts, rb = _expected(w, inp, "rank")
    s = ep.shape(w.T, w.H, w.E, w.R, w.k, w.fmt)
    b = ep.Buffers(s)
    recv = [torch.full((max(want[r].size - rb, 0) if r == 0 else want[r].size,), FILL,
                       dtype=torch.uint8, device="cuda") for r in range(w.R)]
    cnt = [torch.zeros(1, dtype=torch.int32, device="cuda") for r in range(w.R)]
    ring = ep.Ring(w.depth, w.channels, w.max_inflight, 5_000_000_000)
    ring.set_loopback(b.send_buf, recv, cnt)
    ring.proxy_start(2, 0)
    log("[loopback] region of rank 0 one row short")
    b.layout(dev(inp["topk_idx"]))
    b.dispatch(dev_bf16(inp["x"]), dev(inp["topk_idx"]), dev(inp["topk_w"]), ring=ring)
    torch.cuda.synchronize()
    with pytest.raises(ep.EpError):
        ring.wait_complete(10_000_000_000)
    st = ring.loopback_stats()
    ring.proxy_stop(0)
    assert st["errors"] >= 1
    # the other ranks are still delivered
    for r in range(1, w.R):
        assert np.array_equal(recv[r].cpu().numpy(), want[r])


def _query(ring, channels, tickets):
    """done flags of ep_ring_check_completion for (channel, ticket) pairs."""
    import torch
    ch = torch.tensor(channels, dtype=torch.int32, device="cuda")
    tk = torch.tensor(tickets, dtype=torch.int64, device="cuda")
    done = torch.full((len(channels),), 9, dtype=torch.uint8, device="cuda")
    ring.check_completion(ch, tk, done)
    torch.cuda.synchronize()
    return done.cpu().numpy()


@pytest.mark.parametrize("name,loopback", [("decode", True), ("train", False)])
def test_check_completion_on_the_gpu(name, loopback):
    """The GPU's CheckCompletion query: nothing reads complete on a fresh
    ring; once ep_ring_wait_complete has returned, every published ticket of
    every channel reads complete and tickets beyond a channel's last read
    incomplete; a channel outside the ring reads 2."""
    import combine_topk_rank_amd as ep
    import torch
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    s = ep.shape(w.T, w.H, w.E, w.R, w.k, w.fmt)
    b = ep.Buffers(s)
    ring = ep.Ring(w.depth, w.channels, w.max_inflight, 5_000_000_000)
    C = w.channels
    assert list(_query(ring, list(range(C)) + [C, -1], [0] * C + [0, 0])) == [0] * C + [2, 2]
    if loopback:
        want, counts, rb = _expected(w, inp, "rank")
        recv = [torch.empty(max(want[r].size, 1), dtype=torch.uint8, device="cuda")
                for r in range(w.R)]
        cnt = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(w.R)]
        ring.set_loopback(b.send_buf, recv, cnt)
    ring.proxy_start(4, 0)
    log(f"[completion] {name} loopback={loopback}")
    d_idx = dev(inp["topk_idx"])
    b.layout(d_idx)
    b.dispatch(dev_bf16(inp["x"]), d_idx, dev(inp["topk_w"]), ring=ring)
    torch.cuda.synchronize()
    assert int(b.dev_status.item()) == 0
    ring.wait_complete(10_000_000_000)
    heads = [ring.completed(c) for c in range(C)]
    lg, nd = ring.proxy_stop(0)
    assert sum(heads) == nd > 0
    chans, tks, exp = [], [], []
    for c in range(C):
        for t in range(heads[c]):
            chans.append(c), tks.append(t), exp.append(1)
        for t in (heads[c], heads[c] + 1, heads[c] + 1000):
            chans.append(c), tks.append(t), exp.append(0)
    got = _query(ring, chans, tks)
    assert np.array_equal(got, np.array(exp, np.uint8))
    ring.destroy()
