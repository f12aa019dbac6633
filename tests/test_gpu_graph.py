"""Layout, dispatch (with a live ring) and combine captured in one HIP graph
and replayed: every replay, with the program's own eager work in between,
gives the eager results, and every replay publishes its whole command stream
(a ring's state carries over from one replay to the next)."""

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import assert_descriptors, assert_stream_in_order, dev, dev_bf16, log

pytestmark = pytest.mark.gpu


def _streams_by_call(lg, want, C, calls):
    by_ch = {}
    for d in sorted(lg, key=lambda d: int(d["seq"])):
        by_ch.setdefault(int(d["dst_rank"]) % C, []).append(d)
    for c in range(C):
        exp_c = [d for d in want if int(d["dst_rank"]) % C == c]
        got_c = by_ch.get(c, [])
        assert len(got_c) == calls * len(exp_c)
        for i in range(calls):
            assert_descriptors(got_c[i * len(exp_c):(i + 1) * len(exp_c)], exp_c, C)


@pytest.mark.parametrize("name,mode,fused", [("decode", "rank", False), ("tiny", "ll", False),
                                             ("train", "rank", False), ("decode", "rank", True),
                                             ("decode", "ll", True)])
def test_graph_replays_match_eager(name, mode, fused):
    import combine_topk_rank_amd as ep
    import torch
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    s = ep.shape(w.T, w.H, w.E, w.R, w.k, w.fmt)
    b = ep.BuffersLL(s) if mode == "ll" else ep.Buffers(s)
    d_x, d_idx, d_w = dev_bf16(inp["x"]), dev(inp["topk_idx"]), dev(inp["topk_w"])
    y = torch.from_numpy(W.make_expert_outputs(b.capacity_rows, w.H, 9).view(np.int16)).cuda() \
        .view(torch.bfloat16)
    ring = ep.Ring(w.depth, w.channels, w.max_inflight, 5_000_000_000)
    ring.proxy_start(4, 1 << 20)

    def step():
        if fused:   # the one-call layout + pack
            b.dispatch_fused(d_x, d_idx, d_w, ring=ring)
        else:
            b.layout(d_idx)
            b.dispatch(d_x, d_idx, d_w, ring=ring)
        b.combine(y, d_idx, d_w)

    log(f"[graph] {name} {mode} fused={fused}: eager")
    step()
    torch.cuda.synchronize()
    keys = (["expert_slot", "expert_offset", "send_buf", "slot_src", "slot_w", "out"] if mode == "ll"
            else ["send_slot", "rank_offset", "send_buf", "slot_src", "slot_local_idx", "out"])
    # rows past P (Q) are not written by any call: compare the written ones
    n_rows = int((b.expert_offset if mode == "ll" else b.rank_offset)[-1].item())
    row_keys = {"send_buf", "slot_src", "slot_w", "slot_local_idx"}

    def view(k_):
        t_ = getattr(b, k_)
        return t_[:n_rows] if k_ in row_keys else t_

    ref = {k_: view(k_).clone() for k_ in keys}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    replays = 3
    for i in range(replays):
        log(f"[graph] {name} {mode} fused={fused}: replay {i}")
        for k_ in keys:
            getattr(b, k_).fill_(0 if getattr(b, k_).dtype != torch.bfloat16 else 1.0)
        scratch.fill_(i)                      # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert int(b.dev_status.item()) == 0
        for k_ in keys:
            a_, r_ = view(k_), ref[k_]
            assert torch.equal(a_.view(torch.uint8) if a_.dtype == torch.bfloat16 else a_,
                               r_.view(torch.uint8) if r_.dtype == torch.bfloat16 else r_), \
                f"replay {i}: {k_} differs from the eager run"
    lg, nd = ring.proxy_stop(1 << 20)
    calls = 2 + replays                       # eager, side-stream warm-up, replays
    if mode == "ll":
        L = oracle.ll_layout(inp["topk_idx"], w.E)
        want = oracle.ll_descriptors(L["num_tokens_per_expert"], L["expert_offset"], w.R,
                                     oracle.row_bytes(w.H, w.fmt), w.channels)
        assert nd == calls * len(want)
        assert_stream_in_order(lg, want, w.channels, calls=calls)
    else:
        L = oracle.layout(inp["topk_idx"], w.E, w.R)
        want = oracle.descriptors(L["num_tokens_per_rank"], L["rank_offset"],
                                  oracle.row_bytes(w.H, w.fmt), w.channels)
        assert nd == calls * len(want)
        _streams_by_call(lg, want, w.channels, calls)
