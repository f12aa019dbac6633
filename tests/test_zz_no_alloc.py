"""ep_dispatch_fused_noalloc -- the one-call dispatch on the library's own
device scratch, for callers that cannot allocate -- against ep_dispatch_fused
with a caller workspace, through the C ABI.

Three calls in a row share the one scratch array: a large batch (layout and
pack kernels), then a smaller one (one kernel), then the large one again (the
counters the first two left must be clean).  Every output must equal the
workspace call's bit for bit, and the command streams must be the same
multiset with the same per-channel order rules."""

import numpy as np
import pytest

import workloads as W
from gpu_helpers import POISON, assert_descriptors, cmd_key, dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu

RING_TIMEOUT_NS = 5_000_000_000
OUT_KEYS = ("num_tokens_per_rank", "num_tokens_per_expert", "rank_offset", "expert_offset",
            "is_token_in_rank", "send_slot", "send_buf", "slot_src", "slot_local_idx",
            "slot_local_w", "dev_status")

# (T, H, E, R, k, fmt, channels): the second call is smaller than the first
CALLS = [
    (2048, 7168, 256, 32, 8, 0, 8),
    (100, 512, 64, 16, 4, 1, 4),
    (2048, 7168, 256, 32, 8, 0, 8),
]


def _run(case, inp, noalloc, clear=False):
    import combine_topk_rank_amd as ep
    import torch
    T, H, E, R, k, fmt, C = case
    s = ep.shape(T, H, E, R, k, fmt)
    buf = ep.Buffers(s)
    buf.send_buf.fill_(POISON)
    buf.slot_src.fill_(-7)
    buf.slot_local_idx.fill_(-7)
    buf.slot_local_w.fill_(float("nan"))
    buf.send_slot.fill_(-99)
    buf.is_token_in_rank.fill_(7)
    if noalloc:
        buf.workspace.fill_(0xCC)   # must not be touched: the call has its own scratch
    ring = ep.Ring(1024, C, 256, RING_TIMEOUT_NS)
    ring.proxy_start(2, 1 << 16)
    x, idx, w = dev_bf16(inp["x"]), dev(inp["topk_idx"]), dev(inp["topk_w"])
    if noalloc:
        buf.dispatch_fused_noalloc(x, idx, w, ring=ring, clear_scratch=clear)
    else:
        buf.dispatch_fused(x, idx, w, ring=ring)
    torch.cuda.synchronize()
    lg, nd = ring.proxy_stop(1 << 16)
    ring.destroy()
    out = {key: host(getattr(buf, key)) for key in OUT_KEYS}
    if noalloc:
        assert np.all(host(buf.workspace) == 0xCC), "the caller's workspace was written"
    return out, lg, nd


def test_noalloc_matches_workspace_call():
    for i, case in enumerate(CALLS):
        T, H, E, R, k, fmt, C = case
        inp = W.make_random_case(np.random.default_rng(500 + T), T, H, E, R, k, drop_prob=0.05)
        log(f"[noalloc] call {i}: T={T} H={H} E={E} R={R} k={k} fmt={fmt} channels={C}")
        want, lg_w, nd_w = _run(case, inp, noalloc=False)
        got, lg_g, nd_g = _run(case, inp, noalloc=True)
        assert got["dev_status"][0] == 0 and want["dev_status"][0] == 0
        for key in OUT_KEYS:
            a, b = got[key], want[key]
            same = np.array_equal(a.view(np.uint8), b.view(np.uint8))
            assert same, f"call {i}: {key} differs from the workspace call"
        assert nd_g == nd_w == len(lg_w)
        assert_descriptors(lg_g, lg_w, C, first_seq=1)
        if T <= 256:
            # one kernel, closed-form publication: the same stream in order
            order = lambda lg: [cmd_key(d) for d in sorted(lg, key=lambda d: (
                int(d["dst_rank"]) % C, int(d["seq"])))]
            assert order(lg_g) == order(lg_w)


def test_noalloc_clear_and_reject():
    import ctypes

    import combine_topk_rank_amd as ep
    case = CALLS[1]
    T, H, E, R, k, fmt, C = case
    inp = W.make_random_case(np.random.default_rng(600), T, H, E, R, k)
    log("[noalloc] explicit clear, then a shape beyond the scratch")
    want, lg_w, _ = _run(case, inp, noalloc=False)
    got, lg_g, _ = _run(case, inp, noalloc=True, clear=True)
    for key in OUT_KEYS:
        assert np.array_equal(got[key].view(np.uint8), want[key].view(np.uint8)), key
    assert_descriptors(lg_g, lg_w, C, first_seq=1)
    big = ep.shape(65536, 64, 4096, 64, 8)
    assert ep.ep_workspace_bytes(big) > (4 << 20)
    st = ep.lib.ep_dispatch_fused_noalloc(ctypes.byref(big), *([None] * 10), 0, *([None] * 4), 0,
                                          None, None)
    assert st == ep.EP_ERR_INVALID_ARG
    assert b"4 MiB" in ep.lib.ep_last_error()
