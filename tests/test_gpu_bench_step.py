"""The step bench.py times, in its own launch configuration (buffer sets it
rotates over, a live ring with proxy threads, combine reading y from a
buffer of its own), checked against the oracle at full size: after several
rotating steps every set's layout, packed rows and combined output equal the
oracle's, and every step drained exactly the oracle's number of commands."""

import argparse

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import combine_tolerance_check, log

pytestmark = pytest.mark.gpu


def _args(mode="rank"):
    return argparse.Namespace(mode=mode, fused="auto", loopback=False, graph=False,
                              proxy_threads=4, warmup=2)


@pytest.mark.parametrize("name", ["train", "fp8", "skewed", "decode"])
def test_bench_step_matches_oracle(name):
    import torch

    import bench
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    L = oracle.layout(inp["topk_idx"], w.E, w.R)
    P = L["P"]
    pk = oracle.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R, w.fmt,
                     capacity_rows=P)
    want_cmds = len(oracle.descriptors(L["num_tokens_per_rank"], L["rank_offset"],
                                       oracle.row_bytes(w.H, w.fmt), w.channels))
    log(f"[bench step] {name}: two buffer sets, four rotating steps")
    run = bench.Runner(w, inp, _args(), 2, torch.device("cuda", 0))
    try:
        drained0 = run.ring.proxy_drained()
        for i in range(4):
            run.step(i)
        torch.cuda.synchronize()
        assert run.status() == 0
        assert run.P == P
        import time
        t0 = time.time()
        while run.ring.proxy_drained() - drained0 < 4 * want_cmds and time.time() - t0 < 10:
            time.sleep(0.01)
        assert run.ring.proxy_drained() - drained0 == 4 * want_cmds
        for j, st in enumerate(run.sets):
            b = st["b"]
            assert np.array_equal(b.send_slot.cpu().numpy(), L["send_slot"]), j
            assert np.array_equal(b.rank_offset.cpu().numpy(), L["rank_offset"]), j
            assert np.array_equal(b.send_buf[:P].cpu().numpy(), pk["send_buf"][:P]), j
            y = st["y"].view(torch.int16).cpu().numpy().view(np.uint16)
            ref = oracle.combine(y, inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R)
            got = W.bf16_bits_to_f32(b.out.view(torch.int16).cpu().numpy().view(np.uint16))
            combine_tolerance_check(got.astype(np.float64), ref, f"{name} set {j}")
    finally:
        run.close()
