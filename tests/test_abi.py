"""The C ABI without a GPU: the library loads, exports every function that
include/*.h declares, and validates arguments on the host (no kernel is
launched for an invalid call).  Also checks that the HIP library and the CPU
oracle share no code."""

import ctypes
import glob
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(ep_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def ep():
    import combine_topk_rank_amd as ep
    return ep


def test_exports_every_declared_symbol(ep):
    names = declared_functions()
    assert len(names) >= 16
    lib = ctypes.CDLL(ep.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_row_bytes(ep):
    assert ep.ep_row_bytes(7168, ep.EP_FMT_BF16) == 14336
    # fp8: codes, scales, zero pad to a whole number of 128-byte lines
    assert ep.ep_row_bytes(7168, ep.EP_FMT_FP8_E4M3_B128) == 7424
    assert ep.ep_row_bytes(4096, ep.EP_FMT_FP8_E4M3_B128) == 4224
    assert ep.ep_row_bytes(512, ep.EP_FMT_FP8_E4M3_B128) == 640
    assert ep.ep_row_bytes(512, ep.EP_FMT_BF16) == 1024
    # fp8 at any multiple of 128: 384 codes + 3 scales = 396 -> 512
    assert ep.ep_row_bytes(384, ep.EP_FMT_FP8_E4M3_B128) == 512
    assert ep.ep_row_bytes(7168 + 64, ep.EP_FMT_FP8_E4M3_B128) == 0
    assert ep.ep_row_bytes(7, ep.EP_FMT_BF16) == 0
    assert ep.ep_row_bytes(7168, 9) == 0


def test_workspace_bytes(ep):
    assert ep.ep_workspace_bytes(ep.shape(4096, 7168, 256, 32, 8)) > 0
    for H in (128, 384, 640, 6400, 8320):   # fp8 needs H % 128 == 0 only
        assert ep.ep_workspace_bytes(ep.shape(16, H, 16, 4, 2, 1)) > 0
    assert ep.ep_workspace_bytes(ep.shape(0, 64, 16, 4, 2)) > 0
    for bad in [ep.shape(-1, 64, 16, 4, 2), ep.shape(16, 7, 16, 4, 2), ep.shape(16, 64, 15, 4, 2),
                ep.shape(16, 64, 16, 65, 2), ep.shape(16, 64, 16, 4, 0), ep.shape(16, 64, 16, 4, 17),
                ep.shape(16, 64, 8192, 4, 2), ep.shape(16, 7168 + 64, 256, 32, 8, 1),
                ep.shape(16, 64, 16, 4, 2, 5), ep.shape(16, 64, 64, 4, 33)]:
        assert ep.ep_workspace_bytes(bad) == 0


def test_fused_plan_on_the_host(ep):
    """The path ep_dispatch_fused takes: one kernel up to 256 tokens; the
    two calls for shapes the one-kernel large path never takes (fewer than
    1024 tokens, rows of at most 1024 elements, rows that take more than one
    wavefront); an invalid shape is rejected."""
    L = ep.lib
    for s in [ep.shape(1, 64, 16, 4, 2), ep.shape(256, 7168, 256, 32, 8),
              ep.shape(256, 7168, 256, 32, 8, 1)]:
        assert ep.ep_dispatch_fused_plan(s) == ep.EP_FUSED_ONE_KERNEL_SMALL
    for s in [ep.shape(1000, 7168, 256, 32, 8), ep.shape(4096, 1024, 256, 32, 8),
              ep.shape(4096, 16384, 256, 32, 8), ep.shape(4096, 8192, 256, 32, 8, 1)]:
        assert ep.ep_dispatch_fused_plan(s) == ep.EP_FUSED_TWO_CALLS
        assert ep.ep_dispatch_fused_plan(s, with_ring=False) == ep.EP_FUSED_TWO_CALLS
    assert L.ep_dispatch_fused_plan(ctypes.byref(ep.shape(16, 7, 16, 4, 2)), 1) == 1
    assert len({ep.EP_FUSED_ONE_KERNEL_SMALL, ep.EP_FUSED_ONE_KERNEL_LARGE, ep.EP_FUSED_TWO_CALLS,
                ep.EP_OK, ep.EP_ERR_INVALID_ARG, ep.EP_ERR_BAD_EXPERT, ep.EP_ERR_CAPACITY,
                ep.EP_ERR_RING_TIMEOUT, ep.EP_ERR_HIP, ep.EP_ERR_BUSY, ep.EP_ERR_TIMEOUT}) == 11


def test_host_validation_rejects_without_launch(ep):
    L = ep.lib
    bad = ep.shape(16, 7, 16, 4, 2)
    assert L.ep_dispatch_layout(ctypes.byref(bad), *([None] * 7), None, 0, None, None) == 1
    good = ep.shape(16, 64, 16, 4, 2)
    # null outputs / missing workspace
    assert L.ep_dispatch_layout(ctypes.byref(good), *([None] * 7), None, 0, None, None) == 1
    assert L.ep_dispatch(ctypes.byref(good), *([None] * 6), 0, None, None, None, None, None, 0,
                         None, None) == 1
    assert L.ep_combine(ctypes.byref(good), None, 0, None, None, None, None, None, None) == 1
    # misaligned x
    assert L.ep_dispatch(ctypes.byref(good), 8, 16, 16, 16, 16, 256, 10, 16, 16, 16, None, 256,
                         1 << 20, 16, None) == 1
    # one-call layout + dispatch: bad shape, null outputs, misaligned x, short workspace
    assert L.ep_dispatch_fused(ctypes.byref(bad), *([None] * 9), None, 0, None, None, None, None,
                               None, 0, None, None) == 1
    assert L.ep_dispatch_fused(ctypes.byref(good), *([None] * 9), None, 0, None, None, None, None,
                               None, 0, None, None) == 1
    assert L.ep_dispatch_fused(ctypes.byref(good), 8, *([16] * 8), 256, 10, 16, 16, 16, None,
                               256, 1 << 20, 16, None) == 1
    assert L.ep_dispatch_fused(ctypes.byref(good), *([16] * 9), 256, 10, 16, 16, 16, None,
                               256, 0, 16, None) == 1
    # one-call per-expert dispatch: bad shape, beyond its bounds, null outputs
    assert L.ep_dispatch_ll_fused(ctypes.byref(bad), *([16] * 6), 256, 10, 16, 16, None, 256,
                                  1 << 20, 16, None) == 1
    for big in [ep.shape(257, 64, 16, 4, 2), ep.shape(16, 64, 2048, 4, 2)]:
        assert L.ep_dispatch_ll_fused(ctypes.byref(big), *([16] * 6), 256, 10, 16, 16, None, 256,
                                      1 << 30, 16, None) == 1
    assert L.ep_dispatch_ll_fused(ctypes.byref(good), *([None] * 6), None, 0, None, None, None,
                                  None, 0, None, None) == 1
    # one-call per-expert layout: bad shape, E beyond its bound, null outputs, short workspace
    assert L.ep_dispatch_ll_layout(ctypes.byref(bad), 16, 16, 16, 16, 16, 1 << 20, 16, None) == 1
    assert L.ep_dispatch_ll_layout(ctypes.byref(ep.shape(16, 64, 2048, 4, 2)), 16, 16, 16, 16, 16,
                                   1 << 30, 16, None) == 1
    assert b"E > 1024" in L.ep_last_error()
    assert L.ep_dispatch_ll_layout(ctypes.byref(good), 16, None, 16, 16, 16, 1 << 20, 16,
                                   None) == 1
    assert L.ep_dispatch_ll_layout(ctypes.byref(good), 16, 16, 16, 16, 16, 0, 16, None) == 1
    # T = 0 combine is a no-op
    zero = ep.shape(0, 64, 16, 4, 2)
    assert L.ep_combine(ctypes.byref(zero), None, 0, None, None, None, None, 16, None) == 0
    # per-expert mode: bad shape, missing pointers, misaligned buffers
    assert L.ep_dispatch_layout_ll(ctypes.byref(bad), None, 16, 16, 256, 1 << 20, 16, None) == 1
    assert L.ep_dispatch_layout_ll(ctypes.byref(good), None, 16, None, 256, 1 << 20, 16, None) == 1
    assert L.ep_dispatch_layout_ll(ctypes.byref(good), 16, 16, 16, 256, 0, 16, None) == 1
    assert L.ep_dispatch_ll(ctypes.byref(good), *([None] * 6), 0, None, None, None, None, 0,
                            None, None) == 1
    assert L.ep_dispatch_ll(ctypes.byref(good), 8, 16, 16, 16, 16, 256, 10, 16, 16, None, 256,
                            1 << 20, 16, None) == 1
    assert L.ep_combine_ll(ctypes.byref(good), None, 0, None, None, None, None, None, None) == 1
    assert L.ep_combine_ll(ctypes.byref(good), 8, 4, 16, 16, 16, 16, 16, None) == 1
    assert L.ep_combine_ll(ctypes.byref(zero), None, 0, None, None, None, None, 16, None) == 0
    assert L.ep_dispatch_layout_ll(ctypes.byref(zero), None, 16, None, 256, 1 << 20, 16, None) == 0


def test_ring_create_rejects_bad_arguments(ep):
    L = ep.lib
    for args in [(0, 1, 1, 1), (8, 0, 1, 1), (8, 65, 1, 1), (8, 1, 0, 1), (8, 1, 9, 1), (8, 1, 4, 0)]:
        assert not L.ep_ring_create(*args)


def test_status_strings(ep):
    for st in range(8):
        assert ep.status_str(st) != "unknown status"
    assert ep.status_str(99) == "unknown status"


def test_command_record_layout(ep):
    import oracle
    assert ep.CMD_DTYPE.itemsize == 32
    assert ep.CMD_DTYPE == oracle.CMD_DTYPE
    offs = {n: ep.CMD_DTYPE.fields[n][1] for n in ep.CMD_DTYPE.names}
    assert offs == {"seq": 0, "type": 4, "op": 5, "num_tokens": 6, "dst_rank": 8,
                    "size_or_value": 12, "src_offset": 16, "dst_offset": 24}


def test_oracle_and_hip_path_share_nothing():
    prod = glob.glob(os.path.join(ROOT, "combine_topk_rank_amd", "**", "*.*"), recursive=True)
    prod += glob.glob(os.path.join(ROOT, "include", "*.h"))
    for p in prod:
        if p.endswith((".hip", ".h", ".py", ".cpp")):
            text = open(p).read()
            assert "oracle" not in text.lower(), p
    orc = glob.glob(os.path.join(ROOT, "oracle", "*.c")) + glob.glob(os.path.join(ROOT, "oracle", "*.py"))
    for p in orc:
        text = open(p).read()
        assert "combine_topk_rank_amd" not in text and "ep.h" not in text, p


def test_noalloc_rejects_shapes_beyond_its_scratch(ep):
    """The no-allocation one-call dispatch owns 4 MiB of device scratch per
    GPU; a shape that needs more is rejected on the host with a reason,
    before any HIP call."""
    big = ep.shape(65536, 64, 4096, 64, 8)
    assert ep.ep_workspace_bytes(big) > (4 << 20)
    st = ep.lib.ep_dispatch_fused_noalloc(ctypes.byref(big), *([None] * 10), 0, *([None] * 4), 0,
                                          None, None)
    assert st == ep.EP_ERR_INVALID_ARG
    assert b"4 MiB" in ep.lib.ep_last_error()
    bad = ep.shape(16, 7, 16, 4, 2)
    assert ep.lib.ep_dispatch_fused_noalloc(ctypes.byref(bad), *([None] * 10), 0, *([None] * 4),
                                            0, None, None) == ep.EP_ERR_INVALID_ARG
