"""The ring protocol on the CPU: producer threads following the producer
rules (ticket reservation, the in-flight window, four tagged words stored in
any order) against the library's own slot encoding and consumer
(combine_topk_rank_amd/csrc/ep_ring_proto.h), compiled with the host
compiler; see tests/ring_model/ring_model.cpp.

UCCL-EP article (peacm.com/news/835744) s2.2: a FIFO with lock-free head and
tail, batched enqueue, a producer blocked at 256 commands in flight."""

import json
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_topk_rank_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "ring_model", "ring_model.cpp")
PROTO = "ep_ring_proto.h"


def _build(tmp, include_dir, extra=()):
    exe = os.path.join(tmp, "ring_model" + ("_" + "_".join(e.strip("-D").split("=")[0]
                                                             for e in extra) if extra else ""))
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-pthread", "-Wall", "-I", include_dir,
                           *extra, SRC, "-o", exe])
    return exe


def _run(exe, depth, window, producers, pushes, timeout_ms, consume):
    r = subprocess.run([exe, str(depth), str(window), str(producers), str(pushes),
                        str(timeout_ms), str(int(consume))],
                       capture_output=True, text=True, timeout=300)
    return r.returncode, json.loads(r.stdout.strip().splitlines()[-1])


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    return _build(str(tmp_path_factory.mktemp("ring")), CSRC)


@pytest.mark.parametrize("depth,window,producers,pushes", [
    (4, 4, 4, 1_000_000),        # the slot is reused as soon as it is popped
    (4, 3, 3, 1_000_000),
    (1024, 256, 8, 1_000_000),   # the pages' depth and in-flight limit
    (65535, 256, 2, 200_000),    # the largest depth: tags never collide
])
def test_no_lost_or_duplicated_slot(model, depth, window, producers, pushes):
    rc, out = _run(model, depth, window, producers, pushes, 5000, True)
    assert rc == 0, out
    assert out["popped"] == pushes and out["bad"] == 0
    assert out["max_inflight_seen"] <= window


def test_stalled_consumer_times_out(model):
    """Nobody drains: exactly max_inflight commands are written, then every
    producer gives up with a timeout status instead of waiting for ever."""
    rc, out = _run(model, 8, 4, 3, 1000, 50, False)
    assert rc == 0, out
    assert out["timeouts"] >= 1 and out["written"] == 4


def test_model_catches_a_stale_tag_consumer(tmp_path):
    """A consumer that checks the tag of the first word only decodes words
    left by an older command; the model must see it."""
    inc = tmp_path / "inc"
    inc.mkdir()
    src = open(os.path.join(CSRC, PROTO)).read()
    old = "if ((w[i] & 0xFFFFu) != tag) return false;"
    assert src.count(old) == 1
    (inc / PROTO).write_text(src.replace(old, "if (i == 0 && (w[i] & 0xFFFFu) != tag) return false;"))
    exe = _build(str(tmp_path), str(inc))
    rc, out = _run(exe, 4, 4, 4, 1_000_000, 5000, True)
    assert rc != 0 and out["bad"] > 0, out


def test_model_catches_a_window_overrun(tmp_path):
    """Producers that allow one command more than max_inflight in flight."""
    exe = _build(str(tmp_path), CSRC, ["-DRING_MODEL_WINDOW_SLACK=1"])
    rc, out = _run(exe, 8, 4, 4, 200_000, 5000, True)
    assert rc != 0 and out["max_inflight_seen"] > 4, out
