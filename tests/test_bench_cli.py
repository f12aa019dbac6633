"""bench.py's host-side contract without a GPU: one GPU only (a clear exit for
--gpus above 1), and the algorithmic byte model that the reported GB/s and
roofline use, checked against the byte counts written out by hand."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


class _W:
    def __init__(self, T, H, E, R, k, fmt):
        self.T, self.H, self.E, self.R, self.k, self.fmt = T, H, E, R, k, fmt


@pytest.mark.parametrize("fmt", [0, 1])
def test_algorithmic_bytes(fmt):
    import bench
    T, H, E, R, k, P = 4096, 7168, 256, 32, 8, 29810
    w = _W(T, H, E, R, k, fmt)
    ab = bench.algorithmic_bytes(w, P)
    # layout: read the ids; write counts and offsets (R, E, R+1, E+1), membership and slots
    assert ab["layout"] == 4 * T * k + 4 * (R + E + (R + 1) + (E + 1)) + T * R + 4 * T * R
    row = 2 * H if fmt == 0 else H + 4 * (H // 128)   # payload bytes; the fp8 pad is not counted
    # dispatch: read x, ids, gates, slots and R+1 offsets; write P rows and their metadata
    assert ab["dispatch"] == (2 * T * H + 8 * T * k + 4 * T * R + 4 * (R + 1)
                              + P * row + P * (4 + 8 * k))
    # combine: read P returned bf16 rows, ids, gates, slots; write T bf16 rows
    assert ab["combine"] == 2 * P * H + 8 * T * k + 4 * T * R + 2 * T * H
    assert ab["total"] == ab["layout"] + ab["dispatch"] + ab["combine"]
    if fmt == 0:
        # about 238 KB per token at this shape (4H(1 + P/T) plus metadata)
        assert 230e3 < ab["total"] / T < 245e3


def test_row_pitch_is_whole_lines_for_fp8():
    import bench
    assert bench.row_pitch(7168, 1) == 7424 and bench.row_bytes(7168, 1) == 7392
    assert bench.row_pitch(7168, 0) == bench.row_bytes(7168, 0) == 14336


def test_rotation_sets_and_quantiles():
    import bench
    mall = bench.MALL_BYTES
    # enough sets that a set's data was last touched >= 2x the MALL of traffic ago
    for step_bytes in (800_000, 30_000_000, 976_000_000, 3_200_000_000):
        n = bench.rotation_sets(step_bytes)
        assert 2 <= n <= 16
        assert n == 16 or (n - 1) * step_bytes >= 2 * mall
    q = bench.quantiles(list(range(1, 101)))
    assert q["p10"] < q["p50"] < q["p90"] and abs(q["p50"] - 50.5) < 1e-9


def test_cpu_threads_follow_omp_num_threads(monkeypatch):
    import bench
    info = {"nproc": 16, "cpu_count": 64, "model": "x"}
    monkeypatch.setenv("OMP_NUM_THREADS", "4")
    assert bench.cpu_threads_all(info) == 4
    monkeypatch.setenv("OMP_NUM_THREADS", "64")
    assert bench.cpu_threads_all(info) == 16
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.cpu_threads_all(info) == 16


def test_unknown_pre_step_rejected_before_the_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pre-steps", "bogus"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "unknown pre-step" in r.stderr
