"""fp8 pack against the oracle on crafted rows: every finite bf16 value of a
block below the block maximum, for block maxima that put x*(448/amax) on
exact ties (amax = 448 gives inv = 1), on subnormal codes and below the 1e-4
floor.  Codes and scales must match bit for bit."""

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads as W
from gpu_helpers import assert_pack_equal, log, run_hip

pytestmark = pytest.mark.gpu

H = 7168
AMAXES = [448.0, 1.0, 3.0, 0.7, 2.0 ** 10, 2.0 ** -3, 1e-5, 240.0, 3.0e38, 5.0e-3]


def crafted_rows():
    base = pins.all_finite_bf16()
    blocks = []
    for A in AMAXES:
        a_bits = W.f32_to_bf16_bits(np.array([A], np.float32))[0]
        a_val = W.bf16_bits_to_f32(np.array([a_bits]))[0]
        vals = base[np.abs(base) <= a_val]
        vb = W.f32_to_bf16_bits(vals)
        n = int(np.ceil(vb.size / 127))
        pad = np.zeros(n * 127, np.uint16)
        pad[:vb.size] = vb
        blk = np.concatenate([np.full((n, 1), a_bits, np.uint16), pad.reshape(n, 127)], axis=1)
        blocks.append(blk)
    allb = np.concatenate(blocks)
    per_row = H // 128
    nrows = int(np.ceil(allb.shape[0] / per_row))
    rows = np.zeros((nrows * per_row, 128), np.uint16)
    rows[:allb.shape[0]] = allb
    return rows.reshape(nrows, H)


def test_fp8_codes_exhaustive():
    x = crafted_rows()
    T = x.shape[0]
    idx = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    L = oracle.layout(idx, 1, 1)
    pk = oracle.pack(x, idx, w, L["send_slot"], 1, 1, W.FMT_FP8_E4M3_B128, capacity_rows=T + 2)
    log(f"[fp8] crafted rows: T={T}")
    g = run_hip(T, H, 1, 1, 1, W.FMT_FP8_E4M3_B128, x, idx, w, capacity_rows=T + 2, ring_cfg=None)
    assert g["status"] == 0
    a, b = g["send_buf"][:T], pk["send_buf"][:T]
    codes_bad = np.argwhere(a[:, :H] != b[:, :H])
    if codes_bad.size:
        t, c = codes_bad[0]
        blk = c // 128
        raise AssertionError(f"{codes_bad.shape[0]} codes differ; first row {t} col {c}: "
                             f"x=0x{x[t, c]:04x} gpu=0x{a[t, c]:02x} oracle=0x{b[t, c]:02x} "
                             f"block amax bits 0x{x[t, blk * 128]:04x}")
    assert np.array_equal(a[:, H:], b[:, H:]), "scales differ"
    assert_pack_equal(g, pk, T)


@pytest.mark.parametrize("T", [64, 1100], ids=["small_batch", "large_batch"])
def test_fp8_nonfinite(T):
    """NaN and infinite elements: NaNs take no part in a block's maximum, an
    infinity makes it (and the scale) infinite, and a NaN product gets code
    0x7F with the element's sign.  Codes and scales equal the oracle's bit
    for bit, on the small-batch and the large-batch pack."""
    Hn = 1024
    rng = np.random.default_rng(404 + T)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, Hn), dtype=np.float32))
    specials = np.array([0x7FC0, 0xFFC0, 0x7F81, 0xFFFF, 0x7F80, 0xFF80], np.uint16)
    # a few non-finite elements in about a third of the blocks
    nblk = T * Hn // 128
    for b in rng.choice(nblk, nblk // 3, replace=False):
        t, c0 = divmod(int(b) * 128, Hn)
        for _ in range(int(rng.integers(1, 4))):
            x[t, c0 + int(rng.integers(0, 128))] = specials[int(rng.integers(0, specials.size))]
    x[0, :128] = 0x7FC0      # a block of NaNs only: amax 0, the 1e-4 floor
    x[0, 128:256] = 0xFF80   # a block of -inf only
    idx = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    L = oracle.layout(idx, 1, 1)
    pk = oracle.pack(x, idx, w, L["send_slot"], 1, 1, W.FMT_FP8_E4M3_B128, capacity_rows=T + 2)
    log(f"[fp8] non-finite elements: T={T} H={Hn}")
    g = run_hip(T, Hn, 1, 1, 1, W.FMT_FP8_E4M3_B128, x, idx, w, capacity_rows=T + 2,
                ring_cfg=None)
    assert g["status"] == 0
    a, b = g["send_buf"][:T], pk["send_buf"][:T]
    bad = np.argwhere(a != b)
    if bad.size:
        t, c = bad[0]
        raise AssertionError(f"{bad.shape[0]} bytes differ; first row {t} byte {c}: "
                             f"gpu=0x{a[t, c]:02x} oracle=0x{b[t, c]:02x}")
    assert_pack_equal(g, pk, T)
