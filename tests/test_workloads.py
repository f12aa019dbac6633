"""The seeded generator: determinism, shapes and the routing statistics."""

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads as W


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_deterministic(name):
    w = W.WORKLOADS[name]
    a, b = W.make_inputs(w, 0), W.make_inputs(w, 0)
    for key in a:
        assert np.array_equal(a[key], b[key])
    c = W.make_inputs(w, 1)
    assert not np.array_equal(a["x"], c["x"])


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_shapes_and_weights(name):
    w = W.WORKLOADS[name]
    inp = pins.workload_inputs(name)
    assert inp["x"].shape == (w.T, w.H) and inp["x"].dtype == np.uint16
    assert inp["topk_idx"].shape == (w.T, w.k) and inp["topk_idx"].dtype == np.int32
    assert inp["topk_w"].shape == (w.T, w.k) and inp["topk_w"].dtype == np.float32
    idx = inp["topk_idx"]
    assert idx.min() >= 0 and idx.max() < w.E
    # the k experts of a token are distinct
    s = np.sort(idx, axis=1)
    assert np.all(np.diff(s, axis=1) > 0)
    ws = inp["topk_w"].astype(np.float64).sum(axis=1)
    if w.routing == "softmax_top":
        assert np.all(ws < 1.0) and np.all(ws > 0.0)
    else:
        assert np.allclose(ws, 1.0, atol=1e-6)


def test_train_and_fp8_share_inputs():
    a, b = pins.workload_inputs("train"), pins.workload_inputs("fp8")
    for key in a:
        assert np.array_equal(a[key], b[key])


# (P, min cnt_r, max cnt_r, WRITE messages) at seed 0
EXPECTED = {
    "tiny": (237, 52, 69, 31),
    "train": (29810, 880, 992, 3741),
    "decode": (932, 20, 41, 128),
    "skewed": (94646, 236, 16332, 11861),
}


@pytest.mark.parametrize("name", list(EXPECTED))
def test_routing_statistics(name):
    w = W.WORKLOADS[name]
    L = oracle.layout(pins.workload_inputs(name)["topk_idx"], w.E, w.R)
    cnt = L["num_tokens_per_rank"]
    msgs = int(sum((int(c) + 7) // 8 for c in cnt))
    assert (L["P"], int(cnt.min()), int(cnt.max()), msgs) == EXPECTED[name]


def test_skewed_is_zipf_like():
    w = W.WORKLOADS["skewed"]
    idx = pins.workload_inputs("skewed")["topk_idx"]
    cnt = np.bincount(idx.reshape(-1), minlength=w.E)
    # expert 0 is the most popular and popularity falls with the id
    assert cnt.argmax() == 0
    assert cnt[:8].sum() > cnt[-64:].sum()


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    b = W.f32_to_bf16_bits(f)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6)
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]
