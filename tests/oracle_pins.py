"""Pins for the CPU oracle: checks against facts that do not come from the
oracle itself (hand-worked fixtures, brute-force enumeration on tiny inputs,
format definitions, a library cast, invariants and closed forms).

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees.  ``test_oracle_pins.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on deliberately broken builds.
"""

from __future__ import annotations

import collections
import json
import math
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

FMT_BF16, FMT_FP8 = 0, 1

_INPUT_CACHE = {}


def workload_inputs(name: str) -> dict:
    if name not in _INPUT_CACHE:
        _INPUT_CACHE[name] = W.make_inputs(W.WORKLOADS[name], 0)
    return _INPUT_CACHE[name]


# ----------------------------------------------------------------- helpers
def brute_layout(idx: np.ndarray, E: int, R: int):
    """Independent enumeration: the set of (token, rank) pairs, counted with
    collections.Counter, slots by sorting the pairs by (rank, token)."""
    epr = E // R
    T = idx.shape[0]
    pairs = set()
    ecount = collections.Counter()
    for t in range(T):
        for e in idx[t]:
            e = int(e)
            if e == -1:
                continue
            ecount[e] += 1
            pairs.add((t, e // epr))
    cnt_r = collections.Counter(r for (_, r) in pairs)
    ordered = sorted(pairs, key=lambda p: (p[1], p[0]))
    slot = {p: i for i, p in enumerate(ordered)}
    return pairs, ecount, cnt_r, slot


def e4m3_table():
    """Every finite non-negative E4M3 code and its value, from the format
    definition (bias 7, 3 mantissa bits, exponent 0 subnormal, 0x7F NaN)."""
    codes, vals = [], []
    for c in range(0x7F):
        ex, m = c >> 3, c & 7
        v = m * 2.0 ** -9 if ex == 0 else (1 + m / 8) * 2.0 ** (ex - 7)
        codes.append(c)
        vals.append(v)
    return np.array(codes), np.array(vals)


def nearest_code(v: np.ndarray) -> np.ndarray:
    """Brute-force nearest-code search: the finite code closest to |v|, ties to
    the code with an even mantissa, magnitudes above 448 clamp to 448, sign
    copied."""
    codes, vals = e4m3_table()
    a = np.minimum(np.abs(v.astype(np.float64)), 448.0)
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equal distances prefer even code (even mantissa LSB)
    even = (codes % 2 == 0)[None, :]
    score = 2 * cand.astype(np.int32) + (cand & even).astype(np.int32)
    c = codes[np.argmax(score, axis=1)]
    sign = np.signbit(v).astype(np.uint8) << 7
    return (c.astype(np.uint8) | sign)


def all_finite_bf16() -> np.ndarray:
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_bits_to_f32(b)
    return f[np.isfinite(f)]


# ----------------------------------------------------------------- layout
def pin_layout_golden(O):
    g = json.load(open(os.path.join(GOLDEN, "layout_hand_example.json")))
    idx = np.array(g["topk_idx"], np.int32)
    L = O.layout(idx, g["E"], g["R"])
    assert L["status"] == 0
    for key in ("is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert",
                "rank_offset", "expert_offset", "send_slot"):
        assert np.array_equal(L[key], np.array(g[key])), key


def pin_layout_bruteforce(O, n_cases: int = 150, seed: int = 11):
    rng = np.random.default_rng(seed)
    shapes = [(1, 1, 1), (4, 1, 1), (8, 2, 2), (16, 4, 3), (16, 16, 8), (64, 8, 8),
              (64, 64, 8), (128, 64, 6), (32, 2, 1), (12, 3, 2)]
    for c in range(n_cases):
        E, R, k = shapes[c % len(shapes)]
        k = min(k, E)
        T = int(rng.integers(0, 70))
        inp = W.make_random_case(rng, T, 8, E, R, k, drop_prob=0.15 if c % 3 == 0 else 0.0)
        idx = inp["topk_idx"]
        L = O.layout(idx, E, R)
        assert L["status"] == 0
        pairs, ecount, cnt_r, slot = brute_layout(idx, E, R)
        assert L["P"] == len(pairs)
        for r in range(R):
            assert L["num_tokens_per_rank"][r] == cnt_r.get(r, 0)
        for e in range(E):
            assert L["num_tokens_per_expert"][e] == ecount.get(e, 0)
        for t in range(T):
            for r in range(R):
                inr = (t, r) in pairs
                assert L["is_token_in_rank"][t, r] == int(inr)
                assert L["send_slot"][t, r] == (slot[(t, r)] if inr else -1)
        # offsets are exclusive scans of the counts
        assert L["rank_offset"][0] == 0 and L["expert_offset"][0] == 0
        assert np.array_equal(np.diff(L["rank_offset"]), L["num_tokens_per_rank"])
        assert np.array_equal(np.diff(L["expert_offset"]), L["num_tokens_per_expert"])


def pin_layout_invariants(O, names=("tiny", "decode", "train")):
    for name in names:
        w = W.WORKLOADS[name]
        inp = workload_inputs(w.name)
        idx = inp["topk_idx"]
        L = O.layout(idx, w.E, w.R)
        T, R = w.T, w.R
        ss, inr = L["send_slot"], L["is_token_in_rank"]
        # I1: counts sum to the number of distinct (token, rank) pairs
        ranks = idx // w.epr
        distinct = sum(len(set(ranks[t].tolist())) for t in range(T))
        assert L["P"] == distinct == int(L["num_tokens_per_rank"].sum())
        # I2: per-expert counts sum to the number of chosen experts
        assert int(L["num_tokens_per_expert"].sum()) == int((idx >= 0).sum())
        # I3: a rank never receives more tokens than its experts were chosen
        per_rank_e = L["num_tokens_per_expert"].reshape(R, w.epr).sum(axis=1)
        assert np.all(L["num_tokens_per_rank"] <= per_rank_e)
        # I4: slots are a bijection onto [0, P)
        valid = ss[ss >= 0]
        assert valid.size == L["P"]
        assert np.array_equal(np.sort(valid), np.arange(L["P"]))
        assert np.array_equal(ss >= 0, inr.astype(bool))
        # I5: inside each rank segment, the tokens ascend
        for r in range(R):
            toks = np.nonzero(inr[:, r])[0]
            sl = ss[toks, r]
            assert np.all(np.diff(sl) == 1)
            if toks.size:
                assert sl[0] == L["rank_offset"][r]


def pin_layout_expected_fanout(O):
    """Closed form: with k distinct uniformly chosen experts out of E, a token
    misses a rank with probability C(E-epr,k)/C(E,k), so
    E[P/T] = R * (1 - C(E-epr,k)/C(E,k)).  The train workload's routing is
    i.i.d. Gaussian logits (uniform top-k); its P/T must sit within 1% of it."""
    w = W.WORKLOADS["train"]
    inp = workload_inputs(w.name)
    L = O.layout(inp["topk_idx"], w.E, w.R)
    expect = w.R * (1 - math.comb(w.E - w.epr, w.k) / math.comb(w.E, w.k))
    assert abs(L["P"] / w.T - expect) / expect < 0.01, (L["P"] / w.T, expect)


def pin_layout_errors(O):
    idx = np.array([[0, 1], [2, 16]], np.int32)
    assert O.layout(idx, 16, 4)["status"] == 2
    idx = np.array([[0, -2]], np.int32)
    assert O.layout(idx, 16, 4)["status"] == 2
    idx = np.array([[-1, -1], [3, -1]], np.int32)
    L = O.layout(idx, 16, 4)
    assert L["status"] == 0 and L["P"] == 1 and L["send_slot"][0].max() == -1


# ----------------------------------------------------------------- fp8
def pin_e4m3_golden(O):
    rows = []
    for line in open(os.path.join(GOLDEN, "e4m3_ocp_values.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        v, c = line.split()[:2]
        rows.append((float(v), int(c, 16)))
    vals = np.array([r[0] for r in rows], np.float32)
    got = O.e4m3_encode(vals)
    for (v, c), g in zip(rows, got):
        assert g == c, (v, hex(c), hex(int(g)))
    for (v, c) in rows:
        if abs(v) <= 448 and v != 0:
            d = O.e4m3_decode(c)
            # decode of the code is the nearest representable value
            assert abs(d - v) <= abs(v) * 2 ** -4 + 2 ** -10


def pin_e4m3_nearest(O, n_scales: int = 6):
    """All finite bf16 values, times a set of scales, against the brute-force
    nearest-code search."""
    base = all_finite_bf16()
    scales = [1.0, 448.0 / 3.0, 448.0 / 0.7, 2.0 ** -7, 37.5, 448.0 / 2.75][:n_scales]
    for s in scales:
        with np.errstate(over="ignore"):
            v = (base * np.float32(s)).astype(np.float32)
        v = v[np.isfinite(v)]
        got = O.e4m3_encode(v)
        want = nearest_code(v)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (s, v[bad[:5]], got[bad[:5]], want[bad[:5]])


def pin_e4m3_torch(O):
    """torch's float8_e4m3fn cast (round to nearest even) agrees for every
    value within the finite range (it does not saturate beyond 448)."""
    import torch
    base = all_finite_bf16()
    v = base[np.abs(base) <= 448.0]
    got = O.e4m3_encode(v)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def pin_quantize(O, seed: int = 5):
    rng = np.random.default_rng(seed)
    H = 512
    for trial in range(20):
        x = rng.standard_normal(H).astype(np.float32) * (10.0 ** rng.uniform(-3, 3))
        if trial == 0:
            x[:128] = 0.0                         # all-zero block
        if trial == 1:
            x[128:256] = 1e-6                     # block below the 1e-4 floor
        xb = W.f32_to_bf16_bits(x)
        xf = W.bf16_bits_to_f32(xb).astype(np.float64)
        row = O.quantize_row(xb)
        nb = H // 128
        # the row: H codes, nb float32 scales, zero bytes up to a pitch that
        # is the smallest whole number of 128-byte lines holding them
        payload = H + 4 * nb
        assert row.size % 128 == 0 and payload <= row.size < payload + 128
        assert not row[payload:].any(), "pad bytes not zero"
        codes = row[:H]
        scales = row[H:payload].view(np.float32).astype(np.float64)
        for b in range(nb):
            blk = slice(b * 128, (b + 1) * 128)
            amax = np.abs(xf[blk]).max()
            mag = codes[blk] & 0x7F
            deq = np.array([O.e4m3_decode(int(c)) for c in codes[blk]]) * scales[b]
            if amax >= 1e-4:
                # I7: the block maximum maps to the largest code, 448
                assert mag.max() == 0x7E
                # the scale returns the block maximum: 448 * s == amax
                assert abs(448.0 * scales[b] - amax) <= 1e-6 * amax
            else:
                assert abs(scales[b] - 1e-4 / 448.0) <= 1e-6 * 1e-4 / 448.0
            # error bound: half a step of a 3-bit mantissa, or half the
            # subnormal step (2^-9) in code units, plus float rounding
            err = np.abs(xf[blk] - deq)
            bound = 2.0 ** -4 * np.abs(xf[blk]) + 2.0 ** -10 * scales[b] + 1e-6 * np.abs(xf[blk])
            assert np.all(err <= bound + 1e-30)
            # signs survive
            nz = np.abs(xf[blk]) > 2.0 ** -9 * scales[b]
            assert np.all((codes[blk][nz] >> 7) == (xf[blk][nz] < 0))


def pin_quantize_golden(O):
    """Hand-worked fp8 rows (tests/golden/fp8_quant_hand_example.json): one
    whose two possible operation orders, x * (448 / a) and x / (a / 448),
    round to different codes, and one with NaN and infinite elements."""
    g = json.load(open(os.path.join(GOLDEN, "fp8_quant_hand_example.json")))
    for row in g["rows"]:
        H = row["H"]
        x = np.zeros(H, np.uint16)
        for i, b in row["x_bf16"].items():
            x[int(i)] = int(b, 16)
        want = np.zeros(H, np.uint8)
        for i, c in row["codes"].items():
            want[int(i)] = int(c, 16)
        out = O.quantize_row(x)
        bad = np.nonzero(out[:H] != want)[0]
        assert bad.size == 0, (row["name"], [(int(i), hex(int(out[i])), hex(int(want[i])))
                                             for i in bad[:4]])
        nb = H // 128
        scales = out[H:H + 4 * nb].copy().view(np.uint32)
        assert [hex(int(v)) for v in scales] == row["scales_f32_bits"], row["name"]
        assert not out[H + 4 * nb:].any()


# ----------------------------------------------------------------- pack
def pin_pack_golden(O):
    g = json.load(open(os.path.join(GOLDEN, "layout_hand_example.json")))
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    T, H, E, R = g["T"], g["H"], g["E"], g["R"]
    x = (np.arange(T * H, dtype=np.uint32) * 7 + 1).astype(np.uint16).reshape(T, H)
    ss = np.array(g["send_slot"], np.int32)
    pk = O.pack(x, idx, w, ss, E, R, FMT_BF16, capacity_rows=10)
    assert pk["status"] == 0
    assert np.array_equal(pk["slot_src"][:8], np.array(g["slot_src"]))
    assert np.array_equal(pk["slot_local_idx"][:8], np.array(g["slot_local_idx"]))
    assert np.array_equal(pk["slot_local_w"][:8], np.array(g["slot_local_w"], np.float32))
    for s, t in enumerate(g["slot_src"]):
        assert np.array_equal(pk["send_buf"][s].view(np.uint16), x[t])
    assert np.all(pk["send_buf"][8:] == 0xA5)


def pin_pack_bruteforce(O, n_cases: int = 40, seed: int = 3):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        E, R, k = [(8, 4, 2), (16, 4, 3), (32, 8, 8), (4, 2, 4), (64, 64, 4)][c % 5]
        T = int(rng.integers(0, 40))
        H = 128 * int(rng.integers(1, 3)) if c % 2 else 8 * int(rng.integers(1, 9))
        fmt = FMT_FP8 if (c % 2 and H % 128 == 0) else FMT_BF16
        inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=0.2 if c % 4 == 0 else 0.0)
        idx, w, x = inp["topk_idx"], inp["topk_w"], inp["x"]
        pairs, _, _, slot = brute_layout(idx, E, R)
        ss = np.full((T, R), -1, np.int32)
        for (t, r), s in slot.items():
            ss[t, r] = s
        P = len(pairs)
        cap = P + 3
        pk = O.pack(x, idx, w, ss, E, R, fmt, capacity_rows=cap)
        assert pk["status"] == 0
        epr = E // R
        for (t, r), s in slot.items():
            if fmt == FMT_BF16:
                assert np.array_equal(pk["send_buf"][s].view(np.uint16), x[t])
            else:
                assert np.array_equal(pk["send_buf"][s], O.quantize_row(x[t]))
            assert pk["slot_src"][s] == t
            for j in range(k):
                e = int(idx[t, j])
                if e >= 0 and e // epr == r:
                    assert pk["slot_local_idx"][s, j] == e % epr
                    assert pk["slot_local_w"][s, j] == w[t, j]
                else:
                    assert pk["slot_local_idx"][s, j] == -1
                    assert pk["slot_local_w"][s, j] == 0.0
        assert np.all(pk["send_buf"][P:] == 0xA5)
        assert np.all(pk["slot_src"][P:] == -7)
        # capacity shortfall is reported and rows below capacity still land
        if P >= 2:
            pk2 = O.pack(x, idx, w, ss, E, R, fmt, capacity_rows=P - 1)
            assert pk2["status"] == 3
            assert np.array_equal(pk2["send_buf"], pk["send_buf"][:P - 1])


# ----------------------------------------------------------------- descriptors
def brute_descriptors(cnt, off, rb, C):
    """Group slot indices: slot s of rank r belongs to message (s - o_r) // 8.
    Returns {channel: list of records in channel order}."""
    R = len(cnt)
    P = int(off[R])
    groups = collections.OrderedDict()
    for s in range(P):
        r = int(np.searchsorted(off, s, side="right") - 1)
        while cnt[r] == 0:
            r += 1
        m = (s - int(off[r])) // 8
        groups.setdefault((r, m), []).append(s)
    chans = collections.defaultdict(list)
    for r in range(R):
        for (rr, m), slots in groups.items():
            if rr != r:
                continue
            chans[r % C].append((1, 0, len(slots), r, len(slots) * rb,
                                 slots[0] * rb, (slots[0] - int(off[r])) * rb))
        chans[r % C].append((2, 1, 0, r, int(cnt[r]), 0, 0))
    return chans


def _rec(d):
    return (int(d["type"]), int(d["op"]), int(d["num_tokens"]), int(d["dst_rank"]),
            int(d["size_or_value"]), int(d["src_offset"]), int(d["dst_offset"]))


def pin_descriptors_golden(O):
    g = json.load(open(os.path.join(GOLDEN, "layout_hand_example.json")))
    d = O.descriptors(np.array(g["num_tokens_per_rank"], np.int32),
                      np.array(g["rank_offset"], np.int32), g["row_bytes_bf16"], g["channels"])
    want = [(x["type"], x["op"], x["num_tokens"], x["dst_rank"], x["size_or_value"],
             x["src_offset"], x["dst_offset"]) for x in g["descriptors_channel_order"]]
    assert [_rec(x) for x in d] == want


def pin_descriptors(O, n_cases: int = 60, seed: int = 9):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        R = int(rng.integers(1, 65))
        C = int(rng.integers(1, 9))
        cnt = rng.integers(0, 40, size=R).astype(np.int32)
        if c % 5 == 0:
            cnt[rng.integers(0, R)] = 0
        off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
        rb = int(rng.choice([16, 1024, 14336, 7392]))
        d = O.descriptors(cnt, off, rb, C)
        chans = brute_descriptors(cnt, off, rb, C)
        # channel-major order equals the brute-force grouping
        flat = [x for ch in range(C) for x in chans[ch]]
        assert [_rec(x) for x in d] == flat
        # I8 coverage: WRITE intervals tile [0, P*rb) without overlap
        wr = sorted((int(x["src_offset"]), int(x["size_or_value"])) for x in d if x["type"] == 1)
        pos = 0
        for s, n in wr:
            assert s == pos and n > 0
            pos = s + n
        assert pos == int(off[-1]) * rb
        nwrite = sum(1 for x in d if x["type"] == 1)
        assert nwrite == sum((int(n) + 7) // 8 for n in cnt)
        assert all(1 <= x["num_tokens"] <= 8 for x in d if x["type"] == 1)
        atomics = [x for x in d if x["type"] == 2]
        assert sorted(int(x["dst_rank"]) for x in atomics) == list(range(R))
        for x in atomics:
            assert x["size_or_value"] == cnt[x["dst_rank"]] and x["size_or_value"] < 2 ** 28


# ----------------------------------------------------------------- combine
def pin_combine_golden(O):
    g = json.load(open(os.path.join(GOLDEN, "layout_hand_example.json")))
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    ss = np.array(g["send_slot"], np.int32)
    H = g["H"]
    y = np.repeat(W.f32_to_bf16_bits(np.arange(1, 9, dtype=np.float32))[:, None], H, axis=1)
    out = O.combine(y, idx, w, ss, g["E"], g["R"])
    want = np.array(g["combine_y_row_value_is_slot_plus_1"])
    assert np.array_equal(out, np.repeat(want[:, None], H, axis=1))


def pin_combine_bruteforce(O, n_cases: int = 30, seed: int = 21):
    """Per-expert form: out[t] = sum over valid j of w[t,j] * Y[slot(t, rank(e_j))],
    looping over experts instead of ranks."""
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        E, R, k = [(8, 4, 2), (16, 4, 4), (32, 8, 8), (64, 64, 6)][c % 4]
        T = int(rng.integers(0, 30))
        H = 8 * int(rng.integers(1, 6))
        inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=0.2 if c % 2 else 0.0)
        idx, w = inp["topk_idx"], inp["topk_w"]
        pairs, _, _, slot = brute_layout(idx, E, R)
        ss = np.full((T, R), -1, np.int32)
        for (t, r), s in slot.items():
            ss[t, r] = s
        P = len(pairs)
        y = W.f32_to_bf16_bits(rng.standard_normal((max(P, 1), H), dtype=np.float32))
        yf = W.bf16_bits_to_f32(y).astype(np.float64)
        out = O.combine(y, idx, w, ss, E, R, H=H)
        want = np.zeros((T, H))
        for t in range(T):
            for j in range(k):
                e = int(idx[t, j])
                if e < 0:
                    continue
                want[t] += float(w[t, j]) * yf[slot[(t, e // (E // R))]]
        assert np.allclose(out, want, rtol=1e-12, atol=1e-12)


def pin_combine_identity(O, names=("tiny", "decode")):
    """Identity experts: Y = the packed rows, so out = (sum_j w_j) * x."""
    for name in names:
        w = W.WORKLOADS[name]
        inp = workload_inputs(w.name)
        L = O.layout(inp["topk_idx"], w.E, w.R)
        pk = O.pack(inp["x"], inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R,
                    FMT_BF16, capacity_rows=L["P"])
        y = pk["send_buf"].view(np.uint16).reshape(L["P"], w.H)
        out = O.combine(y, inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R)
        xf = W.bf16_bits_to_f32(inp["x"]).astype(np.float64)
        wsum = inp["topk_w"].astype(np.float64).sum(axis=1)
        assert np.allclose(out, wsum[:, None] * xf, rtol=1e-12, atol=1e-300)
        # probe: Y == 1 gives the weight sum in every column
        ones = np.full_like(y, 0x3F80)
        o1 = O.combine(ones, inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R)
        assert np.allclose(o1, np.repeat(wsum[:, None], w.H, axis=1), rtol=1e-12)
        # exact scaling: Y -> 2Y doubles the output bit for bit
        y2 = W.f32_to_bf16_bits(2.0 * W.bf16_bits_to_f32(y))
        o2 = O.combine(y2, inp["topk_idx"], inp["topk_w"], L["send_slot"], w.E, w.R)
        assert np.array_equal(o2, 2.0 * out)


# ----------------------------------------------------------------- per-expert mode
def brute_ll(idx: np.ndarray, E: int):
    """Independent enumeration of the per-expert layout: the list of kept
    choices (t, j, e) sorted by (e, t, j); a choice's row is its position."""
    T, k = idx.shape
    choices = [(int(idx[t, j]), t, j) for t in range(T) for j in range(k) if int(idx[t, j]) != -1]
    ordered = sorted(choices)
    slot = {(t, j): i for i, (_, t, j) in enumerate(ordered)}
    cnt = collections.Counter(e for (e, _, _) in choices)
    return ordered, slot, cnt


def brute_ll_descriptors(ordered, E, R, rb, C):
    """Group the rows of each expert into messages of 8 by walking them; one
    count record per expert.  Returns records in channel-major order."""
    epr = E // R
    first = {}
    rows = collections.defaultdict(list)
    for i, (e, _, _) in enumerate(ordered):
        rows[e].append(i)
    recs = []
    for c in range(C):
        for r in range(c, R, C):
            base = None
            for le in range(epr):
                e = r * epr + le
                if base is None:
                    # the rank's first row: the first row of any of its experts
                    # (or, if none has rows, where the next expert would start)
                    cand = [rows[r * epr + q][0] for q in range(epr) if rows[r * epr + q]]
                    base = min(cand) if cand else 0
                rs = rows[e]
                for m in range(0, len(rs), 8):
                    part = rs[m:m + 8]
                    recs.append((1, 0, len(part), r, len(part) * rb, part[0] * rb, (part[0] - base) * rb))
                recs.append((2, 1, 0, r, len(rs), 0, 4 * le))
    return recs


def pin_ll_golden(O):
    g = json.load(open(os.path.join(GOLDEN, "ll_hand_example.json")))
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    T, H, E, R = g["T"], g["H"], g["E"], g["R"]
    L = O.ll_layout(idx, E)
    assert L["status"] == 0
    assert np.array_equal(L["num_tokens_per_expert"], np.array(g["num_tokens_per_expert"]))
    assert np.array_equal(L["expert_offset"], np.array(g["expert_offset"]))
    assert np.array_equal(L["expert_slot"], np.array(g["expert_slot"]))
    x = (np.arange(T * H, dtype=np.uint32) * 5 + 3).astype(np.uint16).reshape(T, H)
    pk = O.ll_pack(x, w, L["expert_slot"], FMT_BF16, capacity_rows=9)
    assert pk["status"] == 0
    assert np.array_equal(pk["slot_src"][:7], np.array(g["slot_src"]))
    assert np.array_equal(pk["slot_w"][:7], np.array(g["slot_w"], np.float32))
    for s, t in enumerate(g["slot_src"]):
        assert np.array_equal(pk["send_buf"][s].view(np.uint16), x[t])
    assert np.all(pk["send_buf"][7:] == 0xA5)
    d = O.ll_descriptors(L["num_tokens_per_expert"], L["expert_offset"], R, g["row_bytes_bf16"],
                         g["channels"])
    want = [(x_["type"], x_["op"], x_["num_tokens"], x_["dst_rank"], x_["size_or_value"],
             x_["src_offset"], x_["dst_offset"]) for x_ in g["descriptors_channel_order"]]
    assert [_rec(x_) for x_ in d] == want
    y = np.repeat(W.f32_to_bf16_bits(np.arange(1, 8, dtype=np.float32))[:, None], H, axis=1)
    out = O.ll_combine(y, idx, w, L["expert_slot"])
    want_c = np.array(g["combine_y_row_value_is_slot_plus_1"])
    assert np.array_equal(out, np.repeat(want_c[:, None], H, axis=1))


def pin_ll_bruteforce(O, n_cases: int = 60, seed: int = 31):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        E, R, k = [(8, 4, 2), (16, 4, 3), (32, 8, 8), (4, 2, 4), (64, 64, 4), (256, 32, 8)][c % 6]
        T = int(rng.integers(0, 40))
        H = 128 * int(rng.integers(1, 3)) if c % 2 else 8 * int(rng.integers(1, 9))
        fmt = FMT_FP8 if (c % 2 and H % 128 == 0) else FMT_BF16
        inp = W.make_random_case(rng, T, H, E, R, k, drop_prob=0.2 if c % 3 == 0 else 0.0)
        idx, w, x = inp["topk_idx"], inp["topk_w"], inp["x"]
        if c % 7 == 0 and T > 0:
            idx = idx.copy()
            idx[0, :] = idx[0, 0]            # one token naming one expert k times
        ordered, slot, cnt = brute_ll(idx, E)
        Q = len(ordered)
        L = O.ll_layout(idx, E)
        assert L["status"] == 0 and L["Q"] == Q
        assert np.array_equal(L["num_tokens_per_expert"], np.array([cnt[e] for e in range(E)]))
        want_slot = np.full((T, k), -1, np.int32)
        for (t, j), s in slot.items():
            want_slot[t, j] = s
        assert np.array_equal(L["expert_slot"], want_slot)
        # pack: each row is its token's row (or its fp8 row), metadata per choice
        cap = Q + 3
        pk = O.ll_pack(x, w, L["expert_slot"], fmt, capacity_rows=cap)
        assert pk["status"] == 0
        for (t, j), s in slot.items():
            if fmt == FMT_BF16:
                assert np.array_equal(pk["send_buf"][s].view(np.uint16), x[t])
            else:
                assert np.array_equal(pk["send_buf"][s], O.quantize_row(x[t]))
            assert pk["slot_src"][s] == t and pk["slot_w"][s] == w[t, j]
        assert np.all(pk["send_buf"][Q:] == 0xA5) and np.all(pk["slot_src"][Q:] == -7)
        if Q >= 2:
            pk2 = O.ll_pack(x, w, L["expert_slot"], fmt, capacity_rows=Q - 1)
            assert pk2["status"] == 3
            assert np.array_equal(pk2["send_buf"], pk["send_buf"][:Q - 1])
        # descriptors: brute-force grouping, and the WRITEs tile [0, Q*rb)
        rb = O.row_bytes(H, fmt)
        C = int(rng.integers(1, 9))
        d = O.ll_descriptors(L["num_tokens_per_expert"], L["expert_offset"], R, rb, C)
        assert [_rec(x_) for x_ in d] == brute_ll_descriptors(ordered, E, R, rb, C)
        wr = sorted((int(x_["src_offset"]), int(x_["size_or_value"])) for x_ in d if x_["type"] == 1)
        pos = 0
        for s0, n in wr:
            assert s0 == pos and n > 0
            pos = s0 + n
        assert pos == Q * rb
        # combine: loop over the choices of each token
        if fmt == FMT_BF16:
            y = W.f32_to_bf16_bits(rng.standard_normal((max(Q, 1), H), dtype=np.float32))
            yf = W.bf16_bits_to_f32(y).astype(np.float64)
            out = O.ll_combine(y, idx, w, L["expert_slot"], H=H)
            want = np.zeros((T, H))
            for (t, j), s in slot.items():
                want[t] += float(w[t, j]) * yf[s]
            assert np.allclose(out, want, rtol=1e-12, atol=1e-12)


def pin_ll_invariants(O, names=("tiny", "decode", "train")):
    """The per-expert counts and offsets equal the rank layout's; the rows are
    a bijection onto [0, Q) with Q = T*k minus drops; inside an expert the
    source tokens ascend."""
    for name in names:
        w = W.WORKLOADS[name]
        inp = workload_inputs(name)
        idx = inp["topk_idx"]
        L = O.ll_layout(idx, w.E)
        R0 = O.layout(idx, w.E, w.R)
        assert np.array_equal(L["num_tokens_per_expert"], R0["num_tokens_per_expert"])
        assert np.array_equal(L["expert_offset"], R0["expert_offset"])
        es = L["expert_slot"]
        kept = idx != -1
        assert L["Q"] == int(kept.sum())
        assert np.array_equal(np.sort(es[kept]), np.arange(L["Q"]))
        assert np.all(es[~kept] == -1)
        t_of = np.repeat(np.arange(w.T), w.k).reshape(w.T, w.k)
        src = np.empty(L["Q"], np.int64)
        src[es[kept]] = t_of[kept]
        e_of = np.empty(L["Q"], np.int64)
        e_of[es[kept]] = idx[kept]
        assert np.all(np.diff(e_of) >= 0)
        same = np.diff(e_of) == 0
        assert np.all(np.diff(src)[same] >= 0)


def pin_ll_combine_identity(O, names=("tiny", "decode")):
    """Identity experts: per-expert combine gives (sum_j w_j) * x, the same
    as the rank-deduplicated combine on its own identity rows."""
    for name in names:
        w = W.WORKLOADS[name]
        inp = workload_inputs(name)
        L = O.ll_layout(inp["topk_idx"], w.E)
        pk = O.ll_pack(inp["x"], inp["topk_w"], L["expert_slot"], FMT_BF16, capacity_rows=L["Q"])
        y = pk["send_buf"].view(np.uint16).reshape(L["Q"], w.H)
        out = O.ll_combine(y, inp["topk_idx"], inp["topk_w"], L["expert_slot"])
        xf = W.bf16_bits_to_f32(inp["x"]).astype(np.float64)
        wsum = inp["topk_w"].astype(np.float64).sum(axis=1)
        assert np.allclose(out, wsum[:, None] * xf, rtol=1e-12, atol=1e-300)
        R0 = O.layout(inp["topk_idx"], w.E, w.R)
        pr = O.pack(inp["x"], inp["topk_idx"], inp["topk_w"], R0["send_slot"], w.E, w.R,
                    FMT_BF16, capacity_rows=R0["P"])
        yr = pr["send_buf"].view(np.uint16).reshape(R0["P"], w.H)
        outr = O.combine(yr, inp["topk_idx"], inp["topk_w"], R0["send_slot"], w.E, w.R)
        assert np.allclose(out, outr, rtol=1e-12, atol=1e-300)


ALL_PINS = [
    pin_layout_golden, pin_layout_bruteforce, pin_layout_invariants,
    pin_layout_expected_fanout, pin_layout_errors,
    pin_e4m3_golden, pin_e4m3_nearest, pin_e4m3_torch, pin_quantize, pin_quantize_golden,
    pin_pack_golden, pin_pack_bruteforce,
    pin_descriptors_golden, pin_descriptors,
    pin_combine_golden, pin_combine_bruteforce, pin_combine_identity,
    pin_ll_golden, pin_ll_bruteforce, pin_ll_invariants, pin_ll_combine_identity,
]
