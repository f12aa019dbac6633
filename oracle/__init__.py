"""CPU oracle for MoE expert-parallel dispatch/combine (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It wraps ``ep_oracle.c`` (plain C loops, built
with ``-O2 -fno-fast-math -ffp-contract=off``) with ctypes and numpy and shares
no code with the HIP library.

``Oracle(path)`` binds one build of the C source; the module-level functions
use the default build next to this file.  Tests also load deliberately mutated
builds through ``Oracle`` to show that the pins catch plausible mistakes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")

FMT_BF16 = 0
FMT_FP8 = 1
OK, ERR_INVALID_ARG, ERR_BAD_EXPERT, ERR_CAPACITY = 0, 1, 2, 3
CMD_WRITE, CMD_ATOMIC = 1, 2
ATOMIC_ADD = 1

# 32-byte transfer command record (field order of the proxy's WRITE call:
# dst_rank, src_offset, dst_offset, size; plus the op/value pair).
CMD_DTYPE = np.dtype([
    ("seq", "<u4"), ("type", "u1"), ("op", "u1"), ("num_tokens", "<u2"),
    ("dst_rank", "<u4"), ("size_or_value", "<u4"),
    ("src_offset", "<u8"), ("dst_offset", "<u8"),
])
assert CMD_DTYPE.itemsize == 32

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-fopenmp",
             "-Wall", "-Wextra", "-fPIC", "-shared"]


def compile_source(src: str, out: str) -> str:
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle's shared library with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SRC):
        compile_source(SRC, _LIB)
    return _LIB


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """numpy-level wrapper around one build of ep_oracle.c."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_row_bytes.argtypes = [i32, i32]
        L.oracle_row_bytes.restype = i64
        L.oracle_layout.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_layout.restype = i32
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode_array.argtypes = [i64, P, P]
        L.oracle_e4m3_encode_array.restype = None
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_float
        L.oracle_quantize_row.argtypes = [i32, P, P]
        L.oracle_quantize_row.restype = None
        L.oracle_pack.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, i64, P, P, P]
        L.oracle_pack.restype = i32
        L.oracle_descriptors.argtypes = [i32, i32, P, P, i64, P, i64]
        L.oracle_descriptors.restype = i64
        L.oracle_combine.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P]
        L.oracle_combine.restype = None
        L.oracle_ll_layout.argtypes = [i32, i32, i32, P, P, P, P]
        L.oracle_ll_layout.restype = i32
        L.oracle_ll_pack.argtypes = [i32, i32, i32, i32, P, P, P, P, i64, P, P]
        L.oracle_ll_pack.restype = i32
        L.oracle_ll_descriptors.argtypes = [i32, i32, i32, P, P, i64, P, i64]
        L.oracle_ll_descriptors.restype = i64
        L.oracle_ll_combine.argtypes = [i32, i32, i32, P, P, P, P, P]
        L.oracle_ll_combine.restype = None
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_set_threads.restype = i32
        self.L = L
        self.path = path

    def row_bytes(self, H: int, fmt: int) -> int:
        return int(self.L.oracle_row_bytes(H, fmt))

    def set_threads(self, n: int) -> int:
        """Threads for the token loops of pack and combine; returns the number
        in effect.  Results do not depend on it."""
        return int(self.L.oracle_set_threads(n))

    def layout(self, topk_idx: np.ndarray, E: int, R: int) -> dict:
        """Rank membership, histograms, offsets and send slots."""
        idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
        T, k = idx.shape
        out = {
            "num_tokens_per_rank": np.zeros(R, np.int32),
            "num_tokens_per_expert": np.zeros(E, np.int32),
            "rank_offset": np.zeros(R + 1, np.int32),
            "expert_offset": np.zeros(E + 1, np.int32),
            "is_token_in_rank": np.zeros((T, R), np.uint8),
            "send_slot": np.zeros((T, R), np.int32),
        }
        st = self.L.oracle_layout(T, E, R, k, _p(idx), _p(out["num_tokens_per_rank"]),
                                  _p(out["num_tokens_per_expert"]), _p(out["rank_offset"]),
                                  _p(out["expert_offset"]), _p(out["is_token_in_rank"]),
                                  _p(out["send_slot"]))
        out["status"] = int(st)
        out["P"] = int(out["rank_offset"][R])
        return out

    def e4m3_encode(self, v) -> np.ndarray:
        a = np.ascontiguousarray(np.asarray(v, dtype=np.float32).reshape(-1))
        out = np.zeros(a.size, np.uint8)
        self.L.oracle_e4m3_encode_array(a.size, _p(a), _p(out))
        return out.reshape(np.shape(v))

    def e4m3_decode(self, c: int) -> float:
        return float(self.L.oracle_e4m3_decode(ctypes.c_uint8(c)))

    def quantize_row(self, xrow_bits: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(xrow_bits, dtype=np.uint16)
        H = x.size
        out = np.full(self.row_bytes(H, FMT_FP8), 0xA5, np.uint8)   # every byte is written
        self.L.oracle_quantize_row(H, _p(x), _p(out))
        return out

    def pack(self, x: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray,
             send_slot: np.ndarray, E: int, R: int, fmt: int,
             capacity_rows: int, poison: int = 0xA5) -> dict:
        """Pack rows into the rank-contiguous send buffer with per-slot
        metadata.  Unwritten bytes keep the ``poison`` fill;
        unwritten metadata keeps -7 / -7 / NaN."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
        w = np.ascontiguousarray(topk_w, dtype=np.float32)
        ss = np.ascontiguousarray(send_slot, dtype=np.int32)
        T, H = x.shape
        k = idx.shape[1]
        rb = self.row_bytes(H, fmt)
        buf = np.full((capacity_rows, rb), poison, np.uint8)
        slot_src = np.full(capacity_rows, -7, np.int32)
        sli = np.full((capacity_rows, k), -7, np.int32)
        slw = np.full((capacity_rows, k), np.nan, np.float32)
        st = self.L.oracle_pack(T, H, E, R, k, fmt, _p(x), _p(idx), _p(w), _p(ss), _p(buf),
                                capacity_rows, _p(slot_src), _p(sli), _p(slw))
        return {"status": int(st), "send_buf": buf, "slot_src": slot_src,
                "slot_local_idx": sli, "slot_local_w": slw}

    def descriptors(self, num_tokens_per_rank: np.ndarray, rank_offset: np.ndarray,
                    row_bytes_: int, channels: int) -> np.ndarray:
        """Closed-form TransferCmd stream, channel-major order."""
        cnt = np.ascontiguousarray(num_tokens_per_rank, dtype=np.int32)
        off = np.ascontiguousarray(rank_offset, dtype=np.int32)
        R = cnt.size
        cap = int(sum((int(c) + 7) // 8 for c in cnt)) + R + 16
        out = np.zeros(cap, CMD_DTYPE)
        n = self.L.oracle_descriptors(R, channels, _p(cnt), _p(off), row_bytes_, _p(out), cap)
        if n < 0:
            raise RuntimeError("descriptor buffer too small")
        return out[:n]

    def combine(self, y: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray,
                send_slot: np.ndarray, E: int, R: int, H: Optional[int] = None) -> np.ndarray:
        """Gate-weighted gather-reduce of the returned rows, float64."""
        y = np.ascontiguousarray(y, dtype=np.uint16)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
        w = np.ascontiguousarray(topk_w, dtype=np.float32)
        ss = np.ascontiguousarray(send_slot, dtype=np.int32)
        T, k = idx.shape
        if H is None:
            H = y.shape[1]
        out = np.zeros((T, H), np.float64)
        if T and H:
            self.L.oracle_combine(T, H, E, R, k, _p(y), _p(idx), _p(w), _p(ss), _p(out))
        return out

    # ---------------------------------------------------------- per-expert mode
    def ll_layout(self, topk_idx: np.ndarray, E: int) -> dict:
        """Per-expert counts, offsets and the row of every kept choice."""
        idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
        T, k = idx.shape
        out = {
            "num_tokens_per_expert": np.zeros(E, np.int32),
            "expert_offset": np.zeros(E + 1, np.int32),
            "expert_slot": np.zeros((T, k), np.int32),
        }
        st = self.L.oracle_ll_layout(T, E, k, _p(idx), _p(out["num_tokens_per_expert"]),
                                     _p(out["expert_offset"]), _p(out["expert_slot"]))
        out["status"] = int(st)
        out["Q"] = int(out["expert_offset"][E])
        return out

    def ll_pack(self, x: np.ndarray, topk_w: np.ndarray, expert_slot: np.ndarray, fmt: int,
                capacity_rows: int, poison: int = 0xA5) -> dict:
        """Pack one row per kept choice into the per-expert send buffer, with
        slot_src / slot_w metadata (unwritten: poison bytes, -7, NaN)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(topk_w, dtype=np.float32)
        es = np.ascontiguousarray(expert_slot, dtype=np.int32)
        T, H = x.shape
        k = es.shape[1]
        rb = self.row_bytes(H, fmt)
        buf = np.full((capacity_rows, rb), poison, np.uint8)
        slot_src = np.full(capacity_rows, -7, np.int32)
        slot_w = np.full(capacity_rows, np.nan, np.float32)
        st = self.L.oracle_ll_pack(T, H, k, fmt, _p(x), _p(w), _p(es), _p(buf), capacity_rows,
                                   _p(slot_src), _p(slot_w))
        return {"status": int(st), "send_buf": buf, "slot_src": slot_src, "slot_w": slot_w}

    def ll_descriptors(self, num_tokens_per_expert: np.ndarray, expert_offset: np.ndarray,
                       R: int, row_bytes_: int, channels: int) -> np.ndarray:
        """Closed-form per-expert TransferCmd stream, channel-major order."""
        cnt = np.ascontiguousarray(num_tokens_per_expert, dtype=np.int32)
        off = np.ascontiguousarray(expert_offset, dtype=np.int32)
        E = cnt.size
        cap = int(sum((int(c) + 7) // 8 for c in cnt)) + E + 16
        out = np.zeros(cap, CMD_DTYPE)
        n = self.L.oracle_ll_descriptors(E, R, channels, _p(cnt), _p(off), row_bytes_, _p(out),
                                         cap)
        if n < 0:
            raise RuntimeError("descriptor buffer too small or E % R != 0")
        return out[:n]

    def ll_combine(self, y: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray,
                   expert_slot: np.ndarray, H: Optional[int] = None) -> np.ndarray:
        """Gate-weighted sum of the per-expert rows of each token, float64."""
        y = np.ascontiguousarray(y, dtype=np.uint16)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
        w = np.ascontiguousarray(topk_w, dtype=np.float32)
        es = np.ascontiguousarray(expert_slot, dtype=np.int32)
        T, k = idx.shape
        if H is None:
            H = y.shape[1]
        out = np.zeros((T, H), np.float64)
        if T and H:
            self.L.oracle_ll_combine(T, H, k, _p(y), _p(idx), _p(w), _p(es), _p(out))
        return out


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SRC):
            build(force=True)
        _default = Oracle(_LIB)
    return _default


def row_bytes(H, fmt):
    return default().row_bytes(H, fmt)


def set_threads(n):
    return default().set_threads(n)


def layout(topk_idx, E, R):
    return default().layout(topk_idx, E, R)


def e4m3_encode(v):
    return default().e4m3_encode(v)


def e4m3_decode(c):
    return default().e4m3_decode(c)


def quantize_row(xrow_bits):
    return default().quantize_row(xrow_bits)


def pack(*a, **kw):
    return default().pack(*a, **kw)


def descriptors(*a, **kw):
    return default().descriptors(*a, **kw)


def combine(*a, **kw):
    return default().combine(*a, **kw)


def ll_layout(*a, **kw):
    return default().ll_layout(*a, **kw)


def ll_pack(*a, **kw):
    return default().ll_pack(*a, **kw)


def ll_descriptors(*a, **kw):
    return default().ll_descriptors(*a, **kw)


def ll_combine(*a, **kw):
    return default().ll_combine(*a, **kw)
