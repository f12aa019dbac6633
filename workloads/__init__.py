"""Seeded synthetic inputs for MoE expert-parallel dispatch/combine.

This module only draws random numbers and lays them out.  It holds none of the
dispatch/combine arithmetic (no rank membership, counts, slots, packing,
quantisation or reduction); both the CPU oracle and the HIP path consume what it
returns.

The source pages measure dispatch/combine only on a real
DeepSeek-V3 training cluster and on a "MoE simulated load" (UCCL-EP article,
peacm.com, section 6 "performance data"; NCCL GIN article, bjdmk.com.cn,
section 4.3 "benchmark methods").  Neither the model nor its routing traces are
available, so five seeded synthetic workloads stand in for them:

  tiny      T=128,   H=512,  E=16,  R=4,  k=2, bf16, softmax of the chosen 2
  train     T=4096,  H=7168, E=256, R=32, k=8, bf16, renormalised softmax
  decode    T=128,   H=7168, E=256, R=32, k=8, bf16, ring with 1 channel
  skewed    T=16384, H=7168, E=256, R=64, k=8, bf16, Zipf(1.2) routing,
            Dirichlet(1) gate weights
  fp8       as train, rows packed as e4m3 codes + per-128 fp32 scales

Draw order from ``numpy.random.default_rng(seed)``: x, then router logits (or
Gumbel noise), then gate weights (skewed only).  ``train`` and ``fp8`` share x
and routing.  The synthetic expert outputs Y come from a second generator,
``default_rng([seed, 1])``, so that they do not depend on the routing result.
"""

from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np

FMT_BF16 = 0
FMT_FP8_E4M3_B128 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    R: int
    k: int
    fmt: int
    routing: str          # "softmax_top", "softmax_renorm" or "zipf_dirichlet"
    channels: int         # TransferCmd channels (FIFOs) of the ring
    depth: int = 1024     # ring depth per channel
    max_inflight: int = 256

    @property
    def epr(self) -> int:
        return self.E // self.R


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 128, 512, 16, 4, 2, FMT_BF16, "softmax_top", 1),
    "train": Workload("train", 4096, 7168, 256, 32, 8, FMT_BF16, "softmax_renorm", 8),
    "decode": Workload("decode", 128, 7168, 256, 32, 8, FMT_BF16, "softmax_renorm", 1),
    "skewed": Workload("skewed", 16384, 7168, 256, 64, 8, FMT_BF16, "zipf_dirichlet", 8),
    "fp8": Workload("fp8", 4096, 7168, 256, 32, 8, FMT_FP8_E4M3_B128, "softmax_renorm", 8),
}

ZIPF_S = 1.2


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # process in slices to bound the temporary memory at large sizes
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_u.size, step):
        v = flat_u[i:i + step].astype(np.uint64)
        v = v + 0x7FFF + ((v >> 16) & 1)
        flat_o[i:i + step] = (v >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _topk_desc(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row; ties go to the lower index."""
    order = np.argsort(-keys, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k].astype(np.int32))


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Return x (uint16 bf16 bits [T,H]), topk_idx (int32 [T,k]) and
    topk_w (float32 [T,k]) for workload ``w``."""
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(_normal_f32(rng, (w.T, w.H)))
    if w.routing in ("softmax_top", "softmax_renorm"):
        logits = _normal_f32(rng, (w.T, w.E))
        idx = _topk_desc(logits, w.k)
        chosen = np.take_along_axis(logits, idx, axis=1).astype(np.float64)
        if w.routing == "softmax_top":
            # probabilities of the chosen experts under the softmax over all E
            lg = logits.astype(np.float64)
            m = lg.max(axis=1, keepdims=True)
            z = np.exp(lg - m).sum(axis=1, keepdims=True)
            wts = np.exp(chosen - m) / z
        else:
            m = chosen.max(axis=1, keepdims=True)
            e = np.exp(chosen - m)
            wts = e / e.sum(axis=1, keepdims=True)
    elif w.routing == "zipf_dirichlet":
        # k experts drawn without replacement with probability
        # p_e proportional to (e+1)^-s: Gumbel-top-k over log p_e.
        logp = -ZIPF_S * np.log(np.arange(1, w.E + 1, dtype=np.float64))
        g = rng.gumbel(size=(w.T, w.E))
        idx = _topk_desc(logp[None, :] + g, w.k)
        ex = rng.standard_exponential(size=(w.T, w.k))
        wts = ex / ex.sum(axis=1, keepdims=True)
    else:
        raise ValueError(w.routing)
    return {
        "x": np.ascontiguousarray(x),
        "topk_idx": idx,
        "topk_w": np.ascontiguousarray(wts.astype(np.float32)),
    }


def make_expert_outputs(rows: int, H: int, seed: int = 0) -> np.ndarray:
    """Synthetic returned expert outputs Y: bf16 bits [rows, H], N(0,1)."""
    rng = np.random.default_rng([seed, 1])
    out = np.empty((rows, H), dtype=np.uint16)
    step = max(1, (1 << 24) // max(H, 1))
    for i in range(0, rows, step):
        n = min(step, rows - i)
        out[i:i + n] = f32_to_bf16_bits(_normal_f32(rng, (n, H)))
    return out


def make_random_case(rng: np.random.Generator, T: int, H: int, E: int, R: int,
                     k: int, drop_prob: float = 0.0) -> dict:
    """A small random case for property and parity tests: k distinct experts
    per token (uniform), some entries optionally replaced by -1 (dropped)."""
    keys = rng.random((T, E))
    idx = _topk_desc(keys, k) if T > 0 else np.zeros((0, k), np.int32)
    if drop_prob > 0 and T > 0:
        drop = rng.random((T, k)) < drop_prob
        idx = np.where(drop, -1, idx).astype(np.int32)
    wts = rng.random((T, k)).astype(np.float32)
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    return {"x": np.ascontiguousarray(x), "topk_idx": np.ascontiguousarray(idx),
            "topk_w": np.ascontiguousarray(wts)}
