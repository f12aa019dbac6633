"""Python binding of libep.so (include/ep.h): MoE expert-parallel dispatch and
combine on one MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
libep.so; torch supplies device memory and streams.  There is no fallback:
importing this package fails loudly when libep.so has not been built
(``python combine_topk_rank_amd/build.py``).

The functions keep the C names:

    ep_row_bytes(H, fmt) -> int
    ep_workspace_bytes(shape) -> int
    ep_dispatch_layout(shape, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                       rank_offset, expert_offset, is_token_in_rank, send_slot,
                       workspace, dev_status, stream=None)
    ep_dispatch(shape, x, topk_idx, topk_w, rank_offset, send_slot, send_buf,
                slot_src, slot_local_idx, slot_local_w, ring, workspace,
                dev_status, stream=None)
    ep_dispatch_fused_plan(shape, with_ring=True) -> int
    ep_dispatch_fused_noalloc(shape, x, topk_idx, topk_w, <layout outputs>, send_buf,
                              slot_src, slot_local_idx, slot_local_w, ring, dev_status,
                              stream=None, clear_scratch=False)
    ep_dispatch_ll_layout(shape, topk_idx, num_tokens_per_expert, expert_offset, expert_slot,
                          workspace, dev_status, stream=None)
    ep_combine(shape, y, topk_idx, topk_w, send_slot, out, dev_status, stream=None)
        (y_rows is y.shape[0])
    Ring(depth, channels, max_inflight, timeout_ns)   # ep_ring_* calls

Tensors are torch tensors on the current HIP device (contiguous); ``stream``
defaults to torch's current stream.  A non-OK return raises EpError.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep.so")

EP_OK = 0
EP_ERR_INVALID_ARG = 1
EP_ERR_BAD_EXPERT = 2
EP_ERR_CAPACITY = 3
EP_ERR_RING_TIMEOUT = 4
EP_ERR_HIP = 5
EP_ERR_BUSY = 6
EP_ERR_TIMEOUT = 7
EP_FUSED_ONE_KERNEL_SMALL = 101
EP_FUSED_ONE_KERNEL_LARGE = 102
EP_FUSED_TWO_CALLS = 103
EP_FMT_BF16 = 0
EP_FMT_FP8_E4M3_B128 = 1
EP_CMD_WRITE = 1
EP_CMD_ATOMIC = 2
EP_ATOMIC_ADD = 1

# ep_transfer_cmd_t, 32 bytes
CMD_DTYPE = np.dtype([
    ("seq", "<u4"), ("type", "u1"), ("op", "u1"), ("num_tokens", "<u2"),
    ("dst_rank", "<u4"), ("size_or_value", "<u4"),
    ("src_offset", "<u8"), ("dst_offset", "<u8"),
])


class EpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = ""
        if status == EP_ERR_HIP:
            detail = " [" + lib.ep_last_error().decode() + "]"
        super().__init__(f"{where}: {status_str(status)} ({status}){detail}")


class ep_shape_t(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("R", ctypes.c_int32), ("k", ctypes.c_int32), ("fmt", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime (file libamdhip64.so, soname
    # libamdhip64.so.7).  Loading torch first lets libep.so's dependency on
    # libamdhip64.so.7 resolve to that same runtime; the other order puts two
    # HIP runtimes in the process and the second one finds no device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python combine_topk_rank_amd/build.py` "
                          "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    S = ctypes.POINTER(ep_shape_t)
    L.ep_row_bytes.argtypes = [i32, i32]
    L.ep_row_bytes.restype = sz
    L.ep_workspace_bytes.argtypes = [S]
    L.ep_workspace_bytes.restype = sz
    L.ep_dispatch_layout.argtypes = [S, P, P, P, P, P, P, P, P, sz, P, P]
    L.ep_dispatch_layout.restype = ctypes.c_int
    L.ep_dispatch.argtypes = [S, P, P, P, P, P, P, i64, P, P, P, P, P, sz, P, P]
    L.ep_dispatch.restype = ctypes.c_int
    L.ep_dispatch_fused.argtypes = [S, P, P, P, P, P, P, P, P, P, P, i64, P, P, P, P, P, sz, P,
                                    P]
    L.ep_dispatch_fused.restype = ctypes.c_int
    L.ep_dispatch_fused_plan.argtypes = [S, i32]
    L.ep_dispatch_fused_plan.restype = ctypes.c_int
    L.ep_dispatch_fused_noalloc.argtypes = [S, P, P, P, P, P, P, P, P, P, P, i64, P, P, P, P,
                                            i32, P, P]
    L.ep_dispatch_fused_noalloc.restype = ctypes.c_int
    L.ep_combine.argtypes = [S, P, i64, P, P, P, P, P, P]
    L.ep_combine.restype = ctypes.c_int
    L.ep_dispatch_layout_ll.argtypes = [S, P, P, P, P, sz, P, P]
    L.ep_dispatch_layout_ll.restype = ctypes.c_int
    L.ep_dispatch_ll_layout.argtypes = [S, P, P, P, P, P, sz, P, P]
    L.ep_dispatch_ll_layout.restype = ctypes.c_int
    L.ep_dispatch_ll.argtypes = [S, P, P, P, P, P, P, i64, P, P, P, P, sz, P, P]
    L.ep_dispatch_ll.restype = ctypes.c_int
    L.ep_dispatch_ll_fused.argtypes = [S, P, P, P, P, P, P, P, i64, P, P, P, P, sz, P, P]
    L.ep_dispatch_ll_fused.restype = ctypes.c_int
    L.ep_combine_ll.argtypes = [S, P, i64, P, P, P, P, P, P]
    L.ep_combine_ll.restype = ctypes.c_int
    L.ep_ring_create.argtypes = [i32, i32, i32, i64]
    L.ep_ring_create.restype = P
    L.ep_ring_destroy.argtypes = [P]
    L.ep_ring_destroy.restype = ctypes.c_int
    L.ep_ring_reset.argtypes = [P]
    L.ep_ring_reset.restype = ctypes.c_int
    L.ep_ring_drain.argtypes = [P, i32, P, i32, ctypes.POINTER(i32)]
    L.ep_ring_drain.restype = ctypes.c_int
    L.ep_ring_proxy_start.argtypes = [P, i32, i64]
    L.ep_ring_proxy_start.restype = ctypes.c_int
    L.ep_ring_proxy_stop.argtypes = [P, P, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.ep_ring_proxy_stop.restype = ctypes.c_int
    L.ep_ring_proxy_drained.argtypes = [P]
    L.ep_ring_proxy_drained.restype = i64
    u64p = ctypes.POINTER(ctypes.c_uint64)
    L.ep_ring_set_loopback.argtypes = [P, P, ctypes.c_uint64, i32, ctypes.POINTER(P), u64p,
                                       ctypes.POINTER(P), u64p]
    L.ep_ring_set_loopback.restype = ctypes.c_int
    L.ep_ring_completed.argtypes = [P, i32]
    L.ep_ring_completed.restype = i64
    L.ep_ring_check_completion.argtypes = [P, P, P, i32, P, P]
    L.ep_ring_check_completion.restype = ctypes.c_int
    L.ep_ring_wait_complete.argtypes = [P, i64]
    L.ep_ring_wait_complete.restype = ctypes.c_int
    i64p = ctypes.POINTER(i64)
    dp = ctypes.POINTER(ctypes.c_double)
    L.ep_ring_loopback_stats.argtypes = [P, i64p, i64p, i64p, dp, dp]
    L.ep_ring_loopback_stats.restype = ctypes.c_int
    L.ep_status_str.argtypes = [ctypes.c_int]
    L.ep_status_str.restype = ctypes.c_char_p
    L.ep_last_error.argtypes = []
    L.ep_last_error.restype = ctypes.c_char_p
    return L


lib = _load()


def status_str(st: int) -> str:
    return lib.ep_status_str(int(st)).decode()


def _check(st: int, where: str) -> None:
    if st != EP_OK:
        raise EpError(st, where)


def shape(T: int, H: int, E: int, R: int, k: int, fmt: int = EP_FMT_BF16) -> ep_shape_t:
    return ep_shape_t(T, H, E, R, k, fmt)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def ep_row_bytes(H: int, fmt: int) -> int:
    return int(lib.ep_row_bytes(H, fmt))


def ep_workspace_bytes(s: ep_shape_t) -> int:
    return int(lib.ep_workspace_bytes(ctypes.byref(s)))


def ep_dispatch_layout(s, topk_idx, num_tokens_per_rank, num_tokens_per_expert, rank_offset,
                       expert_offset, is_token_in_rank, send_slot, workspace, dev_status,
                       stream=None) -> None:
    st = lib.ep_dispatch_layout(ctypes.byref(s), _ptr(topk_idx), _ptr(num_tokens_per_rank),
                                _ptr(num_tokens_per_expert), _ptr(rank_offset),
                                _ptr(expert_offset), _ptr(is_token_in_rank), _ptr(send_slot),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _ptr(dev_status), _stream(stream))
    _check(st, "ep_dispatch_layout")


def ep_dispatch(s, x, topk_idx, topk_w, rank_offset, send_slot, send_buf, slot_src,
                slot_local_idx, slot_local_w, ring, workspace, dev_status, stream=None,
                capacity_rows: Optional[int] = None) -> None:
    cap = send_buf.shape[0] if capacity_rows is None else capacity_rows
    st = lib.ep_dispatch(ctypes.byref(s), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                         _ptr(rank_offset), _ptr(send_slot), _ptr(send_buf), cap,
                         _ptr(slot_src), _ptr(slot_local_idx), _ptr(slot_local_w),
                         ring.handle if ring is not None else None, _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _ptr(dev_status),
                         _stream(stream))
    _check(st, "ep_dispatch")


def ep_dispatch_fused(s, x, topk_idx, topk_w, num_tokens_per_rank, num_tokens_per_expert,
                      rank_offset, expert_offset, is_token_in_rank, send_slot, send_buf, slot_src,
                      slot_local_idx, slot_local_w, ring, workspace, dev_status, stream=None,
                      capacity_rows: Optional[int] = None) -> None:
    cap = send_buf.shape[0] if capacity_rows is None else capacity_rows
    st = lib.ep_dispatch_fused(ctypes.byref(s), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                               _ptr(num_tokens_per_rank), _ptr(num_tokens_per_expert),
                               _ptr(rank_offset), _ptr(expert_offset), _ptr(is_token_in_rank),
                               _ptr(send_slot), _ptr(send_buf), cap, _ptr(slot_src),
                               _ptr(slot_local_idx), _ptr(slot_local_w),
                               ring.handle if ring is not None else None, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(dev_status),
                               _stream(stream))
    _check(st, "ep_dispatch_fused")


def ep_dispatch_fused_plan(s, with_ring: bool = True) -> int:
    """EP_FUSED_ONE_KERNEL_SMALL, EP_FUSED_ONE_KERNEL_LARGE or
    EP_FUSED_TWO_CALLS: the path ep_dispatch_fused takes for shape s."""
    st = lib.ep_dispatch_fused_plan(ctypes.byref(s), 1 if with_ring else 0)
    if st not in (EP_FUSED_ONE_KERNEL_SMALL, EP_FUSED_ONE_KERNEL_LARGE, EP_FUSED_TWO_CALLS):
        _check(st, "ep_dispatch_fused_plan")
    return st


def ep_dispatch_fused_noalloc(s, x, topk_idx, topk_w, num_tokens_per_rank,
                              num_tokens_per_expert, rank_offset, expert_offset, is_token_in_rank,
                              send_slot, send_buf, slot_src, slot_local_idx, slot_local_w, ring,
                              dev_status, stream=None, capacity_rows: Optional[int] = None,
                              clear_scratch: bool = False) -> None:
    cap = send_buf.shape[0] if capacity_rows is None else capacity_rows
    st = lib.ep_dispatch_fused_noalloc(
        ctypes.byref(s), _ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(num_tokens_per_rank),
        _ptr(num_tokens_per_expert), _ptr(rank_offset), _ptr(expert_offset),
        _ptr(is_token_in_rank), _ptr(send_slot), _ptr(send_buf), cap, _ptr(slot_src),
        _ptr(slot_local_idx), _ptr(slot_local_w), ring.handle if ring is not None else None,
        1 if clear_scratch else 0, _ptr(dev_status), _stream(stream))
    _check(st, "ep_dispatch_fused_noalloc")


def ep_combine(s, y, topk_idx, topk_w, send_slot, out, dev_status, stream=None) -> None:
    st = lib.ep_combine(ctypes.byref(s), _ptr(y), y.shape[0], _ptr(topk_idx), _ptr(topk_w),
                        _ptr(send_slot), _ptr(out), _ptr(dev_status), _stream(stream))
    _check(st, "ep_combine")


def ep_dispatch_layout_ll(s, topk_idx, expert_offset, expert_slot, workspace, dev_status,
                          stream=None) -> None:
    st = lib.ep_dispatch_layout_ll(ctypes.byref(s), _ptr(topk_idx), _ptr(expert_offset),
                                   _ptr(expert_slot), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _ptr(dev_status), _stream(stream))
    _check(st, "ep_dispatch_layout_ll")


def ep_dispatch_ll_layout(s, topk_idx, num_tokens_per_expert, expert_offset, expert_slot,
                          workspace, dev_status, stream=None) -> None:
    st = lib.ep_dispatch_ll_layout(ctypes.byref(s), _ptr(topk_idx), _ptr(num_tokens_per_expert),
                                   _ptr(expert_offset), _ptr(expert_slot), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _ptr(dev_status), _stream(stream))
    _check(st, "ep_dispatch_ll_layout")


def ep_dispatch_ll(s, x, topk_idx, topk_w, expert_offset, expert_slot, send_buf, slot_src,
                   slot_w, ring, workspace, dev_status, stream=None,
                   capacity_rows: Optional[int] = None) -> None:
    cap = send_buf.shape[0] if capacity_rows is None else capacity_rows
    st = lib.ep_dispatch_ll(ctypes.byref(s), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                            _ptr(expert_offset), _ptr(expert_slot), _ptr(send_buf), cap,
                            _ptr(slot_src), _ptr(slot_w),
                            ring.handle if ring is not None else None, _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _ptr(dev_status),
                            _stream(stream))
    _check(st, "ep_dispatch_ll")


def ep_dispatch_ll_fused(s, x, topk_idx, topk_w, num_tokens_per_expert, expert_offset,
                         expert_slot, send_buf, slot_src, slot_w, ring, workspace, dev_status,
                         stream=None, capacity_rows: Optional[int] = None) -> None:
    cap = send_buf.shape[0] if capacity_rows is None else capacity_rows
    st = lib.ep_dispatch_ll_fused(ctypes.byref(s), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                                  _ptr(num_tokens_per_expert), _ptr(expert_offset),
                                  _ptr(expert_slot), _ptr(send_buf), cap, _ptr(slot_src),
                                  _ptr(slot_w), ring.handle if ring is not None else None,
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _ptr(dev_status), _stream(stream))
    _check(st, "ep_dispatch_ll_fused")


def ep_combine_ll(s, y, topk_idx, topk_w, expert_slot, out, dev_status, stream=None) -> None:
    st = lib.ep_combine_ll(ctypes.byref(s), _ptr(y), y.shape[0], _ptr(topk_idx), _ptr(topk_w),
                           _ptr(expert_slot), _ptr(out), _ptr(dev_status), _stream(stream))
    _check(st, "ep_combine_ll")


class Ring:
    """ep_ring_t: TransferCmd FIFO with `channels` channels of `depth` slots."""

    def __init__(self, depth: int = 1024, channels: int = 1, max_inflight: int = 256,
                 timeout_ns: int = 2_000_000_000):
        h = lib.ep_ring_create(depth, channels, max_inflight, timeout_ns)
        if not h:
            raise EpError(EP_ERR_INVALID_ARG, "ep_ring_create")
        self.handle = h
        self.depth, self.channels, self.max_inflight = depth, channels, max_inflight

    def destroy(self) -> None:
        if self.handle:
            _check(lib.ep_ring_destroy(self.handle), "ep_ring_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def reset(self) -> None:
        _check(lib.ep_ring_reset(self.handle), "ep_ring_reset")

    def drain(self, channel: int, max_n: int = 1 << 16) -> np.ndarray:
        out = np.zeros(max_n, CMD_DTYPE)
        n = ctypes.c_int32(0)
        _check(lib.ep_ring_drain(self.handle, channel, out.ctypes.data, max_n, ctypes.byref(n)),
               "ep_ring_drain")
        return out[:n.value]

    def proxy_start(self, threads: int = 4, log_capacity: int = 0) -> None:
        _check(lib.ep_ring_proxy_start(self.handle, threads, log_capacity), "ep_ring_proxy_start")

    def proxy_stop(self, log_max: int = 0):
        out = np.zeros(max(log_max, 0), CMD_DTYPE)
        nl, nd = ctypes.c_int64(0), ctypes.c_int64(0)
        _check(lib.ep_ring_proxy_stop(self.handle, out.ctypes.data if log_max > 0 else None,
                                      log_max, ctypes.byref(nl), ctypes.byref(nd)),
               "ep_ring_proxy_stop")
        return out[:min(nl.value, max(log_max, 0))], nd.value

    def set_loopback(self, src, dst_list, count_list) -> None:
        """Execute popped commands against local memory: src is the send
        buffer, dst_list / count_list one device tensor (or None) per rank."""
        if src is None:
            _check(lib.ep_ring_set_loopback(self.handle, None, 0, 0, None, None, None, None),
                   "ep_ring_set_loopback")
            self._lb_keep = None
            return
        R = len(dst_list)
        P = ctypes.c_void_p
        dst = (P * R)(*[_ptr(t) for t in dst_list])
        dsz = (ctypes.c_uint64 * R)(*[0 if t is None else t.numel() * t.element_size()
                                      for t in dst_list])
        cnt = (P * R)(*[_ptr(t) for t in count_list])
        csz = (ctypes.c_uint64 * R)(*[0 if t is None else t.numel() * t.element_size()
                                      for t in count_list])
        self._lb_keep = (src, list(dst_list), list(count_list))   # keep the memory alive
        _check(lib.ep_ring_set_loopback(self.handle, _ptr(src), src.numel() * src.element_size(),
                                        R, dst, dsz, cnt, csz), "ep_ring_set_loopback")

    def completed(self, channel: int) -> int:
        return int(lib.ep_ring_completed(self.handle, channel))

    def check_completion(self, channels, tickets, done, stream=None) -> None:
        """ep_ring_check_completion: device tensors channels (int32), tickets
        (uint64 as int64) and done (uint8), all of length n."""
        _check(lib.ep_ring_check_completion(self.handle, _ptr(channels), _ptr(tickets),
                                            int(done.numel()), _ptr(done), _stream(stream)),
               "ep_ring_check_completion")

    def wait_complete(self, timeout_ns: int = 10_000_000_000) -> None:
        _check(lib.ep_ring_wait_complete(self.handle, timeout_ns), "ep_ring_wait_complete")

    def loopback_stats(self) -> dict:
        n, e, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        mean, mx = ctypes.c_double(), ctypes.c_double()
        _check(lib.ep_ring_loopback_stats(self.handle, ctypes.byref(n), ctypes.byref(e),
                                          ctypes.byref(c), ctypes.byref(mean), ctypes.byref(mx)),
               "ep_ring_loopback_stats")
        return {"completed": n.value, "errors": e.value, "copies": c.value,
                "mean_latency_us": mean.value, "max_latency_us": mx.value}

    def proxy_drained(self) -> int:
        return int(lib.ep_ring_proxy_drained(self.handle))


class Buffers:
    """Device buffers of one dispatch/combine pass for shape ``s`` (plumbing:
    torch allocations sized from the shape; nothing here computes)."""

    def __init__(self, s: ep_shape_t, capacity_rows: Optional[int] = None, device="cuda"):
        import torch
        T, H, E, R, k = s.T, s.H, s.E, s.R, s.k
        cap = T * min(k, R) if capacity_rows is None else capacity_rows
        rb = ep_row_bytes(H, s.fmt)
        i32 = dict(dtype=torch.int32, device=device)
        self.shape = s
        self.capacity_rows = cap
        self.row_bytes = rb
        self.num_tokens_per_rank = torch.empty(R, **i32)
        self.num_tokens_per_expert = torch.empty(E, **i32)
        self.rank_offset = torch.empty(R + 1, **i32)
        self.expert_offset = torch.empty(E + 1, **i32)
        self.is_token_in_rank = torch.empty((T, R), dtype=torch.uint8, device=device)
        self.send_slot = torch.empty((T, R), **i32)
        self.send_buf = torch.empty((cap, rb), dtype=torch.uint8, device=device)
        self.slot_src = torch.empty(cap, **i32)
        self.slot_local_idx = torch.empty((cap, k), **i32)
        self.slot_local_w = torch.empty((cap, k), dtype=torch.float32, device=device)
        # zero-filled once; the library keeps it consistent afterwards
        self.workspace = torch.zeros(max(ep_workspace_bytes(s), 256), dtype=torch.uint8,
                                     device=device)
        self.dev_status = torch.zeros(1, **i32)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=device)

    def layout(self, topk_idx, stream=None):
        ep_dispatch_layout(self.shape, topk_idx, self.num_tokens_per_rank,
                           self.num_tokens_per_expert, self.rank_offset, self.expert_offset,
                           self.is_token_in_rank, self.send_slot, self.workspace,
                           self.dev_status, stream)

    def dispatch(self, x, topk_idx, topk_w, ring=None, stream=None):
        ep_dispatch(self.shape, x, topk_idx, topk_w, self.rank_offset, self.send_slot,
                    self.send_buf, self.slot_src, self.slot_local_idx, self.slot_local_w, ring,
                    self.workspace, self.dev_status, stream)

    def dispatch_fused(self, x, topk_idx, topk_w, ring=None, stream=None):
        """layout + dispatch in one call (one kernel for T <= 256)"""
        ep_dispatch_fused(self.shape, x, topk_idx, topk_w, self.num_tokens_per_rank,
                          self.num_tokens_per_expert, self.rank_offset, self.expert_offset,
                          self.is_token_in_rank, self.send_slot, self.send_buf, self.slot_src,
                          self.slot_local_idx, self.slot_local_w, ring, self.workspace,
                          self.dev_status, stream)

    def dispatch_fused_noalloc(self, x, topk_idx, topk_w, ring=None, stream=None,
                               clear_scratch=False):
        """layout + dispatch in one call on the library's own device scratch
        (no workspace; the buffers' own workspace is not used)"""
        ep_dispatch_fused_noalloc(self.shape, x, topk_idx, topk_w, self.num_tokens_per_rank,
                                  self.num_tokens_per_expert, self.rank_offset,
                                  self.expert_offset, self.is_token_in_rank, self.send_slot,
                                  self.send_buf, self.slot_src, self.slot_local_idx,
                                  self.slot_local_w, ring, self.dev_status, stream,
                                  clear_scratch=clear_scratch)

    def combine(self, y, topk_idx, topk_w, stream=None):
        ep_combine(self.shape, y, topk_idx, topk_w, self.send_slot, self.out, self.dev_status,
                   stream)


class BuffersLL(Buffers):
    """Buffers of one per-expert (low-latency) pass: the rank layout's
    buffers (its counts, offsets and workspace are reused) plus the per-expert
    rows, metadata and row table.  Capacity defaults to T*k rows."""

    def __init__(self, s: ep_shape_t, capacity_rows: Optional[int] = None, device="cuda"):
        import torch
        super().__init__(s, capacity_rows=0, device=device)
        T, k = s.T, s.k
        cap = T * k if capacity_rows is None else capacity_rows
        self.capacity_rows = cap
        self.expert_slot = torch.empty((T, k), dtype=torch.int32, device=device)
        self.send_buf = torch.empty((cap, self.row_bytes), dtype=torch.uint8, device=device)
        self.slot_src = torch.empty(cap, dtype=torch.int32, device=device)
        self.slot_w = torch.empty(cap, dtype=torch.float32, device=device)

    def layout(self, topk_idx, stream=None):
        super().layout(topk_idx, stream)
        ep_dispatch_layout_ll(self.shape, topk_idx, self.expert_offset, self.expert_slot,
                              self.workspace, self.dev_status, stream)

    def layout_one_call(self, topk_idx, stream=None):
        """the per-expert layout in one kernel (ep_dispatch_ll_layout; E <=
        1024); the rank-layout buffers are left untouched"""
        ep_dispatch_ll_layout(self.shape, topk_idx, self.num_tokens_per_expert,
                              self.expert_offset, self.expert_slot, self.workspace,
                              self.dev_status, stream)

    def dispatch(self, x, topk_idx, topk_w, ring=None, stream=None):
        ep_dispatch_ll(self.shape, x, topk_idx, topk_w, self.expert_offset, self.expert_slot,
                       self.send_buf, self.slot_src, self.slot_w, ring, self.workspace,
                       self.dev_status, stream)

    def dispatch_fused(self, x, topk_idx, topk_w, ring=None, stream=None):
        """per-expert layout, row table and pack in one kernel (T <= 256,
        E <= 1024); the rank-layout buffers are left untouched"""
        ep_dispatch_ll_fused(self.shape, x, topk_idx, topk_w, self.num_tokens_per_expert,
                             self.expert_offset, self.expert_slot, self.send_buf, self.slot_src,
                             self.slot_w, ring, self.workspace, self.dev_status, stream)

    def combine(self, y, topk_idx, topk_w, stream=None):
        ep_combine_ll(self.shape, y, topk_idx, topk_w, self.expert_slot, self.out,
                      self.dev_status, stream)
