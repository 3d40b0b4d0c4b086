"""Python binding of libep_layout.so: MoE expert-parallel dispatch/combine on
one MI355X (gfx950).

Argument marshalling only: every step of layout, dispatch and combine runs in
the library's HIP kernels.  PyTorch provides device memory and streams; the
library is loaded after torch so that both share torch's HIP runtime.  Import
fails loudly when the library has not been built (``python
combine_ep_layout_amd/build.py``).

The names follow the C ABI in include/ep_layout.h (ep_handle_create,
ep_layout, ep_dispatch, ep_combine, ...); ``EpHandle`` bundles them.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libep_layout.so")

EP_OK = 0
EP_ERR_INVALID_ARGUMENT = 1
EP_ERR_UNSUPPORTED = 2
EP_ERR_OUT_OF_MEMORY = 3
EP_ERR_HANDLE_STATE = 4
EP_ERR_BAD_ROUTING = 5
EP_ERR_TIMEOUT = 6
EP_ERR_HIP = 7

EP_DISPATCH_FP8 = 1 << 0
EP_DISPATCH_TILE_READY = 1 << 1
EP_DISPATCH_BORROW = 1 << 2
EP_CONSUME_GATHER = 1 << 3
EP_SCALE_F32 = 1 << 4
EP_SCALE_ROUND = 1 << 5
EP_SCALE_MN_MAJOR = 1 << 6
EP_CONSUME_SIGNAL_DONE = 1 << 7
EP_CONSUME_STAMPS = 1 << 8

# scale flavours by name: flags, element dtype
SCALE_KINDS = {
    "ue8m0": (0, torch.uint8),
    "f32": (EP_SCALE_F32, torch.float32),
    "pow2_f32": (EP_SCALE_F32 | EP_SCALE_ROUND, torch.float32),
}

ARRAYS = {
    "expert_counts": (0, torch.int32),
    "expert_pool_block_offset": (1, torch.int32),
    "num_tiles": (2, torch.int32),
    "tile_expert": (3, torch.int32),
    "pool_arrival_target": (4, torch.int32),
    "pool_arrival_count": (5, torch.int32),
    "tile_ready": (6, torch.int32),
    "slot_to_pool_row": (7, torch.int32),
    "pool_recv_token": (8, torch.int32),
    "topk_weights": (9, torch.float32),
    "y_done_per_token": (10, torch.int32),
    "tile_stamp": (11, torch.int64),
}

EXPORTS = [
    "ep_handle_create", "ep_handle_destroy", "ep_pool_capacity_rows", "ep_max_tiles",
    "ep_num_tokens", "ep_layout", "ep_dispatch", "ep_combine", "ep_handle_get_view",
    "ep_array_bytes", "ep_copy_array", "ep_counts_to_host", "ep_handle_sync_status",
    "ep_tile_consume", "ep_status_string", "ep_borrow_release", "ep_combine_backward",
    "ep_dispatch_backward", "ep_combine_gated", "ep_fp8_cast_back", "ep_scale_ld",
    "ep_layout_noalloc", "ep_set_density_hint", "ep_layout_density", "ep_layout_dispatch",
]

EP_DENSITY_AUTO = 0
EP_DENSITY_SPARSE = 1
EP_DENSITY_DENSE = 2


class EpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.ep_status_string(status).decode()} (status {status})")


class _Config(ctypes.Structure):
    _fields_ = [("max_tokens", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("block_m", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          f"'python combine_ep_layout_amd/build.py' (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64
    st = ctypes.c_int
    sig = {
        "ep_handle_create": (st, [ctypes.POINTER(_Config), ctypes.POINTER(P)]),
        "ep_handle_destroy": (st, [P]),
        "ep_pool_capacity_rows": (I64, [P]),
        "ep_max_tiles": (I32, [P]),
        "ep_num_tokens": (I32, [P]),
        "ep_layout": (st, [P, P, P, I32, P, ctypes.POINTER(U32)]),
        "ep_dispatch": (st, [P, P, I32, P, P, U32, P, ctypes.POINTER(U32)]),
        "ep_layout_dispatch": (st, [P, P, P, I32, P, I32, P, P, U32, P, ctypes.POINTER(U32),
                                    ctypes.POINTER(U32)]),
        "ep_combine": (st, [P, U32, P, I32, P, P]),
        "ep_handle_get_view": (st, [P, P]),
        "ep_array_bytes": (I64, [P, ctypes.c_int]),
        "ep_copy_array": (st, [P, ctypes.c_int, P, I64, P]),
        "ep_counts_to_host": (st, [P, P, P, P]),
        "ep_handle_sync_status": (st, [P, P]),
        "ep_tile_consume": (st, [P, U32, P, P, I32, U32, P, I32, U32, P]),
        "ep_status_string": (ctypes.c_char_p, [st]),
        "ep_borrow_release": (st, [P, P]),
        "ep_combine_backward": (st, [P, U32, P, P, I32, P, P, P]),
        "ep_dispatch_backward": (st, [P, U32, P, I32, P, P]),
        "ep_combine_gated": (st, [P, U32, P, I32, P, U32, U32, P]),
        "ep_fp8_cast_back": (st, [P, P, U32, I64, I64, I32, P, P]),
        "ep_scale_ld": (I64, [P]),
        "ep_layout_noalloc": (st, [P, I32, I32, I32, I32, I64, P, P, P, P, P, P, P, P, P]),
        "ep_set_density_hint": (st, [P, I32]),
        "ep_layout_density": (I32, [P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != EP_OK:
        raise EpError(status, where)


def _require(t: torch.Tensor, dtype, name: str, device: torch.device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


# --------------------------------------------------- functions of the C ABI --

def ep_handle_create(max_tokens: int, top_k: int, num_experts: int, block_m: int) -> ctypes.c_void_p:
    cfg = _Config(max_tokens, top_k, num_experts, block_m)
    h = ctypes.c_void_p()
    _check(_lib.ep_handle_create(ctypes.byref(cfg), ctypes.byref(h)), "ep_handle_create")
    return h


def ep_handle_destroy(h) -> None:
    _check(_lib.ep_handle_destroy(h), "ep_handle_destroy")


def ep_layout(h, topk_idx: torch.Tensor, topk_weights: torch.Tensor, stream=None) -> int:
    epoch = ctypes.c_uint32()
    T = topk_idx.shape[0]
    _check(_lib.ep_layout(h, _ptr(topk_idx), _ptr(topk_weights), T, _stream(stream),
                          ctypes.byref(epoch)), "ep_layout")
    return epoch.value


def ep_dispatch(h, x: torch.Tensor, pool: torch.Tensor, pool_scales: Optional[torch.Tensor],
                flags: int, stream=None) -> int:
    seq = ctypes.c_uint32()
    _check(_lib.ep_dispatch(h, _ptr(x), x.shape[1], _ptr(pool), _ptr(pool_scales), flags,
                            _stream(stream), ctypes.byref(seq)), "ep_dispatch")
    return seq.value


def ep_layout_dispatch(h, topk_idx: torch.Tensor, topk_weights: torch.Tensor, x: torch.Tensor,
                       pool: torch.Tensor, pool_scales: Optional[torch.Tensor], flags: int,
                       stream=None) -> tuple:
    epoch = ctypes.c_uint32()
    seq = ctypes.c_uint32()
    _check(_lib.ep_layout_dispatch(h, _ptr(topk_idx), _ptr(topk_weights), topk_idx.shape[0], _ptr(x),
                                   x.shape[1], _ptr(pool), _ptr(pool_scales), flags, _stream(stream),
                                   ctypes.byref(epoch), ctypes.byref(seq)), "ep_layout_dispatch")
    return epoch.value, seq.value


def ep_combine(h, epoch: int, expert_out: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    _check(_lib.ep_combine(h, epoch, _ptr(expert_out), expert_out.shape[1], _ptr(y),
                           _stream(stream)), "ep_combine")


def ep_combine_gated(h, epoch: int, expert_out: torch.Tensor, y: torch.Tensor, round: int,
                     spin_limit_us: int, stream=None) -> None:
    _check(_lib.ep_combine_gated(h, epoch, _ptr(expert_out), expert_out.shape[1], _ptr(y), round,
                                 spin_limit_us, _stream(stream)), "ep_combine_gated")


def ep_fp8_cast_back(q: torch.Tensor, scales: torch.Tensor, flags: int, rows: int, scale_ld: int,
                     out: torch.Tensor, stream=None) -> None:
    _check(_lib.ep_fp8_cast_back(_ptr(q), _ptr(scales), flags, rows, scale_ld, q.shape[1], _ptr(out),
                                 _stream(stream)), "ep_fp8_cast_back")


def scale_shape(rows: int, hidden: int, kind: str, mn_major: bool, ld: Optional[int] = None):
    """Shape and dtype of a scale array for `rows` pool rows."""
    _, dtype = SCALE_KINDS[kind]
    G = hidden // 128
    if not mn_major:
        return (rows, G), dtype
    ld = rows if ld is None else ld
    if kind == "ue8m0":
        return ((G + 3) // 4, ld), torch.int32      # packed words
    return (G, ld), dtype


def scale_flags(kind: str, mn_major: bool) -> int:
    return SCALE_KINDS[kind][0] | (EP_SCALE_MN_MAJOR if mn_major else 0)


def cast_back(q: torch.Tensor, scales: torch.Tensor, kind: str = "ue8m0", mn_major: bool = False,
              rows: Optional[int] = None, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """per_token_cast_back: bf16 [rows, H] from e4m3fn codes and their scales."""
    if q.dtype != torch.uint8 or not q.is_contiguous() or q.dim() != 2:
        raise TypeError("q must be a contiguous uint8 [rows, hidden] tensor")
    rows = q.shape[0] if rows is None else int(rows)
    H = q.shape[1]
    if rows > q.shape[0]:
        raise ValueError("rows exceeds q")
    shape, dtype = scale_shape(rows, H, kind, mn_major, scales.shape[1] if mn_major else None)
    if mn_major:      # [groups or words, ld >= rows]
        ok = scales.dim() == 2 and scales.shape[0] == shape[0] and scales.shape[1] >= rows
    else:             # [>= rows, groups]
        ok = scales.dim() == 2 and scales.shape[0] >= rows and scales.shape[1] == shape[1]
    if scales.dtype != dtype or not scales.is_contiguous() or not ok:
        raise ValueError(f"scales must be {dtype} {shape}")
    if out is None:
        out = torch.empty(rows, H, dtype=torch.bfloat16, device=q.device)
    if out.dtype != torch.bfloat16 or not out.is_contiguous() or out.shape[0] < rows or out.shape[1] != H:
        raise ValueError("out must be bf16 [rows, hidden]")
    ld = scales.shape[1] if mn_major else 0
    ep_fp8_cast_back(q, scales, scale_flags(kind, mn_major), rows, ld, out, stream)
    return out


def ep_tile_consume(h, seq: int, pool: torch.Tensor, pool_scales: Optional[torch.Tensor],
                    hidden: int, flags: int, out: torch.Tensor, workgroups: int,
                    spin_limit_us: int, stream=None) -> None:
    _check(_lib.ep_tile_consume(h, seq, _ptr(pool), _ptr(pool_scales), hidden, flags, _ptr(out),
                                workgroups, spin_limit_us, _stream(stream)), "ep_tile_consume")


def ep_combine_backward(h, epoch: int, grad_y: torch.Tensor, expert_out: torch.Tensor,
                        grad_expert_out: torch.Tensor, grad_weights: torch.Tensor,
                        stream=None) -> None:
    _check(_lib.ep_combine_backward(h, epoch, _ptr(grad_y), _ptr(expert_out), grad_y.shape[1],
                                    _ptr(grad_expert_out), _ptr(grad_weights), _stream(stream)),
           "ep_combine_backward")


def ep_dispatch_backward(h, epoch: int, grad_pool: torch.Tensor, grad_x: torch.Tensor,
                         stream=None) -> None:
    _check(_lib.ep_dispatch_backward(h, epoch, _ptr(grad_pool), grad_pool.shape[1], _ptr(grad_x),
                                     _stream(stream)), "ep_dispatch_backward")


def ep_borrow_release(h, consumer_stream=None) -> None:
    _check(_lib.ep_borrow_release(h, _stream(consumer_stream)), "ep_borrow_release")


def ep_handle_sync_status(h, stream=None) -> int:
    return int(_lib.ep_handle_sync_status(h, _stream(stream)))


# ------------------------------------------------------------- convenience --

class EpHandle:
    """One layout's metadata on the current device (owns an ep_handle)."""

    def __init__(self, max_tokens: int, top_k: int, num_experts: int, block_m: int):
        self.max_tokens, self.top_k = int(max_tokens), int(top_k)
        self.num_experts, self.block_m = int(num_experts), int(block_m)
        self.device = torch.device("cuda", torch.cuda.current_device())
        self._h = ep_handle_create(max_tokens, top_k, num_experts, block_m)
        self.capacity_rows = int(_lib.ep_pool_capacity_rows(self._h))
        self.max_tiles = int(_lib.ep_max_tiles(self._h))
        self.scale_ld = int(_lib.ep_scale_ld(self._h))

    @property
    def raw(self):
        return self._h

    @property
    def num_tokens(self) -> int:
        return int(_lib.ep_num_tokens(self._h))

    def close(self):
        if self._h is not None and self._h.value:
            ep_handle_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def layout(self, topk_idx: torch.Tensor, topk_weights: torch.Tensor, stream=None) -> int:
        _require(topk_idx, torch.int32, "topk_idx", self.device)
        _require(topk_weights, torch.float32, "topk_weights", self.device)
        if topk_idx.dim() != 2 or topk_idx.shape[1] != self.top_k or topk_weights.shape != topk_idx.shape:
            raise ValueError("topk_idx / topk_weights must both be [num_tokens, top_k]")
        return ep_layout(self._h, topk_idx, topk_weights, stream)

    def scale_shape(self, hidden: int, kind: str = "ue8m0", mn_major: bool = False):
        return scale_shape(self.capacity_rows, hidden, kind, mn_major, self.scale_ld)

    def new_pool(self, hidden: int, fp8: bool = False, scale_kind: str = "ue8m0",
                 mn_major: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
        if fp8:
            shape, dtype = self.scale_shape(hidden, scale_kind, mn_major)
            return (torch.empty(self.capacity_rows, hidden, dtype=torch.uint8, device=self.device),
                    torch.empty(shape, dtype=dtype, device=self.device))
        return torch.empty(self.capacity_rows, hidden, dtype=torch.bfloat16, device=self.device), None

    def dispatch(self, x: torch.Tensor, pool: torch.Tensor, pool_scales: Optional[torch.Tensor] = None,
                 fp8: bool = False, tile_ready: bool = False, stream=None,
                 scale_kind: str = "ue8m0", mn_major: bool = False) -> int:
        _require(x, torch.bfloat16, "x", self.device)
        if x.dim() != 2 or x.shape[0] != self.num_tokens:
            raise ValueError("x must be [num_tokens of the layout, hidden]")
        H = x.shape[1]
        if pool.shape[0] < self.capacity_rows or pool.shape[1] != H:
            raise ValueError(f"pool must be at least [{self.capacity_rows}, {H}]")
        _require(pool, torch.uint8 if fp8 else torch.bfloat16, "pool", self.device)
        if fp8:
            shape, dtype = self.scale_shape(H, scale_kind, mn_major)
            if pool_scales is None or tuple(pool_scales.shape) != shape:
                raise ValueError(f"pool_scales must be {shape}")
            _require(pool_scales, dtype, "pool_scales", self.device)
        elif scale_kind != "ue8m0" or mn_major:
            raise ValueError("scale flavours apply to FP8 dispatch only")
        flags = (EP_DISPATCH_FP8 | scale_flags(scale_kind, mn_major) if fp8 else 0) | \
                (EP_DISPATCH_TILE_READY if tile_ready else 0)
        return ep_dispatch(self._h, x, pool, pool_scales if fp8 else None, flags, stream)

    def layout_dispatch(self, topk_idx: torch.Tensor, topk_weights: torch.Tensor, x: torch.Tensor,
                        pool: torch.Tensor, pool_scales: Optional[torch.Tensor] = None, fp8: bool = False,
                        stream=None, scale_kind: str = "ue8m0", mn_major: bool = False) -> tuple:
        """layout() and dispatch() in one call (one kernel launch for batches
        of at most 2048 slots); returns (epoch, dispatch sequence number)."""
        _require(topk_idx, torch.int32, "topk_idx", self.device)
        _require(topk_weights, torch.float32, "topk_weights", self.device)
        if topk_idx.dim() != 2 or topk_idx.shape[1] != self.top_k or topk_weights.shape != topk_idx.shape:
            raise ValueError("topk_idx / topk_weights must both be [num_tokens, top_k]")
        _require(x, torch.bfloat16, "x", self.device)
        if x.dim() != 2 or x.shape[0] != topk_idx.shape[0]:
            raise ValueError("x must be [num_tokens, hidden]")
        H = x.shape[1]
        if pool.shape[0] < self.capacity_rows or pool.shape[1] != H:
            raise ValueError(f"pool must be at least [{self.capacity_rows}, {H}]")
        _require(pool, torch.uint8 if fp8 else torch.bfloat16, "pool", self.device)
        if fp8:
            shape, dtype = self.scale_shape(H, scale_kind, mn_major)
            if pool_scales is None or tuple(pool_scales.shape) != shape:
                raise ValueError(f"pool_scales must be {shape}")
            _require(pool_scales, dtype, "pool_scales", self.device)
        elif scale_kind != "ue8m0" or mn_major:
            raise ValueError("scale flavours apply to FP8 dispatch only")
        flags = EP_DISPATCH_FP8 | scale_flags(scale_kind, mn_major) if fp8 else 0
        return ep_layout_dispatch(self._h, topk_idx, topk_weights, x, pool, pool_scales if fp8 else None,
                                  flags, stream)

    def combine_backward(self, epoch: int, grad_y: torch.Tensor, expert_out: torch.Tensor,
                         grad_expert_out: Optional[torch.Tensor] = None, stream=None):
        """Returns (grad_expert_out [capacity_rows, H] bf16, grad_weights [T, K] fp32)."""
        _require(grad_y, torch.bfloat16, "grad_y", self.device)
        _require(expert_out, torch.bfloat16, "expert_out", self.device)
        H = grad_y.shape[1]
        if grad_y.shape[0] != self.num_tokens or expert_out.shape[0] < self.capacity_rows \
                or expert_out.shape[1] != H:
            raise ValueError("grad_y must be [num_tokens, H], expert_out [capacity_rows, H]")
        if grad_expert_out is None:
            grad_expert_out = torch.empty(self.capacity_rows, H, dtype=torch.bfloat16, device=self.device)
        _require(grad_expert_out, torch.bfloat16, "grad_expert_out", self.device)
        if grad_expert_out.shape[0] < self.capacity_rows or grad_expert_out.shape[1] != H:
            raise ValueError("grad_expert_out must be at least [capacity_rows, H]")
        grad_w = torch.empty(self.num_tokens, self.top_k, dtype=torch.float32, device=self.device)
        ep_combine_backward(self._h, epoch, grad_y, expert_out, grad_expert_out, grad_w, stream)
        return grad_expert_out, grad_w

    def dispatch_backward(self, epoch: int, grad_pool: torch.Tensor,
                          grad_x: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        _require(grad_pool, torch.bfloat16, "grad_pool", self.device)
        H = grad_pool.shape[1]
        if grad_pool.shape[0] < self.capacity_rows:
            raise ValueError("grad_pool must have at least capacity_rows rows")
        if grad_x is None:
            grad_x = torch.empty(self.num_tokens, H, dtype=torch.bfloat16, device=self.device)
        _require(grad_x, torch.bfloat16, "grad_x", self.device)
        if grad_x.shape != (self.num_tokens, H):
            raise ValueError("grad_x must be [num_tokens, H]")
        ep_dispatch_backward(self._h, epoch, grad_pool, grad_x, stream)
        return grad_x

    def borrow(self, x: torch.Tensor, stream=None) -> int:
        """Dispatch without a copy: lend x through the row map
        (pool_recv_token).  Holds the handle's lease until release()."""
        _require(x, torch.bfloat16, "x", self.device)
        if x.dim() != 2 or x.shape[0] != self.num_tokens:
            raise ValueError("x must be [num_tokens of the layout, hidden]")
        return ep_dispatch(self._h, x, None, None, EP_DISPATCH_BORROW, stream)

    def release(self, consumer_stream=None) -> None:
        ep_borrow_release(self._h, consumer_stream)

    def combine(self, epoch: int, expert_out: torch.Tensor, y: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
        _require(expert_out, torch.bfloat16, "expert_out", self.device)
        H = expert_out.shape[1]
        if expert_out.shape[0] < self.capacity_rows:
            raise ValueError(f"expert_out must have at least {self.capacity_rows} rows")
        if y is None:
            y = torch.empty(max(self.num_tokens, 0), H, dtype=torch.bfloat16, device=self.device)
        _require(y, torch.bfloat16, "y", self.device)
        if y.shape != (self.num_tokens, H):
            raise ValueError("y must be [num_tokens of the layout, hidden]")
        ep_combine(self._h, epoch, expert_out, y, stream)
        return y

    def combine_gated(self, epoch: int, expert_out: torch.Tensor, round: int = 1,
                      y: Optional[torch.Tensor] = None, spin_limit_us: int = 2_000_000,
                      stream=None) -> torch.Tensor:
        """combine behind the per-token gate: token t waits until
        y_done_per_token[t] >= round * (its unmasked slots)."""
        _require(expert_out, torch.bfloat16, "expert_out", self.device)
        H = expert_out.shape[1]
        if expert_out.shape[0] < self.capacity_rows:
            raise ValueError(f"expert_out must have at least {self.capacity_rows} rows")
        if y is None:
            y = torch.empty(max(self.num_tokens, 0), H, dtype=torch.bfloat16, device=self.device)
        _require(y, torch.bfloat16, "y", self.device)
        if y.shape != (self.num_tokens, H):
            raise ValueError("y must be [num_tokens of the layout, hidden]")
        ep_combine_gated(self._h, epoch, expert_out, y, round, spin_limit_us, stream)
        return y

    def tile_consume(self, seq: int, pool: torch.Tensor, pool_scales: Optional[torch.Tensor],
                     hidden: int, out: torch.Tensor, fp8: bool = False, workgroups: int = 32,
                     spin_limit_us: int = 2_000_000, stream=None, gather: bool = False,
                     signal_done: bool = False, scale_kind: str = "ue8m0",
                     mn_major: bool = False, stamps: bool = False) -> None:
        _require(out, torch.bfloat16, "out", self.device)
        if out.shape[0] < self.capacity_rows or out.shape[1] != hidden:
            raise ValueError("out must be at least [capacity_rows, hidden]")
        if gather:
            # pool is the borrowed slab x [num_tokens, hidden]
            _require(pool, torch.bfloat16, "slab", self.device)
            if pool.shape != (self.num_tokens, hidden):
                raise ValueError("the gathered slab must be [num_tokens, hidden]")
        elif pool.shape[0] < self.capacity_rows:
            raise ValueError("pool must have at least capacity_rows rows")
        if not fp8 and (scale_kind != "ue8m0" or mn_major):
            raise ValueError("scale flavours apply to FP8 pools only")
        flags = (EP_DISPATCH_FP8 | scale_flags(scale_kind, mn_major) if fp8 else 0) | \
                (EP_CONSUME_GATHER if gather else 0) | (EP_CONSUME_SIGNAL_DONE if signal_done else 0) | \
                (EP_CONSUME_STAMPS if stamps else 0)
        ep_tile_consume(self._h, seq, pool, pool_scales if fp8 else None, hidden, flags, out,
                        workgroups, spin_limit_us, stream)

    def array(self, name: str, stream=None) -> torch.Tensor:
        """Device copy of one metadata array (see ARRAYS)."""
        which, dtype = ARRAYS[name]
        nbytes = int(_lib.ep_array_bytes(self._h, which))
        out = torch.empty(nbytes // dtype.itemsize, dtype=dtype, device=self.device)
        _check(_lib.ep_copy_array(self._h, which, _ptr(out), nbytes, _stream(stream)), "ep_copy_array")
        return out

    def counts_to_host(self, stream=None) -> Tuple[np.ndarray, int]:
        counts = np.empty(self.num_experts, np.int32)
        nt = np.zeros(1, np.int32)
        _check(_lib.ep_counts_to_host(self._h, counts.ctypes.data_as(ctypes.c_void_p),
                                      nt.ctypes.data_as(ctypes.c_void_p), _stream(stream)),
               "ep_counts_to_host")
        return counts, int(nt[0])

    def set_density_hint(self, hint: int) -> None:
        """EP_DENSITY_AUTO / _SPARSE / _DENSE: launch shape of the combine calls (forward
        and both backward calls) and of the bf16 dispatch of at least 64 MiB of x."""
        _check(_lib.ep_set_density_hint(self._h, int(hint)), "ep_set_density_hint")

    def layout_density(self, stream=None) -> int:
        """The density the current layout reported (EP_DENSITY_SPARSE / _DENSE)."""
        return int(_lib.ep_layout_density(self._h, _stream(stream)))

    def sync_status(self, stream=None) -> int:
        return ep_handle_sync_status(self._h, stream)
