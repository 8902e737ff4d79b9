"""Thin ctypes binding over libmoe_dispatch.so.

Argument marshalling only: every step of routing, dispatch and combine runs in
the library's HIP kernels.  torch supplies device memory and the stream.  The
names and arguments follow the C ABI in include/moe_dispatch.h.  Importing this
module loads the library and raises ImportError when it has not been built
(``python -m combine_moe_dispatch_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_dispatch.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m combine_moe_dispatch_amd.build` (hipcc, gfx950)")
_lib = ctypes.CDLL(LIB_PATH)

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, 1, 2, 3
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_PAYLOAD_BF16, MOE_PAYLOAD_FP8_E4M3_B128 = 0, 1
MOE_DEV_CAPACITY, MOE_DEV_BAD_ID = 1, 2
MOE_MAX_EXPERTS, MOE_MAX_TOP_K = 1024, 32


class _Shape(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("num_ranks", ctypes.c_int32), ("rank_capacity", ctypes.c_int32),
                ("payload", ctypes.c_int32)]


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "expert_counts", "expert_offsets", "rank_counts", "rank_offsets",
        "token_row", "row_src", "status")]


_vp, _i32 = ctypes.c_void_p, ctypes.c_int32
_lib.moe_recv_rows.argtypes = [ctypes.POINTER(_Shape)]
_lib.moe_recv_rows.restype = ctypes.c_int64
_lib.moe_dispatch_workspace_size.argtypes = [ctypes.POINTER(_Shape)]
_lib.moe_dispatch_workspace_size.restype = ctypes.c_size_t
_lib.moe_route_topk.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
_lib.moe_route_topk.restype = _i32
_lib.moe_route_topk_grouped.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
_lib.moe_route_topk_grouped.restype = _i32
_lib.moe_dispatch.argtypes = [ctypes.POINTER(_Shape), _vp, _vp, _vp, _vp,
                              ctypes.POINTER(_Layout), _vp, ctypes.c_size_t, _vp]
_lib.moe_dispatch.restype = _i32
_lib.moe_expert_scale.argtypes = [ctypes.POINTER(_Shape), _vp, _vp, ctypes.POINTER(_Layout),
                                  _vp, _vp, _vp, _vp]
_lib.moe_expert_scale.restype = _i32
_lib.moe_combine.argtypes = [ctypes.POINTER(_Shape), _vp, _vp, ctypes.POINTER(_Layout),
                             _vp, _vp, _vp]
_lib.moe_combine.restype = _i32
_lib.moe_status_string.argtypes = [_i32]
_lib.moe_status_string.restype = ctypes.c_char_p


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {_lib.moe_status_string(status).decode()}")


def _check(status: int, call: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, call)


@dataclasses.dataclass(frozen=True)
class Shape:
    """Sizes of one problem (mirrors moe_shape)."""
    num_tokens: int
    hidden: int
    num_experts: int
    top_k: int
    num_ranks: int
    rank_capacity: int   # 0 = packed regions
    payload: int = MOE_PAYLOAD_BF16

    def c(self) -> _Shape:
        return _Shape(self.num_tokens, self.hidden, self.num_experts, self.top_k,
                      self.num_ranks, self.rank_capacity, self.payload)

    @property
    def fp8(self) -> bool:
        return self.payload == MOE_PAYLOAD_FP8_E4M3_B128


@dataclasses.dataclass
class Layout:
    """Device metadata tensors (mirrors moe_layout); row_src may be None."""
    expert_counts: torch.Tensor
    expert_offsets: torch.Tensor
    rank_counts: torch.Tensor
    rank_offsets: torch.Tensor
    token_row: torch.Tensor
    row_src: Optional[torch.Tensor]
    status: torch.Tensor

    def c(self) -> _Layout:
        p = lambda t: None if t is None else t.data_ptr()
        return _Layout(p(self.expert_counts), p(self.expert_offsets), p(self.rank_counts),
                       p(self.rank_offsets), p(self.token_row), p(self.row_src), p(self.status))

    @staticmethod
    def empty(shape: Shape, device, with_row_src: bool = False) -> "Layout":
        i = dict(dtype=torch.int32, device=device)
        rows = moe_recv_rows(shape)
        return Layout(torch.empty(shape.num_experts, **i), torch.empty(shape.num_experts, **i),
                      torch.empty(shape.num_ranks, **i), torch.empty(shape.num_ranks, **i),
                      torch.empty(shape.num_tokens, shape.top_k, **i),
                      torch.full((rows,), -1, **i) if with_row_src else None,
                      torch.zeros(1, **i))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


# ---------------------------------------------------------------------------
# Argument checks made before each C call: every tensor must be a contiguous
# GPU tensor of the expected element type holding at least the elements the
# shape addresses (a wrong view or an undersized buffer would otherwise be
# read or written out of bounds by the kernels).  Shapes the library rejects
# are left to it, so its status code is what the caller sees.
# ---------------------------------------------------------------------------
def _gpu(t, name: str, call: str, *, dtype=None, itemsize: Optional[int] = None,
         numel: int = 0, optional: bool = False) -> None:
    if t is None:
        if optional or numel == 0:
            return
        raise ValueError(f"{call}: {name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{call}: {name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{call}: {name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{call}: {name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{call}: {name} must be {dtype} (got {t.dtype})")
    if itemsize is not None and t.element_size() != itemsize:
        raise TypeError(f"{call}: {name} must have {itemsize}-byte elements (got {t.dtype})")
    if t.numel() < numel:
        raise ValueError(f"{call}: {name} holds {t.numel()} elements, the shape needs {numel}")


def _rows(shape: Shape) -> Optional[int]:
    """Receive rows of a valid shape, or None (the C call then reports it)."""
    n = _lib.moe_recv_rows(ctypes.byref(shape.c()))
    return None if n < 0 else int(n)


def _payload_rows(shape: Shape, rows: int, t, ts, name: str, call: str,
                  scales_optional: bool = False) -> None:
    """A buffer of `rows` payload rows (bf16, or e4m3 codes plus fp32 scales)."""
    if shape.fp8:
        _gpu(t, name, call, itemsize=1, numel=rows * shape.hidden)
        _gpu(ts, name + " scales", call, dtype=torch.float32,
             numel=rows * (shape.hidden // 128), optional=scales_optional)
    else:
        _gpu(t, name, call, itemsize=2, numel=rows * shape.hidden)


def _layout(lay: "Layout", shape: Shape, rows: int, call: str) -> None:
    if lay is None:
        raise ValueError(f"{call}: layout is required")
    E, N = shape.num_experts, shape.num_ranks
    for f, n in (("expert_counts", E), ("expert_offsets", E), ("rank_counts", N),
                 ("rank_offsets", N), ("status", 1)):
        _gpu(getattr(lay, f), "layout." + f, call, dtype=torch.int32, numel=n)
    _gpu(lay.token_row, "layout.token_row", call, dtype=torch.int32,
         numel=shape.num_tokens * shape.top_k)
    _gpu(lay.row_src, "layout.row_src", call, dtype=torch.int32, numel=rows, optional=True)


def _route_args(call, logits, bias, k, topk_ids, topk_weights):
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError(f"{call}: logits must be a 2-D tensor [T, E]")
    T, E = logits.shape
    _gpu(logits, "logits", call, dtype=torch.float32, numel=T * E)
    _gpu(bias, "bias", call, dtype=torch.float32, numel=E, optional=True)
    _gpu(topk_ids, "topk_ids", call, dtype=torch.int32, numel=T * k)
    _gpu(topk_weights, "topk_weights", call, dtype=torch.float32, numel=T * k)


def moe_recv_rows(shape: Shape) -> int:
    n = _lib.moe_recv_rows(ctypes.byref(shape.c()))
    if n < 0:
        raise MoeError(MOE_ERR_INVALID_ARG, "moe_recv_rows")
    return int(n)


def moe_dispatch_workspace_size(shape: Shape) -> int:
    return int(_lib.moe_dispatch_workspace_size(ctypes.byref(shape.c())))


def moe_route_topk(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int, score: int,
                   topk_ids: Optional[torch.Tensor] = None,
                   topk_weights: Optional[torch.Tensor] = None, stream=None):
    """Top-k routing; returns (topk_ids int32 [T,k], topk_weights fp32 [T,k])."""
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _route_args("moe_route_topk", logits, bias, k, topk_ids, topk_weights)
    _check(_lib.moe_route_topk(_ptr(logits), _ptr(bias), T, E, k, score, _ptr(topk_ids),
                               _ptr(topk_weights), _stream(stream)), "moe_route_topk")
    return topk_ids, topk_weights


def moe_route_topk_grouped(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int, score: int,
                           n_groups: int, topk_groups: int,
                           topk_ids: Optional[torch.Tensor] = None,
                           topk_weights: Optional[torch.Tensor] = None, stream=None):
    """Group-limited top-k routing; returns (topk_ids, topk_weights)."""
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _route_args("moe_route_topk_grouped", logits, bias, k, topk_ids, topk_weights)
    _check(_lib.moe_route_topk_grouped(_ptr(logits), _ptr(bias), T, E, k, score, n_groups,
                                       topk_groups, _ptr(topk_ids), _ptr(topk_weights),
                                       _stream(stream)), "moe_route_topk_grouped")
    return topk_ids, topk_weights


def moe_dispatch(shape: Shape, x: torch.Tensor, topk_ids: torch.Tensor, recv_x: torch.Tensor,
                 recv_scales: Optional[torch.Tensor], layout: Layout,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rows = _rows(shape)
    if rows is not None:
        c = "moe_dispatch"
        T, H, k = shape.num_tokens, shape.hidden, shape.top_k
        _gpu(x, "x", c, itemsize=2, numel=T * H)
        _gpu(topk_ids, "topk_ids", c, dtype=torch.int32, numel=T * k)
        _payload_rows(shape, rows, recv_x, recv_scales, "recv_x", c)
        _layout(layout, shape, rows, c)
        # the library compares the workspace's bytes with what the shape needs
        _gpu(workspace, "workspace", c, optional=True)
    _check(_lib.moe_dispatch(ctypes.byref(shape.c()), _ptr(x), _ptr(topk_ids), _ptr(recv_x),
                             _ptr(recv_scales), ctypes.byref(layout.c()), _ptr(workspace),
                             ws_bytes, _stream(stream)), "moe_dispatch")


_lib.moe_dispatch_static.argtypes = [ctypes.POINTER(_Shape), _vp, _vp, _vp, _vp,
                                     ctypes.POINTER(_Layout), _vp]
_lib.moe_dispatch_static.restype = _i32
MOE_STATIC_SCRATCH_BYTES = 4 << 20


def moe_dispatch_static(shape: Shape, x: torch.Tensor, topk_ids: torch.Tensor,
                        recv_x: torch.Tensor, recv_scales: Optional[torch.Tensor],
                        layout: Layout, stream=None) -> None:
    """moe_dispatch without a workspace: the library's per-GPU scratch array
    serves the multi-kernel layout path (calls on one GPU must not overlap)."""
    rows = _rows(shape)
    if rows is not None:
        c = "moe_dispatch_static"
        T, H, k = shape.num_tokens, shape.hidden, shape.top_k
        _gpu(x, "x", c, itemsize=2, numel=T * H)
        _gpu(topk_ids, "topk_ids", c, dtype=torch.int32, numel=T * k)
        _payload_rows(shape, rows, recv_x, recv_scales, "recv_x", c)
        _layout(layout, shape, rows, c)
    _check(_lib.moe_dispatch_static(ctypes.byref(shape.c()), _ptr(x), _ptr(topk_ids),
                                    _ptr(recv_x), _ptr(recv_scales), ctypes.byref(layout.c()),
                                    _stream(stream)), "moe_dispatch_static")


_lib.moe_dispatch_sources.argtypes = [ctypes.POINTER(_Shape), _i32, _vp, _vp, _vp, _vp,
                                      ctypes.POINTER(_Layout), _vp, _vp, _vp, ctypes.c_size_t,
                                      _vp]
_lib.moe_dispatch_sources.restype = _i32


def world_shape(shape: Shape, num_sources: int) -> Shape:
    """The shape of all sources together (num_tokens = S*T)."""
    return dataclasses.replace(shape, num_tokens=shape.num_tokens * num_sources)


def moe_dispatch_sources(shape: Shape, num_sources: int, x: torch.Tensor,
                         topk_ids: torch.Tensor, recv_x: torch.Tensor,
                         recv_scales: Optional[torch.Tensor], layout: Layout,
                         source_counts: torch.Tensor, source_offsets: torch.Tensor,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Every source rank dispatching at once; shape holds one source's sizes."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    world = world_shape(shape, num_sources) if num_sources >= 1 else shape
    rows = _rows(world)
    if rows is not None and num_sources >= 1:
        c = "moe_dispatch_sources"
        T, H, k = world.num_tokens, world.hidden, world.top_k
        _gpu(x, "x", c, itemsize=2, numel=T * H)
        _gpu(topk_ids, "topk_ids", c, dtype=torch.int32, numel=T * k)
        _payload_rows(world, rows, recv_x, recv_scales, "recv_x", c)
        _layout(layout, world, rows, c)
        _gpu(source_counts, "source_counts", c, dtype=torch.int32,
             numel=num_sources * shape.num_experts)
        _gpu(source_offsets, "source_offsets", c, dtype=torch.int32,
             numel=num_sources * shape.num_experts)
    _check(_lib.moe_dispatch_sources(ctypes.byref(shape.c()), num_sources, _ptr(x),
                                     _ptr(topk_ids), _ptr(recv_x), _ptr(recv_scales),
                                     ctypes.byref(layout.c()), _ptr(source_counts),
                                     _ptr(source_offsets), _ptr(workspace), ws_bytes,
                                     _stream(stream)), "moe_dispatch_sources")


def moe_expert_scale(shape: Shape, recv_x: torch.Tensor, recv_scales: Optional[torch.Tensor],
                     layout: Layout, alpha: torch.Tensor, y: torch.Tensor,
                     y_scales: Optional[torch.Tensor], stream=None) -> None:
    rows = _rows(shape)
    if rows is not None:
        c = "moe_expert_scale"
        _payload_rows(shape, rows, recv_x, recv_scales, "recv_x", c)
        _payload_rows(shape, rows, y, y_scales, "y", c)
        _gpu(alpha, "alpha", c, dtype=torch.float32, numel=shape.num_experts)
        _layout(layout, shape, rows, c)
    _check(_lib.moe_expert_scale(ctypes.byref(shape.c()), _ptr(recv_x), _ptr(recv_scales),
                                 ctypes.byref(layout.c()), _ptr(alpha), _ptr(y), _ptr(y_scales),
                                 _stream(stream)), "moe_expert_scale")


def moe_combine(shape: Shape, expert_y: torch.Tensor, expert_scales: Optional[torch.Tensor],
                layout: Layout, topk_weights: torch.Tensor, out: torch.Tensor,
                stream=None) -> None:
    rows = _rows(shape)
    if rows is not None:
        c = "moe_combine"
        T, H, k = shape.num_tokens, shape.hidden, shape.top_k
        _payload_rows(shape, rows, expert_y, expert_scales, "expert_y", c)
        _layout(layout, shape, rows, c)
        _gpu(topk_weights, "topk_weights", c, dtype=torch.float32, numel=T * k)
        _gpu(out, "out", c, itemsize=2, numel=T * H)
    _check(_lib.moe_combine(ctypes.byref(shape.c()), _ptr(expert_y), _ptr(expert_scales),
                            ctypes.byref(layout.c()), _ptr(topk_weights), _ptr(out),
                            _stream(stream)), "moe_combine")


_lib.moe_combine_partial_send.argtypes = [ctypes.POINTER(_Shape), _vp, _vp, ctypes.POINTER(_Layout),
                                  _vp, _vp, _vp, _vp, _vp]
_lib.moe_combine_partial_send.restype = _i32
_lib.moe_combine_partial_recv.argtypes = [ctypes.POINTER(_Shape), _vp, _vp, _vp, _vp]
_lib.moe_combine_partial_recv.restype = _i32


def partial_slots(shape: Shape) -> int:
    """M = min(k, N): partial rows per token of the two-stage combine."""
    return min(shape.top_k, shape.num_ranks)


def moe_combine_partial_send(shape: Shape, expert_y: torch.Tensor, expert_scales: Optional[torch.Tensor],
                     layout: Layout, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                     partial: torch.Tensor, partial_rank: torch.Tensor, stream=None) -> None:
    """Stage 1 of the two-stage combine: one bf16 row per (token, rank)."""
    rows = _rows(shape)
    if rows is not None:
        c = "moe_combine_partial_send"
        T, H, k, M = shape.num_tokens, shape.hidden, shape.top_k, partial_slots(shape)
        _payload_rows(shape, rows, expert_y, expert_scales, "expert_y", c)
        _layout(layout, shape, rows, c)
        _gpu(topk_ids, "topk_ids", c, dtype=torch.int32, numel=T * k)
        _gpu(topk_weights, "topk_weights", c, dtype=torch.float32, numel=T * k)
        _gpu(partial, "partial", c, itemsize=2, numel=T * M * H)
        _gpu(partial_rank, "partial_rank", c, dtype=torch.int32, numel=T * M)
    _check(_lib.moe_combine_partial_send(ctypes.byref(shape.c()), _ptr(expert_y), _ptr(expert_scales),
                                 ctypes.byref(layout.c()), _ptr(topk_ids), _ptr(topk_weights),
                                 _ptr(partial), _ptr(partial_rank), _stream(stream)),
           "moe_combine_partial_send")


def moe_combine_partial_recv(shape: Shape, partial: torch.Tensor, partial_rank: torch.Tensor,
                     out: torch.Tensor, stream=None) -> None:
    """Stage 2: sum of each token's partial rows."""
    if _rows(shape) is not None:
        c = "moe_combine_partial_recv"
        T, H, M = shape.num_tokens, shape.hidden, partial_slots(shape)
        _gpu(partial, "partial", c, itemsize=2, numel=T * M * H)
        _gpu(partial_rank, "partial_rank", c, dtype=torch.int32, numel=T * M)
        _gpu(out, "out", c, itemsize=2, numel=T * H)
    _check(_lib.moe_combine_partial_recv(ctypes.byref(shape.c()), _ptr(partial), _ptr(partial_rank),
                                 _ptr(out), _stream(stream)), "moe_combine_partial_recv")


_lib.moe_dispatch_recv.argtypes = [ctypes.POINTER(_Shape), _vp, _vp, ctypes.POINTER(_Layout),
                                   _vp, _vp, _vp, _vp]
_lib.moe_dispatch_recv.restype = _i32
_lib.moe_combine_send.argtypes = [ctypes.POINTER(_Shape), _vp, _vp, ctypes.POINTER(_Layout),
                                  _vp, _vp, _vp]
_lib.moe_combine_send.restype = _i32


def moe_dispatch_recv(shape: Shape, recv_x: torch.Tensor, recv_scales: Optional[torch.Tensor],
                      layout: Layout, gemm_x: torch.Tensor, gemm_scales: Optional[torch.Tensor],
                      gemm_offsets: torch.Tensor, stream=None) -> None:
    """Receive half of dispatch: receive regions -> dense grouped-GEMM input."""
    rows = _rows(shape)
    if rows is not None:
        c = "moe_dispatch_recv"
        _payload_rows(shape, rows, recv_x, recv_scales, "recv_x", c)
        _payload_rows(shape, shape.num_tokens * shape.top_k, gemm_x, gemm_scales, "gemm_x", c)
        _layout(layout, shape, rows, c)
        _gpu(gemm_offsets, "gemm_offsets", c, dtype=torch.int32, numel=shape.num_experts + 1)
    _check(_lib.moe_dispatch_recv(ctypes.byref(shape.c()), _ptr(recv_x), _ptr(recv_scales),
                                  ctypes.byref(layout.c()), _ptr(gemm_x), _ptr(gemm_scales),
                                  _ptr(gemm_offsets), _stream(stream)), "moe_dispatch_recv")


def moe_combine_send(shape: Shape, gemm_y: torch.Tensor, gemm_scales: Optional[torch.Tensor],
                     layout: Layout, expert_y: torch.Tensor,
                     expert_scales: Optional[torch.Tensor], stream=None) -> None:
    """Send half of the combine: dense expert outputs -> receive-region layout."""
    rows = _rows(shape)
    if rows is not None:
        c = "moe_combine_send"
        _payload_rows(shape, shape.num_tokens * shape.top_k, gemm_y, gemm_scales, "gemm_y", c)
        _payload_rows(shape, rows, expert_y, expert_scales, "expert_y", c)
        _layout(layout, shape, rows, c)
    _check(_lib.moe_combine_send(ctypes.byref(shape.c()), _ptr(gemm_y), _ptr(gemm_scales),
                                 ctypes.byref(layout.c()), _ptr(expert_y), _ptr(expert_scales),
                                 _stream(stream)), "moe_combine_send")


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def alloc_recv(shape: Shape, device, fill: Optional[int] = None):
    """Receive buffer (bf16 rows or e4m3 codes) and, for fp8, its scales."""
    rows = moe_recv_rows(shape)
    if shape.fp8:
        buf = torch.empty(rows, shape.hidden, dtype=torch.uint8, device=device)
        sc = torch.empty(rows, shape.hidden // 128, dtype=torch.float32, device=device)
    else:
        buf = torch.empty(rows, shape.hidden, dtype=torch.int16, device=device)
        sc = None
    if fill is not None:
        buf.fill_(fill if shape.fp8 else (fill - 0x10000 if fill >= 0x8000 else fill))
        if sc is not None:
            sc.fill_(float("nan"))
    return buf, sc


def alloc_workspace(shape: Shape, device) -> Optional[torch.Tensor]:
    n = moe_dispatch_workspace_size(shape)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)
