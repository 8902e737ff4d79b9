"""CPU oracle for MoE dispatch and combine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps the plain C implementation in
``moe_oracle.c`` (which shares nothing with the HIP library) with numpy
marshalling; every function documents which passage of the pages it follows:

* "Enabling trillion-parameter models on AWS EFA" -- the EFA page;
* "Lower Latency and Higher Throughput with Multi-Node DeepSeek Deployment"
  -- the DeepSeek-deployment page.

bf16 values travel as ``uint16`` bit patterns and e4m3 values as ``uint8``
codes, so nothing here depends on a numpy float type the method uses.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

ST_CAPACITY = 1
ST_BAD_ID = 2
SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1


def build() -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math, no contraction)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        vp = ctypes.c_void_p
        lib.oracle_f32_to_bf16.argtypes = [f32]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f64_to_bf16.argtypes = [f64]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = f32
        lib.oracle_f32_to_e4m3.argtypes = [f32]
        lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
        lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_f32.restype = f32
        lib.oracle_route_topk.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
        lib.oracle_route_topk.restype = i32
        lib.oracle_route_topk_grouped.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
        lib.oracle_route_topk_grouped.restype = i32
        lib.oracle_layout.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                      vp, vp, i64, vp]
        lib.oracle_layout.restype = i32
        lib.oracle_dispatch_bf16.argtypes = [vp, i32, i32, i32, vp, vp]
        lib.oracle_dispatch_bf16.restype = None
        lib.oracle_quantize_row_fp8.argtypes = [vp, i32, vp, vp]
        lib.oracle_quantize_row_fp8.restype = None
        lib.oracle_dispatch_fp8.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        lib.oracle_dispatch_fp8.restype = None
        lib.oracle_expert_scale_bf16.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
        lib.oracle_expert_scale_bf16.restype = None
        lib.oracle_expert_scale_fp8.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
        lib.oracle_expert_scale_fp8.restype = None
        lib.oracle_combine_exact.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
        lib.oracle_combine_exact.restype = None
        lib.oracle_combine_f32_ordered.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
        lib.oracle_combine_f32_ordered.restype = None
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# --- scalar codecs ---------------------------------------------------------

def f32_to_bf16(v: float) -> int:
    return int(_load().oracle_f32_to_bf16(float(v)))


def f64_to_bf16(v: float) -> int:
    return int(_load().oracle_f64_to_bf16(float(v)))


def bf16_to_f32(b: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(b)))


def f32_to_e4m3(v: float) -> int:
    return int(_load().oracle_f32_to_e4m3(float(v)))


def e4m3_to_f32(c: int) -> float:
    return float(_load().oracle_e4m3_to_f32(int(c)))


# --- steps of the path -----------------------------------------------------

def route_topk(logits: np.ndarray, bias: Optional[np.ndarray], k: int, score: int):
    """Top-k routing (EFA page, Introduction; DeepSeek-deployment page, MoE
    Router).  Returns (ids int32 [T,k], weights float32 [T,k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = _load().oracle_route_topk(_ptr(logits), _ptr(b), T, E, k, score, _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_route_topk: invalid arguments or non-finite logits")
    return ids, w


def route_topk_grouped(logits: np.ndarray, bias: Optional[np.ndarray], k: int, score: int,
                       n_groups: int, topk_groups: int):
    """Group-limited top-k (DeepSeek-deployment page, MoE Router): keep the
    topk_groups groups with the largest sum of their two best biased logits,
    then the plain top-k over their experts."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = _load().oracle_route_topk_grouped(_ptr(logits), _ptr(b), T, E, k, score, n_groups,
                                           topk_groups, _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_route_topk_grouped: invalid arguments or non-finite logits")
    return ids, w


def recv_rows(T: int, k: int, N: int, C: int) -> int:
    return N * C if C > 0 else T * k


def layout(ids: np.ndarray, E: int, N: int, C: int, with_row_src: bool = True):
    """Counts, offsets and destination rows (EFA page, Send and Receive
    Buffers; Dispatch and Combine).  Returns a dict of numpy arrays plus the
    status bits; row_src entries of rows that receive no pair are -1."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    rows = recv_rows(T, k, N, C)
    out = {
        "expert_counts": np.empty(E, np.int32),
        "expert_offsets": np.empty(E, np.int32),
        "rank_counts": np.empty(N, np.int32),
        "rank_offsets": np.empty(N, np.int32),
        "token_row": np.empty((T, k), np.int32),
        "row_src": np.full(rows, -1, np.int32) if with_row_src else None,
    }
    st = np.zeros(1, np.int32)
    rc = _load().oracle_layout(_ptr(ids), T, k, E, N, C, _ptr(out["expert_counts"]),
                               _ptr(out["expert_offsets"]), _ptr(out["rank_counts"]),
                               _ptr(out["rank_offsets"]), _ptr(out["token_row"]),
                               _ptr(out["row_src"]), rows, _ptr(st))
    if rc != 0:
        raise ValueError("oracle_layout: invalid arguments")
    out["status"] = int(st[0])
    out["rows"] = rows
    return out


def layout_sources(ids: np.ndarray, E: int, N: int, C: int):
    """Every rank dispatching at once (EFA page, Send and Receive Buffers):
    ids [S,T,k]; pairs placed in (rank, expert, source, token, slot) order.
    Returns the layout dict plus source_counts [S,E] and source_offsets [E,S]."""
    ids = _c(ids, np.int32)
    S, T, k = ids.shape
    rows = recv_rows(S * T, k, N, C)
    out = {
        "expert_counts": np.empty(E, np.int32),
        "expert_offsets": np.empty(E, np.int32),
        "rank_counts": np.empty(N, np.int32),
        "rank_offsets": np.empty(N, np.int32),
        "token_row": np.empty((S * T, k), np.int32),
        "source_counts": np.empty((S, E), np.int32),
        "source_offsets": np.empty((E, S), np.int32),
    }
    st = np.zeros(1, np.int32)
    lib = _load()
    lib.oracle_layout_sources.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int] + \
                                         [ctypes.c_void_p] * 8
    lib.oracle_layout_sources.restype = ctypes.c_int
    rc = lib.oracle_layout_sources(_ptr(ids), S, T, k, E, N, C, _ptr(out["expert_counts"]),
                                   _ptr(out["expert_offsets"]), _ptr(out["rank_counts"]),
                                   _ptr(out["rank_offsets"]), _ptr(out["token_row"]),
                                   _ptr(out["source_counts"]), _ptr(out["source_offsets"]),
                                   _ptr(st))
    if rc != 0:
        raise ValueError("oracle_layout_sources: invalid arguments")
    out["status"] = int(st[0])
    out["rows"] = rows
    return out


def dispatch_bf16(x_bits: np.ndarray, token_row: np.ndarray, rows: int,
                  fill: int = 0xFFFF) -> np.ndarray:
    """bf16 dispatch: every placed pair's row receives a copy of its token."""
    x_bits = _c(x_bits, np.uint16)
    T, H = x_bits.shape
    tr = _c(token_row, np.int32)
    k = tr.shape[1] if tr.ndim == 2 else (tr.size // T if T else 1)
    recv = np.full((rows, H), fill, np.uint16)
    _load().oracle_dispatch_bf16(_ptr(x_bits), T, H, k, _ptr(tr), _ptr(recv))
    return recv


def quantize_row_fp8(x_bits_row: np.ndarray):
    x = _c(x_bits_row, np.uint16)
    H = x.shape[0]
    q = np.empty(H, np.uint8)
    s = np.empty(H // 128, np.float32)
    _load().oracle_quantize_row_fp8(_ptr(x), H, _ptr(q), _ptr(s))
    return q, s


def dispatch_fp8(x_bits: np.ndarray, token_row: np.ndarray, rows: int,
                 fill: int = 0x7F, scale_fill: float = np.nan):
    """Block-scaled fp8 dispatch (EFA page, Evaluation; DeepSeek-deployment
    page, Quantization).  Returns (codes uint8 [rows,H], scales f32 [rows,H/128])."""
    x_bits = _c(x_bits, np.uint16)
    T, H = x_bits.shape
    tr = _c(token_row, np.int32)
    k = tr.shape[1]
    recv = np.full((rows, H), fill, np.uint8)
    sc = np.full((rows, H // 128), scale_fill, np.float32)
    _load().oracle_dispatch_fp8(_ptr(x_bits), T, H, k, _ptr(tr), _ptr(recv), _ptr(sc))
    return recv, sc


def expert_scale_bf16(recv: np.ndarray, ids: np.ndarray, token_row: np.ndarray,
                      alpha: np.ndarray, fill: int = 0xFFFF) -> np.ndarray:
    recv = _c(recv, np.uint16)
    ids = _c(ids, np.int32)
    tr = _c(token_row, np.int32)
    T, k = tr.shape
    H = recv.shape[1]
    y = np.full_like(recv, fill)
    _load().oracle_expert_scale_bf16(_ptr(recv), _ptr(ids), _ptr(tr), T, k, H,
                                     _ptr(_c(alpha, np.float32)), _ptr(y))
    return y


def expert_scale_fp8(recv: np.ndarray, recv_scales: np.ndarray, ids: np.ndarray,
                     token_row: np.ndarray, alpha: np.ndarray):
    recv = _c(recv, np.uint8)
    rs = _c(recv_scales, np.float32)
    ids = _c(ids, np.int32)
    tr = _c(token_row, np.int32)
    T, k = tr.shape
    H = recv.shape[1]
    y = np.full_like(recv, 0x7F)
    ys = np.full_like(rs, np.nan)
    _load().oracle_expert_scale_fp8(_ptr(recv), _ptr(rs), _ptr(ids), _ptr(tr), T, k, H,
                                    _ptr(_c(alpha, np.float32)), _ptr(y), _ptr(ys))
    return y, ys


def _combine(fn, y, y_scales, token_row, weights):
    tr = _c(token_row, np.int32)
    w = _c(weights, np.float32)
    T, k = tr.shape
    if y_scales is None:
        y = _c(y, np.uint16)
        ys = None
    else:
        y = _c(y, np.uint8)
        ys = _c(y_scales, np.float32)
    H = y.shape[1]
    out = np.empty((T, H), np.uint16)
    fn(_ptr(y), _ptr(ys), _ptr(tr), _ptr(w), T, k, H, _ptr(out))
    return out


def gemm_io(pack: bool, src: np.ndarray, src_scales, expert_counts, expert_offsets,
            E: int, N: int, C: int, dst_rows: int, fill: int):
    """Receive-side shuffle into the grouped GEMM's dense input (pack) or back
    (EFA page, Dispatch and Combine).  src: [rows][row elements] uint16/uint8.
    Returns (dst, dst_scales or None, dense offsets [E+1])."""
    src = np.ascontiguousarray(src)
    row_bytes = src.shape[1] * src.itemsize
    dst = np.full((dst_rows, src.shape[1]), fill, src.dtype)
    nb = 0 if src_scales is None else src_scales.shape[1]
    ss = None if src_scales is None else _c(src_scales, np.float32)
    ds = None if src_scales is None else np.full((dst_rows, nb), np.nan, np.float32)
    dense = np.empty(E + 1, np.int32)
    lib = _load()
    lib.oracle_gemm_io.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 6 + [ctypes.c_int] * 5 + \
        [ctypes.c_void_p]
    lib.oracle_gemm_io.restype = None
    lib.oracle_gemm_io(1 if pack else 0, _ptr(src), _ptr(ss), _ptr(dst), _ptr(ds),
                       _ptr(_c(expert_counts, np.int32)), _ptr(_c(expert_offsets, np.int32)),
                       E, N, C, row_bytes, nb, _ptr(dense))
    return dst, ds, dense


def combine_send(y, y_scales, token_row, ids, weights, E: int, N: int, exact: bool):
    """Sender-side partial reduction, stage 1 (EFA page, Evaluation): one bf16
    row per (token, distinct destination rank), ranks ascending.  Returns
    (partial uint16 [T,M,H], partial_rank int32 [T,M]) with M = min(k, N);
    rows of unused slots hold the poison 0xFFFF."""
    tr = _c(token_row, np.int32)
    ids = _c(ids, np.int32)
    w = _c(weights, np.float32)
    T, k = tr.shape
    if y_scales is None:
        y = _c(y, np.uint16)
        ys = None
    else:
        y = _c(y, np.uint8)
        ys = _c(y_scales, np.float32)
    H = y.shape[1]
    M = min(k, N)
    partial = np.full((T, M, H), 0xFFFF, np.uint16)
    prank = np.empty((T, M), np.int32)
    lib = _load()
    lib.oracle_combine_send.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + \
        [ctypes.c_void_p] * 2
    lib.oracle_combine_send.restype = None
    lib.oracle_combine_send(_ptr(y), _ptr(ys), _ptr(tr), _ptr(ids), _ptr(w), T, k, H, E, N, M,
                            1 if exact else 0, _ptr(partial), _ptr(prank))
    return partial, prank


def combine_recv(partial, partial_rank, exact: bool) -> np.ndarray:
    """Stage 2: sum of each token's partial rows, in slot order, to bf16."""
    partial = _c(partial, np.uint16)
    prank = _c(partial_rank, np.int32)
    T, M, H = partial.shape
    out = np.empty((T, H), np.uint16)
    lib = _load()
    lib.oracle_combine_recv.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 4 + \
        [ctypes.c_void_p]
    lib.oracle_combine_recv.restype = None
    lib.oracle_combine_recv(_ptr(partial), _ptr(prank), T, M, H, 1 if exact else 0, _ptr(out))
    return out


def combine_exact(y, y_scales, token_row, weights) -> np.ndarray:
    """Weighted sum of each token's returned rows in double precision, rounded
    once to bf16 (EFA page, Introduction; Evaluation)."""
    return _combine(_load().oracle_combine_exact, y, y_scales, token_row, weights)


def combine_f32_ordered(y, y_scales, token_row, weights) -> np.ndarray:
    """Same sum as fp32 fused multiply-adds in slot order from 0, then bf16."""
    return _combine(_load().oracle_combine_f32_ordered, y, y_scales, token_row, weights)
