"""Helpers for the GPU parity tests: run route -> dispatch -> expert stand-in ->
combine through the C ABI on seeded inputs, and compare every stage with the
CPU oracle fed the GPU's exact inputs to that stage."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from combine_moe_dispatch_amd import api, inputs

BF16_POISON = 0xFFFF   # a bf16 NaN pattern: rows nobody may write keep it
FP8_POISON = 0x7F      # the e4m3fn NaN code
CANARY_ROWS = 4        # extra poisoned rows past the end of every buffer

WEIGHT_RTOL = 2.0 ** -20


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def _poisoned(shape: api.Shape, rows: int):
    """Buffer with CANARY_ROWS extra rows; returns (full, view of the first rows)."""
    dev = "cuda"
    if shape.fp8:
        full = torch.full((rows + CANARY_ROWS, shape.hidden), FP8_POISON, dtype=torch.uint8, device=dev)
        sfull = torch.full((rows + CANARY_ROWS, shape.hidden // 128), float("nan"),
                           dtype=torch.float32, device=dev)
        return full, full[:rows], sfull, sfull[:rows]
    full = torch.full((rows + CANARY_ROWS, shape.hidden), BF16_POISON - 0x10000, dtype=torch.int16,
                      device=dev)
    return full, full[:rows], None, None


def run_chain(shape: api.Shape, x_bits: np.ndarray, alpha: np.ndarray, *,
              logits: np.ndarray | None = None, bias: np.ndarray | None = None,
              score: int = api.MOE_SCORE_SIGMOID, ids: np.ndarray | None = None,
              weights: np.ndarray | None = None, with_row_src: bool = True,
              misalign_ids: bool = False) -> dict:
    """Everything on the GPU through the C ABI; results copied back to numpy.
    misalign_ids: the id list handed to dispatch starts 4 bytes past a
    16-byte boundary (a view one element into its allocation)."""
    T, k = shape.num_tokens, shape.top_k
    out = {}
    if logits is not None:
        lg = torch.from_numpy(logits).cuda()
        b = None if bias is None else torch.from_numpy(bias).cuda()
        d_ids, d_w = api.moe_route_topk(lg, b, k, score)
    else:
        d_ids = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
        d_w = torch.from_numpy(np.ascontiguousarray(weights, np.float32)).cuda()
    if misalign_ids:
        buf = torch.full((d_ids.numel() + 1,), -5, dtype=torch.int32, device="cuda")
        buf[1:].copy_(d_ids.flatten())
        d_ids = buf[1:].view(d_ids.shape)
        assert d_ids.data_ptr() % 16 == 4
    rows = api.moe_recv_rows(shape)
    x = dev_u16(x_bits) if T > 0 else torch.empty(0, shape.hidden, dtype=torch.int16, device="cuda")
    lay = api.Layout.empty(shape, "cuda", with_row_src=with_row_src)
    lay.status.fill_(-1)  # dispatch must overwrite it
    ws = api.alloc_workspace(shape, "cuda")
    recv_full, recv, rs_full, rs = _poisoned(shape, rows)
    api.moe_dispatch(shape, x, d_ids, recv, rs, lay, ws)
    y_full, y, ys_full, ys = _poisoned(shape, rows)
    api.moe_expert_scale(shape, recv, rs, lay, torch.from_numpy(alpha).cuda(), y, ys)
    o = torch.full((T, shape.hidden), -1, dtype=torch.int16, device="cuda")
    api.moe_combine(shape, y, ys, lay, d_w, o)
    torch.cuda.synchronize()

    out["ids"] = d_ids.cpu().numpy()
    out["weights"] = d_w.cpu().numpy()
    for f in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "token_row"):
        out[f] = getattr(lay, f).cpu().numpy()
    out["row_src"] = None if lay.row_src is None else lay.row_src.cpu().numpy()
    out["status"] = int(lay.status.item())
    if shape.fp8:
        out["recv_full"] = recv_full.cpu().numpy()
        out["rs_full"] = rs_full.cpu().numpy()
        out["y_full"] = y_full.cpu().numpy()
        out["ys_full"] = ys_full.cpu().numpy()
    else:
        out["recv_full"] = host_u16(recv_full)
        out["y_full"] = host_u16(y_full)
    out["out"] = host_u16(o)
    out["rows"] = rows
    return out


def ulp_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance of bf16 bit patterns on the ordered number line (+0 == -0)."""
    def key(u):
        u = np.asarray(u, np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))


def check_chain(shape: api.Shape, g: dict, x_bits: np.ndarray, alpha: np.ndarray, *,
                logits=None, bias=None, score=api.MOE_SCORE_SIGMOID) -> None:
    """Compare every stage with the oracle, each stage fed the GPU's inputs."""
    T, H, E, k, N, C = (shape.num_tokens, shape.hidden, shape.num_experts, shape.top_k,
                        shape.num_ranks, shape.rank_capacity)
    rows = g["rows"]
    # route: ids bit-exact, weights within 2^-20 relative
    if logits is not None:
        o_ids, o_w = oracle.route_topk(logits, bias, k, score)
        assert np.array_equal(g["ids"], o_ids), "route ids"
        np.testing.assert_allclose(g["weights"], o_w, rtol=WEIGHT_RTOL, atol=0)
    # layout: bit-exact
    lay = oracle.layout(g["ids"], E, N, C)
    for f in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "token_row"):
        assert np.array_equal(g[f].reshape(lay[f].shape), lay[f]), f
    assert g["status"] == lay["status"], ("status", g["status"], lay["status"])
    if g["row_src"] is not None:
        assert np.array_equal(g["row_src"], lay["row_src"]), "row_src"
    tr = lay["token_row"]
    # dispatch: whole buffer bit-exact, including untouched poison and canaries
    canary = CANARY_ROWS
    if shape.fp8:
        o_recv, o_rs = oracle.dispatch_fp8(x_bits, tr, rows + canary, fill=FP8_POISON)
        assert np.array_equal(g["recv_full"], o_recv), "fp8 payload"
        assert np.array_equal(g["rs_full"].view(np.uint32), o_rs.view(np.uint32)), "fp8 scales"
        o_y, o_ys = oracle.expert_scale_fp8(g["recv_full"][:rows], g["rs_full"][:rows], g["ids"],
                                            tr, alpha)
        assert np.array_equal(g["y_full"][:rows], o_y), "expert fp8 payload"
        assert np.array_equal(g["ys_full"][:rows].view(np.uint32), o_ys.view(np.uint32)), "expert scales"
        assert (g["y_full"][rows:] == FP8_POISON).all()
        y, ys = g["y_full"][:rows], g["ys_full"][:rows]
    else:
        o_recv = oracle.dispatch_bf16(x_bits, tr, rows + canary, fill=BF16_POISON)
        assert np.array_equal(g["recv_full"], o_recv), "bf16 rows"
        o_y = oracle.expert_scale_bf16(g["recv_full"][:rows], g["ids"], tr, alpha, fill=BF16_POISON)
        assert np.array_equal(g["y_full"][:rows], o_y), "expert bf16 rows"
        assert (g["y_full"][rows:] == BF16_POISON).all()
        y, ys = g["y_full"][:rows], None
    # combine: within 1 bf16 ulp of the double-precision sum, and bit-exact
    # against the fp32 fused multiply-add chain in slot order
    if T > 0:
        exact = oracle.combine_exact(y, ys, g["token_row"].reshape(T, k), g["weights"])
        d = ulp_dist(g["out"], exact)
        assert d.max() <= 1, ("combine ulp", int(d.max()))
        ordered = oracle.combine_f32_ordered(y, ys, g["token_row"].reshape(T, k), g["weights"])
        assert np.array_equal(g["out"], ordered), "combine fp32 chain"


def workload_shape(w: inputs.Workload) -> api.Shape:
    return api.Shape(w.T, w.H, w.E, w.k, w.N, w.C,
                     api.MOE_PAYLOAD_FP8_E4M3_B128 if w.payload == "fp8" else api.MOE_PAYLOAD_BF16)
