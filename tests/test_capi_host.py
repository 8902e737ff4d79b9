"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/moe_dispatch.h
declares, and reject invalid arguments synchronously, before any launch --
these paths touch no device, so they run on the CPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_dispatch.h")

api = pytest.importorskip("combine_moe_dispatch_amd.api",
                          reason="libmoe_dispatch.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("moe_route_topk", "moe_dispatch", "moe_combine", "moe_expert_scale",
              "moe_recv_rows", "moe_dispatch_workspace_size", "moe_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(api.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(lib, n), n


def test_recv_rows_and_workspace():
    S = api.Shape
    assert api.moe_recv_rows(S(128, 7168, 256, 8, 32, 1024)) == 32768
    assert api.moe_recv_rows(S(4096, 7168, 256, 8, 32, 0)) == 32768
    assert api.moe_recv_rows(S(0, 8, 1, 1, 1, 0)) == 0
    assert api.moe_dispatch_workspace_size(S(128, 7168, 256, 8, 32, 1024)) == 0
    assert api.moe_dispatch_workspace_size(S(512, 7168, 256, 8, 32, 4096, 1)) == 0
    # one launch up to 8192 pairs, so no workspace; past that the layout's
    assert api.moe_dispatch_workspace_size(S(1024, 7168, 256, 8, 32, 8192)) == 0
    assert api.moe_dispatch_workspace_size(S(8192, 64, 8, 1, 1, 0)) == 0
    assert api.moe_dispatch_workspace_size(S(1025, 7168, 256, 8, 32, 8200)) > 0
    ws = api.moe_dispatch_workspace_size(S(4096, 7168, 256, 8, 32, 0))
    assert ws >= 4 * 32768 + 4 * 32 * 256 + 4 * 32
    with pytest.raises(api.MoeError):
        api.moe_recv_rows(S(1, 8, 10, 2, 4, 0))  # E % N != 0


@pytest.mark.parametrize("shape,code", [
    ((4, 12, 8, 2, 2, 0, 0), 1),        # H % 8 != 0 for bf16
    ((4, 64, 8, 2, 2, 0, 1), 1),        # H % 128 != 0 for fp8
    ((4, 64, 8, 9, 2, 0, 0), 1),        # k > E
    ((4, 64, 9, 2, 2, 0, 0), 1),        # E % N != 0
    ((-1, 64, 8, 2, 2, 0, 0), 1),       # T < 0
    ((4, 64, 8, 2, 2, -1, 0), 1),       # C < 0
    ((4, 64, 8, 2, 2, 0, 7), 1),        # unknown payload
    ((4, 64, 2048, 2, 2, 0, 0), 2),     # E beyond the LDS histogram
    ((4, 64, 64, 33, 2, 0, 0), 2),      # k beyond MOE_MAX_TOP_K
])
def test_dispatch_rejects_bad_shapes(shape, code):
    s = api._Shape(*shape)
    lay = api._Layout(16, 16, 16, 16, 16, None, 16)
    rc = api._lib.moe_dispatch(ctypes.byref(s), 16, 16, 16, 16, ctypes.byref(lay), None, 0, None)
    assert rc == code
    rc = api._lib.moe_combine(ctypes.byref(s), 16, 16, ctypes.byref(lay), 16, 16, None)
    assert rc == code


def test_dispatch_rejects_null_and_misaligned_pointers():
    s = api._Shape(4, 64, 8, 2, 2, 0, 0)
    good = api._Layout(16, 16, 16, 16, 16, None, 16)
    f = api._lib.moe_dispatch
    assert f(None, 16, 16, 16, None, ctypes.byref(good), None, 0, None) == 1
    assert f(ctypes.byref(s), 16, 16, 16, None, None, None, 0, None) == 1
    nostatus = api._Layout(16, 16, 16, 16, 16, None, None)
    assert f(ctypes.byref(s), 16, 16, 16, None, ctypes.byref(nostatus), None, 0, None) == 1
    assert f(ctypes.byref(s), 8, 16, 16, None, ctypes.byref(good), None, 0, None) == 1   # x
    assert f(ctypes.byref(s), 16, 16, 24, None, ctypes.byref(good), None, 0, None) == 1  # recv
    s8 = api._Shape(4, 128, 8, 2, 2, 0, 1)
    assert f(ctypes.byref(s8), 16, 16, 16, None, ctypes.byref(good), None, 0, None) == 1  # scales
    big = api._Shape(1100, 64, 8, 8, 2, 0, 0)  # 8800 pairs: needs a workspace
    assert f(ctypes.byref(big), 16, 16, 16, None, ctypes.byref(good), None, 0, None) == 1
    assert f(ctypes.byref(big), 16, 16, 16, None, ctypes.byref(good), 16, 8, None) == 1


def test_combine_and_expert_scale_reject_bad_pointers():
    s = api._Shape(4, 64, 8, 2, 2, 0, 0)
    lay = api._Layout(16, 16, 16, 16, 16, None, 16)
    c = api._lib.moe_combine
    assert c(ctypes.byref(s), None, None, ctypes.byref(lay), 16, 16, None) == 1
    assert c(ctypes.byref(s), 16, None, ctypes.byref(lay), 16, 8, None) == 1
    assert c(ctypes.byref(s), 16, None, None, 16, 16, None) == 1
    x = api._lib.moe_expert_scale
    assert x(ctypes.byref(s), 16, None, ctypes.byref(lay), None, 16, None, None) == 1
    s8 = api._Shape(4, 128, 8, 2, 2, 0, 1)
    assert x(ctypes.byref(s8), 16, None, ctypes.byref(lay), 16, 16, None, None) == 1


def test_route_rejects_bad_arguments():
    r = api._lib.moe_route_topk
    assert r(16, None, 4, 8, 9, 1, 16, 16, None) == 1      # k > E
    assert r(16, None, 4, 8, 2, 5, 16, 16, None) == 1      # bad score
    assert r(None, None, 4, 8, 2, 1, 16, 16, None) == 1    # null logits
    assert r(16, None, 4, 2048, 2, 1, 16, 16, None) == 2   # E too large
    assert r(16, None, -1, 8, 2, 1, 16, 16, None) == 1


def test_status_strings():
    for code in range(4):
        assert api.moe_status_string(code).startswith("MOE_")


def test_grouped_route_rejects_bad_arguments():
    r = api._lib.moe_route_topk_grouped
    assert r(16, None, 4, 16, 2, 1, 3, 1, 16, 16, None) == 1     # E % groups != 0
    assert r(16, None, 4, 16, 2, 1, 4, 5, 16, 16, None) == 1     # topk_groups > groups
    assert r(16, None, 4, 16, 2, 1, 4, 0, 16, 16, None) == 1     # topk_groups < 1
    assert r(16, None, 4, 16, 9, 1, 4, 2, 16, 16, None) == 1     # k > kept experts
    assert r(16, None, 4, 256, 2, 1, 128, 2, 16, 16, None) == 2  # too many groups


def test_dispatch_sources_rejects_bad_arguments():
    f = api._lib.moe_dispatch_sources
    s = api._Shape(4, 64, 8, 2, 2, 0, 0)
    lay = api._Layout(16, 16, 16, 16, 16, None, 16)
    assert f(ctypes.byref(s), 0, 16, 16, 16, None, ctypes.byref(lay), 16, 16, None, 0, None) == 1
    assert f(ctypes.byref(s), 2, 16, 16, 16, None, ctypes.byref(lay), None, 16, None, 0, None) == 1
    assert f(None, 2, 16, 16, 16, None, ctypes.byref(lay), 16, 16, None, 0, None) == 1
    bad = api._Shape(4, 64, 9, 2, 2, 0, 0)
    assert f(ctypes.byref(bad), 2, 16, 16, 16, None, ctypes.byref(lay), 16, 16, None, 0, None) == 1


def test_two_stage_combine_rejects_bad_arguments():
    s = api._Shape(4, 64, 8, 2, 2, 0, 0)
    lay = api._Layout(16, 16, 16, 16, 16, None, 16)
    send, recv = api._lib.moe_combine_partial_send, api._lib.moe_combine_partial_recv
    assert send(ctypes.byref(s), 16, None, ctypes.byref(lay), 16, 16, None, 16, None) == 1
    assert send(ctypes.byref(s), 16, None, ctypes.byref(lay), None, 16, 16, 16, None) == 1
    assert send(ctypes.byref(s), 16, None, ctypes.byref(lay), 16, 16, 8, 16, None) == 1
    assert recv(ctypes.byref(s), 16, None, 16, None) == 1
    assert recv(ctypes.byref(s), 16, 16, 24, None) == 1
    bad = api._Shape(4, 64, 9, 2, 2, 0, 0)
    assert recv(ctypes.byref(bad), 16, 16, 16, None) == 1


def test_split_halves_reject_bad_arguments():
    s = api._Shape(4, 64, 8, 2, 2, 0, 0)
    lay = api._Layout(16, 16, 16, 16, 16, None, 16)
    r, c = api._lib.moe_dispatch_recv, api._lib.moe_combine_send
    assert r(ctypes.byref(s), 16, None, ctypes.byref(lay), 16, None, None, None) == 1  # offsets
    assert r(ctypes.byref(s), 8, None, ctypes.byref(lay), 16, None, 16, None) == 1     # misaligned
    assert r(ctypes.byref(s), 16, None, None, 16, None, 16, None) == 1
    s8 = api._Shape(4, 128, 8, 2, 2, 0, 1)
    assert r(ctypes.byref(s8), 16, None, ctypes.byref(lay), 16, None, 16, None) == 1  # scales
    assert c(ctypes.byref(s), 16, None, ctypes.byref(lay), None, None, None) == 1
    assert c(ctypes.byref(s8), 16, None, ctypes.byref(lay), 16, None, None) == 1


def test_stream_floor_library_loads_and_rejects_bad_arguments():
    """libmoe_ceiling.so (the benchmark's streaming floor kernels) loads, exports
    its entry points, and refuses null or misaligned pointers and bad grids
    without launching."""
    path = os.path.join(os.path.dirname(api.LIB_PATH), "libmoe_ceiling.so")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.moe_ceiling_read.argtypes = [vp, sz, vp, i32, vp]
    lib.moe_ceiling_write.argtypes = [vp, sz, i32, vp]
    lib.moe_ceiling_copy.argtypes = [vp, vp, sz, i32, vp]
    lib.moe_ceiling_write_blocked.argtypes = [vp, sz, i32, vp]
    lib.moe_ceiling_empty.argtypes = [vp]
    assert lib.moe_ceiling_read(None, 16, 256, 64, None) == 1
    assert lib.moe_ceiling_read(4096, 16, None, 64, None) == 1
    assert lib.moe_ceiling_read(4097, 16, 256, 64, None) == 1
    assert lib.moe_ceiling_write(4096, 16, 0, None) == 1
    assert lib.moe_ceiling_write(4096, 16, 70000, None) == 1
    assert lib.moe_ceiling_copy(4096, 4104, 16, 64, None) == 1
    assert lib.moe_ceiling_write_blocked(None, 16, 0, None) == 1
    assert lib.moe_ceiling_write_blocked(4104, 16, 0, None) == 1
    assert lib.moe_ceiling_write_blocked(4096, 0, 0, None) == 1
    assert lib.moe_ceiling_write_blocked(4096, 16, 3, None) == 1
    # the dispatch-shaped copy: (x, rows, dst, T, k, nvec, col_chunks, vpc, rows_total)
    rc = lib.moe_ceiling_rows_copy
    rc.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    assert rc(4096, None, None, 4, 2, 64, 1, 64, 8, None) == 1      # no destination
    assert rc(4104, None, 4096, 4, 2, 64, 1, 64, 8, None) == 1      # misaligned x
    assert rc(4096, None, 4096, 4, 65, 64, 1, 64, 260, None) == 1   # k past a wave
    assert rc(4096, None, 4096, 4, 2, 1024, 1, 1024, 8, None) == 1  # vpc past two per thread
    assert rc(4096, None, 4096, 4, 2, 600, 1, 512, 8, None) == 1    # chunks miss columns
    assert rc(4096, None, 4096, 4, 2, 64, 1, 64, 7, None) == 1      # rows t*k+j past the end
    assert rc(4096, None, 4096, 0, 2, 64, 1, 64, 8, None) == 1      # no tokens
    # read and write of given sizes in one kernel: (src, nr, dst, nw, sink, blocks)
    rw = lib.moe_ceiling_read_write
    rw.argtypes = [vp, sz, vp, sz, vp, i32, vp]
    assert rw(None, 16, 4096, 16, 256, 64, None) == 1   # reads from nowhere
    assert rw(4096, 16, 4104, 16, 256, 64, None) == 1   # misaligned destination
    assert rw(4096, 0, 4096, 0, 256, 64, None) == 1     # nothing to move
    assert rw(4096, 16, 4096, 16, None, 64, None) == 1  # no sink
    assert rw(4096, 16, 4096, 16, 256, 0, None) == 1    # no blocks
    # the combine-shaped gather: (y, rows, out, T, k, nvec, rows_total)
    rg = lib.moe_ceiling_rows_gather
    rg.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    assert rg(None, None, 4096, 4, 2, 64, 8, None) == 1       # no source
    assert rg(4096, None, 4104, 4, 2, 64, 8, None) == 1       # misaligned output
    assert rg(4096, None, 4096, 0, 2, 64, 8, None) == 1       # no tokens
    assert rg(4096, None, 4096, 70000, 2, 64, 140000, None) == 1  # tokens past grid y
    assert rg(4096, None, 4096, 4, 65, 64, 260, None) == 1    # k past a wave
    assert rg(4096, None, 4096, 4, 2, 64, 7, None) == 1       # rows t*k+j past the end


def test_dispatch_columns_follow_the_launcher_rule():
    """bench.py's copy of the bf16 dispatch's column split: two chunks of 448
    vectors at 128 tokens (256 blocks for 256 compute units) and up to the
    one-launch limit of 8192 pairs, one vector per thread past it, whole
    128-column chunks."""
    import bench
    from combine_moe_dispatch_amd import inputs
    W = inputs.WORKLOADS
    assert bench.dispatch_columns(W["dsv3_decode"]) == (2, 448)
    assert bench.dispatch_columns(W["skewed_prefill"]) == (4, 224)
    assert bench.dispatch_columns(W["tiny"]) == (1, 32)
    # the one-launch path ends at 8192 pairs
    assert bench.dispatch_columns(inputs.with_tokens(W["dsv3_decode"], 1024)) == (2, 448)
    assert bench.dispatch_columns(inputs.with_tokens(W["dsv3_decode"], 1025)) == (4, 224)
    assert bench.ONE_LAUNCH_MAX_PAIRS == 8192
    for w in W.values():
        cc, vpc = bench.dispatch_columns(w)
        assert vpc % 16 == 0 and cc * vpc >= w.H // 8 > (cc - 1) * vpc and vpc <= 512


def test_static_dispatch_rejects_what_its_scratch_cannot_hold():
    """moe_dispatch_static refuses, before touching any device, a shape whose
    multi-kernel layout needs more scratch than the library's array holds,
    and rejects bad shapes like moe_dispatch."""
    f = api._lib.moe_dispatch_static
    good = api._Layout(16, 16, 16, 16, 16, None, 16)
    big = api.Shape(600_000, 8, 64, 8, 8, 0)   # 4.8M pairs
    assert api.moe_dispatch_workspace_size(big) > api.MOE_STATIC_SCRATCH_BYTES
    assert f(ctypes.byref(big.c()), 16, 16, 16, None, ctypes.byref(good), None) == 2
    bad = api._Shape(4, 12, 8, 2, 2, 0, 0)     # H % 8 != 0
    assert f(ctypes.byref(bad), 16, 16, 16, None, ctypes.byref(good), None) == 1
    assert f(None, 16, 16, 16, None, ctypes.byref(good), None) == 1


def test_binding_refuses_host_tensors_before_the_call():
    """The binding checks its tensors before calling the library: a host
    (CPU) tensor where device memory is required is refused with a message
    naming the argument."""
    import torch
    shape = api.Shape(4, 64, 8, 2, 2, 0)
    with pytest.raises(ValueError, match="logits must be a GPU tensor"):
        api.moe_route_topk(torch.zeros(4, 8), None, 2, api.MOE_SCORE_SOFTMAX,
                           torch.zeros(4, 2, dtype=torch.int32),
                           torch.zeros(4, 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="x must be a GPU tensor"):
        api.moe_dispatch(shape, torch.zeros(4, 64, dtype=torch.int16),
                         torch.zeros(4, 2, dtype=torch.int32),
                         torch.zeros(8, 64, dtype=torch.int16), None, None)
