"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: route ids, layout metadata, dispatch rows, fp8 codes and scales and the
expert stand-in bit-exact; combine within 1 bf16 ulp of the double-precision
weighted sum (and bit-exact against the fp32 fused multiply-add chain in slot
order); route weights within 2^-20 relative.  Every buffer is poisoned before
the call and carries canary rows past its end, so a stray or missing write
fails the whole-buffer comparison.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_amd import api, inputs

from gpu_chain import (BF16_POISON, check_chain, run_chain, workload_shape, dev_u16,
                       host_u16, ulp_dist)

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("name", inputs.WORKLOAD_ORDER)
def test_workload_chain(name):
    """The five workloads at full size, routed on the GPU."""
    w = inputs.WORKLOADS[name]
    _announce(f"workload {name} {w}")
    inp = inputs.generate_for(w)
    shape = workload_shape(w)
    g = run_chain(shape, inp.x_bits, inp.alpha, logits=inp.logits, bias=inp.bias, score=w.score)
    check_chain(shape, g, inp.x_bits, inp.alpha, logits=inp.logits, bias=inp.bias, score=w.score)
    if w.expert == "identity":
        # identity experts with normalised weights give the input back exactly
        assert np.array_equal(g["out"], inp.x_bits)


def test_end_to_end_against_oracle_chain():
    """Oracle route -> layout -> dispatch -> expert -> combine on its own, vs the GPU."""
    w = inputs.WORKLOADS["dsv3_decode"]
    inp = inputs.generate_for(w)
    shape = workload_shape(w)
    g = run_chain(shape, inp.x_bits, inp.alpha, logits=inp.logits, score=w.score)
    ids, wt = oracle.route_topk(inp.logits, None, w.k, w.score)
    lay = oracle.layout(ids, w.E, w.N, w.C)
    recv = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"])
    y = oracle.expert_scale_bf16(recv, ids, lay["token_row"], inp.alpha)
    out = oracle.combine_exact(y, None, lay["token_row"], wt)
    assert ulp_dist(g["out"], out).max() <= 1


# (T, H, E, k, N, C, payload, distinct ids, hot expert)
SWEEP = [
    (0, 256, 8, 2, 2, 32, 0, True, None),          # no tokens
    (0, 7168, 256, 8, 32, 0, 1, True, None),
    (1, 8, 1, 1, 1, 1, 0, True, None),             # smallest everything
    (1, 7168, 256, 8, 32, 8, 0, True, None),
    (7, 256, 3, 2, 3, 0, 0, True, None),           # E not a power of two, packed
    (7, 128, 64, 8, 8, 56, 1, True, None),
    (128, 7168, 384, 8, 16, 1024, 0, True, None),
    (129, 1000, 64, 2, 4, 0, 0, True, None),       # ragged H/8 chunks, packed
    (200, 2056, 24, 8, 4, 0, 0, False, 5),         # duplicates and a hot expert
    (511, 384, 256, 8, 32, 0, 1, True, None),
    (512, 256, 256, 8, 32, 4096, 0, True, None),   # 4096 pairs: 16 ids per thread
    (513, 256, 256, 8, 32, 4104, 0, True, None),   # one launch, 32 ids per thread
    (1024, 256, 256, 8, 32, 8192, 0, True, None),  # 8192 pairs: one-launch limit
    (1025, 256, 256, 8, 32, 8200, 0, True, None),  # first chunked case (9 chunks)
    (2048, 256, 256, 8, 32, 0, 0, True, None),     # 16 chunks: layout in one launch
    (2049, 256, 256, 8, 32, 0, 0, True, None),     # 17 chunks: layout in two launches
    (1000, 136, 8, 8, 2, 0, 0, False, 3),          # one launch, heavy duplicates
    (1100, 136, 8, 8, 2, 0, 0, False, 3),          # chunked, heavy duplicates
    (1000, 7168, 64, 1, 8, 0, 1, True, None),
    (900, 1024, 32, 8, 4, 0, 1, False, 7),        # fp8, one launch, duplicates
    (1100, 1024, 32, 8, 4, 0, 1, False, 7),       # fp8, chunked path, duplicates
    (3000, 64, 1024, 8, 32, 0, 0, True, None),     # E at the library maximum
    # fixed-capacity regions on the one-launch path, with repeated experts in
    # a token: rows from the in-rank prefix (L <= 32, 16-byte and scalar
    # reads), from the chunk scan (L > 32), repeats found by row shifts
    # (k <= 8) and by the readlane loop (k > 8)
    (256, 512, 32, 8, 4, 2048, 0, False, 5),       # L = 8
    (120, 256, 96, 8, 4, 960, 0, False, 2),        # L = 24
    (200, 512, 64, 8, 4, 800, 0, False, 3),        # L = 16: four 16-byte reads
    (150, 256, 48, 8, 4, 600, 1, True, None),      # L = 12, fp8
    (50, 256, 30, 4, 5, 200, 0, False, None),      # L = 6
    (100, 512, 64, 12, 8, 800, 1, False, 3),       # k = 12, fp8
    (100, 512, 64, 6, 8, 600, 0, True, None),      # k = 6 (compile-time combine)
    (100, 512, 64, 6, 8, 600, 1, False, 2),        # k = 6, fp8, repeats
    (160, 512, 80, 8, 4, 300, 0, False, 3),        # L = 20: sums of whole vectors plus a
    (140, 256, 112, 8, 4, 280, 1, False, 5),       # partial one (L = 28, fp8); both overflow
    (64, 256, 256, 8, 2, 512, 0, False, 9),        # L = 128
    (2048, 512, 256, 32, 256, 0, 0, True, None),   # k at the library maximum
    (64, 32768, 64, 4, 8, 0, 0, True, None),       # wide rows: 8 column chunks per token
    (40, 16384, 32, 8, 4, 320, 1, True, None),     # wide fp8 rows, 128 scale blocks
    (700, 20480, 64, 8, 8, 0, 0, False, 1),        # wide rows, 5600 pairs in one launch
    (1100, 10240, 64, 8, 8, 0, 0, False, 1),       # wide rows on the chunked path
    (600, 2048, 1024, 8, 64, 0, 1, True, None),    # fp8, E at the library maximum
    (1100, 2048, 1024, 8, 64, 0, 1, True, None),   # the same, chunked
    (100, 1024, 512, 32, 16, 3200, 1, False, 3),   # fp8, k at the library maximum, repeats
    # near the 16- and 32-ids-per-thread limits of the one-kernel path with
    # many blocks per compute unit: odd T, repeated experts, rows of two
    # chunks; fp8 with capacity overflow
    (999, 4104, 64, 4, 8, 0, 0, False, 3),
    (1021, 256, 32, 4, 4, 1100, 1, False, 2),
    (2047, 4104, 64, 4, 8, 0, 0, False, 3),
    (2045, 256, 32, 4, 4, 2200, 1, False, 2),
    # runs of tokens per block on the one-launch path (32 ids per thread, six
    # or more blocks per compute unit otherwise), ragged last runs: runs of
    # four (packed; fp8 with a fixed capacity that overflows) and of two
    # (bf16; fp8 with 24 experts per rank and repeats)
    (1023, 7168, 256, 8, 32, 0, 0, False, 5),
    (1021, 7168, 256, 8, 32, 300, 1, False, 5),
    (769, 7168, 256, 8, 32, 0, 0, True, None),
    (771, 7168, 384, 8, 16, 1600, 1, False, 3),
    (70000, 8, 4, 2, 2, 0, 0, True, None),         # more tokens than a grid's y dimension holds
    (5000, 16, 8, 2, 2, 0, 0, False, None),        # combine grid just past 8192 blocks
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "T{}_H{}_E{}_k{}_N{}_C{}_p{}".format(*c[:7]))
def test_sweep_dispatch_combine(case):
    T, H, E, k, N, C, payload, distinct, hot = case
    _announce(f"sweep {case}")
    seed = 7 * T + H + E + k
    inp = inputs.generate(T, H, E, seed)
    ids = inputs.random_ids(T, k, E, seed + 1, distinct=distinct, hot=hot)
    wts = inputs.random_weights(T, k, seed + 2)
    shape = api.Shape(T, H, E, k, N, C, payload)
    g = run_chain(shape, inp.x_bits, inp.alpha, ids=ids, weights=wts)
    check_chain(shape, g, inp.x_bits, inp.alpha)


@pytest.mark.parametrize("T,k,E,N,C,payload", [
    (128, 8, 256, 32, 40, 0),      # fused path, capacity overflow on many ranks
    (1000, 8, 16, 2, 1500, 0),     # chunked path, overflow
    (64, 4, 8, 2, 100, 1),         # fp8, overflow
])
def test_capacity_overflow_skips_last_pairs(T, k, E, N, C, payload):
    _announce(f"capacity T={T} k={k} E={E} N={N} C={C}")
    H = 256
    inp = inputs.generate(T, H, E, 11)
    ids = inputs.random_ids(T, k, E, 12, distinct=True)
    wts = inputs.random_weights(T, k, 13)
    shape = api.Shape(T, H, E, k, N, C, payload)
    g = run_chain(shape, inp.x_bits, inp.alpha, ids=ids, weights=wts)
    assert g["status"] & api.MOE_DEV_CAPACITY
    check_chain(shape, g, inp.x_bits, inp.alpha)


@pytest.mark.parametrize("T", [16, 700])
def test_bad_ids_are_skipped(T):
    _announce(f"bad ids T={T}")
    H, E, k, N = 64, 16, 4, 4
    inp = inputs.generate(T, H, E, 21)
    ids = inputs.random_ids(T, k, E, 22, distinct=True)
    ids[::5, 1] = E + 3
    ids[1::7, 2] = -4
    wts = inputs.random_weights(T, k, 23)
    shape = api.Shape(T, H, E, k, N, 0)
    g = run_chain(shape, inp.x_bits, inp.alpha, ids=ids, weights=wts)
    assert g["status"] == api.MOE_DEV_BAD_ID
    check_chain(shape, g, inp.x_bits, inp.alpha)


def test_deterministic_bytes():
    w = inputs.WORKLOADS["skewed_prefill"]
    inp = inputs.generate_for(w)
    shape = workload_shape(w)
    a = run_chain(shape, inp.x_bits, inp.alpha, logits=inp.logits, bias=inp.bias)
    b = run_chain(shape, inp.x_bits, inp.alpha, logits=inp.logits, bias=inp.bias)
    for key in ("token_row", "expert_offsets", "recv_full", "out"):
        assert np.array_equal(a[key], b[key]), key


def test_route_softmax_and_ties():
    _announce("route ties")
    T, E, k = 300, 384, 8
    rng = np.random.default_rng(5)
    logits = rng.integers(-3, 4, size=(T, E)).astype(np.float32)  # many exact ties
    for score in (api.MOE_SCORE_SOFTMAX, api.MOE_SCORE_SIGMOID):
        ids, w = api.moe_route_topk(torch.from_numpy(logits).cuda(), None, k, score)
        torch.cuda.synchronize()
        o_ids, o_w = oracle.route_topk(logits, None, k, score)
        assert np.array_equal(ids.cpu().numpy(), o_ids)
        np.testing.assert_allclose(w.cpu().numpy(), o_w, rtol=2.0 ** -20, atol=0)


def test_route_signed_zero_logits():
    """-0 and +0 are equal logits: ties go to the lower id, as the float
    comparison has it (the selection keys treat -0 as +0)."""
    _announce("route signed zeros")
    T, E, k = 64, 256, 8
    rng = np.random.default_rng(11)
    logits = rng.choice(np.array([0.0, -0.0, -0.0, 0.0, -1.0, -0.5], np.float32),
                        size=(T, E)).astype(np.float32)
    for score in (api.MOE_SCORE_SOFTMAX, api.MOE_SCORE_SIGMOID):
        ids, _ = api.moe_route_topk(torch.from_numpy(logits).cuda(), None, k, score)
        torch.cuda.synchronize()
        o_ids, _ = oracle.route_topk(logits, None, k, score)
        assert np.array_equal(ids.cpu().numpy(), o_ids)


@pytest.mark.parametrize("grouped", [False, True])
def test_graph_capture_replays_match_eager(grouped):
    """route -> dispatch -> combine captured once and replayed several times,
    with eager work between replays; every replay equals the eager result.
    grouped: the group-limited router (4 of 8 groups) in place of plain top-k."""
    _announce(f"graph capture, grouped router {grouped}")
    w = inputs.WORKLOADS["dsv3_decode"]
    inp = inputs.generate_for(w)
    shape = workload_shape(w)
    lg = torch.from_numpy(inp.logits).cuda()
    x = dev_u16(inp.x_bits)
    ids = torch.empty(w.T, w.k, dtype=torch.int32, device="cuda")
    wt = torch.empty(w.T, w.k, dtype=torch.float32, device="cuda")
    lay = api.Layout.empty(shape, "cuda")
    recv, _ = api.alloc_recv(shape, "cuda", fill=0)
    out = torch.empty(w.T, w.H, dtype=torch.int16, device="cuda")

    def step(stream=None):
        if grouped:
            api.moe_route_topk_grouped(lg, None, w.k, w.score, 8, 4, ids, wt, stream=stream)
        else:
            api.moe_route_topk(lg, None, w.k, w.score, ids, wt, stream=stream)
        api.moe_dispatch(shape, x, ids, recv, None, lay, None, stream=stream)
        api.moe_combine(shape, recv, None, lay, wt, out, stream=stream)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(stream=s)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        step(stream=s)
    for i in range(4):
        out.fill_(0)
        lay.token_row.fill_(-7)
        ids.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        assert (lay.token_row >= 0).all()


def test_fp8_decode_all_codes_through_combine():
    """All 256 e4m3 codes through moe_combine with k=1, weight 1 and scale 1.
    Each finite code comes out as its exact value (e4m3 values are bf16 values),
    except -0, which the fp32 chain fma(1, -0, +0) turns into +0 -- exactly as
    the oracle's chain does; NaN codes come out as NaN."""
    shape = api.Shape(1, 256, 1, 1, 1, 1, api.MOE_PAYLOAD_FP8_E4M3_B128)
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    y = torch.from_numpy(codes).cuda()
    ys = torch.ones(1, 2, dtype=torch.float32, device="cuda")
    lay = api.Layout.empty(shape, "cuda")
    lay.token_row.zero_()
    w = torch.ones(1, 1, dtype=torch.float32, device="cuda")
    out = torch.empty(1, 256, dtype=torch.int16, device="cuda")
    api.moe_combine(shape, y, ys, lay, w, out)
    torch.cuda.synchronize()
    got = host_u16(out)[0]
    ref = oracle.combine_f32_ordered(codes, np.ones((1, 2), np.float32),
                                     np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32))[0]
    for c in range(256):
        v = oracle.e4m3_to_f32(c)
        if np.isnan(v):
            assert (got[c] & 0x7F80) == 0x7F80 and (got[c] & 0x7F) != 0, c
            continue
        assert got[c] == ref[c], (c, hex(got[c]), hex(ref[c]))
        if c != 0x80:
            assert got[c] == oracle.f32_to_bf16(v), (c, hex(got[c]))


@pytest.mark.parametrize("T,k,payload_path", [(64, 8, "fused"), (600, 8, "chunked")])
def test_fp8_quantiser_at_extreme_magnitudes(T, k, payload_path):
    """Blocks of 128 columns scaled by powers of two from 2^-120 to 2^120 (bf16
    subnormals included), all-zero and all-negative-zero blocks, signed zeros
    beside non-zero entries, and blocks whose small entries fall far below the
    smallest e4m3 step next to one large entry: codes and
    scales bit-exact against the oracle's IEEE division and encoder, on both
    sides of the range where the kernel divides per element instead of
    through the reciprocal."""
    print(f"[case] fp8 extreme magnitudes T={T} k={k} ({payload_path})", flush=True)
    H, E, N = 1408, 32, 4
    C = T * min(k, E // N)
    shape = api.Shape(T, H, E, k, N, C, api.MOE_PAYLOAD_FP8_E4M3_B128)
    inp = inputs.generate(T, H, E, seed=4242)
    x = inp.x_bits.view(np.uint16).astype(np.uint32) << 16
    base = x.view(np.float32).reshape(T, H // 128, 128)
    xf = base.copy()
    exps = np.array([-120, -100, -90, -81, -79, -72, -70, -40, 0, 40, 70, 86, 88, 90, 100, 120])
    e = exps[(np.arange(T)[:, None] * 5 + np.arange(H // 128)[None, :]) % len(exps)]
    xf *= np.ldexp(np.float32(1), e)[:, :, None].astype(np.float32)
    xf[::7, 3, :] = 0.0                     # all-zero blocks
    xf[1::5, 5, :] = base[1::5, 5, :] * np.float32(2.0 ** -30)  # tiny entries beside one large one
    xf[1::5, 5, 17] = np.float32(3.0)
    xf[2::3, 6, ::9] = np.float32(-0.0)     # signed zeros beside non-zero entries: their
    xf[2::3, 6, 4::9] = np.float32(0.0)     # quotients are -0 and +0 (codes 0x80 and 0x00)
    xf[::11, 7, :] = np.float32(-0.0)       # an all-negative-zero block (scale 0, codes 0)
    xb = inputs.bf16_bits_from_f32(xf.reshape(T, H))
    ids = inputs.random_ids(T, k, E, seed=4243)
    w = inputs.random_weights(T, k, seed=4244)
    g = run_chain(shape, xb, inp.alpha, ids=ids, weights=w)
    check_chain(shape, g, xb, inp.alpha)


@pytest.mark.parametrize("T,E,G,TG,k,zipf,ties", [
    (128, 256, 8, 4, 8, 0.0, False),   # DeepSeek-V3-style group routing
    (4096, 256, 8, 4, 8, 1.2, False),  # with a popularity bias
    (300, 384, 8, 2, 8, 0.0, True),    # many exact ties
    (64, 64, 64, 5, 4, 0.0, False),    # one expert per group
    (200, 256, 4, 2, 8, 0.0, True),    # 16 lanes per group, ties
    (200, 256, 16, 5, 8, 0.0, True),   # 4 lanes per group, ties
    (100, 256, 32, 6, 8, 0.0, False),  # 2 lanes per group
    (100, 512, 8, 3, 8, 0.0, False),   # 8 lanes per group, 8 logits per lane
    (50, 256, 1, 1, 8, 0.0, False),    # one group: plain top-k
    (90, 320, 8, 3, 8, 0.0, True),     # 5 experts per lane, 8 lanes per group
    (90, 320, 8, 3, 8, 1.2, False),    # the same with a popularity bias
    (70, 96, 3, 2, 6, 0.0, False),     # 3 groups of 16 lanes, lanes 48-63 empty
    (30, 1024, 16, 6, 8, 0.0, True),   # 16 experts per lane, 4 lanes per group
    (40, 8, 4, 2, 2, 0.0, True),       # 2 lanes per group, 56 empty lanes
    (60, 40, 5, 2, 4, 0.0, False),     # 5 groups of 8 lanes
    # groups off whole lanes, or wider than the 16-lane DPP merge: LDS copy,
    # one lane per group
    (100, 160, 8, 3, 8, 0.0, True),    # 20 experts per group, 3 per lane
    (80, 120, 8, 3, 6, 0.0, False),    # 15 experts per group (scalar LDS reads)
    (60, 256, 2, 1, 8, 0.0, True),     # 32 lanes per group
])
def test_grouped_route(T, E, G, TG, k, zipf, ties):
    _announce(f"grouped route T={T} E={E} G={G} TG={TG} k={k}")
    inp = inputs.generate(T, 8, E, 41 + E, zipf=zipf)
    logits = inp.logits
    if ties:
        logits = np.random.default_rng(3).integers(-3, 4, size=(T, E)).astype(np.float32)
    lg = torch.from_numpy(logits).cuda()
    b = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    for score in (api.MOE_SCORE_SIGMOID, api.MOE_SCORE_SOFTMAX):
        ids, w = api.moe_route_topk_grouped(lg, b, k, score, G, TG)
        torch.cuda.synchronize()
        o_ids, o_w = oracle.route_topk_grouped(logits, inp.bias, k, score, G, TG)
        assert np.array_equal(ids.cpu().numpy(), o_ids)
        np.testing.assert_allclose(w.cpu().numpy(), o_w, rtol=2.0 ** -20, atol=0)


@pytest.mark.parametrize("S,T,H,E,k,N,C,payload", [
    (32, 128, 7168, 256, 8, 32, 0, 0),    # the whole DeepSeek-V3 EP32 decode world
    (4, 50, 256, 24, 4, 4, 0, 0),
    (3, 100, 256, 16, 4, 4, 160, 1),      # fixed capacity shared by all sources, overflow
    (5, 0, 64, 8, 2, 2, 8, 0),            # no tokens
    # multi-chunk layouts: capacity overflow with fp8, around the one-launch
    # limit (8192 pairs), ids outside [0, E) on both paths
    (6, 256, 512, 64, 8, 8, 1500, 1),
    (4, 128, 256, 32, 8, 4, 0, 0),
    (8, 128, 256, 32, 8, 4, 0, 0),
    (9, 128, 256, 32, 8, 4, 0, 0),
    (5, 256, 256, 48, 4, 6, 900, 0),
    (5, 500, 256, 48, 4, 6, 900, 0),
    (2, 100, 256, 1024, 32, 32, 0, 0),    # E and k at the library maximum, chunked
    # 64 and 72 chunks: whole chunks per source (bases read per source), and
    # sources that split a chunk
    (8, 1024, 64, 256, 8, 32, 0, 0),
    (9, 1024, 64, 256, 8, 32, 0, 0),
    (9, 1000, 64, 64, 8, 8, 0, 0),
])
def test_dispatch_sources(S, T, H, E, k, N, C, payload):
    """Every source rank dispatching at once: segments in (source, token, slot)
    order, the exchanged per-source counts and per-source offsets, then the
    world's combine."""
    _announce(f"sources S={S} T={T} H={H} E={E} k={k} N={N} C={C} p={payload}")
    inp = inputs.generate(S * T, H, E, 77 + S)
    ids = np.stack([inputs.random_ids(T, k, E, 100 + s) for s in range(S)]) if T else \
        np.zeros((S, 0, k), np.int32)
    if T and C == 900:
        ids[1, 3, 2] = E + 5  # ids outside [0, E) are skipped and flagged
        ids[3, 7, 0] = -1
    wts = inputs.random_weights(S * T, k, 5)
    one = api.Shape(T, H, E, k, N, C, payload)
    world = api.world_shape(one, S)
    dev = "cuda"
    x = dev_u16(inp.x_bits) if T else torch.empty(0, H, dtype=torch.int16, device=dev)
    d_ids = torch.from_numpy(ids.reshape(S * T, k).copy()).to(dev)
    lay = api.Layout.empty(world, dev)
    recv, rs = api.alloc_recv(world, dev, fill=0x7F if payload else 0xFFFF)
    ws = api.alloc_workspace(world, dev)
    sc = torch.full((S, E), -9, dtype=torch.int32, device=dev)
    so = torch.full((E, S), -9, dtype=torch.int32, device=dev)
    api.moe_dispatch_sources(one, S, x, d_ids, recv, rs, lay, sc, so, ws)
    torch.cuda.synchronize()
    o = oracle.layout_sources(ids, E, N, C)
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "token_row",
                "source_counts", "source_offsets"):
        got = {"source_counts": sc, "source_offsets": so}.get(key)
        got = getattr(lay, key) if got is None else got
        assert np.array_equal(got.cpu().numpy().reshape(o[key].shape), o[key]), key
    assert int(lay.status.item()) == o["status"]
    if T == 0:
        return
    tr = o["token_row"]
    if payload:
        o_recv, o_rs = oracle.dispatch_fp8(inp.x_bits, tr, o["rows"], fill=0x7F)
        assert np.array_equal(recv.cpu().numpy(), o_recv)
        assert np.array_equal(rs.cpu().numpy().view(np.uint32), o_rs.view(np.uint32))
    else:
        o_recv = oracle.dispatch_bf16(inp.x_bits, tr, o["rows"], fill=0xFFFF)
        assert np.array_equal(host_u16(recv), o_recv)
    out = torch.empty(S * T, H, dtype=torch.int16, device=dev)
    api.moe_combine(world, recv, rs, lay, torch.from_numpy(wts).to(dev), out)
    torch.cuda.synchronize()
    y = recv.cpu().numpy() if payload else host_u16(recv)
    ys = rs.cpu().numpy() if payload else None
    assert np.array_equal(host_u16(out), oracle.combine_f32_ordered(y, ys, tr, wts))
