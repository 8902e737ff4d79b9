"""GPU parity on seeded random shapes: dispatch -> expert stand-in -> combine
through the C ABI against the oracle at every stage, with the same bars as the
hand-picked sweep (layout, rows, fp8 codes and scales, the stand-in bit-exact;
combine within 1 bf16 ulp of the double sum and bit-exact against the fp32
chain in slot order; poisoned buffers with canary rows).

Each case draws, from its own seed: the payload (bf16, or fp8 about a third of
the time), H (a multiple of 8, or of 128 for fp8, up to 8192), E up to 1024
with a rank count N dividing it, k up to min(32, E), T up to 3000 (either path
of the dispatch), packed regions or a capacity that may overflow, distinct or
repeated experts per token, now and then ids outside [0, E), and positive
weights.  Sizes are bounded so that the oracle checks each case in about a
second and the receive buffer stays under 256 MB.  A second set draws token
rows with special values -- scaled by 2^e for e in [-135, 120] (bf16
subnormals to near the fp32 limit, all finite), sprinkled with +0 and -0, or
wholly in the bf16 subnormal range -- and now and then one expert per rank.
"""
import numpy as np
import pytest

from combine_moe_dispatch_amd import api, inputs

from gpu_chain import check_chain, run_chain

pytestmark = pytest.mark.gpu

MAX_RECV_BYTES = 256 << 20
MAX_WORK = 24_000_000   # T * k * H: the oracle's double-precision combine


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


def draw_case(seed):
    rng = np.random.default_rng(90_000 + seed)
    payload = 1 if rng.random() < 0.33 else 0
    H = 128 * int(rng.integers(1, 65)) if payload else 8 * int(rng.integers(1, 1025))
    E = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 1025))]))
    divs = [d for d in _divisors(E) if d <= 256]
    N = int(rng.choice(divs))
    k = int(rng.integers(1, min(32, E) + 1))
    T = int(rng.choice([int(rng.integers(0, 65)), int(rng.integers(65, 3001))]))
    T = min(T, max(1, MAX_WORK // (k * H)))
    row_bytes = H + 4 * (H // 128) if payload else 2 * H
    if rng.random() < 0.4 or T == 0:
        C = 0
    else:
        cap = max(1, min(T * k, MAX_RECV_BYTES // (row_bytes * N)))
        C = int(rng.integers(1, cap + 1))
    if C == 0 and T * k * row_bytes > MAX_RECV_BYTES:
        T = max(1, MAX_RECV_BYTES // (k * row_bytes))
    distinct = bool(rng.random() < 0.6)
    bad = bool(rng.random() < 0.15)
    return T, H, E, k, N, C, payload, distinct, bad


CASES = [draw_case(s) for s in range(60)]


@pytest.mark.parametrize("seed", range(len(CASES)))
def test_random_shape_chain(seed):
    T, H, E, k, N, C, payload, distinct, bad = CASES[seed]
    print(f"[case] random shape seed={seed} T={T} H={H} E={E} k={k} N={N} C={C} "
          f"payload={payload} distinct={distinct} bad={bad}", flush=True)
    inp = inputs.generate(T, H, E, 300 + seed)
    ids = inputs.random_ids(T, k, E, 400 + seed, distinct=distinct)
    if bad and T:
        rng = np.random.default_rng(500 + seed)
        for _ in range(1 + T // 50):
            ids[rng.integers(0, T), rng.integers(0, k)] = int(rng.choice([-1, E, E + 7]))
    wts = inputs.random_weights(T, k, 600 + seed)
    shape = api.Shape(T, H, E, k, N, C, payload)
    g = run_chain(shape, inp.x_bits, inp.alpha, ids=ids, weights=wts)
    check_chain(shape, g, inp.x_bits, inp.alpha)


def _special_rows(x_bits, rng):
    """Finite token rows with special values (see the module docstring)."""
    T = x_bits.shape[0]
    xf = (x_bits.astype(np.uint32) << 16).view(np.float32).copy()
    if T == 0:
        return x_bits
    mode = int(rng.integers(0, 4))
    if mode == 1:
        e = rng.integers(-135, 121, size=(T, 1)).astype(np.int32)
        xf *= np.ldexp(np.float32(1), e).astype(np.float32)
    elif mode == 2:
        m = rng.random(xf.shape)
        xf[m < 0.05] = np.float32(0.0)
        xf[(m >= 0.05) & (m < 0.1)] = np.float32(-0.0)
    elif mode == 3:
        xf *= np.float32(2.0 ** -128)
    return inputs.bf16_bits_from_f32(xf)


@pytest.mark.parametrize("seed", range(30))
def test_random_shape_special_values(seed):
    T, H, E, k, N, C, payload, distinct, _ = draw_case(5000 + seed)
    rng = np.random.default_rng(6000 + seed)
    if rng.random() < 0.15:
        N, C = E, (int(rng.integers(1, 4)) if rng.random() < 0.5 else 0)  # one expert per rank
    print(f"[case] random special values seed={seed} T={T} H={H} E={E} k={k} N={N} C={C} "
          f"payload={payload}", flush=True)
    inp = inputs.generate(T, H, E, 7000 + seed)
    xb = _special_rows(inp.x_bits, rng)
    ids = inputs.random_ids(T, k, E, 8000 + seed, distinct=distinct)
    wts = inputs.random_weights(T, k, 9000 + seed)
    shape = api.Shape(T, H, E, k, N, C, payload)
    g = run_chain(shape, xb, inp.alpha, ids=ids, weights=wts)
    check_chain(shape, g, xb, inp.alpha)
