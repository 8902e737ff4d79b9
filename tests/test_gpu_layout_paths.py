"""GPU parity of the multi-kernel layout in both its forms and at many
chunks, and of every dispatch path with an id list that does not start on a
16-byte boundary.

The multi-kernel layout (past 8192 pairs) ranks pairs inside chunks of 1024
(token, slot) pairs and carries bases across chunks.  Up to 16 chunks it is
one launch whose blocks read the id list in 16-byte vectors, so a misaligned
list takes the two-launch form instead.  These cases reach 9, 16, 17, 64 and
65 chunks (ragged last chunks among them), k = 32 and one rank holding every
expert, and the one-kernel path at its limit.  Each case also runs with its id
list one element into its allocation (4 bytes past a 16-byte boundary), which
the C ABI accepts.  Every stage is checked against the oracle with the bars of
the other parity tests."""
import numpy as np
import pytest

from combine_moe_dispatch_amd import api, inputs

from gpu_chain import check_chain, run_chain

pytestmark = pytest.mark.gpu

CASES = [
    # T, H, E, k, N, C, payload, bad ids
    (8192, 64, 256, 8, 32, 0, 0, False),     # 65536 pairs: 64 chunks
    (8193, 64, 256, 8, 32, 0, 0, True),      # 65 chunks, the last one ragged
    (8192, 128, 96, 8, 3, 21000, 1, False),  # fp8, 64 chunks, a capacity that overflows
    (1025, 64, 1024, 8, 4, 0, 0, True),      # 8200 pairs: just past the one-kernel dispatch
    (2000, 64, 256, 8, 32, 0, 0, True),      # 16 chunks, the last one ragged
    (2049, 64, 256, 8, 32, 0, 0, False),     # 17 chunks
    (2048, 64, 96, 32, 3, 21000, 0, False),  # k = 32, 64 chunks, a capacity that overflows
    (10000, 64, 8, 1, 1, 0, 0, False),       # k = 1, one rank, 10 chunks (ragged)
    (300, 256, 256, 8, 32, 0, 0, True),      # one-kernel dispatch (2400 pairs)
    (1024, 128, 256, 8, 32, 64, 1, False),   # one-kernel fp8 dispatch at its limit (8192 pairs)
]


@pytest.mark.parametrize("misalign", [False, True], ids=["aligned", "misaligned"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_layout_many_chunks(case, misalign):
    T, H, E, k, N, C, payload, bad = CASES[case]
    print(f"[case] layout case={case} misalign={misalign} T={T} H={H} E={E} k={k} N={N} "
          f"C={C} payload={payload} bad={bad}", flush=True)
    inp = inputs.generate(T, H, E, 700 + case)
    ids = inputs.random_ids(T, k, E, 710 + case, distinct=True)
    if bad:
        rng = np.random.default_rng(720 + case)
        for _ in range(1 + T // 50):
            ids[rng.integers(0, T), rng.integers(0, k)] = int(rng.choice([-1, E, E + 7]))
    wts = inputs.random_weights(T, k, 730 + case)
    shape = api.Shape(T, H, E, k, N, C, payload)
    g = run_chain(shape, inp.x_bits, inp.alpha, ids=ids, weights=wts, misalign_ids=misalign)
    check_chain(shape, g, inp.x_bits, inp.alpha)
