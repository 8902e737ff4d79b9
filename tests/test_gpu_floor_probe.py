"""The combine-shaped floor probe of libmoe_ceiling.so gathers what it is
asked to: each output vector is the xor of the token's k row vectors (rows
from the list, or rows t*k+j), rows outside the buffer left out.  A floor
that moved other bytes would not measure the combine's data movement."""
import ctypes
import os

import numpy as np
import pytest

from combine_moe_dispatch_amd import api


@pytest.mark.gpu
@pytest.mark.parametrize("T,k,nvec,with_rows", [(5, 3, 70, True), (5, 3, 70, False),
                                                 (3, 9, 130, True)])
def test_rows_gather_probe(T, k, nvec, with_rows):
    import torch
    print(f"[case] rows_gather T={T} k={k} nvec={nvec} rows={with_rows}", flush=True)
    lib = ctypes.CDLL(os.path.join(os.path.dirname(api.LIB_PATH), "libmoe_ceiling.so"))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.moe_ceiling_rows_gather.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    rng = np.random.default_rng(T * 100 + k)
    rows_total = T * k + 4
    y = rng.integers(0, 2 ** 32, size=(rows_total, nvec, 4), dtype=np.uint32)
    rows = rng.integers(-1, rows_total + 2, size=(T, k)).astype(np.int32)
    dev = "cuda:0"
    yd = torch.from_numpy(y.view(np.int32)).to(dev)
    rd = torch.from_numpy(rows).to(dev)
    out = torch.full((T, nvec, 4), -1, dtype=torch.int32, device=dev)
    rc = lib.moe_ceiling_rows_gather(yd.data_ptr(), rd.data_ptr() if with_rows else None,
                                     out.data_ptr(), T, k, nvec, rows_total, None)
    assert rc == 0
    torch.cuda.synchronize()
    want = np.zeros((T, nvec, 4), dtype=np.uint32)
    for t in range(T):
        for j in range(k):
            r = int(rows[t, j]) if with_rows else t * k + j
            if 0 <= r < rows_total:
                want[t] ^= y[r]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
