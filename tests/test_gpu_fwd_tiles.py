"""GPU: the forward GEMM's 128-token tiles (taken where 256-token tiles would leave
CUs idle) give the same bits as its 256-token tiles: every output element sums
the same products in the same order. A batch whose grid fills the chip runs on
256-token tiles; slices of it, run as batches of their own, take 128-token tiles
and must reproduce its rows exactly."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ref
from synthetic import random_linear
from tests._util import TOL, Prepared, dev_bf16, host, rel_err, sample_rows

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy()


# (M, K, N, r, alpha, fmt, slice): with N = 4096 a batch of M = 4096 tokens fills
# the chip with 256-token tiles (16 x 16 workgroups); slices of 1000-1024 tokens
# take 128-token tiles (16 x 8), the 1000-token ones with a ragged last tile;
# also a ragged column count (N = 4000), the rank buckets of 128 and 256 (r = 200
# with its rank rows unaligned), and 300-token slices just above the small-batch
# kernels' 256 tokens (3 tiles of 128, the last one ragged).
CASES = [
    (4096, 512, 4096, 16, 32, 0, 1024),
    (4096, 256, 4096, 16, 24, 0, 1000),
    (4096, 256, 4096, 48, 96, 1, 1024),
    (4096, 256, 4096, 8, 16, 2, 1000),
    (4096, 256, 4000, 16, 32, 0, 1000),
    (4096, 256, 4096, 128, 128, 0, 1024),
    (4096, 320, 4096, 200, 64, 1, 1000),
    (4096, 256, 4096, 16, 32, 2, 300),
]


@pytest.mark.parametrize("M,K,N,r,alpha,fmt,sl", CASES)
def test_forward_128_token_tiles_equal_256_token_tiles_bitwise(M, K, N, r, alpha, fmt, sl):
    print(f"[case] fwd tiles M={M} K={K} N={N} r={r} alpha={alpha} fmt={fmt} slices of {sl}", flush=True)
    import torch
    import parameter_efficient_fine_amd as q
    d = random_linear(72_000 + K + r + fmt, M, K, N, r, alpha=alpha)
    P = Prepared(d["layers"]["proj"], d["s"], fmt=fmt)
    X = dev_bf16(d["X"])
    Y, Z = q.forward(P.dev, X)
    torch.cuda.synchronize()
    Yb, Zb = _bits(Y), _bits(Z)
    for a in range(0, M, sl):
        b = min(M, a + sl)
        if b - a <= 256:  # the small-batch kernels sum in another order
            continue
        Ys, Zs = q.forward(P.dev, X[a:b].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(_bits(Zs), Zb[a:b]), (a, b)
        assert np.array_equal(_bits(Ys), Yb[a:b]), (a, b)
    # and one slice against the oracle on sampled rows of every 128-token tile
    rows = sample_rows(sl, np.random.default_rng(sl + fmt), per_block=2, block=128)
    Ys, _ = q.forward(P.dev, X[:sl].contiguous())
    Yr, _ = ref.linear_fwd(ref.bf16_to_f64(d["X"][:sl])[rows], *P.triple(), P.s)
    assert rel_err(host(Ys)[rows], Yr) <= TOL
