"""GPU parity of the small-batch path (batches of at most 256 tokens, ranks up
to 32: one workgroup per 32 x 32 output tile, its four waves splitting the
reduction and adding their partial products in wave order, the rank-r
products of the tile formed in the same kernel, one-split reductions written
directly) against the full oracle, over ragged batches, widths, ranks and the
three weight formats; and at the boundary (256 and 257 tokens) where the main
kernels take over."""
import numpy as np
import pytest

from synthetic import random_linear
from tests.test_gpu_parity import _linear_case
from tests._util import TOL

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


CASES = [
    (1, 64, 8, 1),        # one token, one block, the narrowest output, rank 1
    (31, 128, 200, 8),    # ragged token tile and output tile (200 = 6 x 32 + 8)
    (33, 192, 264, 13),   # two token tiles, unaligned rank, three 64-column blocks
    (100, 512, 512, 16),
    (256, 512, 512, 8),   # the tiny workload's shape
    (256, 640, 136, 32),  # largest rank of the path, rows past the last full 64-row group
    (200, 4096, 1024, 24),
    (257, 512, 512, 8),   # just past the path: the main kernels
]


@pytest.mark.parametrize("M,K,N,r", CASES)
@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_small_batch_full_oracle(M, K, N, r, fmt):
    _announce(f"small batch M={M} K={K} N={N} r={r} fmt={fmt}")
    d = random_linear(40_000 + M + K + N + r + fmt, M, K, N, r)
    errs = _linear_case(d, fmt=fmt)
    assert max(errs.values()) <= TOL, errs
