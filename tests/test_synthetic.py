"""The counter-based input generator gives the same bits on the host (numpy)
and in torch, and any slice equals the same slice of a full draw."""
import numpy as np

from synthetic import counter_normal


def test_counter_normal_host_and_torch_agree():
    import torch
    idx = np.concatenate([np.arange(0, 1 << 16), np.array([2**31 - 1, 2**31, 2**32 - 1])]).astype(np.int64)
    a = counter_normal(5, idx, 0.02)
    b = counter_normal(5, torch.from_numpy(idx), 0.02).numpy()
    assert a.dtype == np.float32 and b.dtype == np.float32
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_counter_normal_slices_and_moments():
    full = counter_normal(9, np.arange(1 << 20, dtype=np.int64), 1.0)
    part = counter_normal(9, np.arange(4096, 8192, dtype=np.int64), 1.0)
    assert np.array_equal(part, full[4096:8192])
    assert abs(float(full.mean())) < 5e-3 and abs(float(full.std()) - 1.0) < 5e-3
    assert float(np.abs(full).max()) <= np.sqrt(6.0)
    # other seeds give other draws
    assert not np.array_equal(counter_normal(10, np.arange(64, dtype=np.int64)), full[:64])


def test_useful_flops_match_the_per_config_table():
    # useful work of one fwd+bwd, 4MNK + 6Mr(N+K) per projection (no dequant work,
    # no padding): the GFLOP the measurement table gives per workload
    from synthetic import useful_flops
    want = {0: 0.281, 1: 278.1, 2: 2908.0, 4: 14423.0}
    for c, g in want.items():
        assert abs(useful_flops(c) / 1e9 - g) <= 0.5e-3 * g + 1e-3, (c, useful_flops(c))
    for i, g in enumerate((553.0, 556.0, 576.0, 601.0)):  # rank sweep r = 8, 16, 64, 128
        assert abs(useful_flops(3, i) / 1e9 - g) <= 0.6, (i, useful_flops(3, i))
    # the closed form at the attn shape
    M = K = N = 4096
    r = 16
    assert useful_flops(1) == 4 * M * N * K + 6 * M * r * (N + K)
