"""GPU checks of RoPE fused into the q/k projection GEMM ("Unsloth" wiki entry,
Theory: fused RoPE kernel): Y = rope(X.W^T + s.(X.A^T).B^T) through
qlora_forward_rope against the oracle's linear forward followed by its RoPE
(max|err|/max|ref| <= 1e-2), and the cos/sin table against fp64 cos/sin."""
import numpy as np
import pytest

from oracle import normrope, ref
from synthetic import make_workload, packed_positions, random_linear
from tests._util import TOL, Prepared, dev_bf16, host, rel_err, sample_rows

pytestmark = pytest.mark.gpu

D, BASE = 128, 500000.0


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def test_rope_table_matches_fp64_cos_sin():
    _announce("rope table d=128 max_pos=20000")
    import parameter_efficient_fine_amd as q
    t = q.rope_table(D, BASE, 20000).cpu().numpy().astype(np.float64)
    a = normrope.rope_angles(np.arange(20000), D, BASE)
    assert t.shape == (20000, D // 2, 2)
    # fp32 values of fp64 cos/sin: within one fp32 rounding
    assert np.max(np.abs(t[:, :, 0] - np.cos(a))) <= 2.0 ** -24
    assert np.max(np.abs(t[:, :, 1] - np.sin(a))) <= 2.0 ** -24
    assert np.array_equal(t[0, :, 0], np.ones(D // 2)) and not t[0, :, 1].any()  # position 0: the identity


def _case(d, pos, max_pos, rows=None, check_unfused=True, fmt=0):
    import torch
    import parameter_efficient_fine_amd as q
    P = Prepared(d["layers"]["proj"], d["s"], fmt=fmt)
    X = dev_bf16(d["X"])
    table = q.rope_table(D, BASE, max_pos)
    posd = torch.from_numpy(pos.astype(np.int32)).cuda()
    Y, Z = q.forward_rope(P.dev, X, posd, table)
    Xf = ref.bf16_to_f64(d["X"])
    sel = slice(None) if rows is None else rows
    Yl, Zr = ref.linear_fwd(Xf[sel], *P.triple(), P.s)
    Yr = normrope.rope(Yl, pos[sel], D, BASE)
    errs = dict(Y=rel_err(host(Y)[sel], Yr), Z=rel_err(host(Z)[sel], Zr))
    assert max(errs.values()) <= TOL, errs
    # the rotation is visible: the unrotated result is further off than the tolerance
    assert rel_err(Yl, Yr) > TOL
    if check_unfused:
        # the unfused path (bf16 GEMM output, then the standalone RoPE kernel) agrees
        Y2, _ = q.forward(P.dev, X)
        q.rope_forward(Y2, None, posd, D, BASE)
        assert rel_err(host(Y2)[sel], host(Y)[sel]) <= TOL
    return host(Y)


@pytest.mark.parametrize("M,K,N,r", [
    (300, 256, 512, 16),    # ragged token tile, 4 heads
    (77, 192, 384, 8),      # 3 heads: the last column tile holds one head
    (513, 128, 128, 24),    # one head, unaligned rank rows
])
def test_forward_rope_small_full_oracle(M, K, N, r):
    _announce(f"forward_rope M={M} K={K} N={N} r={r}")
    d = random_linear(30_000 + M + K + N + r, M, K, N, r)
    pos = packed_positions(np.random.default_rng(M + N), M, 1000)
    _case(d, pos, 1000)


@pytest.mark.parametrize("fmt", [1, 2])
def test_forward_rope_8bit_weights(fmt):
    # the fused epilogue behind the INT8 and FP8 weight decoders, ragged token tile
    _announce(f"forward_rope fmt={fmt} M=300 K=256 N=512 r=16")
    d = random_linear(30_700 + fmt, 300, 256, 512, 16)
    pos = packed_positions(np.random.default_rng(700 + fmt), 300, 1000)
    _case(d, pos, 1000, fmt=fmt)


def _random_rope_shapes(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(16, 1500)), 64 * int(rng.integers(1, 9)), 128 * int(rng.integers(1, 9)),
             int(rng.integers(1, 129)), int(rng.integers(0, 3)), int(rng.integers(64, 3000))) for _ in range(n)]


@pytest.mark.parametrize("M,K,N,r,fmt,max_pos", _random_rope_shapes(6, 9292))
def test_forward_rope_random_shapes(M, K, N, r, fmt, max_pos):
    _announce(f"forward_rope random M={M} K={K} N={N} r={r} fmt={fmt} max_pos={max_pos}")
    d = random_linear(31_000 + M + K + N + r, M, K, N, r)
    pos = packed_positions(np.random.default_rng(M + max_pos), M, max_pos)
    _case(d, pos, max_pos, fmt=fmt)


def test_forward_rope_attn_q_projection_full_size():
    # the Llama-3-8B q projection (32 heads of 128), M=4096, packed sequences up to 4096
    _announce("forward_rope attn M=4096 K=N=4096 r=16")
    d = make_workload(1)
    pos = packed_positions(np.random.default_rng(41), d["M"], 4096)
    rows = sample_rows(d["M"], np.random.default_rng(42), per_block=1)
    _case(d, pos, 4096, rows)


def test_forward_rope_k_projection_long_context():
    # the GQA k projection (8 heads of 128, 4096 -> 1024) at M=16384 positions
    _announce("forward_rope k-proj M=16384 K=4096 N=1024 r=16")
    d = random_linear(43, 16384, 4096, 1024, 16)
    pos = packed_positions(np.random.default_rng(44), d["M"], 16384)
    rows = sample_rows(d["M"], np.random.default_rng(45), per_block=1, block=512)
    _case(d, pos, 16384, rows)


def test_forward_rope_positions_outside_the_table_give_zero_rows():
    _announce("forward_rope out-of-table positions")
    import torch
    import parameter_efficient_fine_amd as q
    d = random_linear(46, 64, 128, 256, 16)
    pos = np.arange(64, dtype=np.int32)
    pos[[5, 40]] = [100, -3]  # table covers 0..63
    P = Prepared(d["layers"]["proj"], d["s"])
    Y, _ = q.forward_rope(P.dev, dev_bf16(d["X"]), torch.from_numpy(pos).cuda(), q.rope_table(D, BASE, 64))
    Yh = host(Y)
    assert not Yh[5].any() and not Yh[40].any() and Yh[6].any()
