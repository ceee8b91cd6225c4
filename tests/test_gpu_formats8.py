"""GPU parity of the 8-bit frozen-weight formats (INT8, FP8 E4M3; "Rev vs
unsloth", fused quantized-LoRA card) against the oracle (oracle/formats8.py):
codes, scales and dequantized weights bit-exact; the fused layer and the
SwiGLU block to max|err|/max|ref| <= 1e-2, as for the 4-bit format."""
import numpy as np
import pytest

from oracle import formats8 as f8
from synthetic import make_workload, random_linear, random_mlp
from tests._util import TOL, dev_f32, host, sample_rows, tile_major
from tests.test_gpu_parity import _linear_case, _mlp_case

pytestmark = pytest.mark.gpu

FMTS = [f8.FMT_INT8, f8.FMT_FP8]


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _check_quant(W, fmt):
    import parameter_efficient_fine_amd as q
    codes, scale = q.quantize(dev_f32(W), fmt)
    c_ref, s_ref = f8.quantize(W, fmt)
    # stored tile-major (a permutation of the row-major bytes)
    assert np.array_equal(host(codes), tile_major(c_ref, 64))
    assert np.array_equal(host(scale).astype(np.float32).view(np.uint32), tile_major(s_ref, 1).view(np.uint32))
    Wh = q.dequantize(codes, scale, fmt)
    assert np.array_equal(Wh.cpu().numpy().view(np.uint32), f8.dequantize(c_ref, s_ref, fmt).view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_bitexact_on_workload_weights(fmt):
    _announce(f"quantize fmt={fmt} attn and MLP weights")
    d = make_workload(1)
    _check_quant(d["layers"]["proj"]["W"], fmt)
    d = make_workload(2)
    _check_quant(d["layers"]["down"]["W"], fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_bitexact_edge_blocks(fmt):
    _announce(f"quantize fmt={fmt} edge blocks")
    qmax = 127.0 if fmt == f8.FMT_INT8 else 448.0
    W = np.zeros((24, 128), np.float32)
    W[1, :64] = -0.0
    # scale exactly 1: every half-way point between neighbouring codes, and its neighbours
    vals = np.arange(-127, 128, dtype=np.float64) if fmt == f8.FMT_INT8 else f8.E4M3_VALUES[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    for row, arr in ((2, mids), (3, np.nextafter(mids, np.float32(1e9))), (4, np.nextafter(mids, np.float32(-1e9)))):
        n = min(len(arr), 63)
        for blk in range(2):
            sl = arr[blk * 63: blk * 63 + n] if blk * 63 < len(arr) else arr[:n]
            W[row, 64 * blk: 64 * blk + len(sl)] = sl
            W[row, 64 * blk + 63] = qmax
    W[5, :8] = np.array([3e-40, -5e-41, 1e-42, 0, -3e-40, 2e-40, 1e-45, -1e-45], np.float32)  # denormals
    W[6, 64:] = np.float32(1e-38)
    W[7] = np.float32(-7.5)
    rng = np.random.default_rng(4)
    W[8:] = rng.standard_normal((16, 128)).astype(np.float32) * np.float32(100.0)
    _check_quant(W, fmt)


def test_fp8_decode_of_every_code():
    # every finite E4M3 byte through the decoder the GEMMs use, at several scales
    _announce("fp8 decode of all codes")
    import torch
    import parameter_efficient_fine_amd as q
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] * 2, dtype=np.uint8)[:448].reshape(7, 64)
    scale = np.array([[1.0], [2.0 ** -7], [3.0e-3], [1.0 / 448.0], [7.25], [1e-20], [2.0 ** 40]], np.float32)
    Wh = q.dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(), f8.FMT_FP8)
    assert np.array_equal(Wh.cpu().numpy().view(np.uint32), f8.dequantize(codes, scale, f8.FMT_FP8).view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_tiny_full_oracle(fmt):
    _announce(f"linear fmt={fmt} tiny")
    errs = _linear_case(make_workload(0), fmt=fmt)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,N,r", [
    (300, 192, 264, 8),
    (77, 256, 1000, 5),
    (129, 320, 512, 128),
    (700, 448, 200, 132),
])
def test_linear_ragged_full_oracle(fmt, M, K, N, r):
    _announce(f"linear fmt={fmt} ragged M={M} K={K} N={N} r={r}")
    errs = _linear_case(random_linear(20_000 + M + K + N + r, M, K, N, r), fmt=fmt)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_attn_projection_full_size(fmt):
    _announce(f"linear fmt={fmt} attn M=4096 K=N=4096 r=16")
    d = make_workload(1)
    errs = _linear_case(d, sample_rows(d["M"], np.random.default_rng(41)), fmt=fmt)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("fmt", FMTS)
def test_mlp_small_full_oracle(fmt):
    _announce(f"mlp fmt={fmt} M=300 H=256 I=512 r=16")
    errs = _mlp_case(random_mlp(177, 300, 256, 512, 16), fmt=fmt)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("fmt", FMTS)
def test_mlp_full_size(fmt):
    # the SwiGLU block at the Llama-3.1-8B widths (M=4096, H=4096, I=14336, r=16) with
    # 8-bit weights, on sampled rows (the upstream gradient zero elsewhere, so dA and
    # dB are exact over the batch)
    _announce(f"mlp fmt={fmt} M=4096 H=4096 I=14336 r=16")
    d = make_workload(2)
    rows = sample_rows(d["M"], np.random.default_rng(43), per_block=1)
    errs = _mlp_case(d, rows, mask_dy=True, fmt=fmt)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("fmt", FMTS)
def test_decoder_layer_full_size(fmt):
    # the 7 projections of a Llama-3.1-8B decoder layer at M=16384 with 8-bit weights,
    # on sampled rows (the SwiGLU block with its upstream gradient zero elsewhere)
    _announce(f"decoder layer fmt={fmt} M=16384, 7 projections")
    d = make_workload(4)
    M = d["M"]
    rows = sample_rows(M, np.random.default_rng(44), per_block=1, block=1024)
    errs = {}
    for nm, xk in (("q", "X_attn"), ("k", "X_attn"), ("v", "X_attn"), ("o", "X_o")):
        sub = dict(layers={"proj": d["layers"][nm]}, X=d[xk], dY=d["dY_" + nm], s=d["s"], M=M)
        for k, v in _linear_case(sub, rows, check_z=False, fmt=fmt).items():
            errs[f"{nm}.{k}"] = v
    mlp = dict(layers={k: d["layers"][k] for k in ("gate", "up", "down")}, X=d["X_mlp"], dY=d["dY_mlp"], M=M,
               s=d["s"])
    for k, v in _mlp_case(mlp, rows, mask_dy=True, fmt=fmt).items():
        errs["mlp." + k] = v
    assert max(errs.values()) <= TOL, errs
