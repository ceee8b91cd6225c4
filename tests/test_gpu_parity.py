"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact on 4-bit codes, absmax and dequantized weights; max|err|/max|ref|
<= 1e-2 on Y, Z, dX (bf16) and dA, dB (fp32), with fp32 accumulation on the
GPU. At full workload sizes the oracle computes sampled rows of Y and dX (rows
are independent) and the exact dA, dB (they need no weight product); for the
SwiGLU block at full size the upstream gradient is zero outside sampled rows,
so every gradient the GPU produces involves those rows only and the oracle can
compute all of them exactly.
"""
import numpy as np
import pytest

from oracle import ref
from oracle.codebook import NF4_LEVELS, NF4_THRESHOLDS
from synthetic import WORKLOADS, bf16_bits, make_workload, random_linear, random_mlp, projections
from tests._util import TOL, Prepared, dev_bf16, dev_f32, device_codes, host, rel_err, sample_rows, tile_major

pytestmark = pytest.mark.gpu


def _q():
    import parameter_efficient_fine_amd as q
    return q


def _announce(msg):
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------------------
# quantization: bit-exact

def _check_quant(W):
    q = _q()
    codes, absmax = q.quantize(dev_f32(W))
    c_ref, a_ref = ref.quantize(W)
    # the library stores codes and absmax tile-major, NF4 codes in runs of 8 columns
    # (a permutation of the oracle's nibbles)
    assert np.array_equal(host(codes), device_codes(c_ref, 0))
    assert np.array_equal(host(absmax).astype(np.float32).view(np.uint32), tile_major(a_ref, 1).view(np.uint32))
    Wh = q.dequantize(codes, absmax)
    assert np.array_equal(Wh.cpu().numpy().view(np.uint32), ref.dequantize(c_ref, a_ref).view(np.uint32))


@pytest.mark.parametrize("c", [0, 1, 2, 4])
def test_quantize_bitexact_on_workload_weights(c):
    _announce(f"quantize workload {c}")
    projs, r = projections(c)
    rng = np.random.default_rng(1000 * c)
    seen = set()
    for name, K, N in projs:
        if (K, N) in seen:
            continue
        seen.add((K, N))
        W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
        _check_quant(W)


def test_quantize_bitexact_edge_blocks():
    _announce("quantize edge blocks")
    W = np.zeros((40, 128), np.float32)
    W[1, :64] = -0.0
    for j in range(15):  # exact thresholds with absmax 1: ties go to the lower level
        W[2 + j, 0] = 1.0
        W[2 + j, 1] = NF4_THRESHOLDS[j]
        W[2 + j, 2] = np.nextafter(NF4_THRESHOLDS[j], np.float32(2))
        W[2 + j, 3] = np.nextafter(NF4_THRESHOLDS[j], np.float32(-2))
    W[20, :16] = NF4_LEVELS * np.float32(0.037)
    W[21, :8] = np.array([3e-40, -5e-41, 1e-42, 0, -3e-40, 2e-40, 1e-45, -1e-45], np.float32)  # denormals
    W[22, 64:] = np.float32(1e-38)
    W[23] = np.float32(-7.5)
    rng = np.random.default_rng(3)
    W[24:] = rng.standard_normal((16, 128)).astype(np.float32) * np.float32(100.0)
    _check_quant(W)


def test_quantize_reports_nonfinite():
    _announce("quantize non-finite")
    q = _q()
    W = np.zeros((4, 128), np.float32)
    W[2, 70] = np.inf
    with pytest.raises(ValueError):
        q.quantize(dev_f32(W))


# ---------------------------------------------------------------------------
# one projection: full oracle on small shapes

def _linear_case(d, rows=None, check_z=True, fmt=0):
    """Run GPU fwd+bwd on workload dict d (weight format fmt); compare to the oracle (optionally on sampled rows)."""
    q = _q()
    P = Prepared(d["layers"]["proj"], d["s"], fmt=fmt)
    X16, dY16 = d["X"], d["dY"]
    Xd, dYd = dev_bf16(X16), dev_bf16(dY16)
    Y, Z = q.forward(P.dev, Xd)
    dX, dA, dB = q.backward(P.dev, dYd, Xd, Z)
    X = ref.bf16_to_f64(X16)
    dY = ref.bf16_to_f64(dY16)
    sel = slice(None) if rows is None else rows
    Yr, Zr = ref.linear_fwd(X[sel], *P.triple(), P.s)
    dXr, _, _ = ref.linear_bwd(dY[sel], X[sel], *P.triple(), P.s)
    dAr, dBr = ref.adapter_grads(dY, X, P.A, P.B, P.s)
    errs = dict(Y=rel_err(host(Y)[sel], Yr), dX=rel_err(host(dX)[sel], dXr), dA=rel_err(host(dA), dAr),
                dB=rel_err(host(dB), dBr))
    if check_z:
        errs["Z"] = rel_err(host(Z)[sel], Zr)
    # the test can see the adapter: dropping it moves each checked output by more than the tolerance
    Y0, _ = ref.linear_fwd(X[sel], *P.triple(), 0.0)
    dX0, _, _ = ref.linear_bwd(dY[sel], X[sel], *P.triple(), 0.0)
    assert rel_err(Y0, Yr) > TOL and rel_err(dX0, dXr) > TOL
    return errs


def test_linear_tiny_workload_full_oracle():
    _announce("linear tiny M=256 K=N=512 r=8")
    errs = _linear_case(make_workload(0))
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("M,K,N,r", [
    (300, 192, 264, 8),     # ragged M, K not a multiple of the 256 tile, ragged N reduction
    (1, 64, 8, 1),          # smallest shapes, rank 1
    (77, 256, 1000, 5),     # odd rank (unaligned rank rows)
    (513, 640, 136, 24),
    (260, 512, 512, 64),
    (129, 320, 512, 128),
    (64, 128, 256, 256),    # largest rank
    (2000, 1024, 384, 16),  # many row splits in the rank reductions, ragged last split
    (700, 448, 200, 132),   # rank > 128 (reductions in chunks), rank % 8 != 0
    (8200, 128, 136, 24),   # two 16-row fragments per rank-product workgroup, ragged last group
    (16400, 64, 72, 40),    # four fragments per workgroup, ragged last group
    (8232, 64, 80, 200),    # rank 200 with two fragments per workgroup
    (300, 192, 200, 16),    # B read in place (rank 16) with a ragged last 32-row step of G = dY.B
    (77, 256, 136, 32),     # the same at rank 32
    (520, 128, 8, 64),      # N = 8: one ragged step only
])
def test_linear_ragged_shapes_full_oracle(M, K, N, r):
    _announce(f"linear ragged M={M} K={K} N={N} r={r}")
    d = random_linear(10_000 + M + K + N + r, M, K, N, r)
    errs = _linear_case(d)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("r", [48, 80, 96, 112, 144, 160, 192, 240])
def test_linear_ranks_multiple_of_16_not_a_power_of_two(r):
    # B is read in place for G = dY.B only at ranks 16, 32, 64, 128 and 256 (the
    # forms skinny_nt has); these ranks take the transposed copy of B instead
    _announce(f"linear rank {r} M=700 K=256 N=200")
    d = random_linear(61_000 + r, 700, 256, 200, r)
    errs = _linear_case(d)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("M,K,N,r,alpha", [
    (300, 192, 264, 16, 24.0),    # s = 1.5: s.B and s.A^T split into two nonzero bf16 parts
    (513, 640, 136, 24, 7.2),     # s = 0.3
    (129, 320, 512, 128, 12.8),   # s = 0.1, the largest rank bucket of the fused GEMMs
    (200, 256, 256, 8, 12.0),     # s = 1.5 on the small-batch path (M <= 256, r <= 32)
])
def test_linear_scale_not_a_power_of_two(M, K, N, r, alpha):
    # With s a power of two the low parts of the split s-scaled adapter rows are
    # zero and the GEMMs skip their MFMAs; these cases take the low parts.
    _announce(f"linear s={alpha / r:g} M={M} K={K} N={N} r={r}")
    d = random_linear(50_000 + M + K + N + r, M, K, N, r, alpha=alpha)
    errs = _linear_case(d)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("grad_bf16", [False, True])
def test_linear_backward_without_dx_matches_the_one_with_dx(grad_bf16):
    # Without dX the split partials of dA and dB are added by their own reduce
    # launch; with dX, by the backward GEMM's prologue. Same partials, same split
    # order: the gradients agree bit for bit, and with the oracle.
    _announce(f"linear backward without dX M=2000 K=1024 N=384 r=16 bf16={grad_bf16}")
    import torch
    q = _q()
    d = random_linear(4343, 2000, 1024, 384, 16)
    P = Prepared(d["layers"]["proj"], d["s"], grad_dtype=torch.bfloat16 if grad_bf16 else torch.float32)
    Xd, dYd = dev_bf16(d["X"]), dev_bf16(d["dY"])
    _, Z = q.forward(P.dev, Xd)
    _, dA1, dB1 = q.backward(P.dev, dYd, Xd, Z)
    _, dA0, dB0 = q.backward(P.dev, dYd, Xd, Z, need_dX=False)
    bits = (lambda t: t.contiguous().view(torch.int16 if grad_bf16 else torch.int32).cpu().numpy())
    assert np.array_equal(bits(dA0), bits(dA1)) and np.array_equal(bits(dB0), bits(dB1))
    dAr, dBr = ref.adapter_grads(ref.bf16_to_f64(d["dY"]), ref.bf16_to_f64(d["X"]), P.A, P.B, P.s)
    errs = dict(dA=rel_err(host(dA0), dAr), dB=rel_err(host(dB0), dBr))
    assert max(errs.values()) <= TOL, errs


def test_linear_empty_batch_gives_zero_gradients():
    _announce("linear M=0")
    q = _q()
    import torch
    d = random_linear(5, 4, 128, 64, 8)
    P = Prepared(d["layers"]["proj"], d["s"])
    X = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    Y, Z = q.forward(P.dev, X)
    assert Y.shape == (0, 64)
    _, dA, dB = q.backward(P.dev, dY, X, Z, need_dX=False,
                           out=(None, torch.full((8, 128), 7.0, device="cuda"), torch.full((64, 8), 7.0, device="cuda")))
    assert float(dA.abs().max()) == 0.0 and float(dB.abs().max()) == 0.0


# ---------------------------------------------------------------------------
# full-size workloads

def test_linear_attn_projection_full_size():
    _announce("linear attn M=4096 K=N=4096 r=16")
    d = make_workload(1)
    rows = sample_rows(d["M"], np.random.default_rng(1))
    errs = _linear_case(d, rows)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("sub", [0, 1, 2, 3])
def test_rank_sweep_full_size(sub):
    r = WORKLOADS[3]["ranks"][sub]
    _announce(f"rank sweep M=8192 K=N=4096 r={r}")
    d = make_workload(3, sub)
    rows = sample_rows(d["M"], np.random.default_rng(30 + sub), per_block=1)
    errs = _linear_case(d, rows)
    assert max(errs.values()) <= TOL, errs


# ---------------------------------------------------------------------------
# SwiGLU block

def _mlp_case(d, rows=None, mask_dy=False, fmt=0):
    q = _q()
    Ls = {nm: Prepared(d["layers"][nm], d["s"], fmt=fmt) for nm in ("gate", "up", "down")}
    dY16 = d["dY"].copy()
    if mask_dy:
        keep = np.zeros(d["M"], bool)
        keep[rows] = True
        dY16[~keep] = 0
    Xd, dYd = dev_bf16(d["X"]), dev_bf16(dY16)
    f = q.mlp_forward(Ls["gate"].dev, Ls["up"].dev, Ls["down"].dev, Xd)
    b = q.mlp_backward(Ls["gate"].dev, Ls["up"].dev, Ls["down"].dev, dYd, Xd, f)
    X = ref.bf16_to_f64(d["X"])
    dY = ref.bf16_to_f64(dY16)
    sel = slice(None) if rows is None else rows
    trip = [Ls[nm].triple() for nm in ("gate", "up", "down")]
    fr = ref.mlp_fwd(X[sel], *trip, d["s"])
    br = ref.mlp_bwd(dY[sel], X[sel], *trip, d["s"])
    errs = dict(Y=rel_err(host(f["Y"])[sel], fr["Y"]), g=rel_err(host(f["g"])[sel], fr["g"]),
                u=rel_err(host(f["u"])[sel], fr["u"]), h=rel_err(host(f["h"])[sel], fr["h"]),
                dX=rel_err(host(b["dX"])[sel], br["dX"]))
    if rows is None or mask_dy:
        for i, nm in enumerate(("gate", "up", "down")):
            errs["dA_" + nm] = rel_err(host(b["dA"][i]), br["dA_" + nm])
            errs["dB_" + nm] = rel_err(host(b["dB"][i]), br["dB_" + nm])
    if mask_dy:
        other = np.ones(d["M"], bool)
        other[rows] = False
        assert float(np.max(np.abs(host(b["dX"])[other]))) == 0.0
    # adapter visibility: with every adapter off (s = 0) each checked output moves
    # by more than the tolerance; so does Y with only the down adapter off (B_down = 0)
    # and dX with only the gate/up adapters off (B_gate = B_up = 0)
    f0 = ref.mlp_fwd(X[sel], *trip, 0.0)
    b0 = ref.mlp_bwd(dY[sel], X[sel], *trip, 0.0)
    for k in ("Y", "g", "u", "h"):
        assert rel_err(f0[k], fr[k]) > TOL, k
    assert rel_err(b0["dX"], br["dX"]) > TOL
    no_down = trip[:2] + [(trip[2][0], trip[2][1], np.zeros_like(trip[2][2]))]
    assert rel_err(ref.mlp_fwd(X[sel], *no_down, d["s"])["Y"], fr["Y"]) > TOL
    no_gu = [(t[0], t[1], np.zeros_like(t[2])) for t in trip[:2]] + trip[2:]
    assert rel_err(ref.mlp_bwd(dY[sel], X[sel], *no_gu, d["s"])["dX"], br["dX"]) > TOL
    return errs


def test_mlp_small_full_oracle():
    _announce("mlp small M=300 H=256 I=512 r=16")
    errs = _mlp_case(random_mlp(77, 300, 256, 512, 16))
    assert max(errs.values()) <= TOL, errs


def test_mlp_ragged_full_oracle():
    _announce("mlp ragged M=130 H=192 I=320 r=8")
    errs = _mlp_case(random_mlp(78, 130, 192, 320, 8))
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("r", [72, 132, 200])
def test_mlp_high_rank_full_oracle(r):
    # 2r > 128: gate/up dA reductions run as separate launches; r = 200 also
    # splits the forward's paired Z = X.[A_g; A_u]^T (2r > 256)
    _announce(f"mlp high rank M=200 H=128 I=256 r={r}")
    errs = _mlp_case(random_mlp(90 + r, 200, 128, 256, r))
    assert max(errs.values()) <= TOL, errs


def test_mlp_scale_not_a_power_of_two():
    _announce("mlp s=1.5 M=300 H=256 I=512 r=16")
    errs = _mlp_case(random_mlp(81, 300, 256, 512, 16, alpha=24.0))
    assert max(errs.values()) <= TOL, errs


def test_mlp_long_batch_full_oracle():
    # M large enough that the rank products put several 16-row fragments in a workgroup
    _announce("mlp long batch M=16400 H=64 I=128 r=16")
    errs = _mlp_case(random_mlp(79, 16400, 64, 128, 16))
    assert max(errs.values()) <= TOL, errs


def test_mlp_full_size():
    _announce("mlp M=4096 H=4096 I=14336 r=16")
    d = make_workload(2)
    rows = sample_rows(d["M"], np.random.default_rng(2), per_block=1)
    errs = _mlp_case(d, rows, mask_dy=True)
    assert max(errs.values()) <= TOL, errs


def test_decoder_layer_full_size():
    _announce("decoder layer M=16384, 7 projections")
    q = _q()
    d = make_workload(4)
    M = d["M"]
    rows = sample_rows(M, np.random.default_rng(4), per_block=1, block=512)
    errs = {}
    for nm, xk in (("q", "X_attn"), ("k", "X_attn"), ("v", "X_attn"), ("o", "X_o")):
        sub = dict(layers={"proj": d["layers"][nm]}, X=d[xk], dY=d["dY_" + nm], s=d["s"], M=M)
        for k, v in _linear_case(sub, rows, check_z=False).items():
            errs[f"{nm}.{k}"] = v
    mlp = dict(layers={k: d["layers"][k] for k in ("gate", "up", "down")}, X=d["X_mlp"], dY=d["dY_mlp"], M=M,
               s=d["s"])
    for k, v in _mlp_case(mlp, rows, mask_dy=True).items():
        errs["mlp." + k] = v
    assert max(errs.values()) <= TOL, errs


# ---------------------------------------------------------------------------
# determinism, workspace hygiene, streams

def _bits(t):
    import torch
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def test_linear_backward_bitwise_deterministic_and_workspace_independent():
    # the rank-r reductions sum their split partials in a fixed order, so two
    # runs agree bit for bit; a workspace full of NaN bytes and outputs full of
    # NaN bytes change nothing (no uninitialised reads)
    _announce("determinism linear M=2000 K=1024 N=384 r=16")
    import torch
    q = _q()
    d = random_linear(4242, 2000, 1024, 384, 16)
    P = Prepared(d["layers"]["proj"], d["s"])
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    runs = []
    for dirty in (False, True, False):
        M, K, N, r = 2000, 1024, 384, 16
        fill = float("nan") if dirty else 0.0
        Y = torch.full((M, N), fill, dtype=torch.bfloat16, device="cuda")
        Z = torch.full((M, r), fill, dtype=torch.bfloat16, device="cuda")
        q.forward(P.dev, X, Y, Z)
        nb = q.workspace_size(1, M, K, N, r)
        ws = torch.full((nb,), 255 if dirty else 0, dtype=torch.uint8, device="cuda")
        out = (torch.full((M, K), fill, dtype=torch.bfloat16, device="cuda"),
               torch.full((r, K), fill, dtype=torch.float32, device="cuda"),
               torch.full((N, r), fill, dtype=torch.float32, device="cuda"))
        dX, dA, dB = q.backward(P.dev, dY, X, Z, ws=ws, out=out)
        torch.cuda.synchronize()
        runs.append([_bits(t) for t in (Y, Z, dX, dA, dB)])
    for other in runs[1:]:
        for a, b in zip(runs[0], other):
            assert np.array_equal(a, b)


def test_mlp_backward_bitwise_deterministic():
    _announce("determinism mlp M=300 H=256 I=512 r=16")
    import torch
    q = _q()
    d = random_mlp(4243, 300, 256, 512, 16)
    Ls = {nm: Prepared(d["layers"][nm], d["s"]) for nm in ("gate", "up", "down")}
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    runs = []
    for _ in range(2):
        f = q.mlp_forward(Ls["gate"].dev, Ls["up"].dev, Ls["down"].dev, X)
        b = q.mlp_backward(Ls["gate"].dev, Ls["up"].dev, Ls["down"].dev, dY, X, f)
        torch.cuda.synchronize()
        runs.append([_bits(t) for t in [f["Y"], b["dX"]] + b["dA"] + b["dB"]])
    for a, b in zip(*runs):
        assert np.array_equal(a, b)


def test_calls_run_on_the_callers_stream():
    # every launch goes to the current torch stream: a side stream gives the
    # same bits as the default one
    _announce("side stream linear tiny")
    import torch
    q = _q()
    d = make_workload(0)
    P = Prepared(d["layers"]["proj"], d["s"])
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    Y0, Z0 = q.forward(P.dev, X)
    r0 = q.backward(P.dev, dY, X, Z0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Y1, Z1 = q.forward(P.dev, X)
        r1 = q.backward(P.dev, dY, X, Z1)
    s.synchronize()
    for a, b in zip([Y0, Z0, *r0], [Y1, Z1, *r1]):
        assert np.array_equal(_bits(a), _bits(b))


def _random_shapes(n, seed):
    # seeded draws over both paths: M from 1 to ~2600 (the small-batch path up to
    # 256 tokens at r <= 32), K a multiple of 64, N a multiple of 8, r from 1 to 160
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 2600)) if i % 3 else int(rng.integers(1, 257))
        K = 64 * int(rng.integers(1, 13))
        N = 8 * int(rng.integers(1, 97))
        r = int(rng.integers(1, 33)) if i % 2 else int(rng.integers(1, 161))
        out.append((M, K, N, r, i % 3))
    return out


@pytest.mark.parametrize("M,K,N,r,fmt", _random_shapes(12, 2027))
def test_linear_random_shapes_full_oracle(M, K, N, r, fmt):
    _announce(f"linear random fmt={fmt} M={M} K={K} N={N} r={r}")
    d = random_linear(60_000 + M + K + N + r, M, K, N, r)
    errs = _linear_case(d, fmt=fmt)
    assert max(errs.values()) <= TOL, errs
