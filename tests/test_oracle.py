"""Pins for the CPU oracle: it is checked against things other than itself.

  * the NF4 table against its quantile construction and the QLoRA paper's printed values;
  * quantization against brute-force nearest-level search, exact levels, ties,
    idempotence, the error bound and hand-worked byte layouts;
  * the linear layer against central finite differences of L = sum(dY * Y),
    against the explicit merged-weight bracketing x.(W + s.B.A)^T (same answer
    whichever pair is multiplied first: "Unsloth vs PyTorch" video, 1:35-2:00),
    against closed forms (A = 0, B = 0, s = 0) and against naive loops;
  * the SwiGLU MLP against finite differences and silu's textbook values.

The last group plants mistakes in copies of the oracle and shows each pin
catches them, so a plausible bug (a dropped term, a wrong sign, a transposed
operand, a swapped nibble) cannot pass silently.
"""
import os

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import ref
from synthetic import bf16_bits, bf16_to_f32, make_workload, random_linear

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
L = cb.NF4_LEVELS
T = cb.NF4_THRESHOLDS


def f32(x):
    return np.float32(x)


def nextup(x):
    return np.nextafter(np.float32(x), np.float32(np.inf), dtype=np.float32)


def nextdown(x):
    return np.nextafter(np.float32(x), np.float32(-np.inf), dtype=np.float32)


# ---------------------------------------------------------------------------
# codebook

def test_codebook_matches_quantile_construction():
    d = cb.derive_nf4_levels()
    assert np.max(np.abs(d - L.astype(np.float64))) < 5e-7


def test_codebook_matches_golden_printed_values():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "nf4_levels.txt")) if not ln.startswith("#")]
    assert len(rows) == 16
    for i, (idx, val, hx) in enumerate(rows):
        assert int(idx) == i
        assert np.float32(float(val)) == L[i]
        assert int(hx, 16) == int(L.view(np.uint32)[i])


def test_codebook_structure():
    assert np.all(np.diff(L.astype(np.float64)) > 0)
    assert L[0] == -1.0 and L[7] == 0.0 and L[15] == 1.0
    assert (L < 0).sum() == 7 and (L > 0).sum() == 8


def test_thresholds_are_rounded_midpoints():
    from fractions import Fraction
    for j in range(15):
        mid = (Fraction(float(L[j])) + Fraction(float(L[j + 1]))) / 2
        t = T[j]
        assert L[j] < t < L[j + 1]
        # t is an fp32 value nearest to the exact midpoint
        for nb in (nextup(t), nextdown(t)):
            assert abs(Fraction(float(t)) - mid) <= abs(Fraction(float(nb)) - mid)


# ---------------------------------------------------------------------------
# quantization

def _codes(packed):
    return ref.unpack_codes(packed)


def test_quantize_brute_force_nearest_level():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    W[3, :64] *= 1e-30  # tiny block
    packed, a = ref.quantize(W)
    codes = _codes(packed)
    blocks = W.reshape(64, 16, 64).astype(np.float64)
    a64 = np.abs(blocks).max(axis=2)
    x = (blocks / a64[:, :, None]).reshape(64, 1024)
    brute = np.argmin(np.abs(x[:, :, None] - L.astype(np.float64)[None, None, :]), axis=2)
    # exclude elements within a few ulp of a decision threshold
    near = np.zeros_like(x, dtype=bool)
    for t in T.astype(np.float64):
        near |= np.abs(x - t) <= 4 * np.spacing(np.float32(t)).astype(np.float64)
    assert near.sum() < 20
    assert np.array_equal(codes[~near], brute[~near])
    assert np.array_equal(a, np.abs(W.reshape(64, 16, 64)).max(axis=2))


def test_quantize_exact_levels():
    rng = np.random.default_rng(3)
    for a in (f32(0.02), f32(1.0), f32(3.5e-3), f32(1e-39)):  # last one is an fp32 denormal
        c = rng.integers(0, 16, 64)
        c[5], c[17] = 0, 15
        W = (L[c] * a).astype(np.float32)[None, :]
        packed, am = ref.quantize(W)
        assert am[0, 0] == a
        if a > 1e-30:  # denormal scaling loses level precision; checked separately below
            assert np.array_equal(_codes(packed)[0], c)


def test_quantize_ties_go_to_lower_level():
    for j in range(15):
        W = np.zeros((1, 64), np.float32)
        W[0, 0] = 1.0          # absmax = 1, so x = W exactly
        W[0, 1] = T[j]         # exactly on threshold j -> code j
        W[0, 2] = nextup(T[j])  # just above -> code j+1
        W[0, 3] = nextdown(T[j])
        codes = _codes(ref.quantize(W)[0])[0]
        assert codes[0] == 15
        assert codes[1] == j
        assert codes[2] == j + 1
        assert codes[3] == j


def test_quantize_zero_blocks_and_signed_zero():
    W = np.zeros((2, 128), np.float32)
    W[1, :64] = -0.0
    W[1, 64] = 0.5
    packed, a = ref.quantize(W)
    codes = _codes(packed)
    assert np.all(a[0] == 0) and a[1, 0] == 0 and a[1, 1] == f32(0.5)
    assert np.all(codes[0] == 7) and np.all(codes[1, :64] == 7)
    assert codes[1, 64] == 15 and np.all(codes[1, 65:] == 7)
    assert np.all(ref.dequantize(packed, a)[0] == 0)


def test_nibble_order_hand_worked():
    # column 0 = -a -> code 0; column 1 = +a -> code 15; column 2 = 0 -> code 7;
    # column 3 = a*L[12] -> code 12. Byte 0 = 0 | 15<<4 = 0xF0, byte 1 = 7 | 12<<4 = 0xC7.
    W = np.zeros((1, 64), np.float32)
    a = f32(0.25)
    W[0, 0], W[0, 1], W[0, 3] = -a, a, L[12] * a
    packed, am = ref.quantize(W)
    assert packed.shape == (1, 32)
    assert packed[0, 0] == 0xF0 and packed[0, 1] == 0xC7
    assert np.all(packed[0, 2:] == 0x77)
    Wh = ref.dequantize(packed, am)
    assert Wh[0, 0] == -a and Wh[0, 1] == a and Wh[0, 2] == 0 and Wh[0, 3] == f32(L[12] * a)


def test_quantize_idempotent_and_max_element():
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((32, 512)) * 0.02).astype(np.float32)
    packed, a = ref.quantize(W)
    Wh = ref.dequantize(packed, a)
    p2, a2 = ref.quantize(Wh)
    assert np.array_equal(p2, packed) and np.array_equal(a2, a)
    codes = _codes(packed).reshape(32, 8, 64)
    blocks = W.reshape(32, 8, 64)
    imax = np.abs(blocks).argmax(axis=2)
    cmax = np.take_along_axis(codes, imax[:, :, None], axis=2)[:, :, 0]
    sign = np.take_along_axis(blocks, imax[:, :, None], axis=2)[:, :, 0] > 0
    assert np.all(cmax[sign] == 15) and np.all(cmax[~sign] == 0)


def test_quantize_error_bound():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((16, 1024)) * 0.02).astype(np.float32)
    packed, a = ref.quantize(W)
    Wh = ref.dequantize(packed, a)
    gap = np.max(np.diff(L.astype(np.float64))) / 2
    bound = np.repeat(a.astype(np.float64), 64, axis=1) * (gap + 1e-6)
    assert np.all(np.abs(W.astype(np.float64) - Wh) <= bound)


def test_dequantize_is_one_fp32_multiply():
    rng = np.random.default_rng(9)
    packed = rng.integers(0, 256, (4, 64), dtype=np.uint8)
    a = (rng.random((4, 2)) * 0.1).astype(np.float32)
    a[0, 0] = f32(1e-40)  # denormal scale
    Wh = ref.dequantize(packed, a)
    for n in range(4):
        for k in range(128):
            code = (packed[n, k // 2] >> (4 * (k % 2))) & 15
            want = np.float32(np.float32(L[code]) * np.float32(a[n, k // 64]))
            assert Wh[n, k].view(np.uint32) == want.view(np.uint32)


def test_quantize_denormal_block():
    W = np.zeros((1, 64), np.float32)
    W[0, :8] = np.array([3e-40, -5e-41, 1e-42, 0, -3e-40, 2e-40, 1e-45, -1e-45], np.float32)
    packed, a = ref.quantize(W)
    assert a[0, 0] == f32(3e-40)
    codes = _codes(packed)[0]
    x = W[0].astype(np.float64) / float(a[0, 0])
    brute = np.argmin(np.abs(x[:, None] - L.astype(np.float64)[None, :]), axis=1)
    assert np.array_equal(codes, brute)
    assert codes[0] == 15 and codes[4] == 0


def test_quantize_rejects_nonfinite_and_bad_shape():
    W = np.zeros((1, 64), np.float32)
    W[0, 3] = np.inf
    with pytest.raises(ValueError):
        ref.quantize(W)
    W[0, 3] = np.nan
    with pytest.raises(ValueError):
        ref.quantize(W)
    with pytest.raises(ValueError):
        ref.quantize(np.zeros((2, 48), np.float32))


# ---------------------------------------------------------------------------
# linear layer

def _tiny_linear(seed=0, M=3, K=128, N=5, r=2, s=2.0):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wh = ref.dequantize(*ref.quantize(W)).astype(np.float64)
    X = rng.standard_normal((M, K))
    A = rng.standard_normal((r, K)) / np.sqrt(K)
    B = rng.standard_normal((N, r)) * 0.02
    dY = rng.standard_normal((M, N))
    return X, Wh, A, B, dY, s


def _fd_grads(fwd, X, Wh, A, B, dY, s):
    """Central differences of L = sum(dY * Y) with respect to every entry of X, A, B."""
    def loss(X_, A_, B_):
        return float(np.sum(dY * fwd(X_, Wh, A_, B_, s)[0]))
    out = []
    for which in range(3):
        P = [X.copy(), A.copy(), B.copy()]
        g = np.zeros_like(P[which])
        for idx in np.ndindex(*P[which].shape):
            th = P[which][idx]
            h = 1e-6 * max(1.0, abs(th))
            P[which][idx] = th + h
            lp = loss(*P)
            P[which][idx] = th - h
            lm = loss(*P)
            P[which][idx] = th
            g[idx] = (lp - lm) / (2 * h)
        out.append(g)
    return out


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def check_linear_fd(fwd, bwd, seed=0):
    X, Wh, A, B, dY, s = _tiny_linear(seed)
    gX, gA, gB = _fd_grads(fwd, X, Wh, A, B, dY, s)
    dX, dA, dB = bwd(dY, X, Wh, A, B, s)
    return max(_rel(dX, gX), _rel(dA, gA), _rel(dB, gB))


def test_linear_bwd_matches_finite_differences():
    assert check_linear_fd(ref.linear_fwd, ref.linear_bwd) < 1e-6


def check_bracketing(fwd, bwd, seed=1):
    X, Wh, A, B, dY, s = _tiny_linear(seed, M=7, K=192, N=9, r=4, s=1.5)
    Wm = Wh + s * (B @ A)  # merged weight: x.(W + s.B.A)^T
    Y, Z = fwd(X, Wh, A, B, s)
    dX, dA, dB = bwd(dY, X, Wh, A, B, s)
    P = dY.T @ X  # the N x K product the rank-r bracketing avoids
    return max(_rel(Y, X @ Wm.T), _rel(dX, dY @ Wm), _rel(dB, s * (P @ A.T)), _rel(dA, s * (B.T @ P)),
               _rel(Z, X @ A.T))


def test_linear_matches_merged_weight_bracketing():
    assert check_bracketing(ref.linear_fwd, ref.linear_bwd) < 1e-12


def check_closed_forms(fwd, bwd, seed=2):
    X, Wh, A, B, dY, s = _tiny_linear(seed, M=6, K=128, N=8, r=3, s=2.0)
    errs = []
    Z0 = np.zeros_like(A)
    Y, _ = fwd(X, Wh, Z0, B, s)
    dX, dA, dB = bwd(dY, X, Wh, Z0, B, s)
    errs += [_rel(Y, X @ Wh.T), _rel(dX, dY @ Wh), np.max(np.abs(dB)), _rel(dA, s * ((dY @ B).T @ X))]
    B0 = np.zeros_like(B)
    Y, _ = fwd(X, Wh, A, B0, s)
    dX, dA, dB = bwd(dY, X, Wh, A, B0, s)
    errs += [_rel(Y, X @ Wh.T), _rel(dX, dY @ Wh), np.max(np.abs(dA)), _rel(dB, s * (dY.T @ (X @ A.T)))]
    Y, _ = fwd(X, Wh, A, B, 0.0)
    dX, dA, dB = bwd(dY, X, Wh, A, B, 0.0)
    errs += [_rel(Y, X @ Wh.T), np.max(np.abs(dA)), np.max(np.abs(dB))]
    return max(errs)


def test_linear_closed_forms():
    assert check_closed_forms(ref.linear_fwd, ref.linear_bwd) < 1e-12


def check_naive_loops(fwd, bwd, seed=4):
    X, Wh, A, B, dY, s = _tiny_linear(seed, M=5, K=64, N=6, r=3, s=0.75)
    M, K = X.shape
    N, r = B.shape
    Y, _ = fwd(X, Wh, A, B, s)
    dX, dA, dB = bwd(dY, X, Wh, A, B, s)
    Yn = np.zeros((M, N)); dXn = np.zeros((M, K)); dAn = np.zeros((r, K)); dBn = np.zeros((N, r))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                w = Wh[n, k]
                for j in range(r):
                    w += s * B[n, j] * A[j, k]
                acc += X[m, k] * w
            Yn[m, n] = acc
    for m in range(M):
        for k in range(K):
            acc = 0.0
            for n in range(N):
                w = Wh[n, k]
                for j in range(r):
                    w += s * B[n, j] * A[j, k]
                acc += dY[m, n] * w
            dXn[m, k] = acc
    for j in range(r):
        for k in range(K):
            dAn[j, k] = s * sum(dY[m, n] * B[n, j] * X[m, k] for m in range(M) for n in range(N))
    for n in range(N):
        for j in range(r):
            dBn[n, j] = s * sum(dY[m, n] * A[j, k] * X[m, k] for m in range(M) for k in range(K))
    return max(_rel(Y, Yn), _rel(dX, dXn), _rel(dA, dAn), _rel(dB, dBn))


def test_linear_naive_loops():
    assert check_naive_loops(ref.linear_fwd, ref.linear_bwd) < 1e-12


def test_adapter_grads_agree_with_linear_bwd():
    X, Wh, A, B, dY, s = _tiny_linear(8, M=11, K=128, N=7, r=3)
    _, dA, dB = ref.linear_bwd(dY, X, Wh, A, B, s)
    dA2, dB2 = ref.adapter_grads(dY, X, A, B, s)
    assert _rel(dA2, dA) < 1e-14 and _rel(dB2, dB) < 1e-14


def test_linear_rows_are_independent():
    # Row m of Y and dX depends only on row m of X and dY (lets parity tests sample rows).
    X, Wh, A, B, dY, s = _tiny_linear(12, M=9, K=128, N=6, r=2)
    Y, _ = ref.linear_fwd(X, Wh, A, B, s)
    dX, _, _ = ref.linear_bwd(dY, X, Wh, A, B, s)
    rows = [0, 4, 8]
    Ys, _ = ref.linear_fwd(X[rows], Wh, A, B, s)
    dXs, _, _ = ref.linear_bwd(dY[rows], X[rows], Wh, A, B, s)
    assert _rel(Ys, Y[rows]) < 1e-15 and _rel(dXs, dX[rows]) < 1e-15


# ---------------------------------------------------------------------------
# SwiGLU MLP

def test_silu_textbook_values():
    assert ref.silu(0.0) == 0.0
    assert abs(ref.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
    assert abs(ref.silu(-30.0)) < 1e-11 and abs(ref.silu(30.0) - 30.0) < 1e-11
    # derivative of silu at 0 is 1/2, checked through the backward's dg formula (dh = u = 1)
    z = np.array([0.0, 0.3, -1.7, 4.0])
    sig = 1 / (1 + np.exp(-z))
    deriv = sig * (1 + z * (1 - sig))
    assert deriv[0] == 0.5
    h = 1e-6
    fd = (ref.silu(z + h) - ref.silu(z - h)) / (2 * h)
    assert np.max(np.abs(fd - deriv)) < 1e-9


def _tiny_mlp(seed=0, M=3, H=64, I=128, r=2, s=2.0):
    rng = np.random.default_rng(seed)
    def lay(K, N):
        W = (rng.standard_normal((N, K)) * 0.3).astype(np.float32)
        Wh = ref.dequantize(*ref.quantize(W)).astype(np.float64)
        return [Wh, rng.standard_normal((r, K)) / np.sqrt(K), rng.standard_normal((N, r)) * 0.3]
    gate, up, down = lay(H, I), lay(H, I), lay(I, H)
    X = rng.standard_normal((M, H))
    dY = rng.standard_normal((M, H))
    return X, gate, up, down, dY, s


def check_mlp_fd(fwd, bwd, seed=0):
    X, gate, up, down, dY, s = _tiny_mlp(seed)
    got = bwd(dY, X, gate, up, down, s)

    def loss():
        return float(np.sum(dY * fwd(X, gate, up, down, s)["Y"]))

    errs = []
    targets = [("dX", X)]
    for nm, lay in (("gate", gate), ("up", up), ("down", down)):
        targets += [("dA_" + nm, lay[1]), ("dB_" + nm, lay[2])]
    rng = np.random.default_rng(99)
    for key, P in targets:
        fd = np.zeros_like(P)
        # every entry of X; a random subset of 40 entries of each adapter matrix (keeps the test fast)
        idxs = list(np.ndindex(*P.shape))
        if key != "dX":
            idxs = [idxs[i] for i in rng.choice(len(idxs), size=min(40, len(idxs)), replace=False)]
        for idx in idxs:
            th = P[idx]
            h = 1e-6 * max(1.0, abs(th))
            P[idx] = th + h
            lp = loss()
            P[idx] = th - h
            lm = loss()
            P[idx] = th
            fd[idx] = (lp - lm) / (2 * h)
        sel = tuple(np.array(idxs).T)
        errs.append(float(np.max(np.abs(got[key][sel] - fd[sel])) / max(np.max(np.abs(got[key][sel])), 1e-300)))
    return max(errs)


def test_mlp_bwd_matches_finite_differences():
    assert check_mlp_fd(ref.mlp_fwd, ref.mlp_bwd) < 1e-6


def test_mlp_lora_off_reduces_to_base_swiglu():
    X, gate, up, down, dY, s = _tiny_mlp(3)
    f = ref.mlp_fwd(X, gate, up, down, 0.0)
    g = X @ gate[0].T
    u = X @ up[0].T
    Y = (g / (1 + np.exp(-g)) * u) @ down[0].T
    assert _rel(f["Y"], Y) < 1e-13


# ---------------------------------------------------------------------------
# planted mistakes: each pin must fail on a plausible bug in a copy of the oracle

def _bwd_wrong_operand_dB(dY, X, Wh, A, B, s):
    # dB built from G = dY.B instead of Z = X.A^T (the two [M,r] tensors swapped)
    dX, dA, dB = ref.linear_bwd(dY, X, Wh, A, B, s)
    return dX, dA, s * (dY.T @ (dY @ B))


def _bwd_permuted_rank(dY, X, Wh, A, B, s):
    # the rank index of A reversed (a transposed/misindexed operand)
    dX, dA, dB = ref.linear_bwd(dY, X, Wh, A, B, s)
    return dX, dA[::-1], dB


def _bwd_missing_scale(dY, X, Wh, A, B, s):
    dX, dA, dB = ref.linear_bwd(dY, X, Wh, A, B, s)
    return dX, dA / s, dB


def _bwd_dropped_lora_dx(dY, X, Wh, A, B, s):
    return ref.linear_bwd(dY, X, Wh, A, B, s)[0] - s * ((dY @ B) @ A), *ref.linear_bwd(dY, X, Wh, A, B, s)[1:]


def _bwd_wrong_sign(dY, X, Wh, A, B, s):
    dX, dA, dB = ref.linear_bwd(dY, X, Wh, A, B, s)
    return dX, dA, -dB


def _fwd_transposed_adapter(X, Wh, A, B, s):
    Y, Z = ref.linear_fwd(X, Wh, A, B, s)
    return Y - s * (Z @ B.T) + s * (Z @ B[::-1].T), Z


@pytest.mark.parametrize("bad", [_bwd_wrong_operand_dB, _bwd_permuted_rank, _bwd_missing_scale, _bwd_dropped_lora_dx, _bwd_wrong_sign])
def test_planted_backward_mistakes_are_caught(bad):
    assert check_linear_fd(ref.linear_fwd, bad) > 1e-3
    assert check_bracketing(ref.linear_fwd, bad) > 1e-3
    assert check_naive_loops(ref.linear_fwd, bad) > 1e-3


def test_planted_forward_mistake_is_caught():
    assert check_bracketing(_fwd_transposed_adapter, ref.linear_bwd) > 1e-3
    assert check_naive_loops(_fwd_transposed_adapter, ref.linear_bwd) > 1e-3


def test_planted_mlp_mistakes_are_caught(monkeypatch):
    orig_bwd = ref.mlp_bwd

    def bad_sign(dY, X, gate, up, down, s):
        # silu'(g) with the wrong sign in the (1 - sig) term
        out = orig_bwd(dY, X, gate, up, down, s)
        f = out["fwd"]
        g, u = f["g"], f["u"]
        sig = 1 / (1 + np.exp(-g))
        dg = out["dh"] * u * sig * (1 + g * (sig - 1))
        dX_g, dA_g, dB_g = ref.linear_bwd(dg, X, *gate, s)
        dX_u, _, _ = ref.linear_bwd(out["du"], X, *up, s)
        out = dict(out)
        out.update(dX=dX_g + dX_u, dA_gate=dA_g, dB_gate=dB_g)
        return out

    def swapped_gate_up(dY, X, gate, up, down, s):
        out = dict(orig_bwd(dY, X, gate, up, down, s))
        out["dA_gate"], out["dA_up"] = out["dA_up"], out["dA_gate"]
        return out

    assert check_mlp_fd(ref.mlp_fwd, bad_sign) > 1e-3
    assert check_mlp_fd(ref.mlp_fwd, swapped_gate_up) > 1e-3


def test_planted_quantizer_mistakes_are_caught(monkeypatch):
    # ties to the upper level
    W = np.zeros((1, 64), np.float32)
    W[0, 0] = 1.0
    W[0, 1] = T[4]
    x = W / 1.0
    upper = (x[0, 1] >= T).sum()
    assert upper != _codes(ref.quantize(W)[0])[0, 1]
    # swapped nibbles would give 0x0F for the hand-worked byte 0
    W = np.zeros((1, 64), np.float32)
    W[0, 0], W[0, 1] = -1.0, 1.0
    packed, _ = ref.quantize(W)
    swapped = ((packed >> 4) | (packed << 4)).astype(np.uint8)
    assert swapped[0, 0] != 0xF0 and packed[0, 0] == 0xF0


# ---------------------------------------------------------------------------
# synthetic inputs (shared generator; no method arithmetic)

def test_synthetic_inputs_deterministic_and_distributed():
    w1 = make_workload(0)
    w2 = make_workload(0)
    assert np.array_equal(w1["X"], w2["X"]) and np.array_equal(w1["layers"]["proj"]["W"], w2["layers"]["proj"]["W"])
    Lr = w1["layers"]["proj"]
    assert abs(float(np.std(Lr["W"])) - 0.02) < 1e-3
    assert abs(float(np.std(bf16_to_f32(Lr["A"]))) - 1 / np.sqrt(512)) < 3e-3
    assert abs(float(np.std(bf16_to_f32(Lr["B"]))) - 0.02) < 2e-3
    assert abs(float(np.std(bf16_to_f32(w1["X"]))) - 1.0) < 0.02
    assert w1["s"] == 2.0 and w1["r"] == 8


def test_bf16_widening_of_hand_chosen_words():
    # bfloat16 is the top half of an IEEE binary32 word: sign, 8 exponent bits
    # (bias 127), 7 fraction bits. Each word below is decoded by hand.
    words = np.array([0x3F80, 0xC020, 0x0001, 0x8000, 0x7F80, 0xFF80, 0x4049, 0x0080, 0x7F7F, 0x3E80],
                     dtype=np.uint16)
    want = [1.0,                     # exponent 127, fraction 0
            -2.5,                    # sign, exponent 128, fraction 0b0100000 -> -(1 + 1/4) * 2
            2.0 ** -133,             # smallest subnormal: 2^-126 * 2^-7
            -0.0,                    # negative zero
            np.inf, -np.inf,         # exponent all ones, fraction 0
            3.140625,                # exponent 128, fraction 0b1001001 -> (1 + 73/128) * 2
            2.0 ** -126,             # smallest normal
            (2.0 - 2.0 ** -7) * 2.0 ** 127,  # largest finite
            0.25]
    got = ref.bf16_to_f64(words)
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w and np.signbit(g) == np.signbit(w), (g, w)
    # a NaN word stays NaN
    assert np.isnan(ref.bf16_to_f64(np.array([0x7FC0], dtype=np.uint16))[0])
    # exact widening: every finite bf16 word round-trips through float32 bit patterns
    allw = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # the signalling-NaN words are quieted by the widening
        vals = ref.bf16_to_f64(allw)
    fin = np.isfinite(vals)
    back = (vals[fin].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(back, allw[fin])


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, np.inf], np.float32)
    b = bf16_bits(x)
    assert list(bf16_to_f32(b)) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, np.inf]


def test_discrimination_of_lora_term_on_tiny_workload():
    # The parity metric must be able to see the adapter: removing it moves Y and dX by more than 1e-2.
    w = make_workload(0)
    Lr = w["layers"]["proj"]
    Wh = ref.dequantize(*ref.quantize(Lr["W"]))
    X, dY = ref.bf16_to_f64(w["X"]), ref.bf16_to_f64(w["dY"])
    A, B = ref.bf16_to_f64(Lr["A"]), ref.bf16_to_f64(Lr["B"])
    Y, _ = ref.linear_fwd(X, Wh, A, B, w["s"])
    Y0, _ = ref.linear_fwd(X, Wh, A, B, 0.0)
    dX, _, _ = ref.linear_bwd(dY, X, Wh, A, B, w["s"])
    dX0, _, _ = ref.linear_bwd(dY, X, Wh, A, B, 0.0)
    assert _rel(Y0, Y) > 1e-2 and _rel(dX0, dX) > 1e-2


def test_random_linear_shapes():
    d = random_linear(1, 17, 128, 33, 5)
    assert d["X"].shape == (17, 128) and d["layers"]["proj"]["B"].shape == (33, 5)
