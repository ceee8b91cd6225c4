"""Plain CPU definition of the fused QLoRA linear layer (test infrastructure).

Only the tests, the smoke check and bench.py's CPU-baseline leg use this
module. Quantization follows its fp32 procedure exactly (it is a bit-exact
target); everything else is float64 NumPy with one library matmul per product
and no blocking, fusion or reordering beyond the bracketing the method states.

Shapes and names (PyTorch Linear convention, out x in):
  X  [M,K]   activations              W, What [N,K]  frozen weight, dequantized
  A  [r,K]   LoRA down projection     B [N,r]        LoRA up projection
  Y  [M,N]   output                   s = lora_alpha / r
  codes uint8 [N,K/2], two 4-bit codes per byte; absmax fp32 [N,K/64]
"""
from __future__ import annotations

import numpy as np

from .codebook import NF4_LEVELS, NF4_THRESHOLDS

BLOCK = 64  # elements of a weight row that share one absmax


def bf16_to_f64(b) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# 4-bit block quantization of the frozen weight
# ("Unsloth vs The Stack v2", quantized-base card: 4-bit frozen weights;
#  the format -- 64-element row blocks, fp32 absmax, NF4 levels -- is the
#  plainest reading of the bitsandbytes 4-bit checkpoints the pages load.)

def quantize(W) -> tuple[np.ndarray, np.ndarray]:
    """Quantize fp32 W [N,K] to (codes uint8 [N,K/2], absmax fp32 [N,K/64]).

    Per row n and 64-column block b:
      a = max_k |W[n,k]| over the block (exact in fp32);
      x = fp32(W[n,k] / a), correctly rounded;
      code = number of thresholds T[j] with x > T[j]   (ties go to the lower level);
      a block of zeros gets a = 0 and code 7 (the exact zero level).
    Byte k/2 of a row holds the code of the even column in its low nibble and
    the odd column in its high nibble. Non-finite W raises ValueError.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % BLOCK != 0:
        raise ValueError("W must be [N, K] with K a multiple of 64")
    if not np.isfinite(W).all():
        raise ValueError("non-finite weight")
    N, K = W.shape
    blocks = W.reshape(N, K // BLOCK, BLOCK)
    a = np.abs(blocks).max(axis=2)  # fp32
    zero = a == 0
    denom = np.where(zero, np.float32(1.0), a).astype(np.float32)
    x = (blocks / denom[:, :, None]).astype(np.float32)  # IEEE fp32 division
    codes = np.zeros(x.shape, dtype=np.uint8)
    for t in NF4_THRESHOLDS:
        codes += (x > t).astype(np.uint8)
    codes[zero] = 7
    codes = codes.reshape(N, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, a.astype(np.float32)


def unpack_codes(packed) -> np.ndarray:
    """uint8 [N,K/2] -> uint8 [N,K] codes (low nibble = even column)."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, H = packed.shape
    out = np.empty((N, 2 * H), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def dequantize(packed, absmax) -> np.ndarray:
    """What[n,k] = fp32(L[code[n,k]] * absmax[n, k // 64]): one fp32 multiply, rounded to nearest."""
    codes = unpack_codes(packed)
    N, K = codes.shape
    scale = np.repeat(np.asarray(absmax, dtype=np.float32), BLOCK, axis=1)
    return (NF4_LEVELS[codes] * scale).astype(np.float32)


# ---------------------------------------------------------------------------
# LoRA linear layer, forward and hand-derived backward
# ("Rev vs unsloth", fused-LoRA card; "Unsloth" wiki entry, Theory;
#  "Unsloth vs PyTorch" video 0:43-2:11 for the derivatives and the bracketing)

def linear_fwd(X, What, A, B, s):
    """Y = X.What^T + s.(X.A^T).B^T, bracketed so the N x K matrix B.A is never formed.

    Returns (Y, Z) with Z = X.A^T, the tensor the backward reuses. float64.
    """
    X = np.asarray(X, dtype=np.float64)
    Z = X @ np.asarray(A, dtype=np.float64).T
    Y = X @ np.asarray(What, dtype=np.float64).T + s * (Z @ np.asarray(B, dtype=np.float64).T)
    return Y, Z


def linear_bwd(dY, X, What, A, B, s):
    """Gradients of the LoRA linear layer for upstream gradient dY (W is frozen: no dW).

      G  = dY.B
      dX = dY.What + s.G.A
      dB = s.dY^T.(X.A^T)
      dA = s.G^T.X
    Returns (dX, dA, dB). float64.
    """
    dY = np.asarray(dY, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    G = dY @ B
    Z = X @ A.T
    dX = dY @ np.asarray(What, dtype=np.float64) + s * (G @ A)
    dB = s * (dY.T @ Z)
    dA = s * (G.T @ X)
    return dX, dA, dB


def adapter_grads(dY, X, A, B, s):
    """dA and dB alone, by the same formulas as linear_bwd (needs no weight)."""
    dY = np.asarray(dY, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    G = dY @ B
    Z = X @ A.T
    return s * (G.T @ X), s * (dY.T @ Z)


# ---------------------------------------------------------------------------
# SwiGLU MLP with LoRA on gate, up and down
# ("Unsloth" wiki entry, Theory: fused SwiGLU block; "Unsloth" wiki API
#  snippet: target_modules include gate_proj, up_proj, down_proj)

def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def mlp_fwd(X, gate, up, down, s):
    """g = lin_gate(X), u = lin_up(X), h = silu(g)*u, Y = lin_down(h).

    gate/up/down are (What, A, B) tuples. Returns a dict with g, u, h, Y and
    the Z tensors of the three projections. float64 throughout.
    """
    g, Zg = linear_fwd(X, *gate, s)
    u, Zu = linear_fwd(X, *up, s)
    h = silu(g) * u
    Y, Zd = linear_fwd(h, *down, s)
    return dict(g=g, u=u, h=h, Y=Y, Z_gate=Zg, Z_up=Zu, Z_down=Zd)


def mlp_bwd(dY, X, gate, up, down, s):
    """Backward of mlp_fwd for upstream gradient dY.

      dh, dA_down, dB_down = lin_down backward at input h
      sig = sigmoid(g)
      dg = dh * u * sig * (1 + g*(1 - sig))      (d silu / dg = sig*(1 + g*(1-sig)))
      du = dh * silu(g)
      dX = dX_gate(dg) + dX_up(du); dA/dB of gate and up from dg, du and X.
    Returns a dict with dX, dA_*, dB_*, dh, dg, du.
    """
    f = mlp_fwd(X, gate, up, down, s)
    g, u, h = f["g"], f["u"], f["h"]
    dh, dA_d, dB_d = linear_bwd(dY, h, *down, s)
    sig = 1.0 / (1.0 + np.exp(-g))
    dg = dh * u * sig * (1.0 + g * (1.0 - sig))
    du = dh * (g * sig)
    dX_g, dA_g, dB_g = linear_bwd(dg, X, *gate, s)
    dX_u, dA_u, dB_u = linear_bwd(du, X, *up, s)
    return dict(dX=dX_g + dX_u, dA_gate=dA_g, dB_gate=dB_g, dA_up=dA_u, dB_up=dB_u,
                dA_down=dA_d, dB_down=dB_d, dh=dh, dg=dg, du=du, fwd=f)
