"""Plain CPU definition of the steps on either side of the projections:
RMSNorm before them and rotary position embeddings (RoPE) after q and k
(test infrastructure: only the tests, the smoke check and bench.py's
CPU-baseline leg use this module).

The pages name these kernels without formulas ("Unsloth" wiki entry, Theory:
fused kernels for RMSNorm and RoPE; "Unsloth vs PyTorch" video, 2:11-2:22:
rotary embeddings and layer norms rewritten as fused kernels). The readings
below are the standard Llama-3 definitions; everything is float64 NumPy.

RMSNorm over the last axis of x [M,H] with a frozen weight w [H]:
    rstd = 1 / sqrt(mean(x^2) + eps),  y = w * (x * rstd)
and, since w is frozen with the rest of the base model, its backward gives
dx only:  g = w * dy,  n = x * rstd,  dx = rstd * (g - n * mean(g * n)).

RoPE on a head vector v [d] of the token at position p ("rotate half"
pairing: element i goes with element i + d/2), for i < d/2:
    theta_i = base^(-2i/d),  a = p * theta_i
    v'[i]       = v[i] cos a - v[i + d/2] sin a
    v'[i + d/2] = v[i + d/2] cos a + v[i] sin a
The map is a rotation, so its backward is the rotation by -a.
"""
from __future__ import annotations

import numpy as np


def rmsnorm_fwd(x, w, eps):
    """x [M,H], w [H] -> (y [M,H], rstd [M]), float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    y = w[None, :] * (x * rstd[:, None])
    return y, rstd


def rmsnorm_bwd(dy, x, w, eps):
    """dx [M,H] for upstream dy [M,H] (w frozen: no weight gradient)."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    _, rstd = rmsnorm_fwd(x, w, eps)
    n = x * rstd[:, None]
    g = w[None, :] * dy
    return rstd[:, None] * (g - n * np.mean(g * n, axis=1, keepdims=True))


def rope_angles(pos, d, base):
    """[M, d/2] angles p * base^(-2i/d)."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def rope(v, pos, d, base, inverse=False):
    """Rotate every head of v [M, heads*d] by its token's angles (inverse: by -a)."""
    v = np.asarray(v, dtype=np.float64)
    M = v.shape[0]
    heads = v.shape[1] // d
    a = rope_angles(pos, d, base)
    c, s = np.cos(a)[:, None, :], np.sin(a)[:, None, :]
    if inverse:
        s = -s
    h = v.reshape(M, heads, d)
    lo, hi = h[:, :, : d // 2], h[:, :, d // 2:]
    out = np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=2)
    return out.reshape(M, heads * d)


def rope_bwd(dv, pos, d, base):
    """Gradient through rope(): the transpose of a rotation is its inverse."""
    return rope(dv, pos, d, base, inverse=True)
