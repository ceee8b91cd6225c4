"""8-bit formats of the frozen weight (test infrastructure: only the tests,
the smoke check and bench.py's CPU-baseline leg use this module).

The fused quantized-LoRA card ("Rev vs unsloth") names int4, int8 and fp8
quantized base weights and the quantized-base card ("Unsloth vs The Stack
v2") 4-bit and 8-bit ones; neither gives a format. The readings here keep the
4-bit format's blocks (64 consecutive elements of a weight row share one fp32
value) and make that value the block's scale s:

  INT8  s = fp32(a / 127) with a = max |W| over the block;
        q = clamp(rint(fp32(W / s)), -127, 127)  (round half to even),
        stored as a two's-complement byte.
  FP8   OCP E4M3 (1 sign bit, 4 exponent bits biased by 7, 3 mantissa bits,
        subnormals, no infinities; 0x7F and 0xFF are NaN; largest finite 448):
        s = fp32(a / 448); the code is the E4M3 value nearest to fp32(W / s)
        (ties to the even code), at most 448 in magnitude, with W's sign.
  both  a block of zeros has s = 0 and codes 0.
  What  fp32(v * s) for the code's exact value v: one rounding.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64
FMT_NF4, FMT_INT8, FMT_FP8 = 0, 1, 2


def e4m3_value(code: int) -> float:
    """Exact value of an OCP E4M3 byte (NaN for 0x7F / 0xFF)."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_VALUES.setflags(write=False)
_MAG = E4M3_VALUES[:127]  # codes 0x00 .. 0x7E: the finite non-negative values, increasing


def _blocks_scale(W, qmax):
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % BLOCK != 0:
        raise ValueError("W must be [N, K] with K a multiple of 64")
    if not np.isfinite(W).all():
        raise ValueError("non-finite weight")
    N, K = W.shape
    blocks = W.reshape(N, K // BLOCK, BLOCK)
    a = np.abs(blocks).max(axis=2)                       # exact in fp32
    s = (a / np.float32(qmax)).astype(np.float32)        # IEEE fp32 division
    zero = s == 0
    denom = np.where(zero, np.float32(1.0), s).astype(np.float32)
    x = (blocks / denom[:, :, None]).astype(np.float32)  # IEEE fp32 division
    return x, s, zero, (N, K)


def quantize_int8(W):
    """fp32 W [N,K] -> (codes uint8 [N,K] (two's complement), scale fp32 [N,K/64])."""
    x, s, zero, (N, K) = _blocks_scale(W, 127)
    q = np.clip(np.rint(x.astype(np.float64)), -127, 127).astype(np.int64)
    q[zero] = 0
    return (q.reshape(N, K) & 0xFF).astype(np.uint8), s


def quantize_fp8(W):
    """fp32 W [N,K] -> (codes uint8 [N,K] E4M3, scale fp32 [N,K/64])."""
    x, s, zero, (N, K) = _blocks_scale(W, 448)
    ax = np.abs(x.astype(np.float64))
    hi = np.clip(np.searchsorted(_MAG, ax, side="left"), 0, 126)   # first magnitude >= ax
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = ax - _MAG[lo], _MAG[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(ax >= _MAG[126], 126, mag)                        # saturate at 448
    sign = (np.signbit(x)).astype(np.int64) << 7
    codes = (mag | sign).astype(np.int64)
    codes[zero] = 0
    return codes.reshape(N, K).astype(np.uint8), s


def code_values(codes, fmt: int) -> np.ndarray:
    """Exact value of each 8-bit code as float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    if fmt == FMT_INT8:
        return codes.view(np.int8).astype(np.float64)
    if fmt == FMT_FP8:
        return E4M3_VALUES[codes]
    raise ValueError("not an 8-bit format")


def dequantize(codes, scale, fmt: int) -> np.ndarray:
    """What[n,k] = fp32(v[n,k] * s[n, k // 64]), one rounding (v * s is exact in float64:
    at most 8 + 24 significant bits)."""
    v = code_values(codes, fmt)
    s = np.repeat(np.asarray(scale, dtype=np.float32).astype(np.float64), BLOCK, axis=1)
    return (v * s).astype(np.float32)


def quantize(W, fmt: int):
    if fmt == FMT_INT8:
        return quantize_int8(W)
    if fmt == FMT_FP8:
        return quantize_fp8(W)
    raise ValueError("not an 8-bit format")
