"""Seeded synthetic inputs for the fused QLoRA linear layer and its SwiGLU MLP.

This module is the only code shared by the CPU oracle side and the GPU side.
It draws random numbers and rounds them to bf16; it holds none of the
method's arithmetic (no quantization, no matmul, no activation).

Workloads (all shapes follow the Llama-3-8B projections that the Unsloth wiki
entry's example targets: q, k, v, o, gate, up, down with r=16, lora_alpha=32;
see the wiki entry "Unsloth", API snippet):

  tiny     M=256, K=N=512, r=8, alpha=16
  attn     M=4096, K=N=4096, r=16, alpha=32                (one attention projection)
  mlp      M=4096, hidden 4096, intermediate 14336, r=16   (SwiGLU block, LoRA on all 3)
  rsweep   M=8192, K=N=4096, r in {8,16,64,128}, alpha=2r  (rank sweep, sub-run i picks r)
  layer    M=16384, q,o 4096x4096, k,v 4096->1024, MLP as above, r=16  (all 7 projections)

Draw order, per workload with seed = 1000*c + i: for each projection in order
(q, k, v, o, gate, up, down, or the single one) draw W, then A, then B; then
the activations; then one upstream gradient per output.

Distributions: W = 0.02*N(0,1) in fp32 (quantized by the caller);
A = N(0,1)/sqrt(K) -> bf16; B = 0.02*N(0,1) -> bf16; X, dY = N(0,1) -> bf16.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# bf16 helpers (bit patterns stored as uint16)

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the bits as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# counter-based draws for the largest shapes
#
# Element i of stream `seed` depends on (seed, i) alone, so any slice of an
# input (a weight row, one 64-column block of every row, an activation row)
# can be drawn on the host without drawing the rest, and the whole tensor on
# the device with the same arithmetic (numpy int64 on the host, torch int64 on
# the device). The integer hash is the 32-bit "lowbias32" mixer (xorshift and
# multiply rounds, C. Wellons' hash prospector); two hashed uniforms summed give
# a triangular value with mean 0, scaled to unit variance. Every step is an
# exact integer operation or one fp32 rounding in a fixed order, so both sides
# produce identical bits. Indices must stay below 2^32.

_M32 = 0xFFFFFFFF


def _mix32(x):
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & _M32
    x = x ^ (x >> 15)
    x = (x * 0x846CA68B) & _M32
    return x ^ (x >> 16)


def counter_normal(seed: int, idx, scale: float = 1.0):
    """fp32 draws for int64 element indices idx (a numpy array or a torch tensor on
    any device): mean 0, standard deviation `scale`, support +-sqrt(6)*scale.
    numpy computes in uint32 (wrapping products), torch in int64 with masks."""
    host = isinstance(idx, np.ndarray)
    x0 = idx.astype(np.uint32) if host else idx
    u = None
    for j in range(2):
        key = _mix32(4 * seed + j + 1)  # a Python int
        if host:
            x = x0 + np.uint32(key)
            x ^= x >> np.uint32(16)
            x *= np.uint32(0x7FEB352D)
            x ^= x >> np.uint32(15)
            x *= np.uint32(0x846CA68B)
            x ^= x >> np.uint32(16)
            v = (x >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)
        else:
            x = _mix32((x0 + key) & _M32)
            v = (x >> 8).float() * np.float32(2.0 ** -24)
        u = v if u is None else u + v
    return (u - np.float32(1.0)) * np.float32(2.449489742783178 * scale)


# ---------------------------------------------------------------------------
# workload table

WORKLOADS = {
    0: dict(name="tiny", kind="linear", M=256, K=512, N=512, ranks=(8,)),
    1: dict(name="attn", kind="linear", M=4096, K=4096, N=4096, ranks=(16,)),
    2: dict(name="mlp", kind="mlp", M=4096, H=4096, I=14336, ranks=(16,)),
    3: dict(name="rsweep", kind="linear", M=8192, K=4096, N=4096, ranks=(8, 16, 64, 128)),
    4: dict(name="layer", kind="layer", M=16384, H=4096, KV=1024, I=14336, ranks=(16,)),
}


def projections(c: int, sub: int = 0):
    """Return [(name, K, N), ...] for workload c in draw order, and the rank."""
    w = WORKLOADS[c]
    r = w["ranks"][sub]
    if w["kind"] == "linear":
        return [("proj", w["K"], w["N"])], r
    if w["kind"] == "mlp":
        H, I = w["H"], w["I"]
        return [("gate", H, I), ("up", H, I), ("down", I, H)], r
    H, KV, I = w["H"], w["KV"], w["I"]
    return [("q", H, H), ("k", H, KV), ("v", H, KV), ("o", H, H),
            ("gate", H, I), ("up", H, I), ("down", I, H)], r


def _normal(rng, shape, scale=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def make_adapter_layer(rng, K: int, N: int, r: int):
    """Draw one projection: W fp32 [N,K], A bf16 [r,K], B bf16 [N,r] (in that order)."""
    W = _normal(rng, (N, K), 0.02)
    A = bf16_bits(_normal(rng, (r, K), 1.0 / np.sqrt(K)))
    B = bf16_bits(_normal(rng, (N, r), 0.02))
    return dict(W=W, A=A, B=B, K=K, N=N, r=r)


def make_workload(c: int, sub: int = 0, M: int | None = None, seed: int | None = None):
    """Build the seeded inputs of workload c (sub-run `sub`).

    M overrides the token count (the draw order and distributions stay the same).
    Returns dict(layers={name: layer}, r, alpha, s, M, X..., dY...).
    """
    w = WORKLOADS[c]
    projs, r = projections(c, sub)
    alpha = 2 * r
    M = w["M"] if M is None else M
    rng = np.random.default_rng(1000 * c + sub if seed is None else seed)
    layers = {}
    for name, K, N in projs:
        layers[name] = make_adapter_layer(rng, K, N, r)
    out = dict(c=c, sub=sub, name=w["name"], kind=w["kind"], M=M, r=r, alpha=alpha,
               s=float(alpha) / float(r), layers=layers, order=[p[0] for p in projs])
    if w["kind"] == "linear":
        K, N = projs[0][1], projs[0][2]
        out["X"] = bf16_bits(_normal(rng, (M, K)))
        out["dY"] = bf16_bits(_normal(rng, (M, N)))
    elif w["kind"] == "mlp":
        out["X"] = bf16_bits(_normal(rng, (M, w["H"])))
        out["dY"] = bf16_bits(_normal(rng, (M, w["H"])))
    else:
        H, KV = w["H"], w["KV"]
        out["X_attn"] = bf16_bits(_normal(rng, (M, H)))
        out["X_o"] = bf16_bits(_normal(rng, (M, H)))
        out["X_mlp"] = bf16_bits(_normal(rng, (M, H)))
        out["dY_q"] = bf16_bits(_normal(rng, (M, H)))
        out["dY_k"] = bf16_bits(_normal(rng, (M, KV)))
        out["dY_v"] = bf16_bits(_normal(rng, (M, KV)))
        out["dY_o"] = bf16_bits(_normal(rng, (M, H)))
        out["dY_mlp"] = bf16_bits(_normal(rng, (M, H)))
    return out


def random_linear(seed: int, M: int, K: int, N: int, r: int, alpha: float | None = None):
    """A single projection of arbitrary shape with the same distributions (edge-case tests)."""
    rng = np.random.default_rng(seed)
    L = make_adapter_layer(rng, K, N, r)
    X = bf16_bits(_normal(rng, (M, K)))
    dY = bf16_bits(_normal(rng, (M, N)))
    alpha = 2.0 * r if alpha is None else alpha
    return dict(layers={"proj": L}, X=X, dY=dY, M=M, r=r, alpha=alpha, s=float(alpha) / r,
                order=["proj"], kind="linear")


def random_mlp(seed: int, M: int, H: int, I: int, r: int, alpha: float | None = None):
    """A SwiGLU MLP of arbitrary shape with the same distributions (edge-case tests)."""
    rng = np.random.default_rng(seed)
    layers = {"gate": make_adapter_layer(rng, H, I, r), "up": make_adapter_layer(rng, H, I, r),
              "down": make_adapter_layer(rng, I, H, r)}
    X = bf16_bits(_normal(rng, (M, H)))
    dY = bf16_bits(_normal(rng, (M, H)))
    alpha = 2.0 * r if alpha is None else alpha
    return dict(layers=layers, X=X, dY=dY, M=M, r=r, alpha=alpha, s=float(alpha) / r,
                order=["gate", "up", "down"], kind="mlp")


def useful_flops(c: int, sub: int = 0, M: int | None = None) -> float:
    """Useful fwd+bwd FLOPs: 4*M*N*K + 6*M*r*(N+K) per projection (no dW, no dequant work)."""
    projs, r = projections(c, sub)
    M = WORKLOADS[c]["M"] if M is None else M
    return float(sum(4 * M * N * K + 6 * M * r * (N + K) for _, K, N in projs))


# ---------------------------------------------------------------------------
# inputs of the steps around the projections (RMSNorm, RoPE)

def packed_positions(rng, M: int, max_len: int) -> np.ndarray:
    """Positions of M tokens packed from sequences of random length (1..max_len),
    each counting from 0: int32 [M]."""
    pos = np.empty(M, dtype=np.int32)
    m = 0
    while m < M:
        n = int(min(M - m, rng.integers(1, max_len + 1)))
        pos[m:m + n] = np.arange(n, dtype=np.int32)
        m += n
    return pos


def random_norm_rope(seed: int, M: int, H: int, hq: int, hk: int, d: int, max_len: int = 16384):
    """x, dy [M,H] = N(0,1); norm weight w [H] = 1 + 0.1 N(0,1); q [M,hq*d], k [M,hk*d],
    dq, dk = N(0,1); positions of packed sequences up to max_len. All bf16 bits but pos."""
    rng = np.random.default_rng(seed)
    return dict(x=bf16_bits(_normal(rng, (M, H))), dy=bf16_bits(_normal(rng, (M, H))),
                w=bf16_bits(1.0 + 0.1 * _normal(rng, (H,))),
                q=bf16_bits(_normal(rng, (M, hq * d))), k=bf16_bits(_normal(rng, (M, hk * d))),
                dq=bf16_bits(_normal(rng, (M, hq * d))), dk=bf16_bits(_normal(rng, (M, hk * d))),
                pos=packed_positions(rng, M, max_len), M=M, H=H, hq=hq, hk=hk, d=d)


def random_ce(seed: int, M: int, H: int, V: int, ignore_frac: float = 0.1):
    """h [M,H] = N(0,1), LM head W [V,H] = 0.02 N(0,1) (bf16 bits), targets [M] int32
    uniform in [0, V) with about ignore_frac of them -100 (ignored)."""
    rng = np.random.default_rng(seed)
    h = bf16_bits(_normal(rng, (M, H)))
    W = bf16_bits(_normal(rng, (V, H), 0.02))
    t = rng.integers(0, V, M).astype(np.int32)
    t[rng.random(M) < ignore_frac] = -100
    return dict(h=h, W=W, targets=t, M=M, H=H, V=V)
