"""Tensor-level entry points over the C ABI (torch provides device memory and the stream).

Each function checks shapes and dtypes, allocates the outputs and workspace
with torch, and calls one C-ABI entry point on the current HIP stream. No
arithmetic of the layer happens here.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib as C


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, shape, name):
    if t is None:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on GPU, got None")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on GPU, got {t.dtype} {tuple(t.shape)}")


def _need_ws(ws, nbytes: int, name="ws"):
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous() or not ws.is_cuda:
        raise ValueError(f"{name}: expected a contiguous 1-D uint8 GPU tensor")
    if ws.numel() < nbytes:
        raise ValueError(f"{name}: {ws.numel()} bytes, the call needs {nbytes}")


_GRAD_CODE = {torch.bfloat16: C.GRAD_BF16, torch.float32: C.GRAD_F32}


@dataclass
class QLoraLayer:
    """A frozen quantized weight with its LoRA pair (device tensors)."""
    codes: torch.Tensor   # uint8 [N, K/2] (NF4) or [N, K] (INT8, FP8)
    absmax: torch.Tensor  # float32 [N, K/64]: NF4 absmax, 8-bit scale
    A: torch.Tensor       # bfloat16 [r, K]
    B: torch.Tensor       # bfloat16 [N, r]
    s: float
    fmt: int = C.FMT_NF4
    grad_dtype: torch.dtype = torch.bfloat16  # dtype of dA, dB (bfloat16 or float32)

    @property
    def K(self):
        return self.A.shape[1]

    @property
    def N(self):
        return self.B.shape[0]

    @property
    def r(self):
        return self.A.shape[0]

    def c(self) -> C.QLoraLayerC:
        K, N, r = self.K, self.N, self.r
        _need(self.codes, torch.uint8, (N, K // 2 if self.fmt == C.FMT_NF4 else K), "codes")
        _need(self.absmax, torch.float32, (N, K // 64), "absmax")
        _need(self.A, torch.bfloat16, (r, K), "A")
        _need(self.B, torch.bfloat16, (N, r), "B")
        if self.grad_dtype not in _GRAD_CODE:
            raise ValueError(f"grad_dtype must be torch.bfloat16 or torch.float32, got {self.grad_dtype}")
        return C.QLoraLayerC(self.codes.data_ptr(), self.absmax.data_ptr(), self.A.data_ptr(), self.B.data_ptr(),
                             K, N, r, float(self.s), int(self.fmt), _GRAD_CODE[self.grad_dtype])


def quantize(W: torch.Tensor, fmt: int = C.FMT_NF4):
    """fp32 W [N,K] on the GPU -> (codes uint8 [N,K/2] (NF4) or [N,K] (INT8, FP8), block values fp32
    [N,K/64]). Raises on Inf/NaN."""
    N, K = W.shape
    _need(W, torch.float32, (N, K), "W")
    codes = torch.empty((N, K // 2 if fmt == C.FMT_NF4 else K), dtype=torch.uint8, device=W.device)
    absmax = torch.empty((N, K // 64), dtype=torch.float32, device=W.device)
    bad = torch.empty((1,), dtype=torch.int32, device=W.device)
    C.check("qlora_quantize", C.lib().qlora_quantize(fmt, _ptr(W), N, K, _ptr(codes), _ptr(absmax), _ptr(bad),
                                                     _stream()))
    if int(bad.item()) != 0:
        raise ValueError(f"qlora_quantize: {int(bad.item())} block(s) hold non-finite weights")
    return codes, absmax


def quantize_sync(W: torch.Tensor, fmt: int = C.FMT_NF4):
    """As quantize, through the synchronous form of qlora_quantize (no counter passed:
    the call waits for the stream and reports non-finite weights as QLORA_ENONFINITE,
    raised here as QLoraError)."""
    N, K = W.shape
    _need(W, torch.float32, (N, K), "W")
    codes = torch.empty((N, K // 2 if fmt == C.FMT_NF4 else K), dtype=torch.uint8, device=W.device)
    absmax = torch.empty((N, K // 64), dtype=torch.float32, device=W.device)
    C.check("qlora_quantize", C.lib().qlora_quantize(fmt, _ptr(W), N, K, _ptr(codes), _ptr(absmax), None,
                                                     _stream()))
    return codes, absmax


def pack_codes(codes_rowmajor: torch.Tensor, absmax_rowmajor: torch.Tensor, fmt: int = C.FMT_NF4):
    """Codes and block values in checkpoint order (row-major; NF4 column 2c in the low nibble
    of byte c) -> this library's storage order: (codes, absmax) of the same shapes."""
    N, KC = codes_rowmajor.shape
    K = 2 * KC if fmt == C.FMT_NF4 else KC
    _need(codes_rowmajor, torch.uint8, (N, KC), "codes_rowmajor")
    _need(absmax_rowmajor, torch.float32, (N, K // 64), "absmax_rowmajor")
    codes = torch.empty_like(codes_rowmajor)
    absmax = torch.empty_like(absmax_rowmajor)
    C.check("qlora_pack_codes", C.lib().qlora_pack_codes(fmt, _ptr(codes_rowmajor), _ptr(absmax_rowmajor), N, K,
                                                         _ptr(codes), _ptr(absmax), _stream()))
    return codes, absmax


def dequantize(codes: torch.Tensor, absmax: torch.Tensor, fmt: int = C.FMT_NF4) -> torch.Tensor:
    N, KC = codes.shape
    K = 2 * KC if fmt == C.FMT_NF4 else KC
    _need(codes, torch.uint8, (N, KC), "codes")
    _need(absmax, torch.float32, (N, K // 64), "absmax")
    out = torch.empty((N, K), dtype=torch.float32, device=codes.device)
    C.check("qlora_dequantize", C.lib().qlora_dequantize(fmt, _ptr(codes), _ptr(absmax), N, K, _ptr(out),
                                                         _stream()))
    return out


def workspace_size(op: int, M: int, K: int, N: int, r: int) -> int:
    return int(C.lib().qlora_workspace_size(op, M, K, N, r))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)


def forward(L: QLoraLayer, X: torch.Tensor, Y=None, Z=None):
    """Y [M,N] bf16 and Z = X.A^T [M,r] bf16."""
    M = X.shape[0]
    _need(X, torch.bfloat16, (M, L.K), "X")
    Y = torch.empty((M, L.N), dtype=torch.bfloat16, device=X.device) if Y is None else Y
    Z = torch.empty((M, L.r), dtype=torch.bfloat16, device=X.device) if Z is None else Z
    _need(Y, torch.bfloat16, (M, L.N), "Y")
    _need(Z, torch.bfloat16, (M, L.r), "Z")
    lc = L.c()
    C.check("qlora_forward", C.lib().qlora_forward(ctypes.byref(lc), _ptr(X), M, _ptr(Y), _ptr(Z), None, 0,
                                                   _stream()))
    return Y, Z


def backward(L: QLoraLayer, dY, X, Z, need_dX=True, ws=None, out=None):
    """(dX bf16 [M,K] or None, dA [r,K], dB [N,r]; dA, dB in L.grad_dtype)."""
    M = X.shape[0]
    _need(dY, torch.bfloat16, (M, L.N), "dY")
    _need(X, torch.bfloat16, (M, L.K), "X")
    _need(Z, torch.bfloat16, (M, L.r), "Z")
    dev = X.device
    gd = L.grad_dtype
    if out is None:
        dX = torch.empty((M, L.K), dtype=torch.bfloat16, device=dev) if need_dX else None
        dA = torch.empty((L.r, L.K), dtype=gd, device=dev)
        dB = torch.empty((L.N, L.r), dtype=gd, device=dev)
    else:
        dX, dA, dB = out
    if dX is not None:
        _need(dX, torch.bfloat16, (M, L.K), "dX")
    _need(dA, gd, (L.r, L.K), "dA")
    _need(dB, gd, (L.N, L.r), "dB")
    nb = workspace_size(C.OP_BACKWARD, M, L.K, L.N, L.r)
    ws = _workspace(nb, dev) if ws is None else ws
    _need_ws(ws, nb)
    lc = L.c()
    C.check("qlora_backward", C.lib().qlora_backward(ctypes.byref(lc), _ptr(dY), _ptr(X), _ptr(Z), M, _ptr(dX),
                                                     _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(), _stream()))
    return dX, dA, dB


class _LinearFn(torch.autograd.Function):
    """Autograd node of one projection: the library's forward, and its backward for
    dX, dA and dB (the frozen weight gets no gradient)."""

    @staticmethod
    def forward(ctx, X, A, B, L):
        Y, Z = forward(L, X)
        ctx.save_for_backward(X, Z)
        ctx.L = L
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, Z = ctx.saved_tensors
        dX, dA, dB = backward(ctx.L, dY.contiguous(), X, Z, need_dX=ctx.needs_input_grad[0])
        return dX, dA, dB, None


def linear(X: torch.Tensor, L: QLoraLayer) -> torch.Tensor:
    """Y = X.What^T + s.(X.A^T).B^T for bf16 X [..., K] (leading dimensions are the
    tokens), differentiable in X, L.A and L.B through the library's backward. The
    adapters' gradients come in their own dtype, so L.grad_dtype must be bfloat16."""
    if L.grad_dtype != L.A.dtype or L.grad_dtype != L.B.dtype:
        raise ValueError("linear(): the layer's grad_dtype must be the adapters' dtype (torch.bfloat16)")
    lead = X.shape[:-1]
    Y = _LinearFn.apply(X.reshape(-1, L.K), L.A, L.B, L)
    return Y.reshape(*lead, L.N)


class QLoraLinear(torch.nn.Module):
    """One projection for a PyTorch training loop: the frozen quantized weight (codes
    and block values, as buffers) and the trainable bf16 adapters A [r, K], B [N, r]
    (parameters); forward and backward run in the library."""

    def __init__(self, codes: torch.Tensor, absmax: torch.Tensor, A: torch.Tensor, B: torch.Tensor, s: float,
                 fmt: int = C.FMT_NF4):
        super().__init__()
        self.register_buffer("codes", codes)
        self.register_buffer("absmax", absmax)
        self.A = torch.nn.Parameter(A)
        self.B = torch.nn.Parameter(B)
        self.s = float(s)
        self.fmt = int(fmt)

    def layer(self) -> QLoraLayer:
        return QLoraLayer(self.codes, self.absmax, self.A, self.B, self.s, self.fmt)

    def forward(self, X: torch.Tensor) -> torch.Tensor:
        return linear(X, self.layer())


def mlp_forward(gate: QLoraLayer, up: QLoraLayer, down: QLoraLayer, X, out=None):
    """dict(Y, g, u, h, Z) for the SwiGLU block; Z is [3, M, r] (gate, up, down)."""
    M = X.shape[0]
    H, I, r = gate.K, gate.N, gate.r
    _need(X, torch.bfloat16, (M, H), "X")
    dev = X.device
    if out is None:
        out = dict(Y=torch.empty((M, H), dtype=torch.bfloat16, device=dev),
                   g=torch.empty((M, I), dtype=torch.bfloat16, device=dev),
                   u=torch.empty((M, I), dtype=torch.bfloat16, device=dev),
                   h=torch.empty((M, I), dtype=torch.bfloat16, device=dev),
                   Z=torch.empty((3, M, r), dtype=torch.bfloat16, device=dev))
    _need_saved(out, M, H, I, r, ("Y", "g", "u", "h"))
    lg, lu, ld = gate.c(), up.c(), down.c()
    C.check("swiglu_mlp_forward", C.lib().swiglu_mlp_forward(
        ctypes.byref(lg), ctypes.byref(lu), ctypes.byref(ld), _ptr(X), M, _ptr(out["Y"]), _ptr(out["g"]),
        _ptr(out["u"]), _ptr(out["h"]), _ptr(out["Z"]), None, 0, _stream()))
    return out


def _need_saved(t: dict, M, H, I, r, keys):
    shapes = dict(Y=(M, H), g=(M, I), u=(M, I), h=(M, I))
    for k in keys:
        _need(t[k], torch.bfloat16, shapes[k], k)
    _need(t["Z"], torch.bfloat16, (3, M, r), "Z")


def _grads_out(layers, out, M, H, dev, need_dX):
    """Adapter-gradient outputs of a SwiGLU backward (allocated, or the caller's, checked)."""
    gd = layers[0].grad_dtype
    if any(L.grad_dtype != gd for L in layers):
        raise ValueError("the three layers of a SwiGLU block share one grad_dtype")
    if out is None:
        out = dict(dX=torch.empty((M, H), dtype=torch.bfloat16, device=dev) if need_dX else None,
                   dA=[torch.empty((L.r, L.K), dtype=gd, device=dev) for L in layers],
                   dB=[torch.empty((L.N, L.r), dtype=gd, device=dev) for L in layers])
    if out["dX"] is not None:
        _need(out["dX"], torch.bfloat16, (M, H), "dX")
    for i, L in enumerate(layers):
        _need(out["dA"][i], gd, (L.r, L.K), f"dA[{i}]")
        _need(out["dB"][i], gd, (L.N, L.r), f"dB[{i}]")
    return out


def mlp_backward(gate: QLoraLayer, up: QLoraLayer, down: QLoraLayer, dY, X, saved, need_dX=True, ws=None, out=None):
    """dict(dX, dA=[gate, up, down], dB=[...]) with dA, dB in the layers' grad_dtype."""
    M = X.shape[0]
    H, I, r = gate.K, gate.N, gate.r
    _need(dY, torch.bfloat16, (M, H), "dY")
    _need(X, torch.bfloat16, (M, H), "X")
    _need_saved(saved, M, H, I, r, ("g", "u", "h"))
    dev = X.device
    out = _grads_out((gate, up, down), out, M, H, dev, need_dX)
    nb = workspace_size(C.OP_MLP_BACKWARD, M, H, I, r)
    ws = _workspace(nb, dev) if ws is None else ws
    _need_ws(ws, nb)
    dA = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in out["dA"]])
    dB = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in out["dB"]])
    lg, lu, ld = gate.c(), up.c(), down.c()
    C.check("swiglu_mlp_backward", C.lib().swiglu_mlp_backward(
        ctypes.byref(lg), ctypes.byref(lu), ctypes.byref(ld), _ptr(dY), _ptr(X), _ptr(saved["g"]), _ptr(saved["u"]),
        _ptr(saved["h"]), _ptr(saved["Z"]), M, _ptr(out["dX"]), dA, dB, _ptr(ws), ws.numel(), _stream()))
    return out


class _SwiGLUFn(torch.autograd.Function):
    """Autograd node of the SwiGLU block: the library's forward (saving g, u, h and
    the three Z) and its backward for dX and the six adapter gradients."""

    @staticmethod
    def forward(ctx, X, Ag, Bg, Au, Bu, Ad, Bd, layers):
        out = mlp_forward(*layers, X)
        ctx.save_for_backward(X, out["g"], out["u"], out["h"], out["Z"])
        ctx.layers = layers
        return out["Y"]

    @staticmethod
    def backward(ctx, dY):
        X, g, u, h, Z = ctx.saved_tensors
        b = mlp_backward(*ctx.layers, dY.contiguous(), X, dict(g=g, u=u, h=h, Z=Z), need_dX=ctx.needs_input_grad[0])
        (dAg, dAu, dAd), (dBg, dBu, dBd) = b["dA"], b["dB"]
        return b["dX"], dAg, dBg, dAu, dBu, dAd, dBd, None


def swiglu_mlp(X: torch.Tensor, gate: QLoraLayer, up: QLoraLayer, down: QLoraLayer) -> torch.Tensor:
    """The SwiGLU block Y = down(silu(gate(X)) * up(X)) for bf16 X [..., H] (leading
    dimensions are the tokens), differentiable in X and the six adapters through the
    library's backward; the layers' grad_dtype must be the adapters' dtype (bfloat16)."""
    layers = (gate, up, down)
    if any(L.grad_dtype != L.A.dtype or L.grad_dtype != L.B.dtype for L in layers):
        raise ValueError("swiglu_mlp(): the layers' grad_dtype must be the adapters' dtype (torch.bfloat16)")
    lead = X.shape[:-1]
    Y = _SwiGLUFn.apply(X.reshape(-1, gate.K), gate.A, gate.B, up.A, up.B, down.A, down.B, layers)
    return Y.reshape(*lead, down.N)


def mlp_tiled_workspace_size(backward: bool, M: int, H: int, I: int, r: int, tile: int) -> int:
    return int(C.lib().swiglu_mlp_tiled_workspace_size(1 if backward else 0, M, H, I, r, tile))


def mlp_forward_tiled(gate: QLoraLayer, up: QLoraLayer, down: QLoraLayer, X, tile: int, ws=None, out=None):
    """dict(Y, Z) for the SwiGLU block computed `tile` tokens at a time (no g, u, h kept)."""
    M = X.shape[0]
    H, I, r = gate.K, gate.N, gate.r
    _need(X, torch.bfloat16, (M, H), "X")
    dev = X.device
    if out is None:
        out = dict(Y=torch.empty((M, H), dtype=torch.bfloat16, device=dev),
                   Z=torch.empty((3, M, r), dtype=torch.bfloat16, device=dev))
    _need_saved(out, M, H, I, r, ("Y",))
    nb = mlp_tiled_workspace_size(False, M, H, I, r, tile)
    ws = _workspace(nb, dev) if ws is None else ws
    _need_ws(ws, nb)
    lg, lu, ld = gate.c(), up.c(), down.c()
    C.check("swiglu_mlp_forward_tiled", C.lib().swiglu_mlp_forward_tiled(
        ctypes.byref(lg), ctypes.byref(lu), ctypes.byref(ld), _ptr(X), M, tile, _ptr(out["Y"]), _ptr(out["Z"]),
        _ptr(ws), ws.numel(), _stream()))
    return out


def mlp_backward_tiled(gate: QLoraLayer, up: QLoraLayer, down: QLoraLayer, dY, X, Z, tile: int, need_dX=True,
                       ws=None, out=None):
    """dict(dX, dA, dB) of the SwiGLU block, `tile` tokens at a time (g, u, h recomputed per tile)."""
    M = X.shape[0]
    H, I, r = gate.K, gate.N, gate.r
    _need(dY, torch.bfloat16, (M, H), "dY")
    _need(X, torch.bfloat16, (M, H), "X")
    _need(Z, torch.bfloat16, (3, M, r), "Z")
    dev = X.device
    out = _grads_out((gate, up, down), out, M, H, dev, need_dX)
    nb = mlp_tiled_workspace_size(True, M, H, I, r, tile)
    ws = _workspace(nb, dev) if ws is None else ws
    _need_ws(ws, nb)
    dA = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in out["dA"]])
    dB = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in out["dB"]])
    lg, lu, ld = gate.c(), up.c(), down.c()
    C.check("swiglu_mlp_backward_tiled", C.lib().swiglu_mlp_backward_tiled(
        ctypes.byref(lg), ctypes.byref(lu), ctypes.byref(ld), _ptr(dY), _ptr(X), _ptr(Z), M, tile, _ptr(out["dX"]),
        dA, dB, _ptr(ws), ws.numel(), _stream()))
    return out


def rmsnorm_forward(x, w, eps: float, y=None, rstd=None):
    """(y bf16 [M,H], rstd fp32 [M]) = RMSNorm of x [M,H] with the frozen weight w [H] (bf16)."""
    M, H = x.shape
    _need(x, torch.bfloat16, (M, H), "x")
    _need(w, torch.bfloat16, (H,), "w")
    y = torch.empty_like(x) if y is None else y
    rstd = torch.empty((M,), dtype=torch.float32, device=x.device) if rstd is None else rstd
    _need(y, torch.bfloat16, (M, H), "y")
    _need(rstd, torch.float32, (M,), "rstd")
    C.check("qlora_rmsnorm_forward", C.lib().qlora_rmsnorm_forward(_ptr(x), _ptr(w), M, H, float(eps), _ptr(y),
                                                                   _ptr(rstd), _stream()))
    return y, rstd


def rmsnorm_backward(dy, x, w, rstd, dx=None):
    """dx bf16 [M,H] of the RMSNorm (no weight gradient: w is frozen)."""
    M, H = x.shape
    _need(dy, torch.bfloat16, (M, H), "dy")
    _need(x, torch.bfloat16, (M, H), "x")
    _need(w, torch.bfloat16, (H,), "w")
    _need(rstd, torch.float32, (M,), "rstd")
    dx = torch.empty_like(x) if dx is None else dx
    _need(dx, torch.bfloat16, (M, H), "dx")
    C.check("qlora_rmsnorm_backward", C.lib().qlora_rmsnorm_backward(_ptr(dy), _ptr(x), _ptr(w), _ptr(rstd), M, H,
                                                                     _ptr(dx), _stream()))
    return dx


def _rope(fn, q, k, pos, d: int, base: float):
    M = pos.shape[0]
    _need(pos, torch.int32, (M,), "pos")
    hq = 0 if q is None else q.shape[1] // d
    hk = 0 if k is None else k.shape[1] // d
    if q is not None:
        _need(q, torch.bfloat16, (M, hq * d), "q")
    if k is not None:
        _need(k, torch.bfloat16, (M, hk * d), "k")
    C.check(fn, getattr(C.lib(), fn)(_ptr(q), _ptr(k), _ptr(pos), M, hq, hk, d, float(base), _stream()))
    return q, k


def rope_forward(q, k, pos, d: int, base: float):
    """Rotate q [M, hq*d] and k [M, hk*d] (bf16, in place) by positions pos [M] (int32)."""
    return _rope("qlora_rope_forward", q, k, pos, d, base)


def rope_backward(dq, dk, pos, d: int, base: float):
    """Gradients through rope_forward (the inverse rotation, in place)."""
    return _rope("qlora_rope_backward", dq, dk, pos, d, base)


def rope_table(d: int, base: float, max_pos: int, device="cuda"):
    """fp32 cos/sin of the RoPE angles [max_pos, d/2, 2] (fp64 angles and sin/cos)."""
    t = torch.empty((max_pos, d // 2, 2), dtype=torch.float32, device=device)
    C.check("qlora_rope_table", C.lib().qlora_rope_table(d, float(base), max_pos, _ptr(t), _stream()))
    return t


def forward_rope(L: QLoraLayer, X: torch.Tensor, pos, table, d: int = 128, Y=None, Z=None):
    """Y = rope(X.W^T + s.Z.B^T) [M,N] bf16 (RoPE in the GEMM epilogue) and Z = X.A^T [M,r]."""
    M = X.shape[0]
    _need(X, torch.bfloat16, (M, L.K), "X")
    _need(pos, torch.int32, (M,), "pos")
    max_pos = table.shape[0]
    _need(table, torch.float32, (max_pos, d // 2, 2), "table")
    Y = torch.empty((M, L.N), dtype=torch.bfloat16, device=X.device) if Y is None else Y
    Z = torch.empty((M, L.r), dtype=torch.bfloat16, device=X.device) if Z is None else Z
    _need(Y, torch.bfloat16, (M, L.N), "Y")
    _need(Z, torch.bfloat16, (M, L.r), "Z")
    lc = L.c()
    C.check("qlora_forward_rope", C.lib().qlora_forward_rope(ctypes.byref(lc), _ptr(X), M, _ptr(pos), _ptr(table),
                                                             max_pos, d, _ptr(Y), _ptr(Z), _stream()))
    return Y, Z


def lmhead_prepare(W):
    """The frozen LM head W [V, H] (bf16) laid out for chunked_ce's two products: (Wp, Wtp),
    each V*H bf16 values (tiled; see qlora_lmhead_prepare)."""
    V, H = W.shape
    _need(W, torch.bfloat16, (V, H), "W")
    Wp = torch.empty((V * H,), dtype=torch.bfloat16, device=W.device)
    Wtp = torch.empty((V * H,), dtype=torch.bfloat16, device=W.device)
    C.check("qlora_lmhead_prepare", C.lib().qlora_lmhead_prepare(_ptr(W), V, H, _ptr(Wp), _ptr(Wtp), _stream()))
    return Wp, Wtp


def ce_chunk_for_budget(V: int, budget_bytes: int) -> int:
    """Largest chunk (a multiple of 256 tokens, at least 256) whose workspace (fp32 logits and
    bf16 gradient of the chunk) fits the given memory budget."""
    return max(256, (budget_bytes // (6 * V)) // 256 * 256)


def chunked_ce(h, prepared, targets, chunk: int, ws=None, out=None):
    """Cross-entropy of the frozen LM head (prepared = lmhead_prepare(W), W [V,H]) over h [M,H]
    with int32 targets [M] (negative = ignored): dict(loss fp32 [1], loss_rows fp32 [M], dh bf16 [M,H])."""
    M, H = h.shape
    Wp, Wtp = prepared
    V = Wp.numel() // H
    _need(h, torch.bfloat16, (M, H), "h")
    _need(Wp, torch.bfloat16, (V * H,), "Wp")
    _need(Wtp, torch.bfloat16, (V * H,), "Wtp")
    _need(targets, torch.int32, (M,), "targets")
    dev = h.device
    if out is None:
        out = dict(loss=torch.empty((1,), dtype=torch.float32, device=dev),
                   loss_rows=torch.empty((M,), dtype=torch.float32, device=dev),
                   dh=torch.empty((M, H), dtype=torch.bfloat16, device=dev))
    _need(out["loss"], torch.float32, (1,), "loss")
    _need(out["loss_rows"], torch.float32, (M,), "loss_rows")
    _need(out["dh"], torch.bfloat16, (M, H), "dh")
    nb = int(C.lib().qlora_ce_workspace_size(M, V, chunk))
    ws = _workspace(nb, dev) if ws is None else ws
    _need_ws(ws, nb)
    C.check("qlora_chunked_ce", C.lib().qlora_chunked_ce(
        _ptr(h), _ptr(Wp), _ptr(Wtp), _ptr(targets), M, H, V, chunk, _ptr(out["loss"]), _ptr(out["loss_rows"]),
        _ptr(out["dh"]), _ptr(ws), ws.numel(), _stream()))
    return out


class KernelTimer:
    """Per-kernel-class launch durations from hipEvents the library records around
    each of its launches (on the launch's stream). Use as a context manager."""

    def __init__(self, max_launches: int = 100_000):
        self.max_launches = max_launches
        self.result = {}

    def __enter__(self):
        C.check("qlora_profile_begin", C.lib().qlora_profile_begin(self.max_launches))
        return self

    def __exit__(self, *exc):
        buf = (C.KernelTimeC * 64)()
        n = ctypes.c_int(0)
        st = C.lib().qlora_profile_end(buf, 64, ctypes.byref(n))
        self.result = {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(n.value)}
        if st != C.QLORA_OK and exc[0] is None:
            C.check("qlora_profile_end", st)
        return False
