#!/usr/bin/env python3
"""Throughput of the fused QLoRA layer (forward + backward) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload attn|tiny|mlp|rsweep|layer] [--rank R]
                [--mlp-tile T]

A step is one forward and one backward of the workload over one batch of
seeded synthetic inputs already resident in HBM:
  attn   : one Llama-3-8B attention projection, M=4096 tokens, K=N=4096, r=16 (default)
  tiny   : M=256, K=N=512, r=8
  mlp    : SwiGLU block, M=4096, 4096 <-> 14336, LoRA r=16 on gate/up/down
  rsweep : M=8192, K=N=4096, r from --rank (8, 16, 64, 128)
  layer  : the 7 projections of a Llama-3.1-8B GQA decoder layer at M=16384
  normrope: the layer's two RMSNorms (H=4096) and q/k RoPE (32+8 heads of 128), M=16384
  lmhead : chunked cross-entropy over a 128256 x 4096 LM head, M=16384, chunks of 4096
  qkrope : the layer's q and k projections with RoPE (heads of 128, base 500000), fwd+bwd, M=16384;
           RoPE in the GEMM epilogue, or after it as its own pass with --rope-unfused
--mlp-tile T runs the SwiGLU block of mlp/layer token-tiled (T tokens at a
time, g/u/h recomputed in the backward) and reports its activation memory.
Prints one JSON line with tokens/s, useful TFLOP/s (4MNK + 6Mr(N+K) per
projection), the dominant kernel's roofline (live hipEvent durations) and the
CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0
RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # ~312: below it a step is HBM/latency-bound
COLD_STEPS = 30  # the first ~25 cold steps of a run vary by up to ~10% (measured on the attn step)
# Untimed priming before the warm-up steps: back-to-back steps for this much
# wall time. From idle the GPU needs some 30 ms of load before a step reaches
# its steady time (attn: 306 us over the first 25 steps, 272 at 50-75, 266 from
# 100 on, one box), longer than a few warm-up steps take.
PRIME_S = 0.3
SMALL_MAX_M, SMALL_MAX_R = 256, 32  # the library's small-batch path (one wave per 32 x 32 tile)
WL_INDEX = {"tiny": 0, "attn": 1, "mlp": 2, "rsweep": 3, "layer": 4, "normrope": None, "lmhead": None,
            "qkrope": None}
# cross-entropy over the Llama-3-8B LM head (vocabulary 128256, width 4096) for
# the layer workload's 16384 tokens, in chunks of 4096 tokens (3 GB of workspace)
LMHEAD = dict(M=16384, H=4096, V=128256, chunk=4096)
# the steps around the projections of one decoder layer at M=16384: two
# RMSNorms of the 4096-wide residual stream and RoPE of q (32 heads) and k (8)
NORMROPE = dict(M=16384, H=4096, hq=32, hk=8, d=128, eps=1e-5, base=500000.0)
METRIC = "QLoRA linear fwd+bwd tokens/s and useful TFLOP/s (8B shapes); % MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="attn", choices=sorted(WL_INDEX))
    ap.add_argument("--rank", type=int, default=16)
    ap.add_argument("--wfmt", default="nf4", choices=["nf4", "int8", "fp8"],
                    help="format of the frozen weights (NF4 4-bit, INT8, FP8 E4M3; 64-element blocks)")
    ap.add_argument("--rope-unfused", action="store_true",
                    help="qkrope: the forward GEMMs, then RoPE as its own kernel (instead of in the GEMM epilogue)")
    ap.add_argument("--mlp-tile", type=int, default=0,
                    help="token-tiled SwiGLU block with this many tokens per tile (0: whole batch)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-gpu-state", action="store_true",
                    help="skip reading clocks and power with rocm-smi while the step runs")
    ap.add_argument("--prime-s", type=float, default=PRIME_S,
                    help="seconds of untimed back-to-back steps before the warm-up steps (0: none)")
    ap.add_argument("--no-cold", action="store_true",
                    help=f"skip the {COLD_STEPS} cache-cold steps (512 MiB written before each, untimed) timed after the warm ones")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed (reported under 'graph')")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device copies of known size (reference for hardware byte counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# HBM traffic of the dominant kernel, from committed hardware-counter summaries

KERNEL_SOURCES = {  # kernel class -> the sources its code is built from
    "small_fwd": ["small.hip", "common.hpp"],
    "small_bwd": ["small.hip", "common.hpp"],
    "skinny_tn": ["skinny.hip", "common.hpp", "reduce.hpp"],
    "skinny_nt": ["skinny.hip", "common.hpp", "reduce.hpp"],
    "gemm_bwd": ["gemm_bwd.hip", "common.hpp", "reduce.hpp"],
    "gemm_bwd_swiglu": ["gemm_bwd.hip", "common.hpp", "reduce.hpp"],
    "gemm_fwd": ["gemm_fwd.hip", "common.hpp"],
    "gemm_fwd_gateup": ["gemm_fwd.hip", "common.hpp"],
    "rmsnorm_fwd": ["normrope.hip", "common.hpp"],
    "rmsnorm_bwd": ["normrope.hip", "common.hpp"],
    "rope_fwd": ["normrope.hip", "common.hpp"],
    "rope_bwd": ["normrope.hip", "common.hpp"],
    "gemm_nt": ["lmhead.hip", "common.hpp"],
}


def kernel_source_hash(name):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(name, []):
        with open(os.path.join(ROOT, "parameter_efficient_fine_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counted_traffic(name, workload):
    """HBM bytes per launch of kernel class `name` on `workload` from the summary under
    profiles/ (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when there is none or the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{name}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic_bytes_per_launch:") or line.startswith("source_hash:"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip().split()[0]
    if vals.get("source_hash") != kernel_source_hash(name) or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def copy_calibration(steps):
    """Plain copies of 256 MiB (device to device): the byte counters of these
    dispatches, divided by 256 MiB read / written, give the counter scale."""
    import torch
    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": True, "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "copies": steps}), flush=True)


# ---------------------------------------------------------------------------
# workload set-up (outside the timed region)

def dev_bf16(u16):
    import torch
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


WFMT = {"nf4": 0, "int8": 1, "fp8": 2}
WFMT_DESC = {"nf4": "nf4, fp32 absmax per 64-block", "int8": "int8, fp32 scale (absmax/127) per 64-block",
             "fp8": "fp8 e4m3, fp32 scale (absmax/448) per 64-block"}


class Proj:
    """Device tensors and prebuilt C-ABI arguments of one projection's fwd+bwd."""

    def __init__(self, q, C, layer, s, X, dY, fmt=0):
        import torch
        M = X.shape[0]
        codes, absmax = q.quantize(dev_f32(layer["W"]), fmt)
        self.L = q.QLoraLayer(codes, absmax, dev_bf16(layer["A"]), dev_bf16(layer["B"]), s, fmt)
        self.M, self.K, self.N, self.r = M, self.L.K, self.L.N, self.L.r
        self.X, self.dY = X, dY
        dev = X.device
        self.Y = torch.empty((M, self.N), dtype=torch.bfloat16, device=dev)
        self.Z = torch.empty((M, self.r), dtype=torch.bfloat16, device=dev)
        self.dX = torch.empty((M, self.K), dtype=torch.bfloat16, device=dev)
        self.dA = torch.empty((self.r, self.K), dtype=self.L.grad_dtype, device=dev)
        self.dB = torch.empty((self.N, self.r), dtype=self.L.grad_dtype, device=dev)
        nb = q.workspace_size(C.OP_BACKWARD, M, self.K, self.N, self.r)
        self.ws = torch.empty((nb,), dtype=torch.uint8, device=dev)
        self.lc = self.L.c()
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        self.fwd_args = (ctypes.byref(self.lc), p(X), M, p(self.Y), p(self.Z), None, 0)
        self.bwd_args = (ctypes.byref(self.lc), p(dY), p(X), p(self.Z), M, p(self.dX), p(self.dA), p(self.dB),
                         p(self.ws), self.ws.numel())

    def run(self, lib, stream):
        st = lib.qlora_forward(*self.fwd_args, stream)
        if st:
            raise RuntimeError(f"qlora_forward: {st}")
        st = lib.qlora_backward(*self.bwd_args, stream)
        if st:
            raise RuntimeError(f"qlora_backward: {st}")


class MLP:
    def __init__(self, q, C, layers, s, X, dY, tile=0, fmt=0):
        import torch
        Ls = []
        for nm in ("gate", "up", "down"):
            codes, absmax = q.quantize(dev_f32(layers[nm]["W"]), fmt)
            Ls.append(q.QLoraLayer(codes, absmax, dev_bf16(layers[nm]["A"]), dev_bf16(layers[nm]["B"]), s, fmt))
        self.Ls = Ls
        M = X.shape[0]
        H, I, r = Ls[0].K, Ls[0].N, Ls[0].r
        self.M, self.H, self.I, self.r = M, H, I, r
        self.X, self.dY = X, dY
        self.tile = tile
        dev = X.device
        e = lambda shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=dev)
        self.dX = e((M, H))
        self.dA = [e((r, L.K), L.grad_dtype) for L in Ls]
        self.dB = [e((L.N, r), L.grad_dtype) for L in Ls]
        self.lcs = [L.c() for L in Ls]
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        refs = [ctypes.byref(lc) for lc in self.lcs]
        self._dA = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in self.dA])
        self._dB = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in self.dB])
        if tile:
            sv = self.saved = dict(Y=e((M, H)), Z=e((3, M, r)))
            self.ws_f = e((q.mlp_tiled_workspace_size(False, M, H, I, r, tile),), torch.uint8)
            self.ws = e((q.mlp_tiled_workspace_size(True, M, H, I, r, tile),), torch.uint8)
            self.fwd_args = (*refs, p(X), M, tile, p(sv["Y"]), p(sv["Z"]), p(self.ws_f), self.ws_f.numel())
            self.bwd_args = (*refs, p(dY), p(X), p(sv["Z"]), M, tile, p(self.dX), self._dA, self._dB, p(self.ws),
                             self.ws.numel())
            # what the block keeps between its forward and backward, plus the larger workspace
            self.activation_bytes = sv["Z"].numel() * 2 + max(self.ws_f.numel(), self.ws.numel())
        else:
            sv = self.saved = dict(Y=e((M, H)), g=e((M, I)), u=e((M, I)), h=e((M, I)), Z=e((3, M, r)))
            self.ws = e((q.workspace_size(C.OP_MLP_BACKWARD, M, H, I, r),), torch.uint8)
            self.fwd_args = (*refs, p(X), M, p(sv["Y"]), p(sv["g"]), p(sv["u"]), p(sv["h"]), p(sv["Z"]), None, 0)
            self.bwd_args = (*refs, p(dY), p(X), p(sv["g"]), p(sv["u"]), p(sv["h"]), p(sv["Z"]), M, p(self.dX),
                             self._dA, self._dB, p(self.ws), self.ws.numel())
            self.activation_bytes = sum(sv[k].numel() * 2 for k in ("g", "u", "h", "Z")) + self.ws.numel()

    def run(self, lib, stream):
        if self.tile:
            st = lib.swiglu_mlp_forward_tiled(*self.fwd_args, stream)
            if st:
                raise RuntimeError(f"swiglu_mlp_forward_tiled: {st}")
            st = lib.swiglu_mlp_backward_tiled(*self.bwd_args, stream)
            if st:
                raise RuntimeError(f"swiglu_mlp_backward_tiled: {st}")
            return
        st = lib.swiglu_mlp_forward(*self.fwd_args, stream)
        if st:
            raise RuntimeError(f"swiglu_mlp_forward: {st}")
        st = lib.swiglu_mlp_backward(*self.bwd_args, stream)
        if st:
            raise RuntimeError(f"swiglu_mlp_backward: {st}")


class NormRope:
    """RMSNorm fwd+bwd twice and RoPE fwd+bwd of q, k: the steps around one layer's projections."""

    def __init__(self, q, cfg):
        import torch
        from synthetic import random_norm_rope
        d = random_norm_rope(5000, cfg["M"], cfg["H"], cfg["hq"], cfg["hk"], cfg["d"])
        self.d, self.cfg = d, cfg
        M, H = cfg["M"], cfg["H"]
        self.x, self.w, self.dy = dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])
        self.qh, self.kh, self.dq, self.dk = (dev_bf16(d[k]) for k in ("q", "k", "dq", "dk"))
        self.pos = torch.from_numpy(d["pos"]).cuda()
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        self.rstd = torch.empty((M,), dtype=torch.float32, device="cuda")
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        hq, hk, hd = cfg["hq"], cfg["hk"], cfg["d"]
        self.f_args = (p(self.x), p(self.w), M, H, cfg["eps"], p(self.y), p(self.rstd))
        self.b_args = (p(self.dy), p(self.x), p(self.w), p(self.rstd), M, H, p(self.dx))
        self.rf_args = (p(self.qh), p(self.kh), p(self.pos), M, hq, hk, hd, cfg["base"])
        self.rb_args = (p(self.dq), p(self.dk), p(self.pos), M, hq, hk, hd, cfg["base"])

    def run(self, lib, stream):
        for _ in range(2):  # input norm and post-attention norm
            if lib.qlora_rmsnorm_forward(*self.f_args, stream):
                raise RuntimeError("qlora_rmsnorm_forward")
        if lib.qlora_rope_forward(*self.rf_args, stream) or lib.qlora_rope_backward(*self.rb_args, stream):
            raise RuntimeError("qlora_rope")
        for _ in range(2):
            if lib.qlora_rmsnorm_backward(*self.b_args, stream):
                raise RuntimeError("qlora_rmsnorm_backward")

    def bytes_per_launch(self):
        c = self.cfg
        M, H, heads = c["M"], c["H"], c["hq"] + c["hk"]
        rope = 2 * M * heads * c["d"] * 2 + M * 4  # read and write every head element, positions
        return {"rmsnorm_fwd": 2 * M * H * 2 + H * 2 + M * 4, "rmsnorm_bwd": 3 * M * H * 2 + H * 2 + M * 4,
                "rope_fwd": rope, "rope_bwd": rope}


class LMHeadCE:
    """Chunked cross-entropy (loss and dh) over the frozen LM head."""

    def __init__(self, q, cfg):
        import torch
        from synthetic import random_ce
        d = random_ce(6000, cfg["M"], cfg["H"], cfg["V"])
        self.d, self.cfg = d, cfg
        self.h, self.W = dev_bf16(d["h"]), dev_bf16(d["W"])
        self.t = torch.from_numpy(d["targets"]).cuda()
        self.Wp, self.Wtp = q.lmhead_prepare(self.W)
        M, H, V, chunk = cfg["M"], cfg["H"], cfg["V"], cfg["chunk"]
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
        self.loss, self.rows, self.dh = e((1,), torch.float32), e((M,), torch.float32), e((M, H), torch.bfloat16)
        from parameter_efficient_fine_amd import _lib as C
        self.ws = e((int(C.lib().qlora_ce_workspace_size(M, V, chunk)),), torch.uint8)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        self.args = (p(self.h), p(self.Wp), p(self.Wtp), p(self.t), M, H, V, chunk, p(self.loss), p(self.rows),
                     p(self.dh), p(self.ws), self.ws.numel())

    def run(self, lib, stream):
        if lib.qlora_chunked_ce(*self.args, stream):
            raise RuntimeError("qlora_chunked_ce")

    def useful_flops(self):
        c = self.cfg
        return 4.0 * c["M"] * c["V"] * c["H"]  # logits and dh

    def gemm_flops(self):
        c = self.cfg
        out = []
        for r0 in range(0, c["M"], c["chunk"]):
            mc = min(c["chunk"], c["M"] - r0)
            out += [2 * mc * c["V"] * c["H"]] * 2
        return {"gemm_nt": out}


class QKRope:
    """q and k projections of a decoder layer with RoPE on their outputs, forward and backward:
    fused (RoPE in the GEMM epilogue) or unfused (GEMM, then the RoPE kernel on q and k at once).
    The backward rotates dq, dk back in place (one launch), then runs both projection backwards."""

    def __init__(self, q, C, fused, fmt=0):
        import torch
        from synthetic import make_workload, packed_positions
        d = make_workload(4)
        self.d = d
        M = d["M"]
        X = dev_bf16(d["X_attn"])
        self.projs = [Proj(q, C, d["layers"][nm], d["s"], X, dev_bf16(d["dY_" + nm]), fmt) for nm in ("q", "k")]
        pos = packed_positions(np.random.default_rng(4100), M, M)
        self.pos = torch.from_numpy(pos.astype(np.int32)).cuda()
        self.table = q.rope_table(128, 500000.0, M)
        self.fused = fused
        self.M = M
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        self.rope_f = (p(self.projs[0].Y), p(self.projs[1].Y), p(self.pos), M, 32, 8, 128, 500000.0)
        self.rope_b = (p(self.projs[0].dY), p(self.projs[1].dY), p(self.pos), M, 32, 8, 128, 500000.0)
        self.fr = [(ctypes.byref(pr.lc), p(pr.X), M, p(self.pos), p(self.table), M, 128, p(pr.Y), p(pr.Z))
                   for pr in self.projs]

    def run(self, lib, stream):
        if self.fused:
            for a in self.fr:
                if lib.qlora_forward_rope(*a, stream):
                    raise RuntimeError("qlora_forward_rope")
        else:
            for pr in self.projs:
                if lib.qlora_forward(*pr.fwd_args, stream):
                    raise RuntimeError("qlora_forward")
            if lib.qlora_rope_forward(*self.rope_f, stream):
                raise RuntimeError("qlora_rope_forward")
        if lib.qlora_rope_backward(*self.rope_b, stream):  # dq, dk rotated back in place
            raise RuntimeError("qlora_rope_backward")
        for pr in self.projs:
            if lib.qlora_backward(*pr.bwd_args, stream):
                raise RuntimeError("qlora_backward")


def build_workload(name: str, rank: int, mlp_tile: int = 0, fmt: int = 0, rope_unfused: bool = False):
    import torch
    import parameter_efficient_fine_amd as q
    from parameter_efficient_fine_amd import _lib as C
    from synthetic import WORKLOADS, make_workload
    c = WL_INDEX[name]
    if name == "lmhead":
        parts = [LMHeadCE(q, LMHEAD)]
        d = dict(LMHEAD, kind="lmhead", _data=parts[0].d)
        torch.cuda.synchronize()
        return d, parts
    if name == "qkrope":
        part = QKRope(q, C, not rope_unfused, fmt)
        d = dict(kind="qkrope", M=part.M, r=16, fused=not rope_unfused, _data=None)
        torch.cuda.synchronize()
        return d, [part]
    if name == "normrope":
        parts = [NormRope(q, NORMROPE)]
        d = dict(NORMROPE, kind="normrope", _data=parts[0].d)
        torch.cuda.synchronize()
        return d, parts
    sub = WORKLOADS[c]["ranks"].index(rank) if name == "rsweep" else 0
    d = make_workload(c, sub)
    parts = []
    if d["kind"] == "linear":
        parts.append(Proj(q, C, d["layers"]["proj"], d["s"], dev_bf16(d["X"]), dev_bf16(d["dY"]), fmt))
    elif d["kind"] == "mlp":
        parts.append(MLP(q, C, d["layers"], d["s"], dev_bf16(d["X"]), dev_bf16(d["dY"]), mlp_tile, fmt))
    else:
        Xa, Xo = dev_bf16(d["X_attn"]), dev_bf16(d["X_o"])
        for nm, X in (("q", Xa), ("k", Xa), ("v", Xa), ("o", Xo)):
            parts.append(Proj(q, C, d["layers"][nm], d["s"], X, dev_bf16(d["dY_" + nm]), fmt))
        parts.append(MLP(q, C, {k: d["layers"][k] for k in ("gate", "up", "down")}, d["s"], dev_bf16(d["X_mlp"]),
                         dev_bf16(d["dY_mlp"]), mlp_tile, fmt))
    torch.cuda.synchronize()
    return d, parts


def describe(d, name, parts=()):
    if d["kind"] == "qkrope":
        how = "in the GEMM epilogue" if d["fused"] else "as its own kernel after the GEMMs"
        return dict(workload=f"{name}: q (4096->4096) and k (4096->1024) projections with RoPE {how} (heads of 128, "
                             f"base 500000, packed-sequence positions), fwd+bwd, M={d['M']}, r=16",
                    M=d["M"], r=16, rope_fused=d["fused"])
    if d["kind"] == "lmhead":
        return dict(workload=f"{name}: chunked cross-entropy (loss and dh) over a frozen bf16 LM head, V={d['V']}, "
                             f"H={d['H']}, M={d['M']} tokens in chunks of {d['chunk']}, ~10% ignored targets",
                    **{k: d[k] for k in ("M", "H", "V", "chunk")})
    if d["kind"] == "normrope":
        return dict(workload=f"{name}: two RMSNorms (H={d['H']}, eps={d['eps']}) and RoPE of q ({d['hq']} heads) and "
                             f"k ({d['hk']} heads) of {d['d']}, base {d['base']:g}, fwd+bwd, M={d['M']} tokens in "
                             f"packed sequences", **{k: d[k] for k in ("M", "H", "hq", "hk", "d")})
    M, r = d["M"], d["r"]
    mlps = [p for p in parts if isinstance(p, MLP)]
    extra = {}
    if mlps:  # SwiGLU block memory: what its forward keeps for the backward, plus workspace
        extra = dict(mlp_tile=mlps[0].tile or None, mlp_activation_bytes=mlps[0].activation_bytes)
    if d["kind"] == "linear":
        Lr = d["layers"]["proj"]
        K, N = Lr["W"].shape[1], Lr["W"].shape[0]
        return dict(workload=f"{name}: one 4-bit NF4 projection, M={M} tokens, K={K}, N={N}, r={r}, alpha={d['alpha']}",
                    M=M, K=K, N=N, r=r, alpha=d["alpha"], weight_format=WFMT_DESC[d.get("wfmt", "nf4")])
    if d["kind"] == "mlp":
        return dict(workload=f"{name}: SwiGLU block, M={M}, 4096<->14336, LoRA r={r} on gate/up/down",
                    M=M, H=4096, I=14336, r=r, alpha=d["alpha"], weight_format=WFMT_DESC[d.get("wfmt", "nf4")], **extra)
    return dict(workload=f"{name}: 7 projections of a GQA decoder layer (q,o 4096x4096; k,v 4096->1024; "
                         f"gate/up/down 4096<->14336), M={M}, r={r}", M=M, r=r, alpha=d["alpha"],
                weight_format=WFMT_DESC[d.get("wfmt", "nf4")], **extra)


# ---------------------------------------------------------------------------
# algorithmic work per launch of the fused GEMMs (for the roofline)

def gemm_flops(parts):
    """{kernel class: algorithmic FLOPs per launch} of the fused dequant GEMMs."""
    out = {}
    expanded = []
    for p in parts:
        expanded += p.projs if isinstance(p, QKRope) else [p]
    for p in expanded:
        if isinstance(p, NormRope):
            continue
        if isinstance(p, LMHeadCE):
            for k, v in p.gemm_flops().items():
                out.setdefault(k, []).extend(v)
            continue
        if isinstance(p, Proj):
            M, K, N, r = p.M, p.K, p.N, p.r
            out.setdefault("gemm_fwd", []).append(2 * M * N * K + 2 * M * N * r)   # X.W^T + Z.B^T
            out.setdefault("gemm_fwd_rope", []).append(2 * M * N * K + 2 * M * N * r)
            out.setdefault("small_fwd", []).append(2 * M * N * K + 2 * M * N * r + 2 * M * K * r)
            out.setdefault("small_bwd", []).append(2 * M * N * K + 2 * M * K * r + 2 * M * N * r)
            out.setdefault("gemm_bwd", []).append(2 * M * N * K + 2 * M * K * r)   # dY.W + G.A
        else:
            H, I, r = p.H, p.I, p.r
            T = p.tile if p.tile else p.M
            for t0 in range(0, p.M, T):  # one set of launches per token tile
                M = min(T, p.M - t0)
                gateup = 2 * (2 * M * I * H + 2 * M * I * r)
                # a tiled backward recomputes the tile's g, u, h with the same kernel
                out.setdefault("gemm_fwd_gateup", []).extend([gateup] * (2 if p.tile else 1))
                out.setdefault("gemm_fwd", []).append(2 * M * H * I + 2 * M * H * r)
                out.setdefault("gemm_bwd_swiglu", []).append(2 * M * H * I + 2 * M * I * r)
                out.setdefault("gemm_bwd", []).append(2 * (2 * M * I * H + 2 * M * H * r))
    return out


def _wbytes(N, K, fmt):
    """Bytes of a frozen weight [N, K]: codes (0.5 or 1 byte per element) and one fp32 per 64-block."""
    return N * K * (0.5 if fmt == 0 else 1.0) + N * K / 64 * 4


def launch_bytes(parts, fmt=0):
    """{kernel class: [algorithmic HBM bytes of each launch in one step]}: the inputs and
    outputs each launch must read or write once (weights, activations, adapters, results;
    the fp32 split partials of the rank reductions are an implementation detail, not counted)."""
    out = {}

    def add(k, v):
        out.setdefault(k, []).append(float(v))

    for p in parts:
        if isinstance(p, Proj) and p.M <= SMALL_MAX_M and p.r <= SMALL_MAX_R:
            # small-batch kernels: Y and Z in one launch, dX and G in one, then dB and dA
            M, K, N, r = p.M, p.K, p.N, p.r
            add("small_fwd", 2 * M * K + _wbytes(N, K, fmt) + 2 * r * K + 2 * N * r + 2 * M * N + 2 * M * r)
            add("small_bwd", 2 * M * N + _wbytes(N, K, fmt) + 2 * r * K + 2 * N * r + 2 * M * K + 2 * M * r)
            add("skinny_tn", 2 * M * N + 2 * M * r + 2 * M * K + 2 * M * r + 4 * r * (N + K))
        elif isinstance(p, Proj):
            M, K, N, r = p.M, p.K, p.N, p.r
            add("gemm_fwd", 2 * M * K + _wbytes(N, K, fmt) + 2 * M * r + 2 * N * r + 2 * M * N)
            add("gemm_bwd", 2 * M * N + _wbytes(N, K, fmt) + 2 * M * r + 2 * r * K + 2 * M * K)
            add("skinny_nt", 2 * M * K + 2 * r * K + 2 * M * r)      # Z = X.A^T
            add("skinny_nt", 2 * M * N + 2 * N * r + 2 * M * r)      # G = dY.B
            # dB = s.dY^T.Z and dA = s.G^T.X (one launch): operands in, fp32 gradients out
            add("skinny_tn", 2 * M * N + 2 * M * r + 2 * M * K + 2 * M * r + 4 * r * (N + K))
    return out


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload)

def _oracle_weight(W, wfmt):
    """The oracle's dequantized weight in the benched format (float64)."""
    from oracle import formats8, ref
    if wfmt == "nf4":
        return ref.dequantize(*ref.quantize(W)).astype(np.float64)
    f = WFMT[wfmt]
    return formats8.dequantize(*formats8.quantize(W, f), f).astype(np.float64)


def cpu_baseline(d, target_s: float):
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import ref
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        M = d["M"]
        if d["kind"] == "linear":
            Lr = d["layers"]["proj"]
            What = _oracle_weight(Lr["W"], d.get("wfmt", "nf4"))
            A, B = ref.bf16_to_f64(Lr["A"]), ref.bf16_to_f64(Lr["B"])
            X, dY = ref.bf16_to_f64(d["X"]), ref.bf16_to_f64(d["dY"])

            def run(rows):
                ref.linear_fwd(X[:rows], What, A, B, d["s"])
                ref.linear_bwd(dY[:rows], X[:rows], What, A, B, d["s"])
            what = "linear fwd+bwd"
        elif d["kind"] == "lmhead":
            from oracle import ce as ce_oracle
            nd = d["_data"]
            Hh, Wl = ref.bf16_to_f64(nd["h"]), ref.bf16_to_f64(nd["W"])

            def run(rows):
                ce_oracle.ce_fwd_bwd(Hh[:rows], Wl, nd["targets"][:rows])
            what = "cross-entropy over the LM head, loss and dh"
        elif d["kind"] == "qkrope":
            from oracle import normrope as nr
            from synthetic import make_workload, packed_positions
            w4 = make_workload(4)
            pos = packed_positions(np.random.default_rng(4100), M, M)
            X = ref.bf16_to_f64(w4["X_attn"])
            trip = {}
            for nm in ("q", "k"):
                Lr = w4["layers"][nm]
                trip[nm] = (_oracle_weight(Lr["W"], d.get("wfmt", "nf4")), ref.bf16_to_f64(Lr["A"]),
                            ref.bf16_to_f64(Lr["B"]), ref.bf16_to_f64(w4["dY_" + nm]))

            def run(rows):
                for nm, (What, A, B, dY) in trip.items():
                    Y, _ = ref.linear_fwd(X[:rows], What, A, B, w4["s"])
                    nr.rope(Y, pos[:rows], 128, 500000.0)
                    g = nr.rope_bwd(dY[:rows], pos[:rows], 128, 500000.0)
                    ref.linear_bwd(g, X[:rows], What, A, B, w4["s"])
            what = "q and k projections with RoPE, fwd+bwd"
        elif d["kind"] == "normrope":
            from oracle import normrope as nr
            nd = d["_data"]
            X, Wn, DY = ref.bf16_to_f64(nd["x"]), ref.bf16_to_f64(nd["w"]), ref.bf16_to_f64(nd["dy"])
            Q, Kh = ref.bf16_to_f64(nd["q"]), ref.bf16_to_f64(nd["k"])
            DQ, DK = ref.bf16_to_f64(nd["dq"]), ref.bf16_to_f64(nd["dk"])

            def run(rows):
                for _ in range(2):
                    nr.rmsnorm_fwd(X[:rows], Wn, d["eps"])
                for v, f in ((Q, nr.rope), (Kh, nr.rope), (DQ, nr.rope_bwd), (DK, nr.rope_bwd)):
                    f(v[:rows], nd["pos"][:rows], d["d"], d["base"])
                for _ in range(2):
                    nr.rmsnorm_bwd(DY[:rows], X[:rows], Wn, d["eps"])
            what = "two RMSNorms and q/k RoPE, fwd+bwd"
        else:
            names = ("gate", "up", "down")
            lay = d["layers"]
            trip = [(_oracle_weight(lay[n]["W"], d.get("wfmt", "nf4")), ref.bf16_to_f64(lay[n]["A"]),
                     ref.bf16_to_f64(lay[n]["B"])) for n in names]
            xk, dk = ("X", "dY") if d["kind"] == "mlp" else ("X_mlp", "dY_mlp")
            X, dY = ref.bf16_to_f64(d[xk]), ref.bf16_to_f64(d[dk])

            def run(rows):
                ref.mlp_bwd(dY[:rows], X[:rows], *trip, d["s"])  # runs the forward inside
            what = "SwiGLU block fwd+bwd" + (" (MLP part of the layer)" if d["kind"] == "layer" else "")
        rows = min(64, M)
        t0 = time.perf_counter()
        run(rows)
        dt = time.perf_counter() - t0
        # scale the sample (rows, then whole repeats) so it takes about target_s
        rows = int(min(M, max(rows, rows * target_s / max(dt, 1e-3))))
        reps, done = 0, 0
        t0 = time.perf_counter()
        while True:
            run(rows)
            reps += 1
            done += rows
            dt = time.perf_counter() - t0
            if dt >= target_s or reps >= 1000:
                break
    return dict(value=done / dt, unit="tokens/s", cores=threads, kind="oracle", blas=_blas_name(),
                sample=f"NumPy float64 oracle, {what}, {reps} pass(es) over the first {rows} of {M} tokens "
                       f"({dt:.1f} s, {threads} BLAS threads on {cores} host cores)")


def _blas_name():
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # older NumPy: no dict form
        return None


# ---------------------------------------------------------------------------
# Clocks and power state, read while the step runs

_SMI_KEYS = ("sclk", "mclk", "fclk", "performance level", "power")


def gpu_state_under_load(step, sync, cap_s=15.0):
    """rocm-smi's clocks, performance level and power, sampled while `step` runs
    back to back (None when rocm-smi is missing or its output cannot be read)."""
    import shutil
    import subprocess
    exe = shutil.which("rocm-smi")
    if exe is None:
        return None
    try:
        p = subprocess.Popen([exe, "--showclocks", "--showperflevel", "--showpower", "--json"],
                             stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.time()
    while p.poll() is None and time.time() - t0 < cap_s:
        for _ in range(10):
            step()
        sync()
    try:
        out, _ = p.communicate(timeout=5)
    except subprocess.TimeoutExpired:
        p.kill()
        p.communicate()
        return None
    try:
        js = json.loads(out)
    except ValueError:
        return None
    keep = {}
    for card, fields in js.items():
        if isinstance(fields, dict):
            sel = {k: v for k, v in fields.items() if any(x in k.lower() for x in _SMI_KEYS)}
            if sel:
                keep[card] = sel
    return keep or None



# ---------------------------------------------------------------------------

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only: no sharding or collectives are built; "
                                   "run with --gpus 1", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    import torch
    from parameter_efficient_fine_amd import _lib as C
    from parameter_efficient_fine_amd.ops import KernelTimer
    from synthetic import useful_flops

    lib = C.lib()
    d, parts = build_workload(args.workload, args.rank, args.mlp_tile, WFMT[args.wfmt], args.rope_unfused)
    d["wfmt"] = args.wfmt
    c = WL_INDEX[args.workload]
    sub = d["sub"] if args.workload == "rsweep" else 0
    flops = useful_flops(c, sub) if c is not None else None
    if args.workload == "lmhead":
        flops = parts[0].useful_flops()
    if args.workload == "qkrope":  # the two projections' useful work (the rotation is not counted)
        flops = float(sum(4 * p.M * p.N * p.K + 6 * p.M * p.r * (p.N + p.K) for p in parts[0].projs))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step(st=stream):
        for p in parts:
            p.run(lib, st)

    # priming (untimed): steps for args.prime_s seconds, the queue kept short so
    # that the GPU is busy for that wall time
    n_prime, t_prime = 0, time.perf_counter()
    while time.perf_counter() - t_prime < args.prime_s:
        step()
        n_prime += 1
        if n_prime % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    prime = dict(seconds=round(time.perf_counter() - t_prime, 3), steps=n_prime)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K back-to-back steps, one event between consecutive steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    step_stats = dict(median_ms=float(np.median(per_step)), min_ms=float(per_step.min()),
                      p90_ms=float(np.percentile(per_step, 90)))
    if not args.no_cold:
        # cache-cold steps: 512 MiB written between steps (untimed), so the
        # step's inputs come from HBM rather than the last-level cache
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold = []
        for _ in range(COLD_STEPS):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush
        step_stats["cold_median_ms"] = float(np.median(cold))
        step_stats["cold_min_ms"] = float(np.min(cold))
        step_stats["cold_tokens_per_s"] = d["M"] / (step_stats["cold_median_ms"] * 1e-3)

    graph_stats = None
    if args.graph:
        # the whole step captured once (every launch of the library goes to the
        # capture stream) and replayed K times back to back
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        g.replay()
        torch.cuda.synchronize()
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        gev[0].record()
        for i in range(args.steps):
            g.replay()
            gev[i + 1].record()
        torch.cuda.synchronize()
        gms = gev[0].elapsed_time(gev[-1]) / args.steps
        graph_stats = dict(ms_per_step=gms, tokens_per_s=d["M"] / (gms * 1e-3),
                           median_ms=float(np.median([gev[i].elapsed_time(gev[i + 1]) for i in range(args.steps)])))
        del g

    # same steps again with per-launch hipEvents recorded by the library (kernel durations)
    with KernelTimer(max_launches=args.steps * 256 + 64) as kt:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    per_launch_flops = gemm_flops(parts)
    kernels = {}
    for name, (n, tot) in kt.result.items():
        kernels[name] = dict(launches_per_step=n / args.steps, ms_per_step=tot / args.steps, avg_us=1e3 * tot / n)
    step_bytes = None
    if flops is not None and d["kind"] == "linear":
        lb = launch_bytes(parts, WFMT[args.wfmt])
        # the step's algorithmic bytes: every kernel's inputs and outputs once
        step_bytes = sum(sum(v) for v in lb.values())
    low_ai = step_bytes is not None and flops / step_bytes < RIDGE_FLOP_PER_BYTE
    if low_ai:  # below the ridge (small batches): the dominant kernel against HBM bandwidth
        per_launch = {k: float(np.mean(v)) for k, v in launch_bytes(parts, WFMT[args.wfmt]).items()}
        dom = max((k for k in kernels if k in per_launch), key=lambda k: kernels[k]["ms_per_step"])
        avg_s = kernels[dom]["avg_us"] * 1e-6
        achieved = per_launch[dom] / avg_s / 1e9
        roofline = dict(bound="hbm", kernel=dom, achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=achieved / PEAK_HBM_GBS, traffic=counted_traffic(dom, args.workload),
                        traffic_unit="bytes per launch", avg_us=kernels[dom]["avg_us"],
                        bytes_per_launch=per_launch[dom], source_hash=kernel_source_hash(dom))
    elif flops is None:  # HBM-bound steps: algorithmic bytes of the dominant kernel
        per_launch_bytes = parts[0].bytes_per_launch()
        dom = max((k for k in kernels if k in per_launch_bytes), key=lambda k: kernels[k]["ms_per_step"])
        avg_s = kernels[dom]["avg_us"] * 1e-6
        achieved = per_launch_bytes[dom] / avg_s / 1e9
        roofline = dict(bound="hbm", kernel=dom, achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=achieved / PEAK_HBM_GBS, traffic=counted_traffic(dom, args.workload),
                        traffic_unit="bytes per launch", avg_us=kernels[dom]["avg_us"],
                        bytes_per_launch=per_launch_bytes[dom], source_hash=kernel_source_hash(dom))
    else:
        dom = max((k for k in kernels if k in per_launch_flops), key=lambda k: kernels[k]["ms_per_step"])
        fl = per_launch_flops[dom]
        avg_flops = float(np.mean(fl))
        avg_s = kernels[dom]["avg_us"] * 1e-6
        achieved = avg_flops / avg_s / 1e12
        roofline = dict(bound="mfma", kernel=dom, achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                        frac=achieved / PEAK_BF16_TFLOPS, traffic=counted_traffic(dom, args.workload),
                        traffic_unit="bytes per launch", avg_us=kernels[dom]["avg_us"], flops_per_launch=avg_flops,
                        source_hash=kernel_source_hash(dom))

    tokens = d["M"]
    value = tokens / (ms * 1e-3)
    tflops = flops / (ms * 1e-3) / 1e12 if flops is not None else None
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prime": prime,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": {"normrope": "synthetic (seeded N(0,1) activations and gradients, norm weight 1+0.1*N(0,1), "
                             "packed-sequence positions)",
                 "lmhead": "synthetic (seeded N(0,1) hidden states, 0.02*N(0,1) bf16 LM head, uniform targets, "
                           "10% ignored)"}.get(d["kind"],
                                               "synthetic (seeded N(0,1) activations, 0.02*N(0,1) weights quantized"
                                               " to " + d.get("wfmt", "nf4").upper() + ")"),
        "config": describe(d, args.workload, parts),
        "useful_tflops": tflops,
        "mfma_peak_frac": tflops / PEAK_BF16_TFLOPS if tflops is not None else None,
        "useful_gflop_per_step": flops / 1e9 if flops is not None else None,
        "wall_s_timed": wall,
        "step_time": step_stats,
        "roofline": roofline,
        "kernels": kernels,
    }
    if step_bytes is not None:
        # whole-step algorithmic HBM bytes (each kernel's inputs and outputs once) per step time
        out["step_hbm"] = dict(bytes=step_bytes, achieved_gbs=step_bytes / (ms * 1e-3) / 1e9,
                               frac=step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                               arithmetic_intensity=flops / step_bytes)
    if graph_stats is not None:
        out["graph"] = graph_stats
    out["gpu_state"] = None if args.no_gpu_state else gpu_state_under_load(step, torch.cuda.synchronize)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
