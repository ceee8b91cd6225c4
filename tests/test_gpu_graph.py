"""The library's calls can be captured in a HIP graph: a captured fwd+bwd step,
replayed several times with eager work and synchronisations in between, gives
the eager result bit for bit on every replay (no memset nodes, no allocation;
every launch on the caller's stream, or, in the tiled SwiGLU calls, on the
library's second stream, which joins the capture through the events that order
it)."""
import ctypes

import numpy as np
import pytest

from synthetic import random_linear, random_mlp
from tests._util import Prepared, dev_bf16

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _check_graph(run, outputs):
    """run(stream_handle) enqueues the step; outputs() -> tensors to compare."""
    import torch
    run(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    want = [_bits(t) for t in outputs()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    for rep in range(3):
        for t in outputs():
            t.fill_(float("nan") if t.is_floating_point() else 0)   # the replay must rewrite every output
        g.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in outputs()]
        for a, b in zip(want, got):
            assert np.array_equal(a, b), rep
        # eager work between replays
        run(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()


def test_linear_step_in_a_graph():
    _announce("graph linear M=700 K=448 N=200 r=132")
    import torch
    from parameter_efficient_fine_amd import _lib as C
    d = random_linear(71, 700, 448, 200, 132)
    P = Prepared(d["layers"]["proj"], d["s"])
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    M, K, N, r = 700, 448, 200, 132
    e = lambda shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device="cuda")
    Y, Z, dX, dA, dB = e((M, N)), e((M, r)), e((M, K)), e((r, K), torch.float32), e((N, r), torch.float32)
    ws = e((C.lib().qlora_workspace_size(C.OP_BACKWARD, M, K, N, r),), torch.uint8)
    lc = P.dev.c()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    lib = C.lib()

    def run(st):
        assert lib.qlora_forward(ctypes.byref(lc), p(X), M, p(Y), p(Z), None, 0, st) == 0
        assert lib.qlora_backward(ctypes.byref(lc), p(dY), p(X), p(Z), M, p(dX), p(dA), p(dB), p(ws), ws.numel(),
                                  st) == 0
    _check_graph(run, lambda: [Y, Z, dX, dA, dB])


def test_mlp_step_in_a_graph():
    _announce("graph mlp M=300 H=256 I=512 r=16")
    import parameter_efficient_fine_amd as q
    d = random_mlp(72, 300, 256, 512, 16)
    Ls = [Prepared(d["layers"][nm], d["s"]).dev for nm in ("gate", "up", "down")]
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    f = q.mlp_forward(*Ls, X)
    b = q.mlp_backward(*Ls, dY, X, f)
    import torch
    from parameter_efficient_fine_amd import _lib as C
    nb = C.lib().qlora_workspace_size(C.OP_MLP_BACKWARD, 300, 256, 512, 16)
    ws = torch.empty((nb,), dtype=torch.uint8, device="cuda")

    def run(st):
        # the ops enqueue on the current torch stream, which is the capture stream inside the graph
        q.mlp_forward(*Ls, X, out=f)
        q.mlp_backward(*Ls, dY, X, f, ws=ws, out=b)
    _check_graph(run, lambda: [f["Y"], f["h"], b["dX"]] + b["dA"] + b["dB"])


@pytest.mark.parametrize("fmt", [0, 2])
def test_tiled_mlp_step_in_a_graph(fmt):
    # The tiled calls' second stream joins the capture through the events that
    # fork and join it (the stream itself is created by the eager call made
    # before the capture).
    _announce(f"graph tiled mlp M=700 tile=256 H=128 I=256 r=16 fmt={fmt}")
    import torch
    import parameter_efficient_fine_amd as q
    d = random_mlp(73 + fmt, 700, 128, 256, 16)
    Ls = [Prepared(d["layers"][nm], d["s"], fmt=fmt).dev for nm in ("gate", "up", "down")]
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    f = q.mlp_forward_tiled(*Ls, X, 256)
    b = q.mlp_backward_tiled(*Ls, dY, X, f["Z"], 256)
    wsf = torch.empty((q.mlp_tiled_workspace_size(False, 700, 128, 256, 16, 256),), dtype=torch.uint8, device="cuda")
    wsb = torch.empty((q.mlp_tiled_workspace_size(True, 700, 128, 256, 16, 256),), dtype=torch.uint8, device="cuda")

    def run(st):
        q.mlp_forward_tiled(*Ls, X, 256, ws=wsf, out=f)
        q.mlp_backward_tiled(*Ls, dY, X, f["Z"], 256, ws=wsb, out=b)
    _check_graph(run, lambda: [f["Y"], f["Z"], b["dX"]] + b["dA"] + b["dB"])
