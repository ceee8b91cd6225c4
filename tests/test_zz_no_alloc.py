"""GPU check of qlora_backward_noalloc (the backward whose workspace is the
library's own scratch array) through the C ABI: on two calls in a row, the
second with a smaller input, its dX, dA, dB equal qlora_backward's with a
caller workspace bit for bit, and match the oracle."""
import ctypes

import numpy as np
import pytest

from oracle import ref
from synthetic import make_workload, random_linear
from tests._util import TOL, Prepared, dev_bf16, host, rel_err, sample_rows

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _bits(t):
    import torch
    t = t.detach().contiguous()
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def _case(d, grad_dtype, rows=None):
    import torch
    import parameter_efficient_fine_amd as q
    from parameter_efficient_fine_amd import _lib as C
    lib = C.lib()
    P = Prepared(d["layers"]["proj"], d["s"], grad_dtype=grad_dtype)
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    M, K, N, r = X.shape[0], P.dev.K, P.dev.N, P.dev.r
    Y, Z = q.forward(P.dev, X)
    want = q.backward(P.dev, dY, X, Z)  # caller workspace
    nan = float("nan")
    dX = torch.full((M, K), nan, dtype=torch.bfloat16, device="cuda")
    dA = torch.full((r, K), nan, dtype=grad_dtype, device="cuda")
    dB = torch.full((N, r), nan, dtype=grad_dtype, device="cuda")
    lc = P.dev.c()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.qlora_backward_noalloc(ctypes.byref(lc), p(dY), p(X), p(Z), M, p(dX), p(dA), p(dB),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == C.QLORA_OK, lib.qlora_last_error()
    torch.cuda.synchronize()
    for a, b in zip(want, (dX, dA, dB)):
        assert np.array_equal(_bits(a), _bits(b))
    sel = slice(None) if rows is None else rows
    Xf, dYf = ref.bf16_to_f64(d["X"]), ref.bf16_to_f64(d["dY"])
    dXr, _, _ = ref.linear_bwd(dYf[sel], Xf[sel], *P.triple(), P.s)
    dAr, dBr = ref.adapter_grads(dYf, Xf, P.A, P.B, P.s)
    errs = dict(dX=rel_err(host(dX)[sel], dXr), dA=rel_err(host(dA), dAr), dB=rel_err(host(dB), dBr))
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("grad", ["bf16", "f32"])
def test_noalloc_backward_matches_workspace_backward(grad):
    import torch
    gd = torch.bfloat16 if grad == "bf16" else torch.float32
    # first call: the attention projection (M=4096, K=N=4096, r=16)
    _announce(f"noalloc backward attn M=4096 K=N=4096 r=16 grads={grad}")
    d = make_workload(1)
    _case(d, gd, rows=sample_rows(d["M"], np.random.default_rng(12), per_block=1))
    # second call, smaller, on the same scratch: ragged shapes and a rank that needs the B^T copy
    _announce(f"noalloc backward M=300 K=192 N=264 r=8 grads={grad}")
    _case(random_linear(10_764, 300, 192, 264, 8), gd)
