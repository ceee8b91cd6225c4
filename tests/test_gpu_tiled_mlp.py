"""GPU checks of the token-tiled SwiGLU block (tiled feed-forward layers of the
"Unsloth vs PyTorch" video, 4:25-4:36): the batch is processed `tile` tokens
at a time, the backward recomputes each tile's g, u, h, and the adapter
gradients are summed over tiles.

Tiling changes the order of evaluation only, so the oracle is the whole-batch
block: every output is checked against it (max|err|/max|ref| <= 1e-2), and in
addition Y, Z and dX must equal the whole-batch HIP path bit for bit (each
token's row is computed the same way) while dA and dB may differ from it only
by fp32 summation order.
"""
import numpy as np
import pytest

from oracle import ref
from synthetic import random_mlp
from tests._util import TOL, Prepared, dev_bf16, host, rel_err, sample_rows

pytestmark = pytest.mark.gpu

ORDER_TOL = 1e-4  # |tiled - whole| / max|whole| for the fp32 adapter gradients


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _bits(t):
    import torch
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def _run(d, tile):
    import parameter_efficient_fine_amd as q
    Ls = {nm: Prepared(d["layers"][nm], d["s"]) for nm in ("gate", "up", "down")}
    g, u, dn = Ls["gate"].dev, Ls["up"].dev, Ls["down"].dev
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    whole_f = q.mlp_forward(g, u, dn, X)
    whole_b = q.mlp_backward(g, u, dn, dY, X, whole_f)
    tf = q.mlp_forward_tiled(g, u, dn, X, tile)
    tb = q.mlp_backward_tiled(g, u, dn, dY, X, tf["Z"], tile)
    return Ls, whole_f, whole_b, tf, tb


def _compare_to_whole(whole_f, whole_b, tf, tb, same_order):
    for a, b in ((tf["Y"], whole_f["Y"]), (tf["Z"], whole_f["Z"]), (tb["dX"], whole_b["dX"])):
        assert np.array_equal(_bits(a), _bits(b))
    for i in range(3):
        for key in ("dA", "dB"):
            t, w = host(tb[key][i]), host(whole_b[key][i])
            if same_order:
                assert np.array_equal(t.view(np.uint32), w.view(np.uint32)), (key, i)
            else:
                assert rel_err(t, w) <= ORDER_TOL, (key, i, rel_err(t, w))


@pytest.mark.parametrize("M,tile", [
    (1000, 256),   # 3 full tiles and a ragged one
    (1000, 384),   # tile not a multiple of the GEMM's 256-token tile
    (700, 96),     # many small tiles
    (300, 1000),   # one tile holding the whole batch: identical to the whole-batch call
    (1, 64),       # a single token
])
def test_mlp_tiled_full_oracle(M, tile):
    _announce(f"tiled mlp M={M} tile={tile} H=128 I=256 r=16")
    d = random_mlp(500 + M + tile, M, 128, 256, 16)
    Ls, wf, wb, tf, tb = _run(d, tile)
    _compare_to_whole(wf, wb, tf, tb, same_order=tile >= M)
    X, dY = ref.bf16_to_f64(d["X"]), ref.bf16_to_f64(d["dY"])
    trip = [Ls[nm].triple() for nm in ("gate", "up", "down")]
    fr = ref.mlp_fwd(X, *trip, d["s"])
    br = ref.mlp_bwd(dY, X, *trip, d["s"])
    errs = dict(Y=rel_err(host(tf["Y"]), fr["Y"]), dX=rel_err(host(tb["dX"]), br["dX"]))
    for i, nm in enumerate(("gate", "up", "down")):
        errs["dA_" + nm] = rel_err(host(tb["dA"][i]), br["dA_" + nm])
        errs["dB_" + nm] = rel_err(host(tb["dB"][i]), br["dB_" + nm])
    assert max(errs.values()) <= TOL, errs


def test_mlp_tiled_high_rank():
    # 2r > 256: the paired Z_g, Z_u product and the dA reductions split into several launches per tile
    _announce("tiled mlp M=600 tile=256 H=128 I=256 r=200")
    d = random_mlp(611, 600, 128, 256, 200)
    _, wf, wb, tf, tb = _run(d, 256)
    _compare_to_whole(wf, wb, tf, tb, same_order=False)


def test_mlp_tiled_long_batch_full_size():
    # Llama-3.1-8B MLP widths at M=16384 in tiles of 4096 tokens: bitwise rows
    # and order-only gradient differences against the whole-batch call, and the
    # oracle on sampled rows of Y
    _announce("tiled mlp M=16384 tile=4096 H=4096 I=14336 r=16")
    d = random_mlp(4096, 16384, 4096, 14336, 16)
    Ls, wf, wb, tf, tb = _run(d, 4096)
    _compare_to_whole(wf, wb, tf, tb, same_order=False)
    rows = sample_rows(d["M"], np.random.default_rng(9), per_block=1)
    X = ref.bf16_to_f64(d["X"])
    trip = [Ls[nm].triple() for nm in ("gate", "up", "down")]
    fr = ref.mlp_fwd(X[rows], *trip, d["s"])
    assert rel_err(host(tf["Y"])[rows], fr["Y"]) <= TOL


def test_mlp_tiled_backward_independent_of_workspace_and_output_contents():
    # the first tile overwrites dA/dB and later tiles add to them: outputs and a
    # workspace full of NaN bytes must not leak into the result
    _announce("tiled mlp dirty buffers M=700 tile=256")
    import torch
    import parameter_efficient_fine_amd as q
    d = random_mlp(777, 700, 128, 256, 16)
    Ls = {nm: Prepared(d["layers"][nm], d["s"]) for nm in ("gate", "up", "down")}
    g, u, dn = Ls["gate"].dev, Ls["up"].dev, Ls["down"].dev
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    runs = []
    for dirty in (False, True):
        fill = float("nan") if dirty else 0.0
        nbf = q.mlp_tiled_workspace_size(False, 700, 128, 256, 16, 256)
        nbb = q.mlp_tiled_workspace_size(True, 700, 128, 256, 16, 256)
        wsf = torch.full((nbf,), 255 if dirty else 0, dtype=torch.uint8, device="cuda")
        wsb = torch.full((nbb,), 255 if dirty else 0, dtype=torch.uint8, device="cuda")
        f = q.mlp_forward_tiled(g, u, dn, X, 256, ws=wsf,
                                out=dict(Y=torch.full((700, 128), fill, dtype=torch.bfloat16, device="cuda"),
                                         Z=torch.full((3, 700, 16), fill, dtype=torch.bfloat16, device="cuda")))
        out = dict(dX=torch.full((700, 128), fill, dtype=torch.bfloat16, device="cuda"),
                   dA=[torch.full((16, L.K), fill, dtype=torch.float32, device="cuda") for L in (g, u, dn)],
                   dB=[torch.full((L.N, 16), fill, dtype=torch.float32, device="cuda") for L in (g, u, dn)])
        b = q.mlp_backward_tiled(g, u, dn, dY, X, f["Z"], 256, ws=wsb, out=out)
        torch.cuda.synchronize()
        runs.append([_bits(t) for t in [f["Y"], f["Z"], b["dX"]] + b["dA"] + b["dB"]])
    for a, b in zip(*runs):
        assert np.array_equal(a, b)
