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


def _run(d, tile, fmt=0):
    import parameter_efficient_fine_amd as q
    Ls = {nm: Prepared(d["layers"][nm], d["s"], fmt=fmt) for nm in ("gate", "up", "down")}
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


def _oracle_errs(d, Ls, tf, tb):
    X, dY = ref.bf16_to_f64(d["X"]), ref.bf16_to_f64(d["dY"])
    trip = [Ls[nm].triple() for nm in ("gate", "up", "down")]
    fr = ref.mlp_fwd(X, *trip, d["s"])
    br = ref.mlp_bwd(dY, X, *trip, d["s"])
    errs = dict(Y=rel_err(host(tf["Y"]), fr["Y"]), dX=rel_err(host(tb["dX"]), br["dX"]))
    for i, nm in enumerate(("gate", "up", "down")):
        errs["dA_" + nm] = rel_err(host(tb["dA"][i]), br["dA_" + nm])
        errs["dB_" + nm] = rel_err(host(tb["dB"][i]), br["dB_" + nm])
    return errs


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
    errs = _oracle_errs(d, Ls, tf, tb)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("fmt", [1, 2])
def test_mlp_tiled_8bit_weights(fmt):
    # INT8 and FP8 frozen weights through the tiled block: ragged last tile
    _announce(f"tiled mlp fmt={fmt} M=1000 tile=384 H=128 I=256 r=16")
    d = random_mlp(1_400 + fmt, 1000, 128, 256, 16)
    Ls, wf, wb, tf, tb = _run(d, 384, fmt=fmt)
    _compare_to_whole(wf, wb, tf, tb, same_order=False)
    errs = _oracle_errs(d, Ls, tf, tb)
    assert max(errs.values()) <= TOL, errs


def _random_tiled_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 1500))
        tile = int(rng.choice([64, 96, 128, 256, 320, 512, 700]))
        H = 64 * int(rng.integers(1, 5))
        I = 64 * int(rng.integers(1, 7))
        r = int(rng.integers(1, 33)) if i % 3 else int(rng.integers(100, 161))
        out.append((M, tile, H, I, r))
    return out


@pytest.mark.parametrize("M,tile,H,I,r", _random_tiled_shapes(8, 2028))
def test_mlp_tiled_random_shapes(M, tile, H, I, r):
    # seeded shapes: ragged last tiles, 1 to 20 tiles (two streams), ranks that
    # need the B^T copies (r not 16, 32, 64, 128, 256) and reductions in several launches (2r > 256)
    _announce(f"tiled mlp random M={M} tile={tile} H={H} I={I} r={r}")
    d = random_mlp(2_000 + M + tile + H + I + r, M, H, I, r)
    Ls, wf, wb, tf, tb = _run(d, tile)
    _compare_to_whole(wf, wb, tf, tb, same_order=tile >= M)
    errs = _oracle_errs(d, Ls, tf, tb)
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("r", [48, 96])
def test_mlp_rank_multiple_of_16_not_a_power_of_two(r):
    # the G products of such ranks read the transposed copies of B (whole and tiled)
    _announce(f"mlp rank {r} M=600 tile=256 H=128 I=256")
    d = random_mlp(620 + r, 600, 128, 256, r)
    Ls, wf, wb, tf, tb = _run(d, 256)
    _compare_to_whole(wf, wb, tf, tb, same_order=False)
    errs = _oracle_errs(d, Ls, tf, tb)
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
    # The upstream gradient is zero outside sampled rows, so every gradient of
    # the tiled call involves those rows only and the oracle computes dX on them
    # and the exact dA, dB.
    _announce("tiled mlp M=16384 tile=4096 H=4096 I=14336 r=16")
    d = random_mlp(4096, 16384, 4096, 14336, 16)
    rows = sample_rows(d["M"], np.random.default_rng(9), per_block=1)
    keep = np.zeros(d["M"], bool)
    keep[rows] = True
    d["dY"] = np.where(keep[:, None], d["dY"], 0).astype(d["dY"].dtype)
    Ls, wf, wb, tf, tb = _run(d, 4096)
    _compare_to_whole(wf, wb, tf, tb, same_order=False)
    X, dY = ref.bf16_to_f64(d["X"]), ref.bf16_to_f64(d["dY"])
    trip = [Ls[nm].triple() for nm in ("gate", "up", "down")]
    fr = ref.mlp_fwd(X[rows], *trip, d["s"])
    br = ref.mlp_bwd(dY[rows], X[rows], *trip, d["s"])
    errs = dict(Y=rel_err(host(tf["Y"])[rows], fr["Y"]), dX=rel_err(host(tb["dX"])[rows], br["dX"]))
    for i, nm in enumerate(("gate", "up", "down")):
        errs["dA_" + nm] = rel_err(host(tb["dA"][i]), br["dA_" + nm])
        errs["dB_" + nm] = rel_err(host(tb["dB"][i]), br["dB_" + nm])
    assert max(errs.values()) <= TOL, errs
    assert not host(tb["dX"])[~keep].any()


def test_mlp_tiled_second_stream_at_full_width():
    # tiles of 1024 tokens (the last one ragged) at Llama-3.1-8B widths: each
    # tile's down-projection GEMM (forward) and gate/up part (backward) run on
    # the library's second stream beside the next tile's work. Rows must equal
    # the whole-batch call's bit for bit and the gradients up to summation
    # order, and repeated runs must give the first run's bits.
    _announce("tiled mlp second stream M=3500 tile=1024 H=4096 I=14336 r=16")
    import parameter_efficient_fine_amd as q
    d = random_mlp(4100, 3500, 4096, 14336, 16)
    Ls, wf, wb, tf, tb = _run(d, 1024)
    _compare_to_whole(wf, wb, tf, tb, same_order=False)
    g, u, dn = (Ls[nm].dev for nm in ("gate", "up", "down"))
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    for _ in range(2):
        tf2 = q.mlp_forward_tiled(g, u, dn, X, 1024)
        tb2 = q.mlp_backward_tiled(g, u, dn, dY, X, tf2["Z"], 1024)
        for a, b in ((tf2["Y"], tf["Y"]), (tf2["Z"], tf["Z"]), (tb2["dX"], tb["dX"])):
            assert np.array_equal(_bits(a), _bits(b))
        for i in range(3):
            for key in ("dA", "dB"):
                assert np.array_equal(_bits(tb2[key][i]), _bits(tb[key][i])), (key, i)


@pytest.mark.parametrize("tile", [0, 384])
def test_mlp_backward_without_dx_matches_the_one_with_dx(tile):
    # Without dX the gate/up reductions' split partials are added by a reduce
    # launch of their own (on the second stream when the tiles overlap) instead
    # of the dX GEMM's prologue. Same partials, same split order: the gradients
    # agree bit for bit. tile = 0: the whole-batch call.
    _announce(f"mlp backward without dX M=1000 H=128 I=256 r=16 tile={tile}")
    import parameter_efficient_fine_amd as q
    d = random_mlp(1_500 + tile, 1000, 128, 256, 16)
    Ls = {nm: Prepared(d["layers"][nm], d["s"]) for nm in ("gate", "up", "down")}
    g, u, dn = Ls["gate"].dev, Ls["up"].dev, Ls["down"].dev
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    if tile:
        f = q.mlp_forward_tiled(g, u, dn, X, tile)
        b1 = q.mlp_backward_tiled(g, u, dn, dY, X, f["Z"], tile)
        b0 = q.mlp_backward_tiled(g, u, dn, dY, X, f["Z"], tile, need_dX=False)
    else:
        f = q.mlp_forward(g, u, dn, X)
        b1 = q.mlp_backward(g, u, dn, dY, X, f)
        b0 = q.mlp_backward(g, u, dn, dY, X, f, need_dX=False)
    assert b0["dX"] is None and b1["dX"] is not None
    for i in range(3):
        for key in ("dA", "dB"):
            assert np.array_equal(_bits(b0[key][i]), _bits(b1[key][i])), (key, i)


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


@pytest.mark.parametrize("M,H,I,r,tile", [
    (1088, 128, 256, 8, 576),     # the last tile (512 tokens) needs more reduction splits than a full one
    (1344, 128, 384, 16, 704),    # the same with tile 704 (last tile 640 tokens), r = 16
])
def test_mlp_tiled_ragged_last_tile_stays_in_its_workspace(M, H, I, r, tile):
    # a canary region right after a workspace of exactly the size the library
    # asks for must come back untouched; the result must match the oracle
    _announce(f"tiled mlp canary M={M} H={H} I={I} r={r} tile={tile}")
    import torch
    import parameter_efficient_fine_amd as q
    d = random_mlp(900 + M + tile, M, H, I, r)
    Ls = {nm: Prepared(d["layers"][nm], d["s"]) for nm in ("gate", "up", "down")}
    g, u, dn = Ls["gate"].dev, Ls["up"].dev, Ls["down"].dev
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    nb = q.mlp_tiled_workspace_size(True, M, H, I, r, tile)
    canary = 4 << 20
    buf = torch.full((nb + canary,), 0x5A, dtype=torch.uint8, device="cuda")
    f = q.mlp_forward_tiled(g, u, dn, X, tile)
    b = q.mlp_backward_tiled(g, u, dn, dY, X, f["Z"], tile, ws=buf[:nb])
    torch.cuda.synchronize()
    assert bool((buf[nb:] == 0x5A).all()), "the tiled backward wrote past its workspace"
    Xf, dYf = ref.bf16_to_f64(d["X"]), ref.bf16_to_f64(d["dY"])
    trip = [Ls[nm].triple() for nm in ("gate", "up", "down")]
    br = ref.mlp_bwd(dYf, Xf, *trip, d["s"])
    errs = dict(dX=rel_err(host(b["dX"]), br["dX"]))
    for i, nm in enumerate(("gate", "up", "down")):
        errs["dA_" + nm] = rel_err(host(b["dA"][i]), br["dA_" + nm])
        errs["dB_" + nm] = rel_err(host(b["dB"][i]), br["dB_" + nm])
    assert max(errs.values()) <= TOL, errs
