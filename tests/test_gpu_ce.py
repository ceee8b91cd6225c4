"""GPU parity of the chunked cross-entropy over the frozen LM head (through
the C ABI) against the unchunked oracle (oracle/ce.py): per-row losses and dh
to max|err|/max|ref| <= 1e-2, the mean loss to 1e-4 relative; chunking must
not change the result beyond summation order."""
import numpy as np
import pytest

from oracle import ce
from oracle.ref import bf16_to_f64
from synthetic import random_ce
from tests._util import TOL, dev_bf16, host, rel_err, sample_rows

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _run(d, chunk):
    import torch
    import parameter_efficient_fine_amd as q
    h, W = dev_bf16(d["h"]), dev_bf16(d["W"])
    t = torch.from_numpy(d["targets"]).cuda()
    return q.chunked_ce(h, q.lmhead_prepare(W), t, chunk)


@pytest.mark.parametrize("M,H,V,chunk", [
    (300, 128, 1024, 128),   # ragged last chunk
    (300, 128, 1024, 4096),  # one chunk holds the batch
    (97, 64, 2048, 32),      # many small chunks, rows < one GEMM tile
    (1, 64, 64, 1),          # smallest shapes
    (130, 128, 1472, 64),    # vocabulary not a multiple of the 256-column statistics tile
])
def test_ce_full_oracle(M, H, V, chunk):
    _announce(f"ce M={M} H={H} V={V} chunk={chunk}")
    d = random_ce(300 + M + H + V + chunk, M, H, V)
    out = _run(d, chunk)
    loss, rows, dh = ce.ce_fwd_bwd(bf16_to_f64(d["h"]), bf16_to_f64(d["W"]), d["targets"])
    assert abs(float(host(out["loss"])[0]) - loss) <= 1e-4 * max(abs(loss), 1e-12)
    errs = dict(rows=rel_err(host(out["loss_rows"]), rows), dh=rel_err(host(out["dh"]), dh))
    assert max(errs.values()) <= TOL, errs
    # ignored rows give exactly zero
    ign = d["targets"] < 0
    assert not host(out["loss_rows"])[ign].any() and not host(out["dh"])[ign].any()


def _random_ce_shapes(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 700)), 64 * int(rng.integers(1, 5)), 64 * int(rng.integers(1, 70)),
             int(rng.integers(1, 900))) for _ in range(n)]


@pytest.mark.parametrize("M,H,V,chunk", _random_ce_shapes(6, 9191))
def test_ce_random_shapes(M, H, V, chunk):
    _announce(f"ce random M={M} H={H} V={V} chunk={chunk}")
    d = random_ce(700 + M + H + V + chunk, M, H, V)
    out = _run(d, chunk)
    loss, rows, dh = ce.ce_fwd_bwd(bf16_to_f64(d["h"]), bf16_to_f64(d["W"]), d["targets"])
    assert abs(float(host(out["loss"])[0]) - loss) <= 1e-4 * max(abs(loss), 1e-12)
    errs = dict(rows=rel_err(host(out["loss_rows"]), rows), dh=rel_err(host(out["dh"]), dh))
    assert max(errs.values()) <= TOL, errs


def test_ce_all_rows_ignored():
    _announce("ce all ignored")
    d = random_ce(5, 64, 64, 256)
    d["targets"][:] = -100
    out = _run(d, 32)
    assert float(host(out["loss"])[0]) == 0.0 and not host(out["dh"]).any()


def test_ce_chunk_size_changes_nothing_but_order():
    _announce("ce chunk invariance")
    d = random_ce(6, 700, 256, 4096)
    a, b = _run(d, 128), _run(d, 700)
    # each row is computed the same way in any chunk: rows and dh bit for bit
    assert np.array_equal(host(a["loss_rows"]), host(b["loss_rows"]))
    assert np.array_equal(host(a["dh"]), host(b["dh"]))
    assert float(host(a["loss"])[0]) == float(host(b["loss"])[0])


def test_ce_llama3_head_sampled_rows():
    # the Llama-3-8B head (V = 128256, H = 4096), 1024 tokens in chunks of 512;
    # the oracle computes sampled rows (rows are independent given n)
    _announce("ce M=1024 H=4096 V=128256 chunk=512")
    d = random_ce(7, 1024, 4096, 128256)
    out = _run(d, 512)
    rows = sample_rows(1024, np.random.default_rng(7), per_block=4)
    t = d["targets"]
    n = int((t >= 0).sum())
    _, rr, dh = ce.ce_fwd_bwd(bf16_to_f64(d["h"])[rows], bf16_to_f64(d["W"]), t[rows])
    n_s = int((t[rows] >= 0).sum())
    dh = dh * (n_s / n)
    got_rows = host(out["loss_rows"])
    errs = dict(rows=rel_err(got_rows[rows], rr), dh=rel_err(host(out["dh"])[rows], dh))
    assert max(errs.values()) <= TOL, errs
    # the mean over kept rows of the per-row losses
    assert abs(float(host(out["loss"])[0]) - got_rows.sum() / n) <= 1e-5 * abs(got_rows.sum() / n)


def test_ce_bench_configuration():
    # the benchmark's own input and launch configuration: the Llama-3-8B head
    # (V = 128256, H = 4096), M = 16384 tokens in chunks of 4096
    M, H, V, chunk = 16384, 4096, 128256, 4096
    _announce(f"ce M={M} H={H} V={V} chunk={chunk} (bench input)")
    import torch
    import parameter_efficient_fine_amd as q
    d = random_ce(6000, M, H, V)
    prepared = q.lmhead_prepare(dev_bf16(d["W"]))
    t = d["targets"]
    out = q.chunked_ce(dev_bf16(d["h"]), prepared, torch.from_numpy(t).cuda(), chunk)
    Wf = bf16_to_f64(d["W"])
    Hf = bf16_to_f64(d["h"])
    n = int((t >= 0).sum())
    # sampled rows (every 512-row block, so every chunk and GEMM tile is hit): rows
    # are independent given n, so the oracle on the sample scales dh by n_s / n
    rows = sample_rows(M, np.random.default_rng(60), per_block=1, block=512)
    _, rr, dh = ce.ce_fwd_bwd(Hf[rows], Wf, t[rows])
    dh = dh * (int((t[rows] >= 0).sum()) / n)
    errs = dict(rows=rel_err(host(out["loss_rows"])[rows], rr), dh=rel_err(host(out["dh"])[rows], dh))
    assert max(errs.values()) <= TOL, errs
    # the whole batch against the oracle: 64 distinct (hidden row, target) pairs,
    # token m taking pair idx[m] (ignored where the bench's target is), so the
    # oracle's loss over all M tokens and every row of dh follow from its result
    # on the 64 pairs; the GPU runs the same chunked launches over all M tokens
    rng = np.random.default_rng(61)
    idx = rng.integers(0, 64, M)
    t64 = rng.integers(0, V, 64).astype(np.int32)
    keep = t >= 0
    t2 = np.where(keep, t64[idx], -100).astype(np.int32)
    out2 = q.chunked_ce(dev_bf16(d["h"][:64][idx]), prepared, torch.from_numpy(t2).cuda(), chunk)
    _, r64, dh64 = ce.ce_fwd_bwd(Hf[:64], Wf, t64)   # every pair kept: dh64 carries 1/64
    loss = float(np.sum(r64[idx][keep])) / n
    got = float(host(out2["loss"])[0])
    assert abs(got - loss) <= 1e-4 * abs(loss), (got, loss)
    want_rows = np.where(keep, r64[idx], 0.0)
    want_dh = np.where(keep[:, None], dh64[idx] * (64.0 / n), 0.0)
    errs2 = dict(rows=rel_err(host(out2["loss_rows"]), want_rows), dh=rel_err(host(out2["dh"]), want_dh))
    assert max(errs2.values()) <= TOL, errs2
