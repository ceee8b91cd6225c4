"""Calls from several host threads at once (the C ABI promises re-entrant
calls). Each thread runs its own layers on its own stream: linear layers whose
G product reads B in place and through its transposed copy, and token-tiled
SwiGLU blocks, which share the library's second stream. Every result must
equal that of a single-threaded run bit for bit, on every repetition."""
import threading

import numpy as np
import pytest

from synthetic import random_linear, random_mlp
from tests._util import Prepared, dev_bf16

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _bits(t):
    import torch
    t = t.detach().contiguous()
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def _linear_job(seed, M, K, N, r):
    import parameter_efficient_fine_amd as q
    d = random_linear(seed, M, K, N, r)
    P = Prepared(d["layers"]["proj"], d["s"])
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])

    def run():
        Y, Z = q.forward(P.dev, X)
        dX, dA, dB = q.backward(P.dev, dY, X, Z)
        return [Y, Z, dX, dA, dB]
    return run


def _tiled_job(seed, M, H, I, r, tile):
    import parameter_efficient_fine_amd as q
    d = random_mlp(seed, M, H, I, r)
    g, u, dn = (Prepared(d["layers"][nm], d["s"]).dev for nm in ("gate", "up", "down"))
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])

    def run():
        f = q.mlp_forward_tiled(g, u, dn, X, tile)
        b = q.mlp_backward_tiled(g, u, dn, dY, X, f["Z"], tile)
        return [f["Y"], f["Z"], b["dX"], *b["dA"], *b["dB"]]
    return run


def test_concurrent_calls_from_threads():
    import torch
    _announce("threads: 3 linear layers and 2 tiled SwiGLU blocks, 4 repetitions each")
    jobs = [
        _linear_job(70_001, 700, 256, 264, 16),   # B read in place
        _linear_job(70_002, 520, 320, 200, 48),   # B through its transposed copy
        _linear_job(70_003, 200, 512, 512, 8),    # small-batch path
        _tiled_job(70_004, 900, 128, 256, 16, 256),
        _tiled_job(70_005, 700, 192, 320, 24, 128),
    ]
    want = [[_bits(t) for t in job()] for job in jobs]
    torch.cuda.synchronize()
    got = [None] * len(jobs)
    errors = []
    start = threading.Barrier(len(jobs))

    def worker(k):
        try:
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                outs = [jobs[k]() for _ in range(4)]
            s.synchronize()
            got[k] = [[_bits(t) for t in o] for o in outs]
        except Exception as e:  # reported below, with the job
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for k, outs in enumerate(got):
        for rep, o in enumerate(outs):
            for i, (a, b) in enumerate(zip(o, want[k])):
                assert np.array_equal(a, b), (k, rep, i)
