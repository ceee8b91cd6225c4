"""Plain CPU definition of the cross-entropy over the language-model head
(test infrastructure: only the tests, the smoke check and bench.py's
CPU-baseline leg use this module).

The pages name a chunked cross-entropy that never forms the [B, T, V] logits
("Unsloth" wiki entry, Theory; "Unsloth vs PyTorch" video, 3:06-3:51: the
loss is computed slice by slice and each slice discarded, with identical
gradients). Chunking is an evaluation order, so this oracle is the plain,
unchunked definition, in float64:

  logits z = h . W^T                     h [M,H] final hidden states, W [V,H] frozen head
  lse_m    = log sum_v exp(z[m,v])
  loss_m   = lse_m - z[m, t_m]           for targets t_m >= 0; rows with t_m < 0 are ignored
  loss     = sum_m loss_m / n            n = number of rows that are not ignored
  dz       = (softmax(z) - onehot(t)) / n on kept rows, 0 on ignored rows
  dh       = dz . W                      (W is frozen: no weight gradient)
"""
from __future__ import annotations

import numpy as np


def ce_fwd_bwd(h, W, targets):
    """-> (loss, per-row losses [M] (0 on ignored rows), dh [M,H]), float64."""
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    M, V = h.shape[0], W.shape[0]
    keep = t >= 0
    n = int(keep.sum())
    z = h @ W.T
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    s = e.sum(axis=1, keepdims=True)
    lse = (zmax + np.log(s))[:, 0]
    rows = np.arange(M)
    tt = np.where(keep, t, 0)
    loss_rows = np.where(keep, lse - z[rows, tt], 0.0)
    loss = loss_rows.sum() / n if n else 0.0
    dz = e / s
    dz[rows[keep], t[keep]] -= 1.0
    dz[~keep] = 0.0
    dz = dz / n if n else dz * 0.0
    return loss, loss_rows, dz @ W
