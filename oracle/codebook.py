"""The 16-level 4-bit codebook (NormalFloat-4) and its decision thresholds.

The pages only say that the frozen base weights are 4-bit bitsandbytes
checkpoints ("Unsloth" wiki entry, API snippet: load_in_4bit; "Unsloth vs The
Stack v2", quantized-base card). The levels used here are the NormalFloat-4
(NF4) values as printed in the QLoRA paper (Dettmers et al., 2023, appendix on
the NF4 data type): quantiles of N(0,1) taken separately for the negative half
(7 levels) and the positive half (8 levels), joined with an exact zero and
scaled into [-1, 1].

The printed values are the definition (stored as fp32); ``derive_nf4_levels``
rebuilds them from the quantile construction in float64 and agrees to ~2e-7
(the pin in tests/test_oracle.py), which shows the printed table is the
construction and not a typo-ridden copy.
"""
from __future__ import annotations

import numpy as np

# As printed in the QLoRA paper (fp32 values, printed to 17 significant digits).
_NF4_PRINTED = [
    -1.0,
    -0.6961928009986877,
    -0.5250730514526367,
    -0.39491748809814453,
    -0.28444138169288635,
    -0.18477343022823334,
    -0.09105003625154495,
    0.0,
    0.07958029955625534,
    0.16093020141124725,
    0.24611230194568634,
    0.33791524171829224,
    0.44070982933044434,
    0.5626170039176941,
    0.7229568362236023,
    1.0,
]

NF4_LEVELS = np.array(_NF4_PRINTED, dtype=np.float32)
NF4_LEVELS.setflags(write=False)

# The same table as fp32 bit patterns (also written in the HIP sources; a CPU
# test checks the two copies are identical bit for bit).
NF4_HEX = [int(v) for v in NF4_LEVELS.view(np.uint32)]

# Decision thresholds: midpoints of adjacent levels, computed in float64 and
# rounded once to fp32. A code is the number of thresholds strictly below x,
# so a tie x == T[j] goes to the lower level (nearest-level rule).
NF4_THRESHOLDS = ((NF4_LEVELS[:-1].astype(np.float64) + NF4_LEVELS[1:].astype(np.float64)) * 0.5).astype(np.float32)
NF4_THRESHOLDS.setflags(write=False)


def derive_nf4_levels() -> np.ndarray:
    """Rebuild the NF4 levels in float64 from the quantile construction.

    Positive half: the 8 normal quantiles at probabilities evenly spaced from
    delta down to (but excluding) 1/2; negative half: the mirror image of 7
    quantiles spaced the same way. delta sits halfway between the outermost
    quantile positions of a 15- and a 16-point grid, which keeps the extreme
    level finite. The union with 0 is scaled so that its largest magnitude is 1.
    """
    from scipy.special import ndtri

    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    pos = ndtri(np.linspace(delta, 0.5, 9)[:-1])
    neg = -ndtri(np.linspace(delta, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    return v / np.abs(v).max()
