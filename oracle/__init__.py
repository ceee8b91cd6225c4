"""CPU oracle for the fused QLoRA linear layer and its SwiGLU MLP (test infrastructure).

This package is test infrastructure, not product code. Only the tests, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it. It shares no code with the HIP library: it has its own copy of the
codebook, its own quantizer and its own float64 algebra on NumPy/BLAS.

Sources (the pages, by title and passage):
  * "Rev vs unsloth", card on fused quantized LoRA: a frozen quantized weight and
    a LoRA adapter evaluated as one layer, with a custom backward.
  * "Unsloth vs The Stack v2", card on quantized-base fine-tuning: the 4-bit
    weight is frozen, only the adapter trains (so there is no dW).
  * "Unsloth" (wiki entry), Theory: hand-derived backward passes for the LoRA
    path; fused SwiGLU block.
  * "Unsloth vs PyTorch" (video), 0:43-2:11: the six matrix derivatives and the
    associativity argument (bracket the skinny adapter product so the N x K
    matrix is never formed).

Every function that has no pin says "parity unpinned" in its docstring; at
present every function is pinned: ref and codebook by tests/test_oracle.py,
formats8, normrope and ce by tests/test_oracle_formats8.py,
tests/test_oracle_normrope.py and tests/test_oracle_ce.py.
"""
from .codebook import NF4_LEVELS, NF4_THRESHOLDS, derive_nf4_levels  # noqa: F401
from .ref import (  # noqa: F401
    bf16_to_f64,
    quantize,
    dequantize,
    linear_fwd,
    linear_bwd,
    adapter_grads,
    silu,
    mlp_fwd,
    mlp_bwd,
)
