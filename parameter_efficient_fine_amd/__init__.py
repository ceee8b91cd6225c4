"""MI355X (gfx950) fused QLoRA linear layer: 4-bit NF4 frozen weight + rank-r LoRA adapter.

The work runs in libqlora.so (hand-written HIP, C ABI in include/qlora.h);
this package is its thin Python binding. Importing the package does not load
the library; the first call does, and fails loudly if it is not built.
"""
from .ops import (  # noqa: F401
    KernelTimer,
    QLoraLayer,
    QLoraLinear,
    backward,
    ce_chunk_for_budget,
    chunked_ce,
    dequantize,
    forward,
    forward_rope,
    linear,
    lmhead_prepare,
    mlp_backward,
    mlp_backward_tiled,
    mlp_forward,
    mlp_forward_tiled,
    mlp_tiled_workspace_size,
    pack_codes,
    quantize,
    quantize_sync,
    rmsnorm_backward,
    rmsnorm_forward,
    rope_backward,
    rope_forward,
    rope_table,
    swiglu_mlp,
    workspace_size,
)
