"""CPU checks of the C-ABI library: it loads, exports every declared entry point,
carries the same codebook as the oracle, and rejects bad arguments before any
GPU work (these calls return before touching HIP, so they run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle.codebook import NF4_HEX
from parameter_efficient_fine_amd import _lib as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(C.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    lib = C.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_kernel_codebook_matches_oracle_bit_for_bit():
    src = open(os.path.join(ROOT, "parameter_efficient_fine_amd", "csrc", "common.hpp")).read()
    block = src[src.index("kNF4Bits[16]"):]
    block = block[block.index("{") + 1: block.index("}")]
    words = [int(w, 16) for w in re.findall(r"0x([0-9a-fA-F]+)u", block)]
    assert words == NF4_HEX


def _layer(K=512, N=512, r=16, fake=0x10000):
    return C.QLoraLayerC(fake, fake, fake, fake, K, N, r, 2.0)


@pytest.mark.parametrize("K,N,r", [(500, 512, 16), (512, 12, 16), (512, 512, 0), (512, 512, 257), (0, 512, 8)])
def test_forward_rejects_bad_shapes(K, N, r):
    lib = C.lib()
    L = _layer(K, N, r)
    st = lib.qlora_forward(ctypes.byref(L), ctypes.c_void_p(0x10000), 4, ctypes.c_void_p(0x10000),
                           ctypes.c_void_p(0x10000), None, 0, None)
    assert st == C.QLORA_EINVAL


def test_forward_rejects_null_and_misaligned():
    lib = C.lib()
    L = _layer()
    assert lib.qlora_forward(ctypes.byref(L), None, 4, ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10000),
                             None, 0, None) == C.QLORA_EINVAL
    assert lib.qlora_forward(ctypes.byref(L), ctypes.c_void_p(0x10002), 4, ctypes.c_void_p(0x10000),
                             ctypes.c_void_p(0x10000), None, 0, None) == C.QLORA_EINVAL
    bad = C.QLoraLayerC(0, 0x10000, 0x10000, 0x10000, 512, 512, 16, 2.0)
    assert lib.qlora_forward(ctypes.byref(bad), ctypes.c_void_p(0x10000), 4, ctypes.c_void_p(0x10000),
                             ctypes.c_void_p(0x10000), None, 0, None) == C.QLORA_EINVAL
    assert lib.qlora_forward(None, ctypes.c_void_p(0x10000), 4, ctypes.c_void_p(0x10000),
                             ctypes.c_void_p(0x10000), None, 0, None) == C.QLORA_EINVAL


def test_backward_workspace_checks():
    lib = C.lib()
    L = _layer()
    p = ctypes.c_void_p(0x10000)
    need = lib.qlora_workspace_size(C.OP_BACKWARD, 64, 512, 512, 16)
    assert need > 0
    assert lib.qlora_backward(ctypes.byref(L), p, p, p, 64, p, p, p, None, 0, None) == C.QLORA_EWORKSPACE
    assert lib.qlora_backward(ctypes.byref(L), p, p, p, 64, p, p, p, p, need - 1, None) == C.QLORA_EWORKSPACE
    assert lib.qlora_backward(ctypes.byref(L), p, p, p, 64, p, None, p, p, need, None) == C.QLORA_EINVAL


def test_mlp_shape_consistency_checks():
    lib = C.lib()
    g, u, d = _layer(256, 512), _layer(256, 512), _layer(512, 256)
    p = ctypes.c_void_p(0x10000)
    # mismatched down projection (K must equal the intermediate width)
    bad_d = _layer(256, 256)
    assert lib.swiglu_mlp_forward(ctypes.byref(g), ctypes.byref(u), ctypes.byref(bad_d), p, 8, p, p, p, p, p,
                                  None, 0, None) == C.QLORA_EINVAL
    # ranks must agree
    u8 = _layer(256, 512, 8)
    assert lib.swiglu_mlp_forward(ctypes.byref(g), ctypes.byref(u8), ctypes.byref(d), p, 8, p, p, p, p, p,
                                  None, 0, None) == C.QLORA_EINVAL
    # M == 0 is a no-op that succeeds without touching the GPU
    assert lib.swiglu_mlp_forward(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), p, 0, p, p, p, p, p,
                                  None, 0, None) == C.QLORA_OK


def test_quantize_argument_checks():
    lib = C.lib()
    p = ctypes.c_void_p(0x10000)
    for fmt in (C.FMT_NF4, C.FMT_INT8, C.FMT_FP8):
        assert lib.qlora_quantize(fmt, p, 4, 100, p, p, None, None) == C.QLORA_EINVAL
        assert lib.qlora_quantize(fmt, p, 0, 64, p, p, None, None) == C.QLORA_OK
        assert lib.qlora_dequantize(fmt, p, p, 4, 65, p, None) == C.QLORA_EINVAL
    for bad_fmt in (-1, 3):
        assert lib.qlora_quantize(bad_fmt, p, 4, 64, p, p, None, None) == C.QLORA_EINVAL
        assert lib.qlora_dequantize(bad_fmt, p, p, 4, 64, p, None) == C.QLORA_EINVAL
    # 8-bit codes are read in 4-byte groups: they must be aligned
    assert lib.qlora_dequantize(C.FMT_INT8, ctypes.c_void_p(0x10001), p, 4, 64, p, None) == C.QLORA_EINVAL


def test_status_strings():
    lib = C.lib()
    for s in (0, -1, -2, -3):
        assert len(lib.qlora_status_string(s)) > 0
    assert np.isscalar(lib.qlora_workspace_size(C.OP_MLP_BACKWARD, 16, 256, 512, 8))


@pytest.mark.parametrize("op", [C.OP_BACKWARD, C.OP_MLP_BACKWARD])
def test_workspace_size_defined_for_every_batch(op):
    # host-side planning of the row splits must handle every M, including 0
    lib = C.lib()
    for M in (0, 1, 63, 64, 65, 4096, 100_000):
        for K, N in ((64, 8), (4096, 4096), (4096, 14336)):
            for r in (1, 8, 16, 127, 128, 129, 256):
                need = lib.qlora_workspace_size(op, M, K, N, r)
                assert need > 0 and need % 256 == 0
                # the workspace holds at least the rank-r intermediates it must keep
                assert need >= 2 * M * r


def test_forward_rejects_oversized_weights():
    lib = C.lib()
    p = ctypes.c_void_p(0x10000)
    for K, N in ((1 << 22, 8), (64, (1 << 21) + 8), (1 << 20, 1 << 12)):
        L = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, K, N, 16, 2.0)
        assert lib.qlora_forward(ctypes.byref(L), p, 4, p, p, None, 0, None) == C.QLORA_EINVAL


def test_tiled_mlp_workspace_scales_with_the_tile_not_the_batch():
    lib = C.lib()
    H, I = 4096, 14336
    for r in (1, 16, 129, 256):
        for bwd in (0, 1):
            for tile in (1024, 4096):
                one_tile = lib.swiglu_mlp_tiled_workspace_size(bwd, tile, H, I, r, tile)
                assert one_tile > 0 and one_tile % 256 == 0
                # from two tiles on, where a tile's last GEMM (tile x H outputs) has fewer
                # 256 x 256 workgroups than the 256 CUs, one [tile, I] buffer more (h,
                # forward) or two more (dg and du, backward): that GEMM runs beside the
                # next tile's work, reading its own copy
                extra = (2 if bwd else 1) * tile * I * 2 if (tile // 256) * (H // 256) < 256 else 0
                two_tiles = lib.swiglu_mlp_tiled_workspace_size(bwd, 2 * tile, H, I, r, tile)
                assert two_tiles == one_tile + extra, (bwd, tile, r)
                # a longer batch with the same tile needs no more than two tiles do
                assert lib.swiglu_mlp_tiled_workspace_size(bwd, 1 << 20, H, I, r, tile) == two_tiles
                # a tile longer than the batch is sized by the batch
                assert lib.swiglu_mlp_tiled_workspace_size(bwd, tile, H, I, r, 1 << 20) == one_tile
            assert lib.swiglu_mlp_tiled_workspace_size(bwd, 0, H, I, r, 4096) >= 0
        # the tiled backward's workspace holds g, u, h, dg, du of one tile; the whole-batch
        # backward holds dg, du of the batch (g, u, h are saved by its forward)
        assert lib.swiglu_mlp_tiled_workspace_size(1, 4096, H, I, r, 4096) >= 5 * 4096 * I * 2
    assert lib.swiglu_mlp_tiled_workspace_size(1, 4096, H, I, 16, 0) == 0  # tile < 1 is invalid


def test_tiled_mlp_argument_checks():
    lib = C.lib()
    g, u, d = _layer(256, 512), _layer(256, 512), _layer(512, 256)
    p = ctypes.c_void_p(0x10000)
    G = [ctypes.byref(x) for x in (g, u, d)]
    grads = (ctypes.c_void_p * 3)(0x10000, 0x10000, 0x10000)
    need_f = lib.swiglu_mlp_tiled_workspace_size(0, 64, 256, 512, 16, 32)
    need_b = lib.swiglu_mlp_tiled_workspace_size(1, 64, 256, 512, 16, 32)
    assert need_f > 0 and need_b > need_f
    # tile must be >= 1
    assert lib.swiglu_mlp_forward_tiled(*G, p, 64, 0, p, p, p, need_f, None) == C.QLORA_EINVAL
    assert lib.swiglu_mlp_backward_tiled(*G, p, p, p, 64, 0, p, grads, grads, p, need_b, None) == C.QLORA_EINVAL
    # workspace missing or short
    assert lib.swiglu_mlp_forward_tiled(*G, p, 64, 32, p, p, None, 0, None) == C.QLORA_EWORKSPACE
    assert lib.swiglu_mlp_forward_tiled(*G, p, 64, 32, p, p, p, need_f - 1, None) == C.QLORA_EWORKSPACE
    assert lib.swiglu_mlp_backward_tiled(*G, p, p, p, 64, 32, p, grads, grads, p, need_b - 1,
                                         None) == C.QLORA_EWORKSPACE
    # null or misaligned tensors
    assert lib.swiglu_mlp_forward_tiled(*G, None, 64, 32, p, p, p, need_f, None) == C.QLORA_EINVAL
    assert lib.swiglu_mlp_backward_tiled(*G, p, ctypes.c_void_p(0x10002), p, 64, 32, p, grads, grads, p, need_b,
                                         None) == C.QLORA_EINVAL
    bad = (ctypes.c_void_p * 3)(0x10000, 0, 0x10000)
    assert lib.swiglu_mlp_backward_tiled(*G, p, p, p, 64, 32, p, bad, grads, p, need_b, None) == C.QLORA_EINVAL
    # mismatched shapes as for the whole-batch call
    bad_d = _layer(256, 256)
    assert lib.swiglu_mlp_forward_tiled(ctypes.byref(g), ctypes.byref(u), ctypes.byref(bad_d), p, 64, 32, p, p, p,
                                        need_f, None) == C.QLORA_EINVAL
    # an empty batch's forward is a no-op that touches no GPU
    assert lib.swiglu_mlp_forward_tiled(*G, p, 0, 32, p, p, None, 0, None) == C.QLORA_OK


def test_norm_and_rope_argument_checks():
    lib = C.lib()
    p = ctypes.c_void_p(0x10000)
    # RMSNorm: H % 8, H > 0, eps >= 0, alignment; an empty batch is a no-op
    assert lib.qlora_rmsnorm_forward(p, p, 4, 12, 1e-5, p, p, None) == C.QLORA_EINVAL
    assert lib.qlora_rmsnorm_forward(p, p, 4, 0, 1e-5, p, p, None) == C.QLORA_EINVAL
    assert lib.qlora_rmsnorm_forward(p, p, 4, 64, -1.0, p, p, None) == C.QLORA_EINVAL
    assert lib.qlora_rmsnorm_forward(ctypes.c_void_p(0x10002), p, 4, 64, 1e-5, p, p, None) == C.QLORA_EINVAL
    assert lib.qlora_rmsnorm_forward(p, p, 0, 64, 1e-5, p, p, None) == C.QLORA_OK
    assert lib.qlora_rmsnorm_backward(p, p, p, None, 4, 64, p, None) == C.QLORA_EINVAL
    assert lib.qlora_rmsnorm_backward(p, p, p, p, 0, 64, p, None) == C.QLORA_OK
    # RoPE: head size a multiple of 16 in [16, 1024], base > 1, positions given
    for d in (8, 24, 2048):
        assert lib.qlora_rope_forward(p, p, p, 4, 2, 1, d, 10000.0, None) == C.QLORA_EINVAL
    assert lib.qlora_rope_forward(p, p, p, 4, 2, 1, 64, 1.0, None) == C.QLORA_EINVAL
    assert lib.qlora_rope_forward(p, p, None, 4, 2, 1, 64, 10000.0, None) == C.QLORA_EINVAL
    assert lib.qlora_rope_backward(p, None, p, 4, 2, 1, 64, 10000.0, None) == C.QLORA_EINVAL  # k heads need k
    assert lib.qlora_rope_forward(p, None, p, 0, 2, 1, 64, 10000.0, None) == C.QLORA_OK
    assert lib.qlora_rope_forward(None, None, p, 4, 0, 0, 64, 10000.0, None) == C.QLORA_OK


def test_layer_format_checks():
    lib = C.lib()
    p = ctypes.c_void_p(0x10000)
    for fmt, ok in ((0, True), (1, True), (2, True), (3, False), (-1, False)):
        L = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 512, 512, 16, 2.0, fmt)
        st = lib.qlora_forward(ctypes.byref(L), p, 0, p, p, None, 0, None)
        assert st == (C.QLORA_OK if ok else C.QLORA_EINVAL), fmt
    # 8-bit weights hold one byte per element: at most 2^30 elements
    L = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 1 << 16, 1 << 15, 16, 2.0, C.FMT_INT8)
    assert lib.qlora_forward(ctypes.byref(L), p, 4, p, p, None, 0, None) == C.QLORA_EINVAL
    L = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 1 << 16, 1 << 15, 16, 2.0, C.FMT_NF4)
    assert lib.qlora_forward(ctypes.byref(L), p, 0, p, p, None, 0, None) == C.QLORA_OK
    # the three layers of a SwiGLU block share one format
    g = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 256, 512, 16, 2.0, C.FMT_FP8)
    u = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 256, 512, 16, 2.0, C.FMT_FP8)
    d = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 512, 256, 16, 2.0, C.FMT_INT8)
    assert lib.swiglu_mlp_forward(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), p, 8, p, p, p, p, p,
                                  None, 0, None) == C.QLORA_EINVAL


def test_chunked_ce_argument_checks():
    lib = C.lib()
    p = ctypes.c_void_p(0x10000)
    need = lib.qlora_ce_workspace_size(100, 1024, 64)
    assert need >= 64 * 1024 * 6
    # a longer batch with the same chunk needs no more workspace
    assert lib.qlora_ce_workspace_size(1 << 20, 1024, 64) == need
    args = lambda M, H, V, chunk, ws, nb: (p, p, p, p, M, H, V, chunk, p, p, p, ws, nb, None)
    assert lib.qlora_chunked_ce(*args(100, 100, 1024, 64, p, need)) == C.QLORA_EINVAL   # H % 64
    assert lib.qlora_chunked_ce(*args(100, 128, 1000, 64, p, need)) == C.QLORA_EINVAL   # V % 64
    assert lib.qlora_chunked_ce(*args(100, 128, 1024, 0, p, need)) == C.QLORA_EINVAL    # chunk >= 1
    assert lib.qlora_chunked_ce(*args(100, 1 << 16, 1 << 16, 64, p, need)) == C.QLORA_EINVAL  # H*V too large
    assert lib.qlora_chunked_ce(*args(100, 128, 1024, 64, None, 0)) == C.QLORA_EWORKSPACE
    assert lib.qlora_chunked_ce(*args(100, 128, 1024, 64, p, need - 1)) == C.QLORA_EWORKSPACE
    assert lib.qlora_lmhead_prepare(p, 1024, 128, ctypes.c_void_p(0x10002), p, None) == C.QLORA_EINVAL
    assert lib.qlora_lmhead_prepare(p, 1000, 128, p, p, None) == C.QLORA_EINVAL  # V % 64


def test_tile_major_storage_order():
    from tests._util import tile_major
    # N = 66 rows (groups of 64 and 2), K = 128 (two blocks), one value per row and block
    N, nb = 66, 2
    a = np.arange(N * nb).reshape(N, nb)          # a[n, b] = 2n + b
    t = tile_major(a, 1).reshape(-1)
    # row 3, block 1: group 0 (64 rows) -> 1*64 + 3; row 65, block 1: group 64 (2 rows) -> 128 + 1*2 + 1
    assert t[67] == 2 * 3 + 1 and t[131] == 2 * 65 + 1 and t[0] == 0 and t[64] == 1
    assert sorted(t.tolist()) == list(range(N * nb))  # a permutation
    # codes: bb bytes per row and block move together
    c = np.arange(N * nb * 4).reshape(N, nb * 4)
    tc = tile_major(c, 4).reshape(-1)
    assert list(tc[4 * 67: 4 * 68]) == list(c[3, 4:8])


def test_nf4_run_byte_order():
    from tests._util import nf4_runs
    # one row, 16 columns with codes 0..15: the oracle packs bytes 0x10, 0x32, ...; the
    # library pairs column b with column b+4 inside each run of 8 columns
    packed = np.array([[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]], dtype=np.uint8)
    assert list(nf4_runs(packed)[0]) == [0x40, 0x51, 0x62, 0x73, 0xC8, 0xD9, 0xEA, 0xFB]


def _up256(x):
    return (x + 255) // 256 * 256


def _mlp_part_bytes(lib, M, H, I, r):
    """Bytes of the rank reductions' fp32 partials in the whole-batch SwiGLU backward
    workspace: its size minus the documented carve of the other intermediates
    (dg, du [M, I]; G_d [M, r]; G_gate|G_up [M, 2r]; three B^T copies)."""
    total = lib.qlora_workspace_size(C.OP_MLP_BACKWARD, M, H, I, r)
    rest = (2 * _up256(M * I * 2) + _up256(M * r * 2) + _up256(M * 2 * r * 2) + _up256(r * H * 2)
            + 2 * _up256(r * I * 2))
    return total - rest


@pytest.mark.parametrize("H,I", [(4096, 14336), (128, 256), (256, 512), (192, 320)])
def test_tiled_mlp_workspace_covers_every_tile(H, I):
    # the row-split count of a reduction is not monotone in its row count, so
    # the last (ragged) tile of a tiled backward can need more partials than a
    # full tile; the tiled workspace must hold what every tile of the batch needs
    lib = C.lib()
    for r in (1, 8, 16, 64):
        for tile in (256, 576, 1024, 4096):
            for M in (tile + 64, 1088, 1920, 2 * tile - 128, 3 * tile + 896, 16384):
                T = min(tile, M)
                sizes = {T, M - ((M - 1) // T) * T}
                overlap = M > T and -(-T // 256) * -(-H // 256) < 256
                fixed = ((7 if overlap else 5) * _up256(T * I * 2) + _up256(T * r * 2) + _up256(T * 2 * r * 2)
                         + _up256(r * H * 2) + 2 * _up256(r * I * 2))
                need = fixed + max(_mlp_part_bytes(lib, m, H, I, r) for m in sizes)
                got = lib.swiglu_mlp_tiled_workspace_size(1, M, H, I, r, tile)
                assert got >= need, (M, tile, r, H, I, got, need)


def test_pack_codes_argument_checks():
    lib = C.lib()
    p, q2 = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x900000)
    a, b = ctypes.c_void_p(0x2000000), ctypes.c_void_p(0x3000000)
    for fmt in (C.FMT_NF4, C.FMT_INT8, C.FMT_FP8):
        assert lib.qlora_pack_codes(fmt, p, a, 4, 100, q2, b, None) == C.QLORA_EINVAL     # K % 64
        assert lib.qlora_pack_codes(fmt, p, a, 0, 64, q2, b, None) == C.QLORA_OK         # empty: no launch
        assert lib.qlora_pack_codes(fmt, None, a, 4, 64, q2, b, None) == C.QLORA_EINVAL
        assert lib.qlora_pack_codes(fmt, ctypes.c_void_p(0x10004), a, 4, 64, q2, b, None) == C.QLORA_EINVAL
        # destinations must not overlap the sources
        assert lib.qlora_pack_codes(fmt, p, a, 4, 64, ctypes.c_void_p(0x10010), b, None) == C.QLORA_EINVAL
        assert lib.qlora_pack_codes(fmt, p, a, 4, 64, q2, a, None) == C.QLORA_EINVAL
    assert lib.qlora_pack_codes(3, p, a, 4, 64, q2, b, None) == C.QLORA_EINVAL


def test_gradient_dtype_field_checks():
    lib = C.lib()
    p = ctypes.c_void_p(0x10000)
    for gd, ok in ((C.GRAD_BF16, True), (C.GRAD_F32, True), (2, False), (-1, False)):
        L = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 512, 512, 16, 2.0, 0, gd)
        st = lib.qlora_forward(ctypes.byref(L), p, 0, p, p, None, 0, None)
        assert st == (C.QLORA_OK if ok else C.QLORA_EINVAL), gd
    # the three layers of a SwiGLU block share one gradient type
    g = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 256, 512, 16, 2.0, 0, C.GRAD_BF16)
    u = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 256, 512, 16, 2.0, 0, C.GRAD_BF16)
    d = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 512, 256, 16, 2.0, 0, C.GRAD_F32)
    assert lib.swiglu_mlp_forward(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), p, 8, p, p, p, p, p,
                                  None, 0, None) == C.QLORA_EINVAL
    assert lib.qlora_status_string(C.QLORA_ENONFINITE)


def test_noalloc_backward_rejects_workspaces_beyond_its_scratch():
    # the size check comes before any HIP call, so this runs without a GPU
    lib = C.lib()
    p = ctypes.c_void_p(0x10000)
    L = C.QLoraLayerC(0x10000, 0x10000, 0x10000, 0x10000, 4096, 4096, 128, 2.0, 0, 0)
    M = 1 << 20
    assert lib.qlora_workspace_size(C.OP_BACKWARD, M, 4096, 4096, 128) > C.NOALLOC_SCRATCH_BYTES
    assert lib.qlora_backward_noalloc(ctypes.byref(L), p, p, p, M, p, p, p, None) == C.QLORA_EWORKSPACE
    assert b"limit" in lib.qlora_last_error()
    assert lib.qlora_backward_noalloc(None, p, p, p, 4, p, p, p, None) == C.QLORA_EINVAL
    # the header's limit and the binding's constant agree
    text = open(HEADER).read()
    assert "#define QLORA_NOALLOC_SCRATCH_BYTES (64u << 20)" in text and C.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_autograd_wrappers_refuse_gradients_of_another_dtype_than_the_adapters():
    # checked on the host before any call into the library
    import torch
    import parameter_efficient_fine_amd as q
    K, N, r = 128, 64, 8
    L = q.QLoraLayer(torch.zeros((N, K // 2), dtype=torch.uint8), torch.zeros((N, K // 64)),
                     torch.zeros((r, K), dtype=torch.bfloat16), torch.zeros((N, r), dtype=torch.bfloat16), 2.0,
                     grad_dtype=torch.float32)
    X = torch.zeros((4, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        q.linear(X, L)
    with pytest.raises(ValueError):
        q.swiglu_mlp(X, L, L, L)
