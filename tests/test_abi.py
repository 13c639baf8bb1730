"""Host-side checks of the C ABI: the library loads, exports every entry point
include/i8mm.h declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "i8mm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def L():
    ensure_built()
    from int8_mixed_precision_detect_amd._lib import lib
    return lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("int8_quantize_weight", "int8_linear_forward", "int8_linear_workspace_size",
                     "int8_linear_status", "int8_find_outliers", "int8_quantize_rows",
                     "int8_outlier_weights", "int8_gemm_s32"):
        assert required in names


def test_every_declared_symbol_is_exported(L):
    from int8_mixed_precision_detect_amd._lib import SIGNATURES
    names = declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(L, n), f"libi8mm.so does not export {n}"
        assert n in SIGNATURES, f"binding has no signature for {n}"


def test_abi_version_and_status_strings(L):
    assert L.i8mm_abi_version() == 9
    for code, name in [(0, b"I8MM_OK"), (1, b"I8MM_ERR_INVALID_ARG"), (2, b"I8MM_ERR_WORKSPACE"),
                       (3, b"I8MM_ERR_UNSUPPORTED"), (4, b"I8MM_ERR_HIP"),
                       (5, b"I8MM_ERR_OUTLIER_OVERFLOW")]:
        assert L.i8mm_status_string(code) == name


def test_workspace_layout(L):
    from int8_mixed_precision_detect_amd._lib import WsLayout
    for T, N, K, mo in [(16, 64, 64, 64), (2048, 20480, 5120, 5120), (1, 49152, 12288, 12288),
                        (7, 5, 3, 0), (0, 4, 8, 8)]:
        lay = WsLayout()
        assert L.int8_linear_workspace_layout(T, N, K, mo, ctypes.byref(lay)) == 0
        assert lay.splits == 1  # these shapes fill the GPU without splitting K
        # counts and mask first, at fixed offsets (the mask region holds
        # the largest K's mask)
        assert lay.counts == 0 and lay.mask == 256
        regions = [("counts", 16), ("mask", (1 << 18) // 8), ("outliers", max(mo, 1) * 4),
                   ("sx", T * 4), ("xq", T * lay.ldq), ("xo", T * lay.ldo * 2),
                   ("wo", N * lay.ldo * 2), ("zp", max(T, 1) * 4), ("osum", max(N, 1) * 4),
                   ("part", 0)]
        end = 0
        for name, size in regions:
            off = getattr(lay, name)
            assert off % 256 == 0, name
            assert off >= end, name
            end = off + size
        assert lay.total >= end
        assert lay.ldq % 64 == 0 and lay.ldq >= K
        assert lay.ldo % 32 == 0 and lay.ldo >= mo
        assert L.int8_linear_workspace_size(T, N, K, mo) == lay.total


def test_split_k_layout(L):
    # K-heavy down projection (13B: 5120 x 2048 outputs, K = 20480): 128
    # output tiles of 320 x 256 cannot fill 256 compute units, so K is split
    # in two; the workspace gains one int32 partial tile per split and tile.
    # (Without a GPU the planner assumes 256 compute units.)
    from int8_mixed_precision_detect_amd._lib import WsLayout
    T, N, K = 2048, 5120, 20480
    lay = WsLayout()
    assert L.int8_linear_workspace_layout(T, N, K, K, ctypes.byref(lay)) == 0
    assert lay.splits == 2
    tiles = (N // 320) * (T // 256)
    assert lay.total - lay.part >= 2 * tiles * 320 * 256 * 4
    assert lay.part >= lay.osum + N * 4 and lay.osum >= lay.zp + T * 4 >= lay.wo + N * lay.ldo * 2
    # the override: clamped to 4, 0 restores the planner's choice
    try:
        for want, got in [(1, 1), (3, 3), (9, 4)]:
            assert L.i8mm_set_split_override(want) == 0
            assert L.int8_linear_workspace_layout(T, N, K, K, ctypes.byref(lay)) == 0
            assert lay.splits == got
            assert (lay.total - lay.part > 0) == (got > 1)
        assert L.i8mm_set_split_override(-1) == 1
    finally:
        assert L.i8mm_set_split_override(0) == 0
    assert L.int8_linear_workspace_layout(T, N, K, K, ctypes.byref(lay)) == 0
    assert lay.splits == 2


@pytest.mark.parametrize("T,N,K,splits", [
    (2048, 20480, 5120, 1),   # 13B first FF layer: 512 tiles, two full rounds
    (2048, 5120, 5120, 1),    # attention projection: 256 tiles of 320 x 128, one round
    (2048, 16384, 4096, 1),   # 6.7B first FF layer
    (1024, 5120, 5120, 2),
    (256, 5120, 20480, 4),    # K-heavy, few tokens: 20 tiles
    (128, 5120, 5120, 3),     # (two splits measured 3 % faster)
    (512, 4096, 4096, 3),     # LLaMA-like widths (two splits measured 7 % faster)
    (1024, 5120, 20480, 2),   # K-heavy, 1024 tokens: two splits fastest
    (2048, 11008, 4096, 1),
])
def test_planner_choices(L, T, N, K, splits):
    # the split counts the planner's duration model picks for 256 compute
    # units (the fastest measured on MI355X for these shapes, but where a
    # comment gives the measured gap)
    from int8_mixed_precision_detect_amd._lib import WsLayout
    lay = WsLayout()
    assert L.int8_linear_workspace_layout(T, N, K, K, ctypes.byref(lay)) == 0
    assert lay.splits == splits


def test_tile_override_layout(L):
    # the override picks the tile of the product (partial tiles of a forced
    # split show its size); -1 restores the plan, out-of-range values fail
    from int8_mixed_precision_detect_amd._lib import WsLayout
    T, N, K = 2048, 5120, 5120
    lay = WsLayout()
    try:
        assert L.i8mm_set_split_override(2) == 0
        for cfg, bm, bn in [(0, 320, 256), (1, 256, 256), (2, 192, 256), (3, 320, 128)]:
            assert L.i8mm_set_tile_override(cfg) == 0
            assert L.int8_linear_workspace_layout(T, N, K, K, ctypes.byref(lay)) == 0
            tiles = -(-N // bm) * (T // bn)
            assert lay.total - lay.part == 2 * tiles * bm * bn * 4
        for bad in (-2, 4):
            assert L.i8mm_set_tile_override(bad) == 1
    finally:
        assert L.i8mm_set_tile_override(-1) == 0
        assert L.i8mm_set_split_override(0) == 0
    assert L.int8_linear_workspace_layout(T, N, K, K, ctypes.byref(lay)) == 0
    assert lay.splits == 1 and lay.total == lay.part


def test_invalid_arguments_are_rejected_on_the_host(L):
    nan = float("nan")
    fwd = L.int8_linear_forward
    # threshold NaN / <= 0
    for thr in (nan, 0.0, -1.0):
        assert fwd(None, 4, 8, None, None, 4, None, thr, None, None, 0, 8, None) == 1
    # negative sizes, max_outliers outside [0, K]
    assert fwd(None, -1, 8, None, None, 4, None, 6.0, None, None, 0, 8, None) == 1
    assert fwd(None, 4, 8, None, None, 4, None, 6.0, None, None, 0, 9, None) == 1
    assert fwd(None, 4, 8, None, None, 4, None, 6.0, None, None, 0, -1, None) == 1
    # empty problems are no-ops
    assert fwd(None, 0, 8, None, None, 4, None, 6.0, None, None, 0, 8, None) == 0
    assert fwd(None, 4, 8, None, None, 0, None, 6.0, None, None, 0, 8, None) == 0
    # null outputs / workspace
    assert fwd(1 << 20, 4, 8, 1 << 20, 1 << 20, 4, None, 6.0, None, None, 0, 8, None) == 1
    # workspace too small (checked before any launch)
    need = L.int8_linear_workspace_size(4, 4, 8, 8)
    assert fwd(1 << 20, 4, 8, 1 << 20, 1 << 20, 4, None, 6.0, 1 << 20, 1 << 24, need - 1, 8,
               None) == 2
    # misaligned workspace
    assert fwd(1 << 20, 4, 8, 1 << 20, 1 << 20, 4, None, 6.0, 1 << 20, (1 << 24) + 8, need, 8,
               None) == 1
    # the allocation-free forward: the same host checks, and a layout beyond
    # its scratch array is refused before any HIP call
    na = L.int8_linear_forward_noalloc
    assert na(None, 4, 8, None, None, 4, None, 6.0, None, 9, None, None) == 1
    assert na(None, 0, 8, None, None, 4, None, 6.0, None, 8, None, None) == 0
    assert na(1 << 20, 2048, 5120, 1 << 20, 1 << 20, 20480, None, 6.0, 1 << 20, 5120, None,
              None) == 2
    assert na(1 << 20, 4, 8, 1 << 20, 1 << 20, 4, None, 6.0, 1 << 20, 8, (1 << 20) + 2,
              None) == 1  # status not 4-byte aligned
    # too-large K for the LDS mask copy
    assert L.int8_linear_workspace_size(4, 4, (1 << 18) + 1, 0) == 0
    q = L.int8_quantize_weight
    assert q(None, -1, 4, None, None, None) == 1
    assert q(None, 0, 4, None, None, None) == 0
    assert L.int8_gemm_s32(None, 3, None, 4, None, 2, 2, 4, None) == 1   # lda < K
    assert L.int8_find_outliers(None, 4, 8, nan, None, None, None, 8, None) == 1
    assert L.int8_find_outliers(1 << 20, 4, 8, 6.0, None, 1 << 20, 1 << 20, 8, None) == 1
    assert L.int8_quantize_rows(1 << 20, 4, 8, 1 << 20, 8, 1 << 20, 8, 1 << 20, 1 << 20, 32,
                                None) == 1  # ldq % 16 != 0
    assert L.int8_outlier_weights(1 << 20, 1 << 20, 4, 8, 1 << 20, 8, 1 << 20, 16,
                                  None) == 1  # ldo % 32 != 0


def test_python_binding_refuses_cpu_tensors():
    import torch
    import int8_mixed_precision_detect_amd as i8
    with pytest.raises(ValueError):
        i8.quantize_weight(torch.zeros((4, 4), dtype=torch.float16))
    with pytest.raises(TypeError):
        i8.quantize_weight(torch.zeros((4, 4), dtype=torch.float32))
