"""The C-ABI library loads, exports every declared symbol and validates arguments (no GPU needed).

Only calls that must fail validation are made here: they return before any
HIP call, so no device is touched.
"""
import ctypes as C
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "ft_moe.h")


@pytest.fixture(scope="module")
def lib():
    from expert_cached_ffn_amd import _lib
    try:
        return _lib.lib()
    except _lib.LibraryMissing:
        pytest.fail("libftmoe.so is not built (python -m expert_cached_ffn_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ft_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    from expert_cached_ffn_amd import _lib
    assert sorted(_lib.EXPORTS) == names


def test_version(lib):
    from expert_cached_ffn_amd import ops
    assert "gfx950" in ops.version()


def test_layouts():
    from expert_cached_ffn_amd import ops
    L = ops.ft_expert_layout_init(2, 4096, 2048)   # MXFP4 decode-layer shape
    assert L.expert_bytes == 13_369_344
    assert (L.off_gate, L.off_up, L.off_down) == (0, 4_194_304, 8_388_608)
    assert (L.off_sgate, L.off_sup, L.off_sdown) == (12_582_912, 12_845_056, 13_107_200)
    L = ops.ft_expert_layout_init(1, 2048, 768)    # bf16 decode-layer shape
    assert L.expert_bytes == 9_437_184 and L.off_up == 3_145_728 and L.off_down == 6_291_456
    L = ops.ft_expert_layout_init(0, 256, 128)
    assert L.expert_bytes == 393_216
    L = ops.ft_expert_layout_init(3, 2048, 768)    # NVFP4 on the Qwen3-A3B shape
    assert (L.off_gate, L.off_up, L.off_down) == (0, 786_432, 1_572_864)
    assert (L.off_sgate, L.off_sup, L.off_sdown) == (2_359_296, 2_457_600, 2_555_904)  # K/16 scale bytes per row
    assert L.off_tscale == 2_654_208 and L.expert_bytes == 2_658_304
    assert ops.ft_expert_layout_init(2, 2048, 768).off_tscale == 0
    for bad in [(2, 100, 64), (7, 64, 64), (1, 0, 64), (3, 2040, 768)]:
        with pytest.raises(ops.FtError) as e:
            ops.ft_expert_layout_init(*bad)
        assert e.value.status == -1


def test_workspace_sizes():
    from expert_cached_ffn_amd import ops
    assert ops.ft_workspace_bytes(1, 64, 8, 128) == 0               # one-workgroup permutation
    assert ops.ft_workspace_bytes(1, 8192, 6, 256) == 48 * 256 * 4  # 48 blocks of 1024 rows
    assert ops.ft_workspace_bytes(2, 1, 6, 256, 4096, 2048) >= 7 * 2048 * 2
    assert ops.ft_workspace_bytes(9, 1, 1, 1, 1, 1) == 0


def _err(fn, *a, **kw):
    from expert_cached_ffn_amd import ops
    with pytest.raises(ops.FtError) as e:
        fn(*a, **kw)
    return e.value.status


def test_route_validation():
    from expert_cached_ffn_amd import ops
    f = ops.ft_moe_route
    assert _err(f, None, 1, None, None, 4, 64, 8, 9, 0, False, None, None, stream=0) == -2       # k > E
    assert _err(f, None, 1, None, None, 4, 64, 2048, 2, 0, False, None, None, stream=0) == -2    # E > 1024
    assert _err(f, None, 1, None, None, 4, 64, 8, 2, 5, False, None, None, stream=0) == -1       # gating
    assert _err(f, None, 1, None, None, 4, 64, 8, 2, 0, False, None, None, stream=0) == -1       # NULL outputs
    assert _err(f, 16, 1, 16, 16, 4, 100, 8, 2, 0, False, 16, 16, stream=0) == -2                # H % 128
    assert _err(f, 16, 3, 16, 16, 4, 128, 8, 2, 0, False, 16, 16, stream=0) == -1                # x dtype
    assert _err(f, None, 1, None, 8, 4, 0, 8, 2, 0, False, 16, 16, stream=0) == -1               # misaligned logits
    f(None, 1, None, None, 0, 0, 8, 2, 0, False, None, None, stream=0)                            # T = 0: no-op


def test_permute_validation():
    from expert_cached_ffn_amd import ops
    f = ops.ft_moe_permute
    assert _err(f, 16, 4, 2, 5000, 16, 16, 16, None, 0, stream=0) == -2      # E > 4096
    assert _err(f, 16, 4, 0, 8, 16, 16, 16, None, 0, stream=0) == -1         # k = 0
    assert _err(f, None, 4, 2, 8, 16, 16, 16, None, 0, stream=0) == -1       # NULL ids
    assert _err(f, 16, 8192, 6, 256, 16, 16, 16, None, 0, stream=0) == -1   # workspace missing


def test_ffn_validation():
    from expert_cached_ffn_amd import ops
    L4 = ops.ft_expert_layout_init(2, 4096, 2048)
    Lb = ops.ft_expert_layout_init(1, 384, 200)   # I not a multiple of 128
    f = ops.ft_moe_grouped_ffn
    ok = dict(workspace=256, workspace_bytes=1 << 30, stream=0)
    Lbf = ops.ft_expert_layout_init(1, 256, 256)
    assert _err(f, Lbf, 256, None, None, 256, 1, 1, 2, 2, 256, 256, 256, None, 1, **ok) == -2   # mode 1, bf16
    assert _err(f, L4, 256, None, None, 256, 1, 1, 6, 256, 256, 256, 256, None, 2, **ok) == -2   # mode 2
    assert _err(f, L4, 256, None, None, 256, 1, 1, 6, 256, 256, 256, 256, None, 0x400, **ok) == -1  # mode bits
    assert _err(f, L4, 256, None, None, 256, 0, 1, 6, 256, 256, 256, 256, None, 0, **ok) == -1   # x dtype
    assert _err(f, Lb, 256, None, None, 256, 1, 1, 2, 8, 256, 256, 256, None, 0, **ok) == -2     # I % 128
    assert _err(f, L4, 256, None, 256, 256, 1, 1, 6, 256, 256, 256, 256, None, 0, **ok) == -1    # shared w/o y_shared
    assert _err(f, L4, 255, None, None, 256, 1, 1, 6, 256, 256, 256, 256, None, 0, **ok) == -1   # pool alignment
    assert _err(f, L4, 256, None, None, 256, 1, 1, 6, 256, 256, 256, 256, None, 0,
                workspace=256, workspace_bytes=16, stream=0) == -1                                # workspace
    assert _err(f, L4, 256, None, None, 256, 1, 1, 7, 6, 256, 256, 256, None, 0, **ok) == -2     # k > E
    assert _err(f, L4, 256, None, None, 256, 1, 1, 6, 256, 256, 256, 256, None, 0, n_slots=255,
                **ok) == -1                                                # identity table, fewer slots than E
    assert _err(f, L4, 256, 256, None, 256, 1, 1, 6, 256, 256, 256, 256, None, 0, n_slots=0, **ok) == -1
    Lnv = ops.ft_expert_layout_init(3, 2048, 768)
    assert _err(f, Lnv, 256, None, None, 256, 1, 1, 8, 128, 256, 256, 256, None, 1, **ok) == -2  # mode 1, NVFP4
    assert _err(f, ops.ft_expert_layout_init(3, 2048, 784), 256, None, None, 256, 1, 1, 8, 128, 256, 256, 256,
                None, 0, **ok) == -2                                                              # NVFP4 I % 128


def test_mxfp8_quantize_validation():
    from expert_cached_ffn_amd import ops
    f = ops.ft_mxfp8_quantize
    assert _err(f, 16, 48, 2, 48, 16, 16, stream=0) == -1     # K % 32
    assert _err(f, 16, 16, 2, 32, 16, 16, stream=0) == -1     # ldx < K
    assert _err(f, 16, 36, 2, 32, 16, 16, stream=0) == -1     # ldx % 8
    assert _err(f, None, 32, 2, 32, 16, 16, stream=0) == -1   # NULL input
    f(None, 32, 0, 32, None, None, stream=0)                  # n = 0: no-op


def test_combine_validation():
    from expert_cached_ffn_amd import ops
    f = ops.ft_moe_combine
    assert _err(f, 16, 16, 16, None, 2, 65, 64, 1, 16, stream=0) == -2      # k > 64
    assert _err(f, 16, 16, 16, None, 2, 2, 66, 1, 16, stream=0) == -2       # H % 4
    assert _err(f, 16, 16, 16, None, 2, 2, 64, 3, 16, stream=0) == -1       # out dtype
    assert _err(f, 8, 16, 16, None, 2, 2, 64, 1, 16, stream=0) == -1        # misaligned y_rows


def test_read_checksum_validation():
    from expert_cached_ffn_amd import ops
    f = ops.ft_read_checksum
    assert _err(f, 16, 24, 16, stream=0) == -1                 # bytes not a multiple of 16
    assert _err(f, 16, 32, None, stream=0) == -1               # no sink
    assert _err(f, 16, 32, 18, stream=0) == -1                 # misaligned sink
    assert _err(f, 8, 32, 16, stream=0) == -1                  # misaligned buffer
    assert _err(f, None, 32, 16, stream=0) == -1               # no buffer
    assert _err(f, 16, (1 << 31) + 16, 16, stream=0) == -2     # above 2 GiB
    f(None, 0, 16, stream=0)                                   # nothing to read: FT_OK, nothing enqueued


def test_cache_validation():
    from expert_cached_ffn_amd import ops, _lib
    L = ops.ft_expert_layout_init(1, 128, 128)
    lib = _lib.lib()
    h = C.c_void_p()
    assert lib.ft_expert_cache_create(C.byref(L), 0, 8, 4, 256, 256, 1, C.byref(h)) == -1     # n_layers
    assert lib.ft_expert_cache_create(C.byref(L), 1, 8, 70000, 256, 256, 1, C.byref(h)) == -2  # capacity
    assert lib.ft_expert_cache_create(C.byref(L), 1, 8, 4, None, 256, 1, C.byref(h)) == -1     # NULL pool
    assert lib.ft_expert_cache_create(C.byref(L), 1, 8, 4, 256, 256, None, C.byref(h)) == -1   # NULL stream
    assert lib.ft_expert_cache_step(None, 0, None, 1, 1, None, None) == -1
    assert lib.ft_expert_cache_stats(None, None) == -1
    assert lib.ft_expert_cache_resize(None, 4, 256, None) == -1
    assert lib.ft_expert_cache_destroy(None) == 0
    assert b"NULL" in lib.ft_last_error() or lib.ft_last_error() == b""
