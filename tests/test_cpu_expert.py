"""The host CPU expert kernel (hybrid miss execution) against the oracle; runs without a GPU."""
import numpy as np
import pytest

import synth
from oracle import formats, moe
from tests.helpers import Experts, check_close


@pytest.fixture(scope="module")
def ops():
    from expert_cached_ffn_amd import ops as _ops
    _ops.version()
    yield _ops
    _ops.ft_cpu_isa(0)


def _isas():
    """The host kernel's instruction paths this CPU can run."""
    from expert_cached_ffn_amd import _lib
    out = []
    for isa in (_lib.FT_CPU_AVX2, _lib.FT_CPU_AVX512_BF16):
        from expert_cached_ffn_amd import ops as _ops
        try:
            cur = _ops.ft_cpu_isa(-1)
            _ops.ft_cpu_isa(isa)
            _ops.ft_cpu_isa(cur)
            out.append(isa)
        except _ops.FtError:
            pass
    return out


@pytest.fixture(params=["avx2", "avx512-bf16"])
def isa(ops, request):
    from expert_cached_ffn_amd import _lib
    want = {"avx2": _lib.FT_CPU_AVX2, "avx512-bf16": _lib.FT_CPU_AVX512_BF16}[request.param]
    try:
        ops.ft_cpu_isa(want)
    except ops.FtError:
        pytest.skip(f"host CPU lacks {request.param}")
    yield want
    ops.ft_cpu_isa(0)


CASES = [
    ("mxfp4-small", 3, dict(H=512, I=256, E=2, k=1), 1),
    ("mxfp4-three-tokens", 3, dict(H=1024, I=512, E=2, k=1), 3),
    ("mxfp4-two-passes", 3, dict(H=512, I=768, E=2, k=1), 11),
    ("bf16-small", 2, dict(H=256, I=384, E=2, k=1), 5),
    ("mxfp4-full-expert", 3, {}, 2),
]


@pytest.mark.parametrize("name,cfg_id,over,n", CASES, ids=[c[0] for c in CASES])
def test_cpu_expert_matches_oracle(ops, isa, name, cfg_id, over, n):
    from expert_cached_ffn_amd.layer import DTYPES, pack_expert
    cfg = synth.shrink(synth.CONFIGS[cfg_id], **over)
    ex = Experts(cfg)
    lay = ops.ft_expert_layout_init(DTYPES[cfg.wdtype], cfg.H, cfg.I)
    blob = pack_expert(lay, ex.raw(1).arrays)
    x = synth.tokens(cfg, n)
    y = np.full((n, cfg.H), np.nan, np.float32)
    ops.ft_cpu_expert_ffn(lay, blob, np.ascontiguousarray(x), n, y, 4)
    ref = moe.swiglu_expert(formats.activations_to_f64(cfg.xdtype, x), *ex.f64(1))
    check_close(y, ref, what=name)
    # the thread count changes nothing (each output is one fixed-order sum)
    y1 = np.empty_like(y)
    ops.ft_cpu_expert_ffn(lay, blob, np.ascontiguousarray(x), n, y1, 1)
    assert np.array_equal(y, y1)


def test_cpu_expert_validation(ops):
    from expert_cached_ffn_amd.layer import DTYPES
    for wd in ("f32", "nvfp4"):
        lay = ops.ft_expert_layout_init(DTYPES[wd], 256, 128)
        with pytest.raises(ops.FtError) as e:
            ops.ft_cpu_expert_ffn(lay, np.zeros(8, np.uint8), np.zeros(8, np.uint16), 1, np.zeros(8, np.float32))
        assert e.value.status == -2
    lay = ops.ft_expert_layout_init(DTYPES["mxfp4"], 512, 256)
    with pytest.raises(ops.FtError) as e:
        ops.ft_cpu_expert_ffn(lay, None, np.zeros(8, np.uint16), 1, np.zeros(8, np.float32))
    assert e.value.status == -1
    ops.ft_cpu_expert_ffn(lay, None, None, 0, None)  # n = 0: nothing to do


@pytest.mark.parametrize("T,k", [(1, 6), (5, 2), (12, 3)])
def test_cpu_miss_rows_against_oracle(ops, isa, T, k):
    """A step's CPU misses of layer 1 in a two-layer host bank: their permuted rows, nothing else."""
    from expert_cached_ffn_amd.layer import DTYPES, pack_expert
    E, n_layers, layer = 8, 2, 1
    cfg = synth.shrink(synth.CONFIGS[3], H=512, I=256, E=E, k=k)
    ex = Experts(cfg, layer=layer)
    lay = ops.ft_expert_layout_init(DTYPES[cfg.wdtype], cfg.H, cfg.I)
    eb = int(lay.expert_bytes)
    bank = np.zeros((n_layers * E, eb), np.uint8)
    for e in range(E):
        pack_expert(lay, ex.raw(e).arrays, bank[layer * E + e])
    rng = np.random.default_rng(T * 10 + k)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    offsets, sorted_rows, _ = moe.permute(ids, E)
    x = synth.tokens(cfg, T)
    cpu = np.array(sorted(rng.choice(np.unique(ids), size=min(3, len(np.unique(ids))), replace=False)), np.int32)
    y = np.full((T * k, cfg.H), np.nan, np.float32)
    ops.ft_cpu_miss_rows(lay, bank, layer, E, cpu, cpu.size, offsets, sorted_rows, T, k,
                         np.ascontiguousarray(x), y, 3)
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    mine = np.zeros(T * k, bool)
    for e in cpu:
        a, b = int(offsets[e]), int(offsets[e + 1])
        mine[a:b] = True
        ref = moe.swiglu_expert(x64[sorted_rows[a:b] // k], *ex.f64(int(e)))
        check_close(y[a:b], ref, what=f"expert {e}")
    assert np.isnan(y[~mine]).all()


def test_cpu_miss_rows_validation(ops):
    from expert_cached_ffn_amd.layer import DTYPES
    lay = ops.ft_expert_layout_init(DTYPES["mxfp4"], 512, 256)
    off = np.array([0, 1, 2], np.int32)
    rows = np.array([0, 1], np.int32)
    x = np.zeros((2, 512), np.uint16)
    y = np.zeros((2, 512), np.float32)
    bank = np.zeros((2, int(lay.expert_bytes)), np.uint8)
    for experts, offs, srows in [([2], off, rows), ([0], np.array([0, 1, 3], np.int32), rows),
                                 ([1], off, np.array([0, 5], np.int32))]:
        with pytest.raises(ops.FtError) as e:
            ops.ft_cpu_miss_rows(lay, bank, 0, 2, np.array(experts, np.int32), 1, offs, srows, 2, 1, x, y)
        assert e.value.status == -1
    assert (y == 0).all()


def test_isa_selection(ops):
    from expert_cached_ffn_amd import _lib
    best = ops.ft_cpu_isa(_lib.FT_CPU_ISA_BEST)
    assert best in (_lib.FT_CPU_AVX2, _lib.FT_CPU_AVX512_BF16)
    assert ops.ft_cpu_isa(_lib.FT_CPU_ISA_QUERY) == best
    with pytest.raises(ops.FtError) as e:
        ops.ft_cpu_isa(7)
    assert e.value.status == -1
    assert ops.ft_cpu_isa(_lib.FT_CPU_ISA_QUERY) == best


def test_isa_paths_agree(ops):
    """Both paths compute the same products; only the order of fp32 additions differs."""
    from expert_cached_ffn_amd import _lib
    from expert_cached_ffn_amd.layer import DTYPES, pack_expert
    paths = _isas()
    if len(paths) < 2:
        pytest.skip("one instruction path on this host")
    cfg = synth.shrink(synth.CONFIGS[3], H=1024, I=512, E=2, k=1)
    ex = Experts(cfg)
    lay = ops.ft_expert_layout_init(DTYPES[cfg.wdtype], cfg.H, cfg.I)
    blob = pack_expert(lay, ex.raw(0).arrays)
    x = np.ascontiguousarray(synth.tokens(cfg, 3))
    ys = []
    for p in paths:
        ops.ft_cpu_isa(p)
        y = np.empty((3, cfg.H), np.float32)
        ops.ft_cpu_expert_ffn(lay, blob, x, 3, y, 2)
        ys.append(y)
    ops.ft_cpu_isa(_lib.FT_CPU_ISA_BEST)
    scale = np.abs(ys[0]).max()
    assert np.abs(ys[0] - ys[1]).max() <= 1e-3 * scale
