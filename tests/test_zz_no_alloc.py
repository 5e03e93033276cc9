"""The no-allocation grouped FFN (static device scratch) against the workspace entry point.

Two calls in a row on the same GPU, the second with a smaller input, each
compared with ft_moe_grouped_ffn on the same inputs (bit-identical outputs:
the same kernels run on the same operands); the stage-split form through the
static scratch; a size beyond the scratch refused with nothing written.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import moe
from tests.helpers import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from expert_cached_ffn_amd import ops as _ops
    _ops.version()
    return _ops


def _case(ops, cfg, T, seed):
    """Device inputs of one grouped-FFN call over resident experts (slot e = expert e)."""
    from expert_cached_ffn_amd.layer import DTYPES, pack_expert, to_device
    lay = ops.ft_expert_layout_init(DTYPES[cfg.wdtype], cfg.H, cfg.I)
    ids = synth.routing_ids_uniform(cfg, T, case=seed)
    off, rows, _ = moe.permute(ids, cfg.E)
    used = sorted(set(ids.ravel().tolist()))
    pool = np.zeros((cfg.E, int(lay.expert_bytes)), np.uint8)
    for e in used:
        pack_expert(lay, synth.expert_weights(cfg, 0, e).arrays, pool[e])
    x = synth.tokens(cfg, T, case=seed)
    shared = to_device(pack_expert(lay, synth.expert_weights(cfg, 0, cfg.E).arrays)) if cfg.shared else None
    return lay, to_device(pool), shared, to_device(x), to_device(off), to_device(rows), DTYPES[cfg.xdtype]


def _outputs(cfg, T):
    y = torch.full((T * cfg.k, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    ys = torch.full((T, cfg.H), float("nan"), dtype=torch.float32, device="cuda") if cfg.shared else None
    return y, ys


def _run_both(ops, cfg, T, seed, mode=0):
    lay, pool, shared, x, off, rows, xd = _case(ops, cfg, T, seed)
    ya, ysa = _outputs(cfg, T)
    yb, ysb = _outputs(cfg, T)
    wsb = ops.ft_workspace_bytes(2, T, cfg.k, cfg.E, cfg.H, cfg.I)
    ws = torch.empty(max(256, wsb), dtype=torch.uint8, device="cuda")
    ops.ft_moe_grouped_ffn(lay, pool, None, shared, x, xd, T, cfg.k, cfg.E, off, rows, ya, ysa, mode, ws, wsb)
    ops.ft_moe_grouped_ffn_noalloc(lay, pool, None, shared, x, xd, T, cfg.k, cfg.E, off, rows, yb, ysb, mode)
    torch.cuda.synchronize()
    return (ya, ysa), (yb, ysb), (lay, pool, shared, x, off, rows, xd)


def _same(a, b, what):
    assert torch.isfinite(b).all(), what
    assert torch.equal(a, b), what
    check_close(b.cpu().numpy(), a.cpu().numpy(), what=what)


CASES = [
    # name, config, overrides, (first T, second T), mode
    ("bf16-decode", 2, {}, (64, 5), 0),
    ("mxfp4-decode-shared", 3, {}, (32, 1), 0),
    ("mxfp4-native", 3, dict(E=32), (24, 8), 1),
    ("bf16-gemm-then-decode", 2, dict(E=16), (200, 3), 0),
]


@pytest.mark.parametrize("name,cfg_id,over,Ts,mode", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_call(ops, name, cfg_id, over, Ts, mode):
    cfg = synth.shrink(synth.CONFIGS[cfg_id], **over)
    for i, T in enumerate(Ts):                      # two calls in a row, the second smaller
        print(f"noalloc {name} call {i} T={T}", flush=True)
        (ya, ysa), (yb, ysb), _ = _run_both(ops, cfg, T, seed=10 + i, mode=mode)
        _same(ya, yb, f"{name} call {i} y_rows")
        if ysa is not None:
            _same(ysa, ysb, f"{name} call {i} y_shared")


def test_noalloc_stages_through_the_static_scratch(ops):
    """Gate/up alone then down alone through the static scratch equals the one-call result."""
    cfg = synth.CONFIGS[3]
    T = 8
    (ya, ysa), _, (lay, pool, shared, x, off, rows, xd) = _run_both(ops, cfg, T, seed=3)
    yb, ysb = _outputs(cfg, T)
    ops.ft_moe_grouped_ffn_noalloc(lay, pool, None, shared, x, xd, T, cfg.k, cfg.E, off, rows, yb, ysb, 0x100)
    ops.ft_moe_grouped_ffn_noalloc(lay, pool, None, shared, x, xd, T, cfg.k, cfg.E, off, rows, yb, ysb, 0x200)
    torch.cuda.synchronize()
    _same(ya, yb, "staged y_rows")
    _same(ysa, ysb, "staged y_shared")


def test_noalloc_refuses_sizes_beyond_the_scratch(ops):
    cfg = synth.CONFIGS[3]
    T = 1024
    need = ops.ft_workspace_bytes(2, T, cfg.k, cfg.E, cfg.H, cfg.I)
    assert need > ops.ft_noalloc_scratch_bytes()
    lay = ops.ft_expert_layout_init(2, cfg.H, cfg.I)
    y = torch.full((4, cfg.H), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ops.FtError) as e:
        ops.ft_moe_grouped_ffn_noalloc(lay, y, None, None, y, 1, T, cfg.k, cfg.E, y, y, y, None, 0, n_slots=cfg.E)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
