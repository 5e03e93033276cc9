"""Per-call parity of the HIP path against the oracle (route, permute, grouped FFN, combine)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import formats, moe
from tests.helpers import Experts, check_close, route_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from expert_cached_ffn_amd import ops as _ops
    _ops.version()  # loads the library or raises
    return _ops


def dev(a):
    from expert_cached_ffn_amd.layer import to_device
    return to_device(a)


def x_dtype(cfg):
    from expert_cached_ffn_amd.layer import DTYPES
    return DTYPES[cfg.xdtype]


# ----------------------------------------------------------------------------- route

ROUTE_CASES = [(1, 8), (2, 1), (2, 16), (2, 64), (3, 1), (3, 8), (3, 32), (3, 100)]


@pytest.mark.parametrize("cfg_id,T", ROUTE_CASES)
def test_route_with_router_gemv(ops, cfg_id, T):
    from expert_cached_ffn_amd.layer import GATING
    cfg = synth.CONFIGS[cfg_id]
    print(f"route cfg{cfg_id} T={T}", flush=True)
    x = synth.tokens(cfg, T)
    wr = synth.router_weight(cfg)
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    wr64 = formats.activations_to_f64(cfg.xdtype, wr)
    l_ref, ids_ref, w_ref, margin = route_oracle(cfg, x64, wr64)
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    ops.ft_moe_route(dev(x), x_dtype(cfg), dev(wr), logits, T, cfg.H, cfg.E, cfg.k, GATING[cfg.gating],
                     cfg.renormalize, ids, w)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy().astype(np.float64)
    scale = np.abs(x64) @ np.abs(wr64).T
    assert np.all(np.abs(lg - l_ref) <= 3e-5 * scale + 1e-6)
    sure = margin > 1e-4
    assert sure.mean() > 0.9
    got_ids = ids.cpu().numpy()
    assert np.array_equal(got_ids[sure], ids_ref[sure])
    w_at = moe.gating_weights(l_ref, got_ids, cfg.gating, cfg.renormalize)
    np.testing.assert_allclose(w.cpu().numpy()[sure], w_at[sure], rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("gating,renorm,E,k,T", [("sigmoid", False, 256, 6, 8192), ("softmax", True, 128, 8, 333),
                                                  ("softmax", False, 16, 16, 9), ("sigmoid", True, 1000, 40, 17),
                                                  ("softmax", False, 1, 1, 3), ("sigmoid", False, 130, 65, 5)])
def test_route_given_logits_bit_exact_ids(ops, gating, renorm, E, k, T):
    from expert_cached_ffn_amd.layer import GATING
    print(f"route-given {gating} E={E} k={k} T={T}", flush=True)
    if E == 256:
        logits = synth.prefill_logits(synth.CONFIGS[4], T)
    else:
        rng = np.random.default_rng(E * 1000 + k)
        logits = rng.standard_normal((T, E)).astype(np.float32)
        # exact ties and signed zeros
        logits[0, :] = 0.0
        logits[0, ::2] = -0.0
        if T > 1:
            logits[1, :] = np.round(logits[1, :])
    ids_ref = moe.topk(logits, k)
    w_ref = moe.gating_weights(logits, ids_ref, gating, renorm)
    lt = dev(logits)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ops.ft_moe_route(None, 0, None, lt, T, 0, E, k, GATING[gating], renorm, ids, w)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=2e-6, atol=1e-7)


# ----------------------------------------------------------------------------- permute

@pytest.mark.parametrize("T,k,E,kind", [(1, 8, 128, "u"), (16, 8, 128, "u"), (64, 8, 128, "u"), (5, 2, 16, "u"),
                                        (300, 6, 256, "u"), (2048, 6, 256, "zipf"), (8192, 6, 256, "zipf"),
                                        (3000, 3, 4096, "u"), (1, 1, 1, "u"), (0, 4, 8, "u")])
def test_permute_bit_exact(ops, T, k, E, kind):
    print(f"permute T={T} k={k} E={E} {kind}", flush=True)
    if kind == "zipf":
        ids = moe.topk(synth.prefill_logits(synth.CONFIGS[4], T), k).astype(np.int32)
    else:
        rng = np.random.default_rng(T * 7 + E)
        ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], np.int32).reshape(T, k)
    off_ref, rows_ref, pos_ref = moe.permute(ids, E)
    n = max(1, T * k)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    rows = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    pos = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    wsb = ops.ft_workspace_bytes(1, T, k, E)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    ids_d = dev(ids.reshape(-1)) if T else torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.ft_moe_permute(ids_d, T, k, E, off, rows, pos, ws, wsb)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), off_ref)
    if T:
        assert np.array_equal(rows.cpu().numpy(), rows_ref)
        assert np.array_equal(pos.cpu().numpy(), pos_ref)


# ----------------------------------------------------------------------------- grouped FFN

def _ffn_case(ops, cfg, T, ids, shuffle_slots=True, with_shared=None, missing=None):
    """Run the GPU grouped FFN on oracle permutation data; return (gpu y_rows, y_shared, oracle ...)."""
    from expert_cached_ffn_amd.layer import DTYPES, pack_expert
    with_shared = cfg.shared if with_shared is None else with_shared
    ex = Experts(cfg)
    lay = ops.ft_expert_layout_init(DTYPES[cfg.wdtype], cfg.H, cfg.I)
    off, rows, pos = moe.permute(ids, cfg.E)
    used = sorted(set(ids.ravel().tolist()))
    rng = np.random.default_rng(99)
    n_slots = len(used) + 3
    slot_ids = rng.permutation(n_slots)[:len(used)] if shuffle_slots else np.arange(len(used))
    slot_of = np.full(cfg.E, -1, np.int32)
    pool = np.zeros((n_slots, int(lay.expert_bytes)), np.uint8)
    for e, s in zip(used, slot_ids):
        slot_of[e] = s
        pack_expert(lay, ex.raw(e).arrays, pool[s])
    if missing is not None:
        slot_of[missing] = -1
    x = synth.tokens(cfg, T)
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    shared_blob = None
    if with_shared:
        shared_blob = dev(pack_expert(lay, ex.raw(cfg.E).arrays))
    R = T * cfg.k
    y = torch.full((R, cfg.H), np.nan, dtype=torch.float32, device="cuda")
    ys = torch.full((T, cfg.H), np.nan, dtype=torch.float32, device="cuda") if with_shared else None
    wsb = ops.ft_workspace_bytes(2, T, cfg.k, cfg.E, cfg.H, cfg.I)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ops.ft_moe_grouped_ffn(lay, dev(pool), dev(slot_of), shared_blob, dev(x), DTYPES[cfg.xdtype], T, cfg.k,
                           cfg.E, dev(off), dev(rows), y, ys, 0, ws, wsb)
    torch.cuda.synchronize()
    y_ref = moe.grouped_ffn(x64, cfg.k, off, rows, ex.f64)
    ys_ref = moe.swiglu_expert(x64, *ex.f64(cfg.E)) if with_shared else None
    return y.cpu().numpy(), (ys.cpu().numpy() if with_shared else None), y_ref, ys_ref, off


FFN_CASES = [
    # name, cfg overrides, T
    ("f32-cfg1", 1, {}, 8),
    ("bf16-small-ragged", 2, dict(H=384, I=256, E=8, k=2), 5),
    ("bf16-two-col-tiles", 2, dict(H=256, I=384, E=4, k=2), 23),
    ("bf16-cfg2-T16", 2, {}, 16),
    ("fp4-small", 3, dict(H=1024, I=512, E=6, k=2), 37),
    ("fp4-long-segment", 3, dict(H=512, I=1024, E=2, k=1), 150),
    ("fp4-cfg3-T1", 3, {}, 1),
]


@pytest.mark.parametrize("name,cfg_id,over,T", FFN_CASES, ids=[c[0] for c in FFN_CASES])
def test_grouped_ffn_parity(ops, name, cfg_id, over, T):
    print(f"ffn {name}", flush=True)
    cfg = synth.shrink(synth.CONFIGS[cfg_id], **over)
    ids = synth.routing_ids_uniform(cfg, T)
    y, ys, y_ref, ys_ref, _ = _ffn_case(ops, cfg, T, ids)
    check_close(y, y_ref, what=f"{name} y_rows")
    if ys_ref is not None:
        check_close(ys, ys_ref, what=f"{name} y_shared")


def test_grouped_ffn_missing_slot_gives_nan(ops):
    cfg = synth.shrink(synth.CONFIGS[3], H=512, I=512, E=4, k=1, shared=False)
    ids = np.array([[0], [1], [2], [1]], np.int32)
    y, _, y_ref, _, off = _ffn_case(ops, cfg, 4, ids, missing=1)
    a, b = int(off[1]), int(off[2])
    assert np.all(np.isnan(y[a:b]))
    keep = np.r_[0:a, b:len(y)]
    check_close(y[keep], y_ref[keep], what="other experts")


# ----------------------------------------------------------------------------- combine

@pytest.mark.parametrize("T,k,H,shared,bf16", [(1, 8, 2048, False, True), (33, 6, 4096, True, True),
                                               (8, 2, 256, False, False), (5, 3, 12, True, False)])
def test_combine_parity(ops, T, k, H, shared, bf16):
    rng = np.random.default_rng(T + k + H)
    R = T * k
    y_rows = rng.standard_normal((R, H)).astype(np.float32) * 50
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    row_pos = rng.permutation(R).astype(np.int32)
    ysh = rng.standard_normal((T, H)).astype(np.float32) if shared else None
    ref = moe.combine(y_rows, w, row_pos, ysh, T, k)
    out = torch.empty((T, H), dtype=torch.int16 if bf16 else torch.float32, device="cuda")
    ops.ft_moe_combine(dev(y_rows), dev(w), dev(row_pos), dev(ysh) if shared else None, T, k, H,
                       1 if bf16 else 0, out)
    torch.cuda.synchronize()
    if bf16:
        got = formats.bf16_to_f64(out.cpu().numpy().view(np.uint16))
        # fp32 sum then one rounding to nearest even
        assert np.all(np.abs(got - ref) <= 2 * 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())
        check_close(got, ref, bf16_out=True, what="combine bf16")
    else:
        got = out.cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
