"""Per-call parity of the HIP path against the oracle (route, permute, grouped FFN, combine)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import formats, moe
from tests.helpers import Experts, check_close, check_topk_valid, route_oracle

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

ROUTE_CASES = [(1, 8), (2, 1), (2, 3), (2, 16), (2, 64), (3, 1), (3, 2), (3, 3), (3, 4), (3, 5), (3, 8), (3, 32), (3, 100)]


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
    assert np.array_equal(got_ids, moe.topk(lg.astype(np.float32), cfg.k))   # exact on its own logits
    assert np.array_equal(got_ids[sure], ids_ref[sure])
    differ = check_topk_valid(got_ids, l_ref, cfg.k, what=f"cfg{cfg_id} T={T}")   # near ties: a valid top-k
    assert set(differ.tolist()) <= set(np.flatnonzero(~sure).tolist())
    w_at = moe.gating_weights(l_ref, got_ids, cfg.gating, cfg.renormalize)
    np.testing.assert_allclose(w.cpu().numpy(), w_at, rtol=1e-4, atol=1e-6)


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


# ----------------------------------------------------------------------------- route + permute, one call

def _check_permutation(ids, off, rows, pos, E, ids_ref=None):
    """Bit-exact against the oracle's permutation when the ids agree, else the
    defining properties of a stable counting sort of the GPU's own ids."""
    ids = np.asarray(ids)
    if ids_ref is not None and np.array_equal(ids, ids_ref):
        o, r, p = moe.permute(ids_ref, E)
        assert np.array_equal(off, o) and np.array_equal(rows, r) and np.array_equal(pos, p)
        return
    flat = ids.ravel()
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
    assert np.array_equal(np.sort(rows), np.arange(flat.size))
    assert np.array_equal(pos[rows], np.arange(flat.size))
    for e in range(E):
        seg = rows[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def _route_permute(ops, cfg, T, x=None, wr=None, logits=None, ws=None):
    from expert_cached_ffn_amd.layer import GATING
    E, k = cfg.E, cfg.k
    lg = dev(logits) if logits is not None else torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    rows = torch.empty(max(1, T * k), dtype=torch.int32, device="cuda")
    pos = torch.empty(max(1, T * k), dtype=torch.int32, device="cuda")
    wsb = ops.ft_workspace_bytes(3, T, k, E)
    if ws is None:
        ws = torch.zeros(max(256, wsb), dtype=torch.uint8, device="cuda")
    ops.ft_moe_route_permute(None if x is None else dev(x), x_dtype(cfg), None if wr is None else dev(wr), lg,
                             T, cfg.H, E, k, GATING[cfg.gating], cfg.renormalize, ids, w, off, rows, pos, ws, wsb)
    torch.cuda.synchronize()
    return (lg.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), off.cpu().numpy(), rows.cpu().numpy()[:T * k],
            pos.cpu().numpy()[:T * k], ws)


@pytest.mark.parametrize("cfg_id,T", [(2, 1), (2, 16), (2, 64), (3, 1), (3, 8), (3, 32), (3, 100), (2, 65)])
def test_route_permute_with_router(ops, cfg_id, T):
    """Router + one routing launch up to 64 tokens, the two calls above."""
    cfg = synth.CONFIGS[cfg_id]
    print(f"route+permute cfg{cfg_id} T={T}", flush=True)
    ws = None
    for rep in range(3):  # back to back on one workspace
        x = synth.tokens(cfg, T, case=rep)
        wr = synth.router_weight(cfg)
        x64 = formats.activations_to_f64(cfg.xdtype, x)
        wr64 = formats.activations_to_f64(cfg.xdtype, wr)
        l_ref, ids_ref, w_ref, margin = route_oracle(cfg, x64, wr64)
        lg, ids, w, off, rows, pos, ws = _route_permute(ops, cfg, T, x=x, wr=wr, ws=ws)
        scale = np.abs(x64) @ np.abs(wr64).T
        assert np.all(np.abs(lg - l_ref) <= 3e-5 * scale + 1e-6)
        sure = margin > 1e-4
        assert np.array_equal(ids, moe.topk(lg.astype(np.float32), cfg.k))
        assert np.array_equal(ids[sure], ids_ref[sure])
        differ = check_topk_valid(ids, l_ref, cfg.k, what=f"cfg{cfg_id} T={T} rep {rep}")
        assert set(differ.tolist()) <= set(np.flatnonzero(~sure).tolist())
        w_at = moe.gating_weights(l_ref, ids, cfg.gating, cfg.renormalize)
        np.testing.assert_allclose(w, w_at, rtol=1e-4, atol=1e-6)
        _check_permutation(ids, off, rows, pos, cfg.E, ids_ref)


@pytest.mark.parametrize("E,k,T", [(128, 8, 1), (256, 6, 64), (16, 16, 9), (1000, 2, 33), (256, 6, 300),
                                   (16, 16, 4), (1000, 2, 16), (256, 6, 10),
                                   # the one-workgroup tail's chunk sort at its 1024-row limit, one past it
                                   # (block sort), and 64 one-pick tokens (16 waves of 4 tokens, wave sort)
                                   (256, 16, 64), (64, 17, 64), (128, 1, 64),
                                   (1024, 4, 16), (1024, 3, 40)])   # the routing kernels' 1024-expert limit
def test_route_permute_given_logits_bit_exact(ops, E, k, T):
    cfg = synth.shrink(synth.CONFIGS[3], E=E, k=k, shared=False)
    rng = np.random.default_rng(E + k + T)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, :] = 0.0
    logits[0, ::3] = -0.0
    ids_ref = moe.topk(logits, k)
    w_ref = moe.gating_weights(logits, ids_ref, cfg.gating, cfg.renormalize)
    _, ids, w, off, rows, pos, _ = _route_permute(ops, cfg, T, logits=logits)
    assert np.array_equal(ids, ids_ref)
    np.testing.assert_allclose(w, w_ref, rtol=2e-6, atol=1e-7)
    _check_permutation(ids, off, rows, pos, E, ids_ref)


# ----------------------------------------------------------------------------- permute

@pytest.mark.parametrize("T,k,E,kind", [(1, 8, 128, "u"), (16, 8, 128, "u"), (64, 8, 128, "u"), (5, 2, 16, "u"),
                                        (128, 8, 256, "u"), (129, 8, 256, "u"), (40, 2, 257, "u"),  # chunk sort
                                        # at its 1024-row and 256-expert limits and one past each
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

class _FfnRig:
    """Device inputs of one grouped-FFN case built from oracle permutation data."""

    def __init__(self, ops, cfg, T, ids, shuffle_slots=True, with_shared=None, missing=None, skip=None,
                 beyond=None):
        from expert_cached_ffn_amd.layer import DTYPES, pack_expert
        self.ops, self.cfg, self.T = ops, cfg, T
        self.with_shared = cfg.shared if with_shared is None else with_shared
        self.ex = ex = Experts(cfg)
        self.lay = lay = ops.ft_expert_layout_init(DTYPES[cfg.wdtype], cfg.H, cfg.I)
        self.off, self.rows, _ = moe.permute(ids, cfg.E)
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
        if skip is not None:
            slot_of[skip] = -2  # FT_SLOT_SKIP
        if beyond is not None:
            slot_of[beyond] = n_slots + 7  # past the end of the pool
        self.x = synth.tokens(cfg, T)
        self.x64 = formats.activations_to_f64(cfg.xdtype, self.x)
        self.shared_blob = dev(pack_expert(lay, ex.raw(cfg.E).arrays)) if self.with_shared else None
        R = T * cfg.k
        self.y = torch.full((R, cfg.H), np.nan, dtype=torch.float32, device="cuda")
        self.ys = torch.full((T, cfg.H), np.nan, dtype=torch.float32, device="cuda") if self.with_shared else None
        self.wsb = ops.ft_workspace_bytes(2, T, cfg.k, cfg.E, cfg.H, cfg.I)
        self.ws = torch.zeros(self.wsb, dtype=torch.uint8, device="cuda")
        self.dev = (dev(pool), dev(slot_of), dev(self.x), dev(self.off), dev(self.rows))

    def run(self, mode):
        from expert_cached_ffn_amd.layer import DTYPES
        c = self.cfg
        pool, slot_of, x, off, rows = self.dev
        self.ops.ft_moe_grouped_ffn(self.lay, pool, slot_of, self.shared_blob, x, DTYPES[c.xdtype], self.T, c.k,
                                    c.E, off, rows, self.y, self.ys, mode, self.ws, self.wsb)
        torch.cuda.synchronize()

    def hidden(self, n_rows):
        """The bf16 hidden rows the gate/up stage left at the start of the workspace."""
        b = self.ws[:n_rows * self.cfg.I * 2].cpu().numpy().view(np.uint16)
        return formats.bf16_to_f64(b.reshape(n_rows, self.cfg.I))


def _ffn_case(ops, cfg, T, ids, shuffle_slots=True, with_shared=None, missing=None, mode=0, beyond=None):
    """Run the GPU grouped FFN on oracle permutation data; return (gpu y_rows, y_shared, oracle ...).

    mode 1 (native MXFP4) is compared with the oracle's native-mode expert."""
    rig = _FfnRig(ops, cfg, T, ids, shuffle_slots, with_shared, missing, beyond=beyond)
    rig.run(mode)
    fn = moe.swiglu_expert_mx if mode == 1 else moe.swiglu_expert
    y_ref = moe.grouped_ffn(rig.x64, cfg.k, rig.off, rig.rows, rig.ex.f64, fn)
    ys_ref = fn(rig.x64, *rig.ex.f64(cfg.E)) if rig.with_shared else None
    return (rig.y.cpu().numpy(), (rig.ys.cpu().numpy() if rig.with_shared else None), y_ref, ys_ref, rig.off)


FFN_CASES = [
    # name, cfg overrides, T
    ("f32-cfg1", 1, {}, 8),
    ("bf16-small-ragged", 2, dict(H=384, I=256, E=8, k=2), 5),
    ("bf16-two-col-tiles", 2, dict(H=256, I=384, E=4, k=2), 23),
    ("bf16-cfg2-T16", 2, {}, 16),
    ("fp4-small", 3, dict(H=1024, I=512, E=6, k=2), 37),
    ("fp4-long-segment", 3, dict(H=512, I=1024, E=2, k=1), 150),
    # prefill GEMM over 6 chunks a stage: the block-scale groups of 4 chunks end part-way
    ("fp4-prefill-six-chunks", 3, dict(H=768, I=768, E=5, k=3), 130),
    ("fp4-cfg3-T1", 3, {}, 1),
    ("fp4-decode-multigroup", 3, dict(H=512, I=256, E=3, k=2), 60),     # ~40 tokens per expert: 3 groups each
    ("fp4-decode-T64-E16", 3, dict(H=1024, I=1024, E=16, k=4), 64),
    ("nv4-decode-small", 6, dict(H=512, I=512, E=6, k=2), 37),
    ("nv4-decode-shared", 6, dict(H=1024, I=768, E=8, k=2, shared=True), 9),
    ("nv4-decode-multigroup", 6, dict(H=512, I=768, E=3, k=2), 60),
    ("nv4-decode-cfg6-T16", 6, {}, 16),
    ("nv4-prefill-ragged", 6, dict(H=512, I=384, E=8, k=2, shared=True), 200),
    ("nv4-prefill-many-tiles", 6, dict(H=512, I=768, E=24, k=3), 700),
    ("bf16-gemm-ragged", 2, dict(H=512, I=384, E=8, k=2), 200),
    ("fp4-gemm-many-tiles", 3, dict(H=512, I=768, E=24, k=3), 700),
    # the persistent decode kernels' expert-table limit (1024 experts), and one past it (grouped GEMM)
    ("bf16-decode-E1024-limit", 2, dict(H=512, I=768, E=1024, k=8), 64),
    ("fp4-decode-E1024-shared", 3, dict(H=1024, I=1024, E=1024, k=6, shared=True), 64),
    ("bf16-decode-E1100-past-limit", 2, dict(H=512, I=384, E=1100, k=4), 16),
    ("bf16-E4096-max", 2, dict(H=256, I=256, E=4096, k=2), 40),                  # the grouped FFN's expert limit
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


@pytest.mark.parametrize("cfg_id,T,how", [(3, 4, "missing"), (6, 4, "missing"), (2, 4, "missing"),
                                         (3, 150, "missing"), (3, 4, "beyond"), (6, 4, "beyond"),
                                         (2, 4, "beyond"), (3, 150, "beyond"), (2, 150, "beyond"),
                                         (1, 8, "beyond")])
def test_grouped_ffn_missing_slot_gives_nan(ops, cfg_id, T, how):
    """A routed expert with no slot (-1), or with a slot past the end of the pool: nothing is read for
    it and its rows are NaN (decode kernels of every weight format, the prefill GEMM, the fp32 path);
    the other experts' rows are exact."""
    over = dict(E=4, k=1, shared=False) if cfg_id == 1 else dict(H=512, I=512, E=4, k=1, shared=False)
    cfg = synth.shrink(synth.CONFIGS[cfg_id], **over)
    ids = np.array([[0], [1], [2], [1]] * (T // 4) + [[3]] * (T % 4), np.int32)
    y, _, y_ref, _, off = _ffn_case(ops, cfg, T, ids, **{how: 1})
    a, b = int(off[1]), int(off[2])
    assert np.all(np.isnan(y[a:b]))
    keep = np.r_[0:a, b:len(y)]
    check_close(y[keep], y_ref[keep], what="other experts")


SKIP_CASES = [("bf16-decode", 2, dict(H=512, I=512, E=6, k=2), 9, 0),
              ("bf16-stream", 2, dict(H=256, I=256, E=6, k=2), 9, 0),
              ("fp4-decode-xs", 3, dict(H=512, I=512, E=6, k=2, shared=False), 9, 0),
              ("nv4-decode-xs", 6, dict(H=512, I=512, E=6, k=2), 9, 0),
              ("fp4-gemm", 3, dict(H=512, I=512, E=6, k=2, shared=False), 150, 0),
              ("f32", 1, dict(E=6), 9, 0),
              ("fp4-native", 3, dict(H=512, I=512, E=6, k=2, shared=False), 150, 1)]


@pytest.mark.parametrize("name,cfg_id,over,T,mode", SKIP_CASES, ids=[c[0] for c in SKIP_CASES])
def test_grouped_ffn_skip_slot_leaves_rows(ops, name, cfg_id, over, T, mode):
    """FT_SLOT_SKIP experts: their y rows keep what was there (NaN sentinels here), the others are right."""
    cfg = synth.shrink(synth.CONFIGS[cfg_id], **over)
    ids = synth.routing_ids_uniform(cfg, T)
    used = sorted(set(ids.ravel().tolist()))
    skip = used[::2]
    rig = _FfnRig(ops, cfg, T, ids, skip=skip)
    rig.run(mode)
    fn = moe.swiglu_expert_mx if mode == 1 else moe.swiglu_expert
    y_ref = moe.grouped_ffn(rig.x64, cfg.k, rig.off, rig.rows, rig.ex.f64, fn)
    y = rig.y.cpu().numpy()
    skipped = np.zeros(len(y), bool)
    for e in skip:
        skipped[int(rig.off[e]):int(rig.off[e + 1])] = True
    assert skipped.any() and (~skipped).any()
    assert np.all(np.isnan(y[skipped]))
    if mode == 1:
        from tests.helpers import native_mx_expert
        allow = np.zeros_like(y_ref)
        for e in sorted(set(used) - set(skip)):
            a, b = int(rig.off[e]), int(rig.off[e + 1])
            _, allow[a:b] = native_mx_expert(rig.x64[rig.rows[a:b] // cfg.k], *rig.ex.f64(e))
        check_close(y[~skipped], y_ref[~skipped], what=f"{name} computed experts", allow=allow[~skipped])
    else:
        check_close(y[~skipped], y_ref[~skipped], what=f"{name} computed experts")


# ----------------------------------------------------------------------------- native MXFP4 mode

def _bf16_rows(rng, n, K):
    """bf16 bit patterns spanning many binades, with the special cases of the quantizer."""
    mag = rng.standard_normal((n, K)) * np.exp2(rng.integers(-20, 20, size=(n, K // 32)).repeat(32, axis=1))
    v = np.asarray(mag, np.float32).view(np.uint32)
    bits = ((v + 0x7FFF + ((v >> 16) & 1)) >> 16).astype(np.uint16)
    bits[0, :32] = 0                      # an all-zero block
    bits[0, 32:64] = 0x8000               # all -0.0
    bits[1, :32] = np.arange(1, 33)       # bf16 subnormals
    if K >= 128:
        bits[1, 64:96] = 0x4380           # 256.0 everywhere: amax a power of two
        bits[1, 96:128] = rng.integers(0, 65536, 32).astype(np.uint16) & 0x7F7F  # finite mixed signs
    return bits


@pytest.mark.parametrize("n,K,ldx", [(1, 32, 32), (7, 96, 104), (64, 2048, 2048), (257, 4096, 4096)])
def test_mxfp8_quantize_bit_exact(ops, n, K, ldx):
    from oracle import mx
    rng = np.random.default_rng(n * 1000 + K)
    bits = np.zeros((n, ldx), np.uint16)
    bits[:, :K] = _bf16_rows(rng, max(n, 2), K)[:n]
    codes = torch.empty((n, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, K // 32), dtype=torch.uint8, device="cuda")
    ops.ft_mxfp8_quantize(dev(bits), ldx, n, K, codes, scales)
    torch.cuda.synchronize()
    q_ref, s_ref = mx.mxfp8_quantize(formats.bf16_to_f64(bits[:, :K]))
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), q_ref)


MX_CASES = [
    ("mx-small", dict(H=1024, I=512, E=6, k=2), 37),
    ("mx-long-segment", dict(H=512, I=1024, E=2, k=1), 150),
    ("mx-ragged-tiles", dict(H=512, I=768, E=5, k=3), 300),
    ("mx-cfg3-T1", {}, 1),
    ("mx-cfg3-T8", {}, 8),
    # rows of more than 4096 elements: the block scales come in two windows
    ("mx-two-scale-windows", dict(H=4608, I=4352, E=2, k=1), 24),
]


@pytest.mark.parametrize("name,over,T", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_grouped_ffn_native_mx_parity(ops, name, over, T):
    from tests.helpers import native_mx_expert
    print(f"ffn {name}", flush=True)
    cfg = synth.shrink(synth.CONFIGS[3], **over)
    ids = synth.routing_ids_uniform(cfg, T)
    rig = _FfnRig(ops, cfg, T, ids)
    rig.run(1)
    y = rig.y.cpu().numpy()
    y_ref = np.zeros_like(y, dtype=np.float64)
    allow = np.zeros_like(y_ref)
    for e in range(cfg.E):
        a, b = int(rig.off[e]), int(rig.off[e + 1])
        if a < b:
            y_ref[a:b], allow[a:b] = native_mx_expert(rig.x64[rig.rows[a:b] // cfg.k], *rig.ex.f64(e))
    check_close(y, y_ref, what=f"{name} y_rows", allow=allow)
    if rig.with_shared:
        ys_ref, ys_allow = native_mx_expert(rig.x64, *rig.ex.f64(cfg.E))
        check_close(rig.ys.cpu().numpy(), ys_ref, what=f"{name} y_shared", allow=ys_allow)


@pytest.mark.parametrize("mode", [0, 1])
def test_grouped_ffn_stages_through_the_workspace(ops, mode):
    """Gate/up alone leaves the bf16 hidden rows in the workspace; down alone reads them.
    The down stage gets hidden rows written by the test, so both sides quantize the
    same bf16 values (native mode: bit-identical codes) and the bound is the plain one."""
    from oracle import mx
    cfg = synth.shrink(synth.CONFIGS[3], H=1024, I=512, E=6, k=2)
    T = 37
    ids = synth.routing_ids_uniform(cfg, T)
    rig = _FfnRig(ops, cfg, T, ids)
    R, rows_all = T * cfg.k, T * cfg.k + T
    rig.run(mode | 0x100)
    h = rig.hidden(rows_all)
    assert np.all(np.isnan(rig.y.cpu().numpy()))          # gate/up alone writes no output
    x_in = mx.mxfp8_round_trip(rig.x64) if mode == 1 else rig.x64
    h_ref = np.zeros((rows_all, cfg.I))
    for e in range(cfg.E + 1):
        if e < cfg.E:
            a, b = int(rig.off[e]), int(rig.off[e + 1])
            X = x_in[rig.rows[a:b] // cfg.k]
        else:
            a, b = R, rows_all
            X = x_in
        if a < b:
            Wg, Wu, _ = rig.ex.f64(e)
            G, U = X @ Wg.T, X @ Wu.T
            h_ref[a:b] = G * moe.sigmoid(G) * U
    check_close(h, h_ref, bf16_out=True, what=f"mode {mode} hidden rows")
    # down stage from hidden rows of the test's own (seeded, synthetic) making
    rng = np.random.default_rng(7 + mode)
    hv = (rng.standard_normal((rows_all, cfg.I)) * 20).astype(np.float32).view(np.uint32)
    hb = ((hv + 0x7FFF + ((hv >> 16) & 1)) >> 16).astype(np.uint16)
    rig.ws[:hb.nbytes].copy_(torch.from_numpy(hb.view(np.uint8).ravel()))
    rig.run(mode | 0x200)
    h_in = formats.bf16_to_f64(hb)
    if mode == 1:
        h_in = mx.mxfp8_round_trip(h_in)
    y_ref = np.zeros((R, cfg.H))
    for e in range(cfg.E):
        a, b = int(rig.off[e]), int(rig.off[e + 1])
        if a < b:
            y_ref[a:b] = h_in[a:b] @ rig.ex.f64(e)[2].T
    check_close(rig.y.cpu().numpy(), y_ref, what=f"mode {mode} down stage")
    check_close(rig.ys.cpu().numpy(), h_in[R:] @ rig.ex.f64(cfg.E)[2].T, what=f"mode {mode} shared down")


@pytest.mark.parametrize("how", ["missing", "beyond"])
def test_grouped_ffn_native_mx_missing_slot_gives_nan(ops, how):
    from tests.helpers import native_mx_expert
    cfg = synth.shrink(synth.CONFIGS[3], H=512, I=512, E=4, k=1, shared=False)
    ids = np.array([[0], [1], [2], [1]], np.int32)
    rig = _FfnRig(ops, cfg, 4, ids, **{how: 1})
    rig.run(1)
    y = rig.y.cpu().numpy()
    a, b = int(rig.off[1]), int(rig.off[2])
    assert np.all(np.isnan(y[a:b]))
    for e in (0, 2):
        a, b = int(rig.off[e]), int(rig.off[e + 1])
        ref, allow = native_mx_expert(rig.x64[rig.rows[a:b]], *rig.ex.f64(e))
        check_close(y[a:b], ref, what=f"expert {e}", allow=allow)


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


def test_grouped_ffn_nvfp4_decode_shape_not_covered(ops):
    """NVFP4 decode needs a persistent shape for H/128 and I/128: others are refused, nothing written."""
    cfg = synth.shrink(synth.CONFIGS[6], H=256, I=512, E=4, k=1)
    T = 3
    ids = synth.routing_ids_uniform(cfg, T)
    with pytest.raises(ops.FtError) as e:
        _ffn_case(ops, cfg, T, ids)
    assert e.value.status == -2


EDGE_ROUTINGS = [
    # name, cfg id, overrides, T, routing
    ("one-expert-decode-fp4", 3, dict(H=512, I=512, E=8, k=1, shared=True), 64, "one"),
    ("one-expert-decode-bf16", 2, dict(H=512, I=512, E=8, k=1), 64, "one"),
    ("one-expert-prefill-fp4", 3, dict(H=512, I=512, E=8, k=1, shared=False), 1000, "one"),
    ("k-equals-E-fp4", 3, dict(H=512, I=512, E=4, k=4, shared=True), 20, "all"),
    ("k-equals-E-nv4-prefill", 6, dict(H=512, I=512, E=4, k=4), 90, "all"),
    ("single-token-k1-nv4", 6, dict(H=512, I=512, E=8, k=1), 1, "one"),
]


@pytest.mark.parametrize("name,cfg_id,over,T,kind", EDGE_ROUTINGS, ids=[c[0] for c in EDGE_ROUTINGS])
def test_grouped_ffn_edge_routings(ops, name, cfg_id, over, T, kind):
    """Degenerate routings: every token on one expert (one long segment, the rest empty), and k = E
    (every expert takes every token)."""
    cfg = synth.shrink(synth.CONFIGS[cfg_id], **over)
    if kind == "one":
        ids = np.full((T, cfg.k), cfg.E - 1, np.int32)
    else:
        ids = np.tile(np.arange(cfg.E, dtype=np.int32)[::-1], (T, 1))
    y, ys, y_ref, ys_ref, off = _ffn_case(ops, cfg, T, ids)
    check_close(y, y_ref, what=f"{name} y_rows")
    if ys_ref is not None:
        check_close(ys, ys_ref, what=f"{name} y_shared")
