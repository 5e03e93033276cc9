"""End-to-end parity of the whole layer (route -> permute -> FFN -> combine) on every workload shape."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import formats, moe
from tests.helpers import (TOPK_MARGIN, Experts, check_close, check_topk_valid, native_mx_expert,
                           native_mx_token, route_oracle)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from expert_cached_ffn_amd import layer as _layer
    from expert_cached_ffn_amd import ops
    ops.version()
    return _layer


def make_layer(Lm, cfg, T):
    shape = Lm.LayerShape(cfg.H, cfg.I, cfg.E, cfg.k, cfg.wdtype, cfg.xdtype, cfg.gating, cfg.renormalize,
                          cfg.shared)
    return Lm.MoELayer(shape, T)


def build_pool(Lm, layer, ex, experts, n_slots):
    """Device pool with expert e in slot e for e in `experts` (other slots zero, never read)."""
    eb = int(layer.layout.expert_bytes)
    pool = torch.zeros((n_slots, eb), dtype=torch.uint8, device="cuda")
    buf = np.zeros(eb, np.uint8)
    for e in experts:
        buf[:] = 0
        Lm.pack_expert(layer.layout, ex.raw(e).arrays, buf)
        pool[e].copy_(torch.from_numpy(buf))
    return pool


def out_f64(layer, cfg, T):
    o = layer.out[:T].cpu().numpy()
    return formats.bf16_to_f64(o.view(np.uint16)) if cfg.xdtype == "bf16" else o.astype(np.float64)


def check_routing(cfg, got_logits, got_ids, got_w, ref, wr64, x64, what):
    """Routing of a layer call against the oracle's: the GPU's logits within the fp32-accumulation
    bound, its top-k exact on its own logits, bit-exact ids where the oracle margin exceeds 1e-4 and a
    valid top-k elsewhere; gating weights equal to the oracle's at the GPU's ids.  Returns the tokens
    whose ids differ from the oracle's (near ties only) and the oracle weights at the GPU's ids."""
    scale = np.abs(x64) @ np.abs(wr64).T
    assert np.all(np.abs(got_logits - ref["logits"]) <= 3e-5 * scale + 1e-6), f"{what}: logits"
    assert np.array_equal(got_ids, moe.topk(got_logits.astype(np.float32), cfg.k)), f"{what}: top-k of own logits"
    sure = ref["margin"] > TOPK_MARGIN
    assert np.array_equal(got_ids[sure], ref["ids"][sure]), f"{what}: ids above the margin"
    differ = check_topk_valid(got_ids, ref["logits"], cfg.k, what=what)
    assert set(differ.tolist()) <= set(np.flatnonzero(~sure).tolist())
    w_at = moe.gating_weights(ref["logits"], got_ids, cfg.gating, cfg.renormalize)
    np.testing.assert_allclose(got_w, w_at, rtol=1e-4, atol=1e-6)
    print(f"ROUTING {what}: {int((~sure).sum())} of {len(sure)} tokens at or below the 1e-4 margin, "
          f"{len(differ)} with ids other than the oracle's (valid top-k, compared at the GPU's ids)", flush=True)
    return differ, w_at


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg_id,T", [(1, 8), (2, 1), (2, 16), (2, 64), (3, 1), (3, 8), (3, 32), (6, 1), (6, 64)])
def test_layer_router_gemv(L, cfg_id, T):
    """Every token of the layer call against the oracle layer, evaluated expert-major (each expert's
    weights decoded once for all its tokens); tokens whose routing is a near tie at the GPU's own ids."""
    cfg = synth.CONFIGS[cfg_id]
    print(f"layer cfg{cfg_id} T={T}", flush=True)
    ex = Experts(cfg)
    x = synth.tokens(cfg, T)
    wr = synth.router_weight(cfg)
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    wr64 = formats.activations_to_f64(cfg.xdtype, wr)
    ids0 = moe.topk(moe.router_logits(x64, wr64), cfg.k)
    layer = make_layer(L, cfg, T)
    pool = build_pool(L, layer, ex, sorted(set(ids0.ravel().tolist())), cfg.E)
    shared = L.as_device_u8([L.pack_expert(layer.layout, ex.raw(cfg.E).arrays)])[0] if cfg.shared else None
    layer.forward(T, L.to_device(x), pool, w_router=L.to_device(wr), shared_blob=shared)
    torch.cuda.synchronize()
    got = out_f64(layer, cfg, T)
    got_ids = layer.ids[:T].cpu().numpy()
    got_logits = layer.logits[:T].cpu().numpy().astype(np.float64)
    got_w = layer.w[:T].cpu().numpy()
    sh = ex.f64(cfg.E) if cfg.shared else None
    ref = moe.moe_layer(x64, k=cfg.k, E=cfg.E, gating=cfg.gating, renormalize=cfg.renormalize,
                        experts=ex.fresh, shared=sh, w_router=wr64)
    differ, w_at = check_routing(cfg, got_logits, got_ids, got_w, ref, wr64, x64, f"cfg{cfg_id} T={T}")
    out_ref = ref["out"].copy()
    for t in differ:
        out_ref[t] = moe.token_output(x64[t], got_ids[t], w_at[t], ex.fresh, sh)
    check_close(got, out_ref, bf16_out=cfg.xdtype == "bf16", what=f"cfg{cfg_id} T={T} every token")


def _prefill_segments(off_ref):
    """The most and the least popular non-empty experts of a routing."""
    sizes = np.diff(off_ref)
    big = int(np.argmax(sizes))
    small = int(np.argmin(np.where(sizes > 0, sizes, 10 ** 9)))
    return [big, small]


@pytest.mark.timeout(900)
def test_layer_prefill_given_logits(L):
    """Prefill workload (8192 tokens, Zipf-skewed segments), both modes: the whole segments of the
    most and the least popular expert, the shared expert's rows of every token, sampled outputs."""
    cfg = synth.CONFIGS[4]
    T = 8192
    ex = Experts(cfg)
    x = synth.tokens(cfg, T)
    logits = synth.prefill_logits(cfg, T)
    ids = moe.topk(logits, cfg.k)
    w = moe.gating_weights(logits, ids, cfg.gating, cfg.renormalize)
    layer = make_layer(L, cfg, T)
    print("prefill: packing 257 experts", flush=True)
    pool = build_pool(L, layer, ex, range(cfg.E), cfg.E)
    shared = L.as_device_u8([L.pack_expert(layer.layout, ex.raw(cfg.E).arrays)])[0]
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    off_ref, rows_ref, _ = moe.permute(ids, cfg.E)
    segs = _prefill_segments(off_ref)
    toks = [0, 1, 4097, 5000, T - 1]
    for mode in (0, 1):      # exact bf16 MFMA, then the native MXFP4 scaled MFMA
        print(f"prefill: running mode {mode}", flush=True)
        layer.forward(T, L.to_device(x), pool, logits=L.to_device(logits), shared_blob=shared, mode=mode)
        torch.cuda.synchronize()
        assert np.array_equal(layer.ids[:T].cpu().numpy(), ids)
        assert np.array_equal(layer.offsets.cpu().numpy(), off_ref)
        assert np.array_equal(layer.sorted_rows[:T * cfg.k].cpu().numpy(), rows_ref)
        got = out_f64(layer, cfg, T)
        assert np.all(np.isfinite(got))
        assert np.all(np.isfinite(layer.y_rows[:T * cfg.k].cpu().numpy()))
        for e in segs:
            a, b = int(off_ref[e]), int(off_ref[e + 1])
            print(f"prefill mode {mode}: expert {e}, {b - a} rows", flush=True)
            yr = layer.y_rows[a:b].cpu().numpy()
            X = x64[rows_ref[a:b] // cfg.k]
            if mode == 0:
                check_close(yr, moe.swiglu_expert(X, *ex.f64(e)), what=f"prefill mode 0 segment of expert {e}")
            else:
                yref, allow = native_mx_expert(X, *ex.f64(e))
                check_close(yr, yref, what=f"prefill mode 1 segment of expert {e}", allow=allow)
        ysh = layer.y_shared[:T].cpu().numpy()
        if mode == 0:
            check_close(ysh, moe.swiglu_expert(x64, *ex.f64(cfg.E)), what="prefill mode 0 shared expert, every token")
            ref = np.stack([moe.token_output(x64[t], ids[t], w[t], ex.f64, ex.f64(cfg.E)) for t in toks])
            check_close(got[toks], ref, bf16_out=True, what="prefill mode 0 sampled tokens")
        else:
            yref, allow = native_mx_expert(x64, *ex.f64(cfg.E))
            check_close(ysh, yref, what="prefill mode 1 shared expert, every token", allow=allow)
            pairs = [native_mx_token(x64[t], ids[t], w[t], ex.f64, ex.f64(cfg.E)) for t in toks]
            check_close(got[toks], np.stack([p[0] for p in pairs]), bf16_out=True,
                        what="prefill mode 1 sampled tokens", allow=np.stack([p[1] for p in pairs]))
        ex.drop()
        for e in segs + [cfg.E]:
            ex.f64(e)            # keep only the compared experts for the next mode


@pytest.mark.timeout(600)
def test_layer_prefill_nvfp4(L):
    """NVFP4 prefill workload (8192 tokens on the Qwen3-A3B shape): the whole segments of the most and
    the least popular expert, and sampled tokens."""
    cfg = synth.CONFIGS[7]
    T = 8192
    ex = Experts(cfg)
    x = synth.tokens(cfg, T)
    logits = synth.prefill_logits(cfg, T)
    ids = moe.topk(logits, cfg.k)
    w = moe.gating_weights(logits, ids, cfg.gating, cfg.renormalize)
    layer = make_layer(L, cfg, T)
    print("nvfp4 prefill: packing 128 experts", flush=True)
    pool = build_pool(L, layer, ex, range(cfg.E), cfg.E)
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    layer.forward(T, L.to_device(x), pool, logits=L.to_device(logits))
    torch.cuda.synchronize()
    assert np.array_equal(layer.ids[:T].cpu().numpy(), ids)
    got = out_f64(layer, cfg, T)
    assert np.all(np.isfinite(got))
    toks = [0, 3000, T - 1]
    ref = np.stack([moe.token_output(x64[t], ids[t], w[t], ex.f64) for t in toks])
    check_close(got[toks], ref, bf16_out=True, what="nvfp4 prefill sampled tokens")
    off_ref, rows_ref, _ = moe.permute(ids, cfg.E)
    for e in _prefill_segments(off_ref):
        a, b = int(off_ref[e]), int(off_ref[e + 1])
        yref = moe.swiglu_expert(x64[rows_ref[a:b] // cfg.k], *ex.f64(e))
        check_close(layer.y_rows[a:b].cpu().numpy(), yref, what=f"nvfp4 prefill segment of expert {e}")


@pytest.mark.parametrize("cfg_id", [2, 3])
def test_layer_empty_batch_then_small(L, cfg_id):
    """A step of zero tokens through all four calls launches nothing and writes nothing: the
    permutation offsets come back all zero, the output buffer keeps its contents, and the next
    (non-empty) step on the same buffers is still exact."""
    cfg = synth.shrink(synth.CONFIGS[cfg_id], H=512, I=256, E=8, k=2)
    print(f"empty batch cfg{cfg_id}", flush=True)
    ex = Experts(cfg)
    T = 3
    x = synth.tokens(cfg, T)
    wr = synth.router_weight(cfg)
    layer = make_layer(L, cfg, T)
    pool = build_pool(L, layer, ex, range(cfg.E), cfg.E)
    shared = L.as_device_u8([L.pack_expert(layer.layout, ex.raw(cfg.E).arrays)])[0] if cfg.shared else None
    xd, wrd = L.to_device(x), L.to_device(wr)
    layer.offsets.fill_(-7)
    layer.out.fill_(1234)
    layer.forward(0, xd, pool, w_router=wrd, shared_blob=shared)
    torch.cuda.synchronize()
    assert layer.offsets.cpu().numpy().tolist() == [0] * (cfg.E + 1)
    assert bool((layer.out == 1234).all())
    layer.forward(T, xd, pool, w_router=wrd, shared_blob=shared)
    torch.cuda.synchronize()
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    logits, ids, w, margin = route_oracle(cfg, x64, formats.activations_to_f64(cfg.xdtype, wr))
    sure = np.flatnonzero(margin > 1e-4)
    assert len(sure) >= 1
    assert np.array_equal(layer.ids[:T].cpu().numpy()[sure], ids[sure])
    ref = np.stack([moe.token_output(x64[t], ids[t], w[t], ex.f64, ex.f64(cfg.E) if cfg.shared else None)
                    for t in sure])
    check_close(out_f64(layer, cfg, T)[sure], ref, bf16_out=cfg.xdtype == "bf16", what=f"cfg{cfg_id} after empty")


def _near_tie_router(cfg, x64, rng):
    """Router weights [E, H] (bf16 bits) that give the token a near tie at the top-k boundary: experts
    0..k-2 far ahead, then two experts whose rows differ by one bf16 step at the token's smallest
    activation, so their logits differ by far less than the 1e-4 margin (fp32 rounding of the GPU's
    sum may order them either way)."""
    E, H, k = cfg.E, cfg.H, cfg.k
    w = rng.standard_normal((E, H)).astype(np.float32) * np.float32(cfg.w_std)
    sgn = np.sign(x64[0]).astype(np.float32)
    order = rng.permutation(E)
    lead, (a, b) = order[:k - 1], order[k - 1:k + 1]
    for j, e in enumerate(lead):
        w[e] = sgn * np.float32(0.05 + 0.002 * j)
    w[a] = sgn * np.float32(0.01)
    bits = synth.f32_to_bf16_bits(w)
    h = int(np.argmin(np.abs(x64[0])))
    bits[b] = bits[a]
    bits[b, h] = bits[a, h] + 1           # one bf16 step (same sign: the magnitude grows by one ulp)
    return bits, int(a), int(b)


@pytest.mark.parametrize("cfg_id", [2, 3])
def test_layer_near_tie_routing(L, cfg_id):
    """Planted near ties at the top-k boundary: the GPU's ids are a valid top-k of the oracle logits
    (checked against the margin rule), and the token's output equals the oracle's at the GPU's own
    ids and weights."""
    cfg = synth.CONFIGS[cfg_id]
    ex = Experts(cfg)
    layer = make_layer(L, cfg, 1)
    n_tie = n_differ = 0
    for case in range(6):
        x = synth.tokens(cfg, 1, case=100 + case)
        x64 = formats.activations_to_f64(cfg.xdtype, x)
        wr, a, b = _near_tie_router(cfg, x64, np.random.default_rng(case))
        wr64 = formats.activations_to_f64(cfg.xdtype, wr)
        logits = moe.router_logits(x64, wr64)
        ids0 = moe.topk(logits, cfg.k)
        used = sorted(set(ids0.ravel().tolist()) | {a, b})
        pool = build_pool(L, layer, ex, used, cfg.E)
        shared = L.as_device_u8([L.pack_expert(layer.layout, ex.raw(cfg.E).arrays)])[0] if cfg.shared else None
        layer.forward(1, L.to_device(x), pool, w_router=L.to_device(wr), shared_blob=shared)
        torch.cuda.synchronize()
        got_ids = layer.ids[:1].cpu().numpy()
        got_logits = layer.logits[:1].cpu().numpy().astype(np.float64)
        sh = ex.f64(cfg.E) if cfg.shared else None
        ref = moe.moe_layer(x64, k=cfg.k, E=cfg.E, gating=cfg.gating, renormalize=cfg.renormalize,
                            experts=ex.f64, shared=sh, w_router=wr64)
        assert ref["margin"][0] <= TOPK_MARGIN           # the planted near tie
        n_tie += 1
        assert set(got_ids[0].tolist()) & {a, b}         # one of the tied pair made the cut
        scale = np.abs(x64) @ np.abs(wr64).T
        assert np.all(np.abs(got_logits - ref["logits"]) <= 3e-5 * scale + 1e-6)
        assert np.array_equal(got_ids, moe.topk(got_logits.astype(np.float32), cfg.k))
        differ = check_topk_valid(got_ids, ref["logits"], cfg.k, what=f"near tie case {case}")
        n_differ += len(differ)
        w_at = moe.gating_weights(ref["logits"], got_ids, cfg.gating, cfg.renormalize)
        np.testing.assert_allclose(layer.w[:1].cpu().numpy(), w_at, rtol=1e-4, atol=1e-6)
        want = moe.token_output(x64[0], got_ids[0], w_at[0], ex.f64, sh)[None, :]
        check_close(out_f64(layer, cfg, 1), want, bf16_out=True, what=f"cfg{cfg_id} near tie case {case}")
        ex.drop()
    print(f"NEAR-TIE cfg{cfg_id}: {n_tie} planted ties, {n_differ} with ids other than the oracle's", flush=True)


LAYER_CALL_CASES = [
    # name, config, overrides, T -- T <= 4 with a covered shape runs the fused three-launch path
    ("bf16-T1", 2, {}, 1),
    ("bf16-T2", 2, {}, 2),
    ("bf16-T4", 2, {}, 4),
    ("mxfp4-T1", 3, {}, 1),
    ("mxfp4-T3", 3, {}, 3),
    ("nvfp4-T1", 6, {}, 1),
    ("nvfp4-T4", 6, {}, 4),
    # one token: one launch for gate/up + down (k + shared <= 8), in every row-chunk shape ...
    ("bf16-T1-rows4k", 2, dict(I=2048), 1),                            # 4 KiB gate/up and down rows
    ("mxfp4-T1-small", 3, dict(H=512, I=512, E=8, k=2), 1),            # a grid of a few workgroups
    ("nvfp4-T1-shared", 6, dict(shared=True), 1),
    # ... two launches with 9 to 12 down steps, the MFMA kernels past 12
    ("bf16-T1-k10", 2, dict(k=10), 1),
    ("bf16-T1-k16", 2, dict(k=16), 1),
    ("bf16-small-4x1", 2, dict(H=512, I=512, E=8, k=2), 3),            # 4 waves x 1 k-block both stages
    ("bf16-E256-k16", 2, dict(H=512, I=768, E=256, k=16), 4),          # the fused path's E and k limits
    ("mxfp4-no-shared", 3, dict(shared=False), 2),
    ("bf16-T5-four-calls", 2, {}, 5),                                  # past the fused path: the three calls
    ("bf16-T64", 2, dict(H=1024, I=768, E=32), 64),                    # staged down outputs: 64-tile groups, 4 windows
    ("bf16-T33-4x1", 2, dict(H=512, I=512, E=16, k=2), 33),            # experts with two token groups
    # ... whose routing past 16 tokens is one launch after the router (the last workgroup sorts)
    ("bf16-T64-k16-1024rows", 2, dict(H=512, I=512, E=64, k=16), 64),  # 16-wave workgroups, 1024 rows
    ("mxfp4-T17-E256", 3, dict(H=512, I=512), 17),                     # four logits per lane, shared expert
    ("mxfp4-small-four-calls", 3, dict(H=512, I=512, E=8, k=2), 2),    # no persistent shape for H/256 = 2
    ("f32-four-calls", 1, {}, 8),
]


@pytest.mark.parametrize("name,cfg_id,over,T", LAYER_CALL_CASES, ids=[c[0] for c in LAYER_CALL_CASES])
def test_layer_call(L, name, cfg_id, over, T):
    """ft_moe_layer: every token against the oracle layer (near ties at the GPU's ids); topk ids and
    weights as the routing rule fixes them, and the permutation outputs bit-exact for the GPU's ids."""
    cfg = synth.shrink(synth.CONFIGS[cfg_id], **over)
    print(f"layer call {name}", flush=True)
    ex = Experts(cfg)
    x = synth.tokens(cfg, T, case=7)
    wr = synth.router_weight(cfg)
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    wr64 = formats.activations_to_f64(cfg.xdtype, wr)
    ids0 = moe.topk(moe.router_logits(x64, wr64), cfg.k)
    layer = make_layer(L, cfg, T)
    pool = build_pool(L, layer, ex, sorted(set(ids0.ravel().tolist())), cfg.E)
    shared = L.as_device_u8([L.pack_expert(layer.layout, ex.raw(cfg.E).arrays)])[0] if cfg.shared else None
    layer.out.fill_(0)
    layer.forward_layer(T, L.to_device(x), pool, w_router=L.to_device(wr), shared_blob=shared)
    torch.cuda.synchronize()
    got = out_f64(layer, cfg, T)
    got_ids = layer.ids[:T].cpu().numpy()
    sh = ex.f64(cfg.E) if cfg.shared else None
    ref = moe.moe_layer(x64, k=cfg.k, E=cfg.E, gating=cfg.gating, renormalize=cfg.renormalize,
                        experts=ex.f64, shared=sh, w_router=wr64)
    differ, w_at = check_routing(cfg, layer.logits[:T].cpu().numpy().astype(np.float64), got_ids,
                                 layer.w[:T].cpu().numpy(), ref, wr64, x64, name)
    off, rows, pos = moe.permute(got_ids, cfg.E)
    assert np.array_equal(layer.offsets.cpu().numpy(), off)
    assert np.array_equal(layer.sorted_rows[:T * cfg.k].cpu().numpy(), rows)
    assert np.array_equal(layer.row_pos[:T * cfg.k].cpu().numpy(), pos)
    out_ref = ref["out"].copy()
    for t in differ:
        out_ref[t] = moe.token_output(x64[t], got_ids[t], w_at[t], ex.f64, sh)
    check_close(got, out_ref, bf16_out=cfg.xdtype == "bf16", what=f"layer call {name} every token")


def _tie_logits(E, k, pattern, rng):
    """One token's logits with exact ties (float32 values): all equal; a few repeated values; +0.0
    and -0.0 at the top; k - 1 distinct leaders and five equal values across the top-k boundary."""
    if pattern == "all-equal":
        return np.full(E, 0.5, np.float32)
    if pattern == "few-values":
        return rng.choice(np.array([-1.0, 0.0, 0.25, 1.0], np.float32), size=E)
    if pattern == "signed-zeros":
        v = np.full(E, -3.0, np.float32)
        at = rng.choice(E, size=k + 3, replace=False)
        v[at] = np.where(np.arange(k + 3) % 2 == 0, np.float32(0.0), np.float32(-0.0))
        return v
    v = rng.normal(-2.0, 0.5, size=E).astype(np.float32)  # "boundary": the k-th pick among 5 equals
    at = rng.choice(E, size=k + 4, replace=False)
    v[at[:k - 1]] = 2.0 + np.arange(k - 1, dtype=np.float32)
    v[at[k - 1:]] = np.float32(1.5)
    return v


@pytest.mark.parametrize("cfg_id", [2, 3])
@pytest.mark.parametrize("pattern", ["all-equal", "few-values", "signed-zeros", "boundary"])
def test_layer_call_one_token_exact_ties(L, cfg_id, pattern):
    """The one-token layer kernel's routing on given logits with exact ties: ids in the order the
    routing rule fixes (larger logit first, the lower index among equal logits, -0.0 = +0.0), its
    gating weights, and the layer output at those ids."""
    cfg = synth.CONFIGS[cfg_id]
    rng = np.random.default_rng(11)
    lg = _tie_logits(cfg.E, cfg.k, pattern, rng)[None, :]
    ids = moe.topk(lg.astype(np.float64), cfg.k)
    w = moe.gating_weights(lg.astype(np.float64), ids, cfg.gating, cfg.renormalize)
    ex = Experts(cfg)
    x = synth.tokens(cfg, 1, case=3)
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    layer = make_layer(L, cfg, 1)
    pool = build_pool(L, layer, ex, sorted(set(ids.ravel().tolist())), cfg.E)
    shared = L.as_device_u8([L.pack_expert(layer.layout, ex.raw(cfg.E).arrays)])[0] if cfg.shared else None
    print(f"one-token ties cfg{cfg_id} {pattern}", flush=True)
    layer.forward_layer(1, L.to_device(x), pool, logits=L.to_device(lg), shared_blob=shared)
    torch.cuda.synchronize()
    assert np.array_equal(layer.ids[:1].cpu().numpy(), ids), f"{pattern}: ids {layer.ids[:1].cpu().numpy()} != {ids}"
    got_w = layer.w[:1].cpu().numpy().astype(np.float64)
    assert np.allclose(got_w, w, rtol=2e-6, atol=1e-7), f"{pattern}: gating weights"
    sh = ex.f64(cfg.E) if cfg.shared else None
    want = moe.token_output(x64[0], ids[0], w[0], ex.f64, sh)[None, :]
    check_close(out_f64(layer, cfg, 1), want, bf16_out=True, what=f"cfg{cfg_id} one-token ties {pattern}")


@pytest.mark.parametrize("cfg_id", [2, 3])
def test_layer_call_missing_expert_gives_nan(L, cfg_id):
    """The fused path with one picked expert not resident: that token's outputs are NaN, the other
    token's are exact."""
    cfg = synth.CONFIGS[cfg_id]
    T = 2
    ex = Experts(cfg)
    x = synth.tokens(cfg, T, case=9)
    wr = synth.router_weight(cfg)
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    wr64 = formats.activations_to_f64(cfg.xdtype, wr)
    ref = moe.moe_layer(x64, k=cfg.k, E=cfg.E, gating=cfg.gating, renormalize=cfg.renormalize,
                        experts=ex.f64, shared=ex.f64(cfg.E) if cfg.shared else None, w_router=wr64)
    ids = ref["ids"]
    gone = int(ids[0, 0])
    assert gone not in ids[1]
    layer = make_layer(L, cfg, T)
    used = sorted(set(ids.ravel().tolist()))
    pool = build_pool(L, layer, ex, used, cfg.E)
    slot_of = np.arange(cfg.E, dtype=np.int32)
    slot_of[gone] = -1
    shared = L.as_device_u8([L.pack_expert(layer.layout, ex.raw(cfg.E).arrays)])[0] if cfg.shared else None
    layer.forward_layer(T, L.to_device(x), pool, w_router=L.to_device(wr), shared_blob=shared,
                        slot_of_expert=L.to_device(slot_of))
    torch.cuda.synchronize()
    got = out_f64(layer, cfg, T)
    assert np.all(np.isnan(got[0]))
    check_close(got[1:], ref["out"][1:], bf16_out=True, what=f"cfg{cfg_id} token beside a missing expert")


GRAPH_CASES = [
    # name, config, overrides, T
    ("bf16-T1", 2, {}, 1),     # one launch for gate/up + down: the grid-wide wait
    ("mxfp4-T1", 3, {}, 1),
    ("bf16-T64", 2, dict(H=1024, I=768, E=32), 64),  # the grouped decode kernels
]


@pytest.mark.parametrize("name,cfg_id,over,T", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_layer_call_graph_replays(L, name, cfg_id, over, T):
    """The layer call captured in a HIP graph: every replay, with eager calls on other inputs between
    them, gives the eager output bit for bit (the grid-wide wait's counters start each replay at zero
    and the hidden rows are read after every workgroup wrote them).  With more than one token the
    calls leave the wait area as they found it."""
    cfg = synth.shrink(synth.CONFIGS[cfg_id], **over)
    print(f"layer call graph {name}", flush=True)
    ex = Experts(cfg)
    xs = [synth.tokens(cfg, T, case=c) for c in (11, 12)]
    wr = synth.router_weight(cfg)
    wr64 = formats.activations_to_f64(cfg.xdtype, wr)
    used = set()
    for x in xs:
        used |= set(moe.topk(moe.router_logits(formats.activations_to_f64(cfg.xdtype, x), wr64), cfg.k).ravel())
    layer = make_layer(L, cfg, T)
    pool = build_pool(L, layer, ex, sorted(used), cfg.E)
    shared = L.as_device_u8([L.pack_expert(layer.layout, ex.raw(cfg.E).arrays)])[0] if cfg.shared else None
    xd = [L.to_device(x) for x in xs]
    wrd = L.to_device(wr)
    wait_area = layer.ws_layer[:8192].clone()
    eager = []
    for x in xd:
        layer.forward_layer(T, x, pool, w_router=wrd, shared_blob=shared)
        torch.cuda.synchronize()
        eager.append(layer.out[:T].clone())
    assert not torch.equal(eager[0], eager[1])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            layer.forward_layer(T, xd[0], pool, w_router=wrd, shared_blob=shared)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        layer.out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out[:T], eager[0]), f"replay {rep}"
        layer.forward_layer(T, xd[1], pool, w_router=wrd, shared_blob=shared)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(layer.out[:T], eager[1]), f"eager call after replay {rep}"
    if T > 1:
        assert torch.equal(layer.ws_layer[:8192], wait_area), "the calls left the wait area changed"
    print(f"PARITY {name} graph replays: bit-identical to the eager call", flush=True)
