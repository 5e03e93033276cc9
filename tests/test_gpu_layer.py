"""End-to-end parity of the whole layer (route -> permute -> FFN -> combine) on every workload shape."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import formats, moe
from tests.helpers import Experts, check_close, native_mx_expert, native_mx_token, route_oracle

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


@pytest.mark.parametrize("cfg_id,T,sample", [(1, 8, None), (2, 1, None), (2, 16, None), (2, 64, 12),
                                             (3, 1, None), (3, 8, 4), (3, 32, 4), (6, 1, None), (6, 64, 12)])
def test_layer_router_gemv(L, cfg_id, T, sample):
    cfg = synth.CONFIGS[cfg_id]
    print(f"layer cfg{cfg_id} T={T}", flush=True)
    ex = Experts(cfg)
    x = synth.tokens(cfg, T)
    wr = synth.router_weight(cfg)
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    wr64 = formats.activations_to_f64(cfg.xdtype, wr)
    logits, ids, w, margin = route_oracle(cfg, x64, wr64)
    layer = make_layer(L, cfg, T)
    pool = build_pool(L, layer, ex, sorted(set(ids.ravel().tolist())), cfg.E)
    shared = L.as_device_u8([L.pack_expert(layer.layout, ex.raw(cfg.E).arrays)])[0] if cfg.shared else None
    layer.forward(T, L.to_device(x), pool, w_router=L.to_device(wr), shared_blob=shared)
    torch.cuda.synchronize()
    got = out_f64(layer, cfg, T)
    got_ids = layer.ids[:T].cpu().numpy()
    sure = np.flatnonzero(margin > 1e-4)
    assert len(sure) >= 0.9 * T
    assert np.array_equal(got_ids[sure], ids[sure])
    toks = sure if sample is None else np.random.default_rng(T).choice(sure, size=min(sample, len(sure)), replace=False)
    ref = np.stack([moe.token_output(x64[t], ids[t], w[t], ex.f64, ex.f64(cfg.E) if cfg.shared else None)
                    for t in toks])
    check_close(got[toks], ref, bf16_out=cfg.xdtype == "bf16", what=f"cfg{cfg_id} T={T} out")


def test_layer_prefill_given_logits(L):
    """Prefill workload (8192 tokens, Zipf-skewed segments), sampled tokens + whole-output properties."""
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
    sizes = np.diff(off_ref)
    e = int(np.argmin(np.where(sizes > 0, sizes, 10 ** 9)))   # the least popular non-empty expert
    a, b = int(off_ref[e]), int(off_ref[e + 1])
    toks = [0, 4097, T - 1]
    for mode in (0, 1):      # exact bf16 MFMA, then the native MXFP4 scaled MFMA
        print(f"prefill: running mode {mode}", flush=True)
        layer.forward(T, L.to_device(x), pool, logits=L.to_device(logits), shared_blob=shared, mode=mode)
        torch.cuda.synchronize()
        assert np.array_equal(layer.ids[:T].cpu().numpy(), ids)
        assert np.array_equal(layer.offsets.cpu().numpy(), off_ref)
        got = out_f64(layer, cfg, T)
        assert np.all(np.isfinite(got))
        yr = layer.y_rows[a:b].cpu().numpy()
        if mode == 0:
            ref = np.stack([moe.token_output(x64[t], ids[t], w[t], ex.f64, ex.f64(cfg.E)) for t in toks])
            check_close(got[toks], ref, bf16_out=True, what="prefill mode 0 sampled tokens")
            # one expert's whole segment in the permuted expert rows
            yref = moe.swiglu_expert(x64[rows_ref[a:b] // cfg.k], *ex.f64(e))
            check_close(yr, yref, what=f"prefill mode 0 segment of expert {e}")
        else:
            pairs = [native_mx_token(x64[t], ids[t], w[t], ex.f64, ex.f64(cfg.E)) for t in toks]
            check_close(got[toks], np.stack([p[0] for p in pairs]), bf16_out=True,
                        what="prefill mode 1 sampled tokens", allow=np.stack([p[1] for p in pairs]))
            yref, allow = native_mx_expert(x64[rows_ref[a:b] // cfg.k], *ex.f64(e))
            check_close(yr, yref, what=f"prefill mode 1 segment of expert {e}", allow=allow)


def test_layer_prefill_nvfp4(L):
    """NVFP4 prefill workload (8192 tokens on the Qwen3-A3B shape): sampled tokens and one expert's segment."""
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
    sizes = np.diff(off_ref)
    e = int(np.argmax(sizes))                                  # the most popular expert: many token tiles
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
