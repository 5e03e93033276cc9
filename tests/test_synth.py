"""The seeded generators produce what the workloads state (shapes, ranges, routing)."""
import numpy as np

import synth
from oracle import moe


def test_shapes_and_ranges():
    cfg = synth.shrink(synth.CONFIGS[3], H=128, I=64, E=8)
    w = synth.expert_weights(cfg, 0, 3)
    assert w["gate_codes"].shape == (64, 64) and w["down_codes"].shape == (128, 32)
    assert w["gate_scales"].shape == (64, 4) and w["down_scales"].shape == (128, 2)
    assert w["gate_scales"].min() >= 119 and w["gate_scales"].max() <= 123
    # the same expert is regenerated bit-identically, other experts differ
    assert np.array_equal(w["up_codes"], synth.expert_weights(cfg, 0, 3)["up_codes"])
    assert not np.array_equal(w["up_codes"], synth.expert_weights(cfg, 0, 4)["up_codes"])
    x = synth.tokens(synth.CONFIGS[2], 4)
    assert x.dtype == np.uint16 and x.shape == (4, 2048)


def test_zipf_popularity():
    p = synth.zipf_popularity(256, 1.1)
    assert abs(p.sum() - 1) < 1e-12 and np.all(np.diff(p) < 0)
    assert abs(p[0] - 1 / np.sum(np.arange(1, 257) ** -1.1)) < 1e-15


def test_cache_trace_logits_reproduce_ids():
    cfg = synth.CONFIGS[5]
    tr = synth.cache_trace(cfg, steps=40, n_layers=3)
    for s in range(40):
        for l in range(3):
            ids = moe.topk(tr.logits[s, l][None, :], cfg.k)[0]
            assert ids.tolist() == tr.ids[s, l].tolist()
            assert moe.topk_margin(tr.logits[s, l][None, :], cfg.k)[0] >= 3.75
            assert len(set(tr.ids[s, l].tolist())) == cfg.k


def test_prefill_logits_are_skewed():
    cfg = synth.CONFIGS[4]
    l = synth.prefill_logits(cfg, 2048)
    ids = moe.topk(l, cfg.k)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    top = synth.rank_to_expert(cfg, 0)[0]
    assert counts.argmax() == top and counts[top] > 0.7 * 2048


def test_nvfp4_shapes_and_ranges():
    cfg = synth.shrink(synth.CONFIGS[6], H=128, I=64, E=8)
    w = synth.expert_weights(cfg, 0, 2)
    assert w.fmt == "nvfp4"
    assert w["gate_codes"].shape == (64, 64) and w["down_codes"].shape == (128, 32)
    assert w["gate_scales"].shape == (64, 8) and w["down_scales"].shape == (128, 4)
    assert w["gate_scales"].min() >= 0x30 and w["gate_scales"].max() <= 0x40
    ts = w["tensor_scales"]
    assert ts.dtype == np.float32 and ts.shape == (3,) and (ts >= 0.01).all() and (ts <= 0.03).all()
