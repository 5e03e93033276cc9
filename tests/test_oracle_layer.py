"""Pins of the oracle's permutation, SwiGLU expert, combine and whole layer."""
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import formats, moe
import synth


# --------------------------------------------------------------------------- permutation

def _brute_permute(ids, E):
    flat = [int(v) for v in np.asarray(ids).ravel()]
    rows = []
    offsets = [0]
    for e in range(E):
        seg = [r for r in range(len(flat)) if flat[r] == e]
        rows += seg
        offsets.append(len(rows))
    pos = [0] * len(flat)
    for i, r in enumerate(rows):
        pos[r] = i
    return offsets, rows, pos


@settings(max_examples=100, deadline=None)
@given(T=st.integers(0, 12), E=st.integers(1, 9), data=st.data())
def test_permute_brute_force(T, E, data):
    k = data.draw(st.integers(1, E))
    ids = np.array(data.draw(st.lists(st.integers(0, E - 1), min_size=T * k, max_size=T * k)),
                   dtype=np.int32).reshape(T, k)
    off, rows, pos = moe.permute(ids, E)
    bo, br, bp = _brute_permute(ids, E)
    assert off.tolist() == bo and rows.tolist() == br and pos.tolist() == bp


def test_permute_invariants_large():
    cfg = synth.CONFIGS[4]
    l = synth.prefill_logits(cfg, 512)
    ids = moe.topk(l, cfg.k)
    off, rows, pos = moe.permute(ids, cfg.E)
    flat = ids.ravel()
    assert off[0] == 0 and off[-1] == flat.size and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=cfg.E))
    assert np.array_equal(np.sort(rows), np.arange(flat.size))
    for e in range(cfg.E):
        seg = rows[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    assert np.array_equal(pos[rows], np.arange(flat.size))


def test_permute_rejects_out_of_range():
    with pytest.raises(ValueError):
        moe.permute(np.array([[0, 3]]), 3)


# --------------------------------------------------------------------------- SwiGLU expert

def _worked(golden_dir):
    out = []
    with open(os.path.join(golden_dir, "swiglu_worked.txt")) as f:
        for line in f:
            if not line.startswith("case "):
                continue
            parts = [p.strip() for p in line.split(";")]
            _, name, H, I = parts[0].split()
            mat = lambda s: np.array([[float(v) for v in r.split()] for r in s.split("|")])
            out.append(dict(name=name, H=int(H), I=int(I),
                            x=np.array([float(v) for v in parts[1].split()]),
                            wg=mat(parts[2]), wu=mat(parts[3]), wd=mat(parts[4]),
                            y=np.array([float(v) for v in parts[5].split()])))
    return out


def test_swiglu_worked_examples(golden_dir):
    cases = _worked(golden_dir)
    assert len(cases) == 2
    for c in cases:
        assert c["wg"].shape == (c["I"], c["H"]) and c["wd"].shape == (c["H"], c["I"])
        y = moe.swiglu_expert(c["x"][None, :], c["wg"], c["wu"], c["wd"])[0]
        np.testing.assert_allclose(y, c["y"], rtol=1e-15, atol=1e-15, err_msg=c["name"])


def test_swiglu_matches_torch_silu():
    rng = np.random.default_rng(7)
    H, I, n = 24, 10, 5
    X = rng.standard_normal((n, H))
    Wg, Wu, Wd = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    y, h = moe.swiglu_expert(X, Wg, Wu, Wd, return_hidden=True)
    tX = torch.from_numpy(X)
    th = torch.nn.functional.silu(tX @ torch.from_numpy(Wg).T) * (tX @ torch.from_numpy(Wu).T)
    ty = th @ torch.from_numpy(Wd).T
    np.testing.assert_allclose(h, th.numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y, ty.numpy(), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- whole layer

def _tiny_experts(rng, E, H, I):
    W = [(rng.standard_normal((I, H)) * 0.3, rng.standard_normal((I, H)) * 0.3,
          rng.standard_normal((H, I)) * 0.3) for _ in range(E)]
    return W


@pytest.mark.parametrize("gating,renorm", [("softmax", False), ("softmax", True), ("sigmoid", False)])
def test_k_equals_E_collapses_to_dense_mixture(gating, renorm):
    rng = np.random.default_rng(11)
    T, H, I, E = 7, 12, 5, 6
    x = rng.standard_normal((T, H))
    W = _tiny_experts(rng, E, H, I)
    wr = rng.standard_normal((E, H))
    shared = (rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I)))
    r = moe.moe_layer(x, k=E, E=E, gating=gating, renormalize=renorm, experts=lambda e: W[e],
                      shared=shared, w_router=wr)
    # dense: every expert on every token, weighted by its gate; no permutation involved
    l = (x @ wr.T).astype(np.float32).astype(np.float64)
    if gating == "softmax":
        g = np.exp(l - l.max(1, keepdims=True))
        g /= g.sum(1, keepdims=True)
    else:
        g = 1 / (1 + np.exp(-l))
        if renorm:
            g /= g.sum(1, keepdims=True)
    dense = np.zeros((T, H))
    for e in range(E):
        Wg, Wu, Wd = W[e]
        dense += g[:, e:e + 1] * ((x @ Wg.T) / (1 + np.exp(-(x @ Wg.T))) * (x @ Wu.T)) @ Wd.T
    Wg, Wu, Wd = shared
    dense += ((x @ Wg.T) / (1 + np.exp(-(x @ Wg.T))) * (x @ Wu.T)) @ Wd.T
    np.testing.assert_allclose(r["out"], dense, rtol=1e-12, atol=1e-12)


def test_one_hot_routing_reproduces_single_expert():
    rng = np.random.default_rng(12)
    T, H, I, E = 5, 16, 6, 8
    x = rng.standard_normal((T, H))
    W = _tiny_experts(rng, E, H, I)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    target = [3, 0, 7, 3, 5]
    for t, e in enumerate(target):
        logits[t, e] = 30.0
    r = moe.moe_layer(x, k=1, E=E, gating="softmax", renormalize=True, experts=lambda e: W[e],
                      logits=logits)
    assert r["ids"][:, 0].tolist() == target
    np.testing.assert_array_equal(r["w"], 1.0)
    for t, e in enumerate(target):
        Wg, Wu, Wd = (torch.from_numpy(a) for a in W[e])
        xt = torch.from_numpy(x[t:t + 1])
        ref = (torch.nn.functional.silu(xt @ Wg.T) * (xt @ Wu.T)) @ Wd.T
        np.testing.assert_allclose(r["out"][t], ref.numpy()[0], rtol=1e-12, atol=1e-12)


def test_token_output_matches_layer():
    cfg = synth.shrink(synth.CONFIGS[3], H=64, I=32, E=12, k=3)
    T = 6
    x = formats.activations_to_f64("bf16", synth.tokens(cfg, T))
    W = {e: formats.expert_to_f64("mxfp4", synth.expert_weights(cfg, 0, e).arrays) for e in range(cfg.E + 1)}
    wr = formats.bf16_to_f64(synth.router_weight(cfg))
    r = moe.moe_layer(x, k=cfg.k, E=cfg.E, gating="sigmoid", renormalize=False,
                      experts=lambda e: W[e], shared=W[cfg.E], w_router=wr)
    for t in range(T):
        o = moe.token_output(x[t], r["ids"][t], r["w"][t], lambda e: W[e], W[cfg.E])
        np.testing.assert_allclose(o, r["out"][t], rtol=1e-12, atol=1e-12)


def test_combine_uses_row_pos():
    # two tokens, k=2; y_rows in permuted order; w and row_pos picked by hand
    y_rows = np.array([[1.0, 0], [0, 1.0], [10.0, 0], [0, 10.0]])
    w = np.array([[0.5, 2.0], [1.0, 3.0]])
    row_pos = np.array([2, 0, 1, 3])  # (t0,j0)->2, (t0,j1)->0, (t1,j0)->1, (t1,j1)->3
    out = moe.combine(y_rows, w, row_pos, np.array([[1.0, 1.0], [0, 0]]), 2, 2)
    assert out.tolist() == [[0.5 * 10 + 2.0 * 1 + 1, 1.0], [0.0, 1.0 + 30.0]]
