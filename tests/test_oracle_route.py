"""Pins of the oracle's router: top-k against brute force, gating closed forms."""
import itertools
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import moe


def _cases(golden_dir):
    out = []
    with open(os.path.join(golden_dir, "gating_closed_forms.txt")) as f:
        for line in f:
            line = line.strip()
            if not line.startswith("case "):
                continue
            head, logits, ids, w = [p.strip() for p in line.split(";")]
            _, name, E, k, gating, renorm = head.split()
            out.append(dict(name=name, E=int(E), k=int(k), gating=gating, renorm=bool(int(renorm)),
                            logits=np.array([float(v) for v in logits.split()], np.float32),
                            ids=[int(v) for v in ids.split()],
                            w=[float(v) for v in w.split()]))
    return out


def test_gating_closed_forms(golden_dir):
    cases = _cases(golden_dir)
    assert len(cases) >= 6
    for c in cases:
        l = c["logits"][None, :]
        ids = moe.topk(l, c["k"])
        assert ids[0].tolist() == c["ids"], c["name"]
        w = moe.gating_weights(l, ids, c["gating"], c["renorm"])
        np.testing.assert_allclose(w[0], c["w"], rtol=1e-14, atol=0, err_msg=c["name"])


def _brute_topk(row, k):
    """Every ordering of all indices; keep the ones sorted by (-l, idx); take the first k."""
    E = len(row)
    best = None
    for perm in itertools.permutations(range(E)):
        ok = all((-row[perm[i]], perm[i]) < (-row[perm[i + 1]], perm[i + 1]) for i in range(E - 1))
        if ok:
            best = perm
            break
    return list(best[:k])


@settings(max_examples=150, deadline=None)
@given(E=st.integers(1, 6), data=st.data())
def test_topk_brute_force(E, data):
    k = data.draw(st.integers(1, E))
    # small integer-valued logits force many ties
    vals = data.draw(st.lists(st.integers(-2, 2), min_size=E, max_size=E))
    row = np.array(vals, np.float32)
    got = moe.topk(row[None, :], k)[0].tolist()
    assert got == _brute_topk([float(v) for v in row], k)


def test_topk_k_equals_E_is_full_sort_and_ties_to_lower_index():
    rng = np.random.default_rng(1)
    l = rng.integers(-3, 4, size=(20, 9)).astype(np.float32)
    ids = moe.topk(l, 9)
    for t in range(20):
        keys = [(-l[t, e], e) for e in ids[t]]
        assert keys == sorted(keys)
        assert sorted(ids[t].tolist()) == list(range(9))
    # all equal -> 0..k-1
    assert moe.topk(np.zeros((1, 7), np.float32), 4)[0].tolist() == [0, 1, 2, 3]


def test_topk_matches_torch_when_distinct():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((64, 256)).astype(np.float32)
    ids = moe.topk(l, 6)
    ref = torch.topk(torch.from_numpy(l), 6, dim=1, sorted=True).indices.numpy()
    assert np.array_equal(ids, ref)


def test_softmax_k_equals_E_sums_to_one_and_matches_torch():
    rng = np.random.default_rng(3)
    l = (rng.standard_normal((10, 16)) * 4).astype(np.float32)
    ids = moe.topk(l, 16)
    w = moe.gating_weights(l, ids, "softmax", False)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    p = torch.softmax(torch.from_numpy(l).double(), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-13)


def test_sigmoid_matches_torch_and_renorm():
    rng = np.random.default_rng(4)
    l = (rng.standard_normal((10, 32)) * 10).astype(np.float32)
    ids = moe.topk(l, 5)
    w = moe.gating_weights(l, ids, "sigmoid", False)
    s = torch.sigmoid(torch.from_numpy(l).double()).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(s, ids.astype(np.int64), 1), rtol=1e-13)
    wr = moe.gating_weights(l, ids, "sigmoid", True)
    np.testing.assert_allclose(wr.sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(wr, w / w.sum(1, keepdims=True), rtol=1e-14)
    # extreme logits stay finite
    big = np.array([[-800.0, 800.0]], np.float32)
    assert np.all(np.isfinite(moe.gating_weights(big, moe.topk(big, 2), "sigmoid", False)))


def test_router_logits_are_fp32_of_exact_sum():
    x = np.array([[1.0, 2.0 ** -30, -1.0]])
    w = np.array([[1.0, 1.0, 1.0]])
    # float64 keeps 2^-30 through the cancellation; float32 storage keeps it too
    assert moe.router_logits(x, w)[0, 0] == np.float32(2.0 ** -30)


def test_margin():
    l = np.array([[3, 1, 2, 2]], np.float32)
    assert moe.topk_margin(l, 1)[0] == 1.0
    assert moe.topk_margin(l, 2)[0] == 0.0
    assert moe.topk_margin(l, 4)[0] == np.inf


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        moe.topk(np.zeros((1, 3), np.float32), 4)
