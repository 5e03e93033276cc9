"""The parity helpers themselves: the near-tie top-k validity check accepts exactly the valid
alternatives and rejects wrong picks (CPU only)."""
import numpy as np
import pytest

from oracle import moe
from tests.helpers import check_topk_valid


def _logits():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((4, 10)).astype(np.float32)
    # token 1: the 3rd and 4th largest within 5e-5 of each other
    order = np.argsort(-l[1])
    l[1, order[3]] = l[1, order[2]] - np.float32(5e-5)
    return l, order


def test_oracle_ids_are_valid_and_equal():
    l, _ = _logits()
    ids = moe.topk(l, 3)
    assert check_topk_valid(ids, l, 3).size == 0


def test_near_tie_swap_is_valid_and_reported():
    l, order = _logits()
    ids = moe.topk(l, 3)
    ids[1, 2] = order[3]                 # the near-tied 4th instead of the 3rd
    assert check_topk_valid(ids, l, 3).tolist() == [1]


def test_wrong_pick_is_rejected():
    l, _ = _logits()
    ids = moe.topk(l, 3)
    ids[0, 2] = int(np.argmin(l[0]))     # far below the 3rd largest
    with pytest.raises(AssertionError):
        check_topk_valid(ids, l, 3)


def test_duplicate_pick_is_rejected():
    l, _ = _logits()
    ids = moe.topk(l, 3)
    ids[2, 1] = ids[2, 0]
    with pytest.raises(AssertionError):
        check_topk_valid(ids, l, 3)


def test_swap_beyond_the_margin_is_rejected():
    l, order = _logits()
    ids = moe.topk(l, 3)
    ids[0, 2] = np.argsort(-l[0])[3]     # token 0 has no near tie at the boundary
    assert l[0, np.argsort(-l[0])[2]] - l[0, np.argsort(-l[0])[3]] > 1e-4
    with pytest.raises(AssertionError):
        check_topk_valid(ids, l, 3)
