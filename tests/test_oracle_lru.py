"""Pins of the LRU simulator: hand traces, textbook LRU, compulsory misses, capacity."""
import os
from collections import OrderedDict

import numpy as np
import pytest

from oracle.lru import CapacityError, ExpertLRU
from oracle import policy


def _traces(golden_dir):
    traces = []
    cur = None
    with open(os.path.join(golden_dir, "lru_traces.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = line.split()
            if w[0] == "trace":
                kv = dict(p.split("=") for p in w[2:])
                cur = dict(name=w[1], C=int(kv["capacity"]), L=int(kv["layers"]),
                           E=int(kv["experts"]), steps=[])
            elif w[0] == "step":
                left, right = line.split(":", 1)
                lw = left.split()
                ids = [int(v) for v in lw[5].split(",")]
                evs = []
                rt = right.split()
                fill = None
                if "fill" in rt:
                    fill = int(rt[rt.index("fill") + 1])
                    rt = rt[:rt.index("fill")]
                for tok in rt:
                    e, rest = tok.split(":")
                    hm, rest = rest.split("@")
                    if "/" in rest:
                        s, ev = rest.split("/")
                        evl, eve = ev.split(".")
                        evicted = (int(evl), int(eve))
                    else:
                        s, evicted = rest, None
                    evs.append((int(e), hm == "H", int(s), evicted))
                cur["steps"].append((int(lw[1]), int(lw[3]), ids, evs))
                cur.setdefault("fill", {})[len(cur["steps"]) - 1] = fill
            elif w[0] == "prefetch":
                left, right = line.split(":", 1)
                evs = []
                for tok in right.split():
                    e, rest = tok.split(":")
                    hm, rest = rest.split("@")
                    if "/" in rest:
                        s_, ev = rest.split("/")
                        evl, eve = ev.split(".")
                        evicted = (int(evl), int(eve))
                    else:
                        s_, evicted = rest, None
                    evs.append((int(e), hm == "H", int(s_), evicted))
                cur["steps"].append(("prefetch", int(left.split()[1]), None, evs))
            elif w[0] == "resize":
                left, right = line.split(":", 1)
                rw = right.split()
                i = rw.index("drops")
                keeps = [tuple(int(v) for v in t.split(">")) for t in rw[1:i]]
                drops = [tuple(int(v) for v in t.split(".")) for t in rw[i + 1:]]
                cur["steps"].append(("resize", int(left.split()[1]), keeps, drops))
            elif w[0] == "totals":
                cur["totals"] = {k: int(v) for k, v in (p.split("=") for p in w[1:])}
            elif w[0] == "stamps":
                cur["stamps"] = [int(v) for v in w[1].split(",")]
            elif w[0] == "end":
                traces.append(cur)
    return traces


def test_hand_traced_sequences(golden_dir):
    traces = _traces(golden_dir)
    assert [t["name"] for t in traces] == ["A", "B", "C", "D", "E", "F", "G", "H"]
    for tr in traces:
        lru = ExpertLRU(tr["L"], tr["E"], tr["C"])
        for i, (step, layer, ids, want) in enumerate(tr["steps"]):
            if step == "resize":
                assert lru.resize(layer) == (ids, want), (tr["name"], "resize", layer)
                continue
            fill = tr.get("fill", {}).get(i)
            got = lru.prefetch(layer) if step == "prefetch" else lru.step(layer, ids, fill)
            assert [(e.expert, e.hit, e.slot, e.evicted) for e in got] == want, (tr["name"], step, layer)
        assert {k: getattr(lru, k) for k in tr["totals"]} == tr["totals"], tr["name"]
        assert lru.stamp == tr["stamps"], tr["name"]


def _textbook_lru(accesses, capacity):
    """Plain LRU with an OrderedDict; returns the hit/miss sequence."""
    od = OrderedDict()
    seq = []
    for key in accesses:
        if key in od:
            od.move_to_end(key)
            seq.append(True)
        else:
            if len(od) >= capacity:
                od.popitem(last=False)
            od[key] = True
            seq.append(False)
    return seq


def test_single_access_steps_equal_textbook_lru():
    rng = np.random.default_rng(0)
    for trial in range(20):
        L, E, C = int(rng.integers(1, 4)), int(rng.integers(2, 12)), int(rng.integers(1, 8))
        acc = [(int(rng.integers(L)), int(rng.integers(E))) for _ in range(300)]
        lru = ExpertLRU(L, E, C)
        ours = [lru.step(l, [e])[0].hit for l, e in acc]
        assert ours == _textbook_lru(acc, C)
        # resident set equals the textbook's most recent distinct keys
        recent = list(OrderedDict.fromkeys(reversed(acc)))[:C]
        assert set(lru.where) == set(recent)


def test_compulsory_misses_only_when_everything_fits():
    rng = np.random.default_rng(1)
    L, E, k = 3, 10, 3
    lru = ExpertLRU(L, E, L * E)
    seen = set()
    for s in range(50):
        for l in range(L):
            ids = rng.choice(E, size=k, replace=False)
            for ev in lru.step(l, ids):
                assert ev.hit == ((l, ev.expert) in seen)
                seen.add((l, ev.expert))
    assert lru.misses == len(seen) and lru.evictions == 0


def test_capacity_error_leaves_state_unchanged():
    lru = ExpertLRU(1, 8, 2)
    lru.step(0, [1])
    before = (list(lru.owner), list(lru.stamp), dict(lru.where), lru.clock, lru.stats())
    with pytest.raises(CapacityError):
        lru.step(0, [2, 3, 4])
    assert (list(lru.owner), list(lru.stamp), dict(lru.where), lru.clock, lru.stats()) == before


def test_a_miss_never_evicts_a_needed_expert():
    rng = np.random.default_rng(2)
    lru = ExpertLRU(2, 16, 6)
    for s in range(400):
        l = int(rng.integers(2))
        ids = rng.choice(16, size=int(rng.integers(1, 7)), replace=False)
        evs = lru.step(l, ids)
        needed = {(l, int(e)) for e in ids}
        for ev in evs:
            assert ev.evicted not in needed
        assert all(lru.lookup(l, int(e)) >= 0 for e in ids)
        slots = [ev.slot for ev in evs]
        assert len(set(slots)) == len(slots)


def test_resize_keeps_the_most_recent_entries_like_a_textbook_lru():
    # one access per step: the cache is a textbook LRU, and shrinking it keeps
    # exactly the most recently used keys (then it goes on as the smaller LRU)
    rng = np.random.default_rng(11)
    for trial in range(30):
        C0, C1 = int(rng.integers(2, 9)), int(rng.integers(1, 12))
        lru = ExpertLRU(1, 12, C0)
        od = OrderedDict()
        seq = rng.integers(0, 12, size=60)
        cut = int(rng.integers(1, 59))
        for t, e in enumerate(seq):
            if t == cut:
                _, dropped = lru.resize(C1)
                while len(od) > C1:
                    k, _ = od.popitem(last=False)
                    assert (0, k) in dropped
                assert sorted(lru.where) == sorted((0, k) for k in od)
                # kept entries sit in slots 0.. in ascending old-slot order
                assert sorted(lru.where.values()) == list(range(len(od)))
            e = int(e)
            ev = lru.step(0, [e])[0]
            hit = e in od
            assert ev.hit == hit
            if hit:
                od.move_to_end(e)
            else:
                if len(od) == lru.capacity:
                    od.popitem(last=False)
                od[e] = True
            assert sorted(k[1] for k in lru.where) == sorted(od)


def test_resize_grow_moves_nothing_and_shrink_never_moves_up():
    rng = np.random.default_rng(12)
    lru = ExpertLRU(2, 50, 20)
    for t in range(40):
        lru.step(t % 2, rng.choice(50, size=5, replace=False))
    before = dict(lru.where)
    moves, dropped = lru.resize(30)
    assert dropped == [] and all(a == b for a, b in moves) and lru.where == before
    moves, dropped = lru.resize(7)
    assert len(dropped) == 13 and all(b <= a for a, b in moves)
    assert lru.evictions >= 13 and len(lru.where) == 7 and lru.owner.count(None) == 0


def test_prefetched_layer_steps_are_all_hits():
    # with room for two layers and the order route(l) -> prefetch(l+1) -> compute(l),
    # every routed access of layer l+1 is a hit, whatever its routing, and a prefetch
    # never evicts the layer being computed
    rng = np.random.default_rng(13)
    L, E = 5, 10
    lru = ExpertLRU(L, E, 2 * E)
    lru.prefetch(0)
    for l in range(L):
        ids = rng.integers(0, E, size=12)
        assert all(ev.hit for ev in lru.step(l, ids))
        if l + 1 < L:
            evs = lru.prefetch(l + 1)
            assert all(ev.evicted is None or ev.evicted[0] != l for ev in evs)
    assert lru.misses == 0 and lru.prefetch_fills == L * E


def test_fill_limit_split():
    # an unlimited step is the plain step; the filled misses are the lowest ids;
    # CPU misses leave the cache exactly as it was
    rng = np.random.default_rng(21)
    for trial in range(40):
        a, b = ExpertLRU(2, 30, 8), ExpertLRU(2, 30, 8)
        for t in range(30):
            layer = int(rng.integers(2))
            ids = rng.choice(30, size=int(rng.integers(1, 6)), replace=False)
            ea = a.step(layer, ids)
            eb = b.step(layer, ids, fill_limit=len(ids))
            assert ea == eb
        before = (dict(b.where), list(b.stamp), b.clock)
        ids = rng.choice(30, size=6, replace=False)
        misses = sorted(int(e) for e in ids if (0, int(e)) not in b.where)
        evs = b.step(0, ids, fill_limit=0)
        hits = [e for e in evs if e.hit]
        assert [e.expert for e in evs if not e.hit] == misses and all(e.slot == -1 for e in evs if not e.hit)
        if not hits:
            assert (dict(b.where), list(b.stamp), b.clock) == before
        q = int(rng.integers(0, len(misses) + 1))
        c = ExpertLRU(1, 30, 8)
        evs = c.step(0, ids, fill_limit=q)
        filled = [e.expert for e in evs if not e.hit and e.slot >= 0]
        assert filled == sorted(int(e) for e in ids)[:q]
        assert c.cpu_misses == len(ids) - q and c.misses == len(ids)


def test_miss_split_policy():
    # equal bandwidths split evenly; monotone in B_p, antitone in B_h; clamped to 0..m
    assert policy.miss_split(6, 1.0, 1.0) == 3
    assert policy.miss_split(0, 5.0, 1.0) == 0
    assert policy.miss_split(4, 1.0, 0.0) == 4 and policy.miss_split(4, 0.0, 1.0) == 0
    prev = -1
    for bp in [0.1, 0.5, 1, 2, 5, 10, 50]:
        q = policy.miss_split(10, bp, 5.0)
        assert 0 <= q <= 10 and q >= prev
        prev = q
    # the integer split sits next to the balance point q* = m Bp / (Bp + Bh)
    rng = np.random.default_rng(3)
    for _ in range(200):
        m = int(rng.integers(1, 40))
        bp, bh = float(rng.uniform(0.1, 100)), float(rng.uniform(0.1, 100))
        q = policy.miss_split(m, bp, bh)
        assert abs(q - m * bp / (bp + bh)) < 1.0
    # worked example: m=7, Bp=3, Bh=11 -> q*=1.5; q=1 gives max(1/3, 6/11)=0.545,
    # q=2 gives max(2/3, 5/11)=0.667, so one fill
    assert policy.miss_split(7, 3.0, 11.0) == 1
    # m=7, Bp=Bh: q=3 -> max(3, 4)=4, q=4 -> max(4, 3)=4: tie -> more fills
    assert policy.miss_split(7, 1.0, 1.0) == 4
    assert policy.split_misses([9, 2, 5], 1.0, 1.0) == ([2, 5], [9])


def test_prefetch_never_takes_the_last_steps_slots():
    # capacity between E and 2E: a prefetch evicts no entry the last routed step needed, fills
    # exactly min(missing, free-of-protection slots) experts (the lowest missing ids), and an
    # expert it leaves out is simply a miss of its own step later
    rng = np.random.default_rng(17)
    for trial in range(60):
        L, E = 3, int(rng.integers(3, 9))
        C = int(rng.integers(E, 2 * E))
        lru = ExpertLRU(L, E, C)
        for st in range(12):
            l = st % L
            ids = rng.integers(0, E, size=int(rng.integers(1, min(E, C) + 1)))
            lru.step(l, ids)
            needed = {(l, int(e)) for e in ids}
            slots_needed = {lru.where[k] for k in needed}
            missing = [e for e in range(E) if ((l + 1) % L, e) not in lru.where]
            room = sum(1 for s in range(C)
                       if lru.owner[s] not in needed and (lru.owner[s] is None or lru.owner[s][0] != (l + 1) % L))
            evs = lru.prefetch((l + 1) % L)
            filled = [ev.expert for ev in evs if not ev.hit and ev.slot >= 0]
            skipped = [ev.expert for ev in evs if not ev.hit and ev.slot < 0]
            assert filled == missing[:min(len(missing), room)] and skipped == missing[len(filled):]
            assert all(ev.slot not in slots_needed for ev in evs if not ev.hit and ev.slot >= 0)
            assert all(lru.where.get(k) is not None for k in needed)      # still resident
