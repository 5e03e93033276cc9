"""Parity of the device LRU expert cache and its miss fills against the oracle simulator."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import formats, moe, policy
from oracle.lru import CapacityError, ExpertLRU
from tests.helpers import Experts, check_close
from tests.test_oracle_lru import _traces

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from expert_cached_ffn_amd import layer, ops
    ops.version()
    return ops, layer


class Rig:
    """A cache over n_layers x E small experts with an identifiable pinned host bank."""

    def __init__(self, ops, n_layers, E, C, H=128, I=128, wdtype=1, fill=True):
        self.ops = ops
        self.lay = ops.ft_expert_layout_init(wdtype, H, I)
        self.eb = int(self.lay.expert_bytes)
        self.n_layers, self.E, self.C = n_layers, E, C
        self.bank = torch.empty((n_layers * E, self.eb), dtype=torch.uint8, pin_memory=True)
        if fill:
            rng = np.random.default_rng(n_layers * 1000 + E)
            self.bank.numpy()[:] = rng.integers(0, 256, size=self.bank.shape, dtype=np.uint8)
        self.pool = torch.zeros((C, self.eb), dtype=torch.uint8, device="cuda")
        self.copy_stream = torch.cuda.Stream()
        self.cache = ops.ExpertCache(self.lay, n_layers, E, C, self.pool, self.bank, self.copy_stream,
                                     trace_events=1 << 20)
        self.slot_of = torch.empty(E, dtype=torch.int32, device="cuda")

    def set_split(self, b_pcie, b_host):
        """Steps of this rig have k = 1 and at most 64 ids."""
        self.cache.set_split(b_pcie, b_host, 64, 1)

    def step(self, layer, ids):
        ids = np.asarray(ids, np.int32).reshape(-1)
        d = torch.from_numpy(ids).cuda() if ids.size else torch.zeros(1, dtype=torch.int32, device="cuda")
        self.cache.step(layer, d, ids.size, 1, self.slot_of)

    def resize(self, C, in_place):
        """Resize to C slots: in the current pool (C <= its slots) or into a fresh one."""
        if not in_place:
            self.pool = torch.zeros((C, self.eb), dtype=torch.uint8, device="cuda")
        self.cache.resize(C, self.pool)
        self.C = C


def _split_for(q, m):
    """Bandwidths (b_pcie, b_host) for which the miss split of m misses is exactly q
    (q = None or q = m: every miss filled; the split is then off)."""
    if q is None or q == m:
        return 1.0, 0.0
    return float(q), float(m - q)


def events_by_step(trace):
    out = {}
    for step, layer, e, hit, slot, ev in trace:
        out.setdefault(step, []).append((e, bool(hit), slot, None if ev < 0 else ev))
    return out


def test_hand_traced_sequences_on_device(env, golden_dir):
    ops, _ = env
    for tr in _traces(golden_dir):
        print(f"trace {tr['name']}", flush=True)
        rig = Rig(ops, tr["L"], tr["E"], tr["C"], fill=False)
        E = tr["E"]
        want, n_steps = [], 0
        for i, (kind, layer, ids, evs) in enumerate(tr["steps"]):
            if kind == "resize":
                rig.resize(layer, in_place=layer <= rig.C)
                continue
            if kind == "prefetch":
                rig.cache.prefetch_layer(layer)
                code = {True: 3, False: 2, None: 5}       # 5: not prefetched for lack of room
            else:
                rig.set_split(*_split_for(tr.get("fill", {}).get(i), sum(not h for _, h, _, _ in evs)))
                rig.step(layer, ids)
                code = {True: 1, False: 0, None: 4}       # 4: left to the host CPU
            want += [(n_steps, layer, e, code[h if s >= 0 or h else None], s,
                      -1 if ev is None else ev[0] * E + ev[1]) for e, h, s, ev in evs]
            n_steps += kind != "prefetch"
        assert rig.cache.trace() == want, tr["name"]
        st = rig.cache.stats()
        assert {k: st[k] for k in tr["totals"]} == tr["totals"]
        rig.cache.destroy()


def _compare_run(rig, steps):
    """steps: list of (layer, ids). Runs both; checks events, slot tables, stats and filled bytes."""
    sim = ExpertLRU(rig.n_layers, rig.E, rig.C)
    E = rig.E
    n_ok = 0
    for layer, ids in steps:
        try:
            want = sim.step(layer, ids)
            cap = False
        except CapacityError:
            cap = True
        if cap:
            with pytest.raises(rig.ops.FtError) as ei:
                rig.step(layer, ids)
            assert ei.value.status == -3
            continue
        rig.step(layer, ids)
        torch.cuda.synchronize()
        table = rig.slot_of.cpu().numpy()
        assert table.tolist() == sim.slot_of_expert(layer)
        n_ok += 1
        # the filled slots hold exactly the host blobs of their (layer, expert)
        for ev in want:
            if not ev.hit:
                src = rig.bank[layer * E + ev.expert]
                assert torch.equal(rig.pool[ev.slot].cpu(), src)
    got = events_by_step(rig.cache.trace())
    want_all = {}
    sim2 = ExpertLRU(rig.n_layers, rig.E, rig.C)
    i = 0
    for layer, ids in steps:
        try:
            evs = sim2.step(layer, ids)
        except CapacityError:
            continue
        if evs:  # a step with no routed rows records no event
            want_all[i] = [(e.expert, e.hit, e.slot, None if e.evicted is None else e.evicted[0] * E + e.evicted[1])
                           for e in evs]
        i += 1
    assert got == want_all
    st = rig.cache.stats()
    assert (st["accesses"], st["hits"], st["misses"], st["evictions"]) == \
        (sim.accesses, sim.hits, sim.misses, sim.evictions)
    assert st["steps"] == n_ok
    assert st["bytes_h2d"] == sim.misses * rig.eb
    return sim


def test_random_multi_token_traces(env):
    ops, _ = env
    rng = np.random.default_rng(5)
    rig = Rig(ops, 3, 20, 9)
    steps = []
    for s in range(150):
        layer = int(rng.integers(3))
        T = int(rng.integers(0, 4))
        ids = [rng.choice(20, size=2, replace=False) for _ in range(T)]
        steps.append((layer, np.array(ids, np.int32).reshape(-1)))
    steps.insert(40, (1, np.arange(12, dtype=np.int32)))   # 12 distinct > 9 slots -> capacity error
    _compare_run(rig, steps)
    rig.cache.destroy()


def test_resize_against_the_simulator(env):
    """Shrink in place, grow into a new pool, shrink into a new pool, between random steps:
    slot table, the bytes of every resident slot, later events and totals follow the oracle."""
    ops, _ = env
    rng = np.random.default_rng(17)
    L, E = 3, 24
    rig = Rig(ops, L, E, 12)
    sim = ExpertLRU(L, E, 12)

    def check_resident():
        for (layer, e), slot in sim.where.items():
            assert rig.cache.lookup(layer, e) == slot
            assert torch.equal(rig.pool[slot].cpu(), rig.bank[layer * E + e])
        n_res = sum(rig.cache.lookup(l, e) >= 0 for l in range(L) for e in range(E))
        assert n_res == len(sim.where)

    plan = {25: (5, True), 50: (16, False), 80: (7, False), 95: (7, True)}
    for t in range(120):
        if t in plan:
            C, in_place = plan[t]
            sim.resize(C)
            rig.resize(C, in_place)
            check_resident()
        layer = int(rng.integers(L))
        ids = rng.choice(E, size=int(rng.integers(1, 4)), replace=False).astype(np.int32)
        want = sim.step(layer, ids)
        rig.step(layer, ids)
        torch.cuda.synchronize()
        assert rig.slot_of.cpu().numpy().tolist() == sim.slot_of_expert(layer)
        for ev in want:
            if not ev.hit:
                assert torch.equal(rig.pool[ev.slot].cpu(), rig.bank[layer * E + ev.expert])
    st = rig.cache.stats()
    assert (st["accesses"], st["hits"], st["misses"], st["evictions"]) == \
        (sim.accesses, sim.hits, sim.misses, sim.evictions)
    rig.cache.destroy()


def test_bad_expert_id_is_rejected_without_state_change(env):
    ops, _ = env
    rig = Rig(ops, 1, 8, 4)
    rig.step(0, [1, 2])
    with pytest.raises(ops.FtError) as ei:
        rig.step(0, [3, 8])
    assert ei.value.status == -1
    rig.step(0, [2, 3])
    evs = events_by_step(rig.cache.trace())
    assert evs[1] == [(2, True, 1, None), (3, False, 2, None)]
    rig.cache.destroy()


def test_full_decode_trace_exact(env):
    """The whole 8-layer x 512-step Zipf + reuse trace at 25 % capacity (small experts)."""
    ops, _ = env
    cfg = synth.CONFIGS[5]
    tr = synth.cache_trace(cfg)
    rig = Rig(ops, cfg.n_layers, cfg.E, cfg.capacity, fill=False)
    steps = [(l, tr.ids[s, l]) for s in range(cfg.steps) for l in range(cfg.n_layers)]
    print(f"trace of {len(steps)} layer-steps", flush=True)
    sim = ExpertLRU(cfg.n_layers, cfg.E, cfg.capacity)
    for layer, ids in steps:
        sim.step(layer, ids)
        rig.step(layer, ids)
    got = rig.cache.trace()
    st = rig.cache.stats()
    assert (st["accesses"], st["hits"], st["misses"], st["evictions"]) == \
        (sim.accesses, sim.hits, sim.misses, sim.evictions)
    assert st["accesses"] == cfg.steps * cfg.n_layers * cfg.k
    # event-by-event equality with a fresh simulator run
    sim2 = ExpertLRU(cfg.n_layers, cfg.E, cfg.capacity)
    want = []
    for i, (layer, ids) in enumerate(steps):
        for e in sim2.step(layer, ids):
            want.append((i, layer, e.expert, int(e.hit), e.slot,
                         -1 if e.evicted is None else e.evicted[0] * cfg.E + e.evicted[1]))
    assert got == want
    print(f"hit rate {st['hits'] / st['accesses']:.4f}", flush=True)
    rig.cache.destroy()


def test_layer_outputs_through_the_cache(env):
    """Reduced decode trace: route (given logits) -> cache step -> permute -> FFN from slots -> combine."""
    ops, Lm = env
    cfg = synth.shrink(synth.CONFIGS[5], H=512, I=512, E=32, n_layers=2, capacity=10, steps=24)
    tr = synth.cache_trace(cfg)
    shape = Lm.LayerShape(cfg.H, cfg.I, cfg.E, cfg.k, cfg.wdtype, cfg.xdtype, cfg.gating, cfg.renormalize, True)
    layer = Lm.MoELayer(shape, 1)
    lay = layer.layout
    eb = int(lay.expert_bytes)
    ex = [Experts(cfg, l) for l in range(cfg.n_layers)]
    bank = torch.empty((cfg.n_layers * cfg.E, eb), dtype=torch.uint8, pin_memory=True)
    for l in range(cfg.n_layers):
        for e in range(cfg.E):
            Lm.pack_expert(lay, ex[l].raw(e).arrays, bank.numpy()[l * cfg.E + e])
    shared = [Lm.as_device_u8([Lm.pack_expert(lay, ex[l].raw(cfg.E).arrays)])[0] for l in range(cfg.n_layers)]
    pool = torch.zeros((cfg.capacity, eb), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    cache = ops.ExpertCache(lay, cfg.n_layers, cfg.E, cfg.capacity, pool, bank, cs)
    slot_of = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    for s in range(cfg.steps):
        for l in range(cfg.n_layers):
            x = synth.tokens(cfg, 1, layer=l, step=s)
            layer.route(1, logits=Lm.to_device(tr.logits[s, l][None, :]))
            cache.step(l, layer.ids, 1, cfg.k, slot_of)
            layer.permute(1)
            layer.ffn(1, Lm.to_device(x), pool, slot_of_expert=slot_of, shared_blob=shared[l])
            layer.combine(1)
            torch.cuda.synchronize()
            got = formats.bf16_to_f64(layer.out[:1].cpu().numpy().view(np.uint16))[0]
            ids = tr.ids[s, l]
            assert layer.ids[0].cpu().numpy().tolist() == ids.tolist()
            w = moe.gating_weights(tr.logits[s, l][None, :], ids[None, :], cfg.gating, cfg.renormalize)[0]
            x64 = formats.activations_to_f64(cfg.xdtype, x)[0]
            ref = moe.token_output(x64, ids, w, ex[l].f64, ex[l].f64(cfg.E))
            check_close(got[None, :], ref[None, :], bf16_out=True, what=f"step {s} layer {l}")
    st = cache.stats()
    assert st["misses"] > 0 and st["hits"] > 0
    cache.destroy()


def test_prefill_double_buffered_through_the_cache(env):
    """Full-layer double buffering: route(l) -> cache step(l) -> prefetch(l+1) -> FFN(l) from the slots.
    With room for two layers every routed access hits; outputs match the oracle; LRU events match."""
    ops, Lm = env
    cfg = synth.shrink(synth.CONFIGS[4], H=512, I=512, E=16, k=4, n_layers=3, capacity=32)
    T = 200
    shape = Lm.LayerShape(cfg.H, cfg.I, cfg.E, cfg.k, cfg.wdtype, cfg.xdtype, cfg.gating, cfg.renormalize, True)
    layer = Lm.MoELayer(shape, T)
    lay = layer.layout
    eb = int(lay.expert_bytes)
    ex = [Experts(cfg, l) for l in range(cfg.n_layers)]
    bank = torch.empty((cfg.n_layers * cfg.E, eb), dtype=torch.uint8, pin_memory=True)
    for l in range(cfg.n_layers):
        for e in range(cfg.E):
            Lm.pack_expert(lay, ex[l].raw(e).arrays, bank.numpy()[l * cfg.E + e])
    shared = [Lm.as_device_u8([Lm.pack_expert(lay, ex[l].raw(cfg.E).arrays)])[0] for l in range(cfg.n_layers)]
    pool = torch.zeros((cfg.capacity, eb), dtype=torch.uint8, device="cuda")
    cache = ops.ExpertCache(lay, cfg.n_layers, cfg.E, cfg.capacity, pool, bank, torch.cuda.Stream())
    slot_of = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    sim = ExpertLRU(cfg.n_layers, cfg.E, cfg.capacity)
    cache.prefetch_layer(0)
    sim.prefetch(0)
    for l in range(cfg.n_layers):
        print(f"prefill layer {l}", flush=True)
        x = synth.tokens(cfg, T, layer=l)
        logits = synth.prefill_logits(cfg, T, layer=l)
        layer.route_permute(T, logits=Lm.to_device(logits))
        cache.step(l, layer.ids, T, cfg.k, slot_of)
        ids = moe.topk(logits, cfg.k)
        assert all(ev.hit for ev in sim.step(l, ids.ravel()))
        if l + 1 < cfg.n_layers:
            cache.prefetch_layer(l + 1)
            sim.prefetch(l + 1)
        layer.ffn(T, Lm.to_device(x), pool, slot_of_expert=slot_of, shared_blob=shared[l])
        layer.combine(T)
        torch.cuda.synchronize()
        got = formats.bf16_to_f64(layer.out[:T].cpu().numpy().view(np.uint16))
        w = moe.gating_weights(logits, ids, cfg.gating, cfg.renormalize)
        x64 = formats.activations_to_f64(cfg.xdtype, x)
        toks = [0, 77, T - 1]
        ref = np.stack([moe.token_output(x64[t], ids[t], w[t], ex[l].f64, ex[l].f64(cfg.E)) for t in toks])
        check_close(got[toks], ref, bf16_out=True, what=f"layer {l}")
    st = cache.stats()
    assert st["misses"] == 0 and st["hits"] == st["accesses"] == sim.accesses
    assert st["prefetch_fills"] == sim.prefetch_fills == cfg.n_layers * cfg.E
    assert st["evictions"] == sim.evictions and st["bytes_h2d"] == cfg.n_layers * cfg.E * eb
    cache.destroy()


def test_split_bandwidths_give_the_intended_fill_count():
    for m in range(0, 9):
        for q in range(0, m + 1):
            bp, bh = _split_for(q, m)
            assert (m if bh == 0 else policy.miss_split(m, bp, bh)) == q


def test_hybrid_split_against_the_simulator(env):
    """Random steps under changing bandwidth pairs: events (CPU misses code 4, slot -1), the CPU
    miss list, slot tables, filled bytes and totals follow the oracle's fill-limited steps."""
    ops, _ = env
    rng = np.random.default_rng(23)
    L, E, C = 3, 24, 10
    rig = Rig(ops, L, E, C)
    sim = ExpertLRU(L, E, C)
    pairs = [(49.3, 0.0), (49.3, 30.0), (25.0, 50.0), (0.0, 10.0), (10.0, 10.0), (3.0, 1.0)]
    want_log = []
    for t in range(160):
        layer = int(rng.integers(L))
        T = int(rng.integers(0, 4))
        ids = np.array([rng.choice(E, size=3, replace=False) for _ in range(T)], np.int32).reshape(-1)
        bp, bh = pairs[int(rng.integers(len(pairs)))]
        needed = sorted(set(ids.tolist()))
        m = sum(sim.slot_of_expert(layer)[e] < 0 for e in needed)
        q = m if bh == 0 else policy.miss_split(m, bp, bh)
        evs = sim.step(layer, ids, fill_limit=q)
        rig.set_split(bp, bh)
        rig.step(layer, ids)
        torch.cuda.synchronize()
        cpu = [e.expert for e in evs if not e.hit and e.slot < 0]
        assert rig.cache.cpu_misses() == cpu
        assert len(cpu) == m - q
        assert rig.slot_of.cpu().numpy().tolist() == sim.slot_of_expert(layer)
        for ev in evs:
            if not ev.hit and ev.slot >= 0:
                assert torch.equal(rig.pool[ev.slot].cpu(), rig.bank[layer * E + ev.expert])
        want_log += [(t, layer, e.expert, 1 if e.hit else (0 if e.slot >= 0 else 4), e.slot,
                      -1 if e.evicted is None else e.evicted[0] * E + e.evicted[1]) for e in evs]
    assert rig.cache.trace() == want_log
    st = rig.cache.stats()
    assert (st["accesses"], st["hits"], st["misses"], st["evictions"], st["cpu_misses"]) == \
        (sim.accesses, sim.hits, sim.misses, sim.evictions, sim.cpu_misses)
    assert sim.cpu_misses > 20
    assert st["bytes_h2d"] == (sim.misses - sim.cpu_misses) * rig.eb
    rig.cache.destroy()


@pytest.mark.parametrize("T,C,hybrid,hits_first", [(1, 10, True, False), (5, 30, True, False),
                                                   (1, 10, False, True), (5, 30, True, True),
                                                   (1, 10, False, "plan"), (5, 30, True, "plan")])
def test_hybrid_layer_outputs(env, T, C, hybrid, hits_first):
    """Decode through the cache, with the CPU miss split (hybrid) and/or the hits-first step (the
    hits' FFN before the fills land, the filled misses' FFN after; "plan": the hits' FFN queued
    between ft_expert_cache_plan and ft_expert_cache_fill): every layer output matches the oracle."""
    ops, Lm = env
    cfg = synth.shrink(synth.CONFIGS[5], H=512, I=512, E=32, n_layers=2, capacity=C, steps=12)
    shape = Lm.LayerShape(cfg.H, cfg.I, cfg.E, cfg.k, cfg.wdtype, cfg.xdtype, cfg.gating, cfg.renormalize, True)
    layer = Lm.MoELayer(shape, T)
    lay = layer.layout
    eb = int(lay.expert_bytes)
    ex = [Experts(cfg, l) for l in range(cfg.n_layers)]
    bank = torch.empty((cfg.n_layers * cfg.E, eb), dtype=torch.uint8, pin_memory=True)
    for l in range(cfg.n_layers):
        for e in range(cfg.E):
            Lm.pack_expert(lay, ex[l].raw(e).arrays, bank.numpy()[l * cfg.E + e])
    shared = [Lm.as_device_u8([Lm.pack_expert(lay, ex[l].raw(cfg.E).arrays)])[0] for l in range(cfg.n_layers)]
    pool = torch.zeros((cfg.capacity, eb), dtype=torch.uint8, device="cuda")
    cache = ops.ExpertCache(lay, cfg.n_layers, cfg.E, cfg.capacity, pool, bank, torch.cuda.Stream())
    if hybrid:
        cache.set_split(2.0, 1.0, T, cfg.k)  # a third of each step's misses on the CPU
    slot_of = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    slot_hits = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    n_cpu = n_two_pass = 0
    for s in range(cfg.steps):
        for l in range(cfg.n_layers):
            x = synth.tokens(cfg, T, layer=l, step=s)
            logits = synth.prefill_logits(cfg, T, case=s, layer=l)
            xd = Lm.to_device(x)
            layer.route_permute(T, logits=Lm.to_device(logits))
            if hits_first == "plan":
                cache.plan(l, layer.ids, T, cfg.k, slot_hits, slot_of)
                layer.ffn(T, xd, pool, slot_of_expert=slot_hits, shared_blob=shared[l])
                n_fill = cache.fill()
            elif hits_first:
                n_fill = cache.step_split(l, layer.ids, T, cfg.k, slot_hits, slot_of)
            else:
                cache.step(l, layer.ids, T, cfg.k, slot_of)
            cpu = cache.cpu_misses()
            n_cpu += len(cpu)
            layer.stage_cpu_misses(cache, T, xd)
            if hits_first:
                if hits_first != "plan":
                    layer.ffn(T, xd, pool, slot_of_expert=slot_hits, shared_blob=shared[l])
                cache.wait_fills()
                if n_fill or cpu:  # the filled misses (and NaN rows for the CPU's, patched next)
                    layer.ffn(T, xd, pool, slot_of_expert=slot_of)
                    n_two_pass += 1
            else:
                layer.ffn(T, xd, pool, slot_of_expert=slot_of, shared_blob=shared[l])
            layer.run_cpu_misses(cache, n_threads=4)
            layer.combine(T)
            torch.cuda.synchronize()
            got = formats.bf16_to_f64(layer.out[:T].cpu().numpy().view(np.uint16))
            ids = moe.topk(logits, cfg.k)
            w = moe.gating_weights(logits, ids, cfg.gating, cfg.renormalize)
            x64 = formats.activations_to_f64(cfg.xdtype, x)
            ref = np.stack([moe.token_output(x64[t], ids[t], w[t], ex[l].f64, ex[l].f64(cfg.E)) for t in range(T)])
            check_close(got, ref, bf16_out=True, what=f"step {s} layer {l} cpu {cpu}")
    st = cache.stats()
    assert n_cpu == st["cpu_misses"] and st["misses"] > st["cpu_misses"]
    assert (n_cpu > 0 and st["cpu_ns"] > 0) if hybrid else n_cpu == 0
    assert n_two_pass > 0 or not hits_first
    cache.destroy()


def test_cpu_miss_calls_validate(env):
    """Run without a stage of the same step, and f32 activations, are refused; no-ops without CPU misses."""
    ops, Lm = env
    rig = Rig(ops, 1, 8, 4, H=256, I=256)
    x = torch.zeros((2, 256), dtype=torch.int16, device="cuda")
    off = torch.tensor([0, 1, 2, 2, 2, 2, 2, 2, 2], dtype=torch.int32, device="cuda")
    rows = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    y = torch.zeros((2, 256), dtype=torch.float32, device="cuda")
    rig.step(0, [0, 1])
    rig.cache.stage_cpu_misses(x, Lm.DTYPES["bf16"], 2, 1, off, rows)  # no CPU miss: nothing happens
    rig.cache.run_cpu_misses(y)
    rig.cache.set_split(0.0, 1.0, 2, 1)                             # every miss on the CPU
    rig.step(0, [2, 3])
    assert rig.cache.cpu_misses() == [2, 3]
    with pytest.raises(ops.FtError) as e:                           # larger than set_split's T_max x k
        rig.cache.stage_cpu_misses(x, Lm.DTYPES["bf16"], 2, 2, off, rows)
    assert e.value.status == -3
    with pytest.raises(ops.FtError) as e:
        rig.cache.run_cpu_misses(y)
    assert e.value.status == -1
    with pytest.raises(ops.FtError) as e:
        rig.cache.stage_cpu_misses(x, Lm.DTYPES["f32"], 2, 1, off, rows)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert (y == 0).all()
    rig.cache.destroy()


def test_split_step_tables_against_the_simulator(env):
    """Hits-first steps (with and without the CPU split; step_split and plan + fill alternating):
    slot_hits holds the hits' slots, slot_misses the filled misses' slots, FT_SLOT_SKIP marks the
    other needed experts, -1 the rest; n_filled counts the fills; events and totals follow the
    oracle."""
    ops, _ = env
    from expert_cached_ffn_amd import _lib
    SKIP = _lib.FT_SLOT_SKIP
    rng = np.random.default_rng(31)
    L, E, C = 3, 24, 10
    rig = Rig(ops, L, E, C)
    sim = ExpertLRU(L, E, C)
    hits_t = torch.empty(E, dtype=torch.int32, device="cuda")
    for t in range(120):
        layer = int(rng.integers(L))
        ids = rng.choice(E, size=int(rng.integers(1, 7)), replace=False).astype(np.int32)
        bp, bh = [(1.0, 0.0), (2.0, 1.0), (0.0, 1.0)][t % 3]
        needed = sorted(set(ids.tolist()))
        m = sum(sim.slot_of_expert(layer)[e] < 0 for e in needed)
        q = m if bh == 0 else policy.miss_split(m, bp, bh)
        evs = {ev.expert: ev for ev in sim.step(layer, ids, fill_limit=q)}
        rig.set_split(bp, bh)
        d = torch.from_numpy(ids).cuda()
        if t % 2:
            n_filled = rig.cache.step_split(layer, d, ids.size, 1, hits_t, rig.slot_of)
        else:  # the same step in two calls
            rig.cache.plan(layer, d, ids.size, 1, hits_t, rig.slot_of)
            n_filled = rig.cache.fill()
        rig.cache.wait_fills()
        torch.cuda.synchronize()
        hits, misses = hits_t.cpu().numpy(), rig.slot_of.cpu().numpy()
        assert n_filled == sum(1 for ev in evs.values() if not ev.hit and ev.slot >= 0)
        for e in range(E):
            ev = evs.get(e)
            if ev is None:
                assert hits[e] == -1 and misses[e] == -1
            elif ev.hit:
                assert hits[e] == ev.slot and misses[e] == SKIP
            elif ev.slot >= 0:
                assert hits[e] == SKIP and misses[e] == ev.slot
                assert torch.equal(rig.pool[ev.slot].cpu(), rig.bank[layer * E + e])
            else:
                assert hits[e] == SKIP and misses[e] == -1
    st = rig.cache.stats()
    assert (st["accesses"], st["hits"], st["misses"], st["evictions"], st["cpu_misses"]) == \
        (sim.accesses, sim.hits, sim.misses, sim.evictions, sim.cpu_misses)
    rig.cache.destroy()


def test_plan_and_fill_call_order(env):
    """fill without a plan, a second plan, and cache-changing calls while a plan waits are refused;
    an LRU error surfaces at fill and leaves the state as it was."""
    ops, _ = env
    rig = Rig(ops, 1, 8, 3)
    hits_t = torch.empty(8, dtype=torch.int32, device="cuda")
    d = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    with pytest.raises(ops.FtError) as e:
        rig.cache.fill()
    assert e.value.status == -1
    rig.cache.plan(0, d, 2, 1, hits_t, rig.slot_of)
    for call in (lambda: rig.cache.plan(0, d, 2, 1, hits_t, rig.slot_of),
                 lambda: rig.cache.step(0, d, 2, 1, rig.slot_of),
                 lambda: rig.cache.step_split(0, d, 2, 1, hits_t, rig.slot_of)):
        with pytest.raises(ops.FtError) as e:
            call()
        assert e.value.status == -1
    assert rig.cache.fill() == 2
    rig.cache.wait_fills()
    before = rig.cache.stats()
    big = torch.tensor([2, 3, 4, 5], dtype=torch.int32, device="cuda")  # 4 distinct experts > 3 slots
    rig.cache.plan(0, big, 4, 1, hits_t, rig.slot_of)
    with pytest.raises(ops.FtError) as e:
        rig.cache.fill()
    assert e.value.status == -3
    assert rig.cache.stats() == before
    rig.cache.plan(0, d, 2, 1, hits_t, rig.slot_of)      # the cache is usable again: two hits
    assert rig.cache.fill() == 0
    torch.cuda.synchronize()
    rig.cache.destroy()


def test_prefetch_with_room_for_less_than_two_layers(env):
    """Capacity between E and 2E, order route(l) -> cache step(l) -> prefetch(l+1) -> FFN(l): the
    prefetch keeps the slots layer l's FFN reads and fills only what fits (events, fills and totals
    follow the simulator, some experts are not prefetched), and every token of every layer matches the
    oracle layer evaluated expert-major."""
    ops, Lm = env
    cfg = synth.shrink(synth.CONFIGS[4], H=512, I=512, E=16, k=4, n_layers=4, capacity=22)
    T = 160
    shape = Lm.LayerShape(cfg.H, cfg.I, cfg.E, cfg.k, cfg.wdtype, cfg.xdtype, cfg.gating, cfg.renormalize, True)
    layer = Lm.MoELayer(shape, T)
    lay = layer.layout
    eb = int(lay.expert_bytes)
    ex = [Experts(cfg, l) for l in range(cfg.n_layers)]
    bank = torch.empty((cfg.n_layers * cfg.E, eb), dtype=torch.uint8, pin_memory=True)
    for l in range(cfg.n_layers):
        for e in range(cfg.E):
            Lm.pack_expert(lay, ex[l].raw(e).arrays, bank.numpy()[l * cfg.E + e])
    shared = [Lm.as_device_u8([Lm.pack_expert(lay, ex[l].raw(cfg.E).arrays)])[0] for l in range(cfg.n_layers)]
    pool = torch.zeros((cfg.capacity, eb), dtype=torch.uint8, device="cuda")
    cache = ops.ExpertCache(lay, cfg.n_layers, cfg.E, cfg.capacity, pool, bank, torch.cuda.Stream(),
                            trace_events=4096)
    slot_of = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    sim = ExpertLRU(cfg.n_layers, cfg.E, cfg.capacity)
    want, n_steps, skipped = [], 0, 0

    def log(kind, l, evs):
        nonlocal skipped
        for e in evs:
            if kind == "prefetch":
                code = 3 if e.hit else (2 if e.slot >= 0 else 5)
                skipped += code == 5
            else:
                code = 1 if e.hit else 0
            want.append((n_steps, l, e.expert, code, e.slot,
                         -1 if e.evicted is None else e.evicted[0] * cfg.E + e.evicted[1]))

    cache.prefetch_layer(0)
    log("prefetch", 0, sim.prefetch(0))
    for l in range(cfg.n_layers):
        print(f"prefetch regime: layer {l}", flush=True)
        x = synth.tokens(cfg, T, layer=l)
        logits = synth.prefill_logits(cfg, T, layer=l)
        layer.route_permute(T, logits=Lm.to_device(logits))
        cache.step(l, layer.ids, T, cfg.k, slot_of)
        ids = moe.topk(logits, cfg.k)
        log("step", l, sim.step(l, ids.ravel()))
        table_want = sim.slot_of_expert(l)
        n_steps += 1
        if l + 1 < cfg.n_layers:
            cache.prefetch_layer(l + 1)
            log("prefetch", l + 1, sim.prefetch(l + 1))
        layer.ffn(T, Lm.to_device(x), pool, slot_of_expert=slot_of, shared_blob=shared[l])
        layer.combine(T)
        torch.cuda.synchronize()
        assert slot_of.cpu().numpy().tolist() == table_want
        got = formats.bf16_to_f64(layer.out[:T].cpu().numpy().view(np.uint16))
        x64 = formats.activations_to_f64(cfg.xdtype, x)
        ref = moe.moe_layer(x64, k=cfg.k, E=cfg.E, gating=cfg.gating, renormalize=cfg.renormalize,
                            experts=ex[l].f64, shared=ex[l].f64(cfg.E), logits=logits)
        check_close(got, ref["out"], bf16_out=True, what=f"prefetch regime layer {l}, every token")
    assert cache.trace() == want
    st = cache.stats()
    assert skipped > 0                                   # the regime: some experts found no room
    assert (st["accesses"], st["hits"], st["misses"], st["evictions"], st["prefetch_fills"]) == \
        (sim.accesses, sim.hits, sim.misses, sim.evictions, sim.prefetch_fills)
    assert st["bytes_h2d"] == (sim.misses + sim.prefetch_fills) * eb
    cache.destroy()


def test_event_ring(env):
    """The event log is off by default; a ring keeps the newest events oldest first and counts the
    ones it overwrote."""
    ops, _ = env
    rig = Rig(ops, 1, 16, 4)
    rig.cache.set_trace(0)
    rig.step(0, [1, 2])
    assert rig.cache.trace() == []
    rig.cache.set_trace(5)
    sim = ExpertLRU(1, 16, 4)
    sim.step(0, [1, 2])
    want = []
    for i, ids in enumerate([[1, 3], [4, 5, 6], [2, 7]]):
        want += [(i + 1, 0, e.expert, int(e.hit), e.slot, -1 if e.evicted is None else e.evicted[1])
                 for e in sim.step(0, ids)]
        rig.step(0, ids)
    assert rig.cache.trace() == want[-5:]
    assert rig.cache.stats()["trace_dropped"] == len(want) - 5
    with pytest.raises(ops.FtError):
        rig.cache.set_trace(-1)
    rig.cache.destroy()
