"""Simulator of the GPU expert cache: one LRU over (layer, expert) entries.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
* a cache entry is one whole logical (layer, expert) pair, with the same
  mapping on the CPU and the GPU (FreeToken rtx 4090 page, "Cómo funciona la
  jerarquía de memoria MoE");
* one LRU policy is shared by all MoE layers, keeps recently selected experts
  resident for later tokens, and follows the router rather than being frozen
  at start-up (FreeToken linux page, "Cómo gestiona FreeToken la memoria MoE";
  rtx 4090 page, same section);
* hits run from the GPU copy; misses are filled into the GPU cache over PCIe
  from pinned host memory (FreeToken quantization page, "Cómo se desplazan los
  pesos MoE cuantizados por la memoria");
* the miss rate is misses over routed expert reads (FreeToken 290b model page,
  "Limitaciones, lista de comprobación y buenas prácticas", metrics table).

The order of updates inside one (layer, step) is not on the pages.  Reading
taken here:  the needed set S is the distinct experts of the step's routing,
visited in ascending expert id.  Phase 1 refreshes every hit.  Phase 2 gives
each miss the least recently used slot not holding a member of S (empty slots
have stamp 0, so they fill lowest index first; stamps are otherwise unique).
Refreshing all hits before any eviction means a miss can never evict an expert
that the same step still needs.  If |S| exceeds the capacity the step is
refused and nothing changes.

Resizing: the runtime can resize and rebuild the GPU expert cache at safe
points of its scheduler when the available GPU memory changes (FreeToken
quantization page, "Flujo de configuración de la cuantización de FreeToken";
FreeToken 290b model page, "Caché elástica").  Reading taken here (the pages
give no rule): between steps, the cache keeps the min(new capacity, resident)
most recently used entries and drops the rest (counted as evictions); the
kept entries move to slots 0, 1, ... in ascending order of their old slot
(never to a higher slot, so the move is safe in place), keep their stamps,
and the clock is unchanged; new slots are empty.

Hybrid execution: a step's misses are either filled into the GPU cache or
run on the CPU, by a split derived from measured bandwidths (FreeToken 290b
model page, "Ejecución híbrida" and "Cómo gestiona FreeToken el prellenado y
la decodificación"; the count is `policy.miss_split`).  Reading taken here:
the lowest expert ids among the misses are filled (as `policy.split_misses`);
the others stay non-resident -- no slot, no eviction, no recency -- and are
still misses.

Full-layer prefetch: in prefill the runtime double-buffers whole layers --
while the GPU computes one layer, the experts of the next are streamed over
PCIe, when the cache has room for them (FreeToken linux page, "Cómo gestiona
FreeToken la memoria MoE"; FreeToken rtx 4090 page, "Prefill"; FreeToken 290b
model page, "Cómo gestiona FreeToken el prellenado y la decodificación"), in
the same cache that serves decode (FreeToken linux page, same section).
Reading taken here: a prefetch of layer l updates the LRU exactly like a step
of layer l whose needed set is all of its experts, but it is not a routed
access: it adds fills and evictions, not accesses, hits or misses.  "When the
cache has room" is read as: the prefetch never takes the slot of an entry the
most recent routed step needed (that step's expert computation may still be
reading it: the intended order is step(l), prefetch(l+1), compute(l)); when no
other slot is left, the remaining experts of the layer (the higher ids) are
not prefetched -- no slot, no eviction, no recency -- and are served as
ordinary misses by their own step.
"""
from __future__ import annotations

from dataclasses import dataclass


class CapacityError(RuntimeError):
    """More distinct experts in one step than the cache has slots."""


@dataclass(frozen=True)
class Event:
    expert: int
    hit: bool
    slot: int
    evicted: tuple | None   # (layer, expert) that left the slot, or None

    def short(self) -> str:
        s = f"{self.expert}:{'H' if self.hit else 'M'}@{self.slot}"
        if self.evicted is not None:
            s += f" evicts {self.evicted[0]}/{self.evicted[1]}"
        return s


class ExpertLRU:
    """Slot table (layer, expert) -> slot with least-recently-used replacement."""

    def __init__(self, n_layers: int, n_experts: int, capacity: int):
        if n_layers < 1 or n_experts < 1 or capacity < 1:
            raise ValueError("n_layers, n_experts and capacity must be positive")
        self.n_layers = n_layers
        self.n_experts = n_experts
        self.capacity = capacity
        self.owner: list[tuple | None] = [None] * capacity   # slot -> key
        self.stamp: list[int] = [0] * capacity                # 0 = never used
        self.where: dict[tuple, int] = {}                     # key -> slot
        self.clock = 0
        self.accesses = 0
        self.hits = 0
        self.misses = 0
        self.evictions = 0
        self.prefetch_fills = 0
        self.cpu_misses = 0
        self.protected: set[tuple] = set()   # keys the most recent routed step needed (resident)

    def lookup(self, layer: int, expert: int) -> int:
        """Slot holding (layer, expert), or -1."""
        return self.where.get((layer, expert), -1)

    def step(self, layer: int, ids, fill_limit: int | None = None) -> list[Event]:
        """Serve one layer of one step; returns events in ascending expert id.

        fill_limit: at most this many of the step's misses (the lowest ids) are
        filled; the others run on the CPU (events with slot -1)."""
        needed = self._needed(layer, ids)
        events = self._serve(layer, needed, fill_limit)
        self.protected = {(layer, ev.expert) for ev in events if ev.slot >= 0}
        self.accesses += len(needed)
        self.hits += sum(1 for ev in events if ev.hit)
        self.misses += sum(1 for ev in events if not ev.hit)
        return events

    def prefetch(self, layer: int) -> list[Event]:
        """Bring the experts of ``layer`` in (full-layer prefetch), as many as fit without taking a
        slot of the most recent step's needed entries; events ascending, slot -1 = not prefetched."""
        events = self._serve(layer, self._needed(layer, range(self.n_experts)), protect=self.protected)
        self.prefetch_fills += sum(1 for ev in events if not ev.hit and ev.slot >= 0)
        return events

    def _needed(self, layer: int, ids) -> list[int]:
        if not 0 <= layer < self.n_layers:
            raise ValueError("layer out of range")
        needed = sorted({int(e) for e in list(ids)})
        for e in needed:
            if not 0 <= e < self.n_experts:
                raise ValueError("expert id out of range")
        if len(needed) > self.capacity:
            raise CapacityError(f"{len(needed)} distinct experts > {self.capacity} slots")
        return needed

    def _serve(self, layer: int, needed: list[int], fill_limit: int | None = None,
               protect: set | None = None) -> list[Event]:
        events: dict[int, Event] = {}
        # Phase 1: every hit becomes most recently used, ascending expert id.
        for e in needed:
            s = self.where.get((layer, e))
            if s is not None:
                self.clock += 1
                self.stamp[s] = self.clock
                events[e] = Event(e, True, s, None)
        # Phase 2: each miss takes the least recently used slot that holds no
        # member of the needed set (nor, for a prefetch, a protected entry),
        # ascending expert id.
        needed_keys = {(layer, e) for e in needed}
        protect = protect or set()
        filled = 0
        for e in needed:
            if e in events:
                continue
            if fill_limit is not None and filled >= fill_limit:
                events[e] = Event(e, False, -1, None)   # runs on the CPU
                self.cpu_misses += 1
                continue
            best = None
            for s in range(self.capacity):
                if self.owner[s] in needed_keys or self.owner[s] in protect:
                    continue
                if best is None or (self.stamp[s], s) < (self.stamp[best], best):
                    best = s
            if best is None:                          # prefetch only: no room left
                events[e] = Event(e, False, -1, None)
                continue
            filled += 1
            evicted = self.owner[best]
            if evicted is not None:
                del self.where[evicted]
                self.evictions += 1
            self.owner[best] = (layer, e)
            self.where[(layer, e)] = best
            self.clock += 1
            self.stamp[best] = self.clock
            events[e] = Event(e, False, best, evicted)
        return [events[e] for e in needed]

    def resize(self, capacity: int) -> tuple[list[tuple[int, int]], list[tuple]]:
        """Change the number of slots; returns (moves old slot -> new slot, dropped keys)."""
        if capacity < 1:
            raise ValueError("capacity must be positive")
        used = [s for s in range(self.capacity) if self.owner[s] is not None]
        keep = set(sorted(used, key=lambda s: self.stamp[s], reverse=True)[:capacity])
        moves, dropped = [], []
        owner: list[tuple | None] = [None] * capacity
        stamp = [0] * capacity
        nxt = 0
        for s in used:                        # ascending old slot
            key = self.owner[s]
            if s in keep:
                owner[nxt], stamp[nxt] = key, self.stamp[s]
                self.where[key] = nxt
                moves.append((s, nxt))
                nxt += 1
            else:
                del self.where[key]
                dropped.append(key)
        self.evictions += len(dropped)
        self.capacity, self.owner, self.stamp = capacity, owner, stamp
        return moves, dropped

    def slot_of_expert(self, layer: int) -> list[int]:
        """Slot of every expert of ``layer`` (-1 if not resident)."""
        return [self.where.get((layer, e), -1) for e in range(self.n_experts)]

    def stats(self) -> dict:
        return dict(accesses=self.accesses, hits=self.hits, misses=self.misses,
                    evictions=self.evictions)
