"""Bandwidth-derived split of a step's cache misses between GPU fill and CPU execution.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages (FreeToken 290b model page, "Cómo gestiona FreeToken el prellenado
y la decodificación", the miss-split formula) measure B_p, the pinned
host-to-device expert transfer bandwidth, and B_h, the effective host
bandwidth seen by the CPU expert kernel, and fill about q* ~ m B_p / B_h of a
step's m misses into the GPU cache; the rest run on the CPU.  A higher PCIe
rate favours more fills and a stronger CPU path leaves more misses on the CPU.

Read literally the printed ratio can exceed m.  Reading taken here: the two
paths run at the same time, so the step waits for the slower one; choose the
integer q in 0..m that minimises max(q S / B_p, (m - q) S / B_h) (S = bytes
of one expert), ties going to the larger q (a filled expert stays cached for
later tokens).  Its real-valued optimum balances the two times,
q* = m B_p / (B_p + B_h); it grows with B_p and shrinks with B_h, as the
pages state.  Which misses are filled is not on the pages; the lowest expert
ids are taken first.
"""
from __future__ import annotations


def miss_split(m: int, b_pcie: float, b_host: float) -> int:
    """Number of the m misses to fill into the GPU cache."""
    if m < 0 or b_pcie < 0 or b_host < 0:
        raise ValueError("negative input")
    if m == 0:
        return 0
    if b_pcie + b_host == 0:
        raise ValueError("both bandwidths are zero")

    def step_time(q):
        fill = (q / b_pcie if b_pcie else float("inf")) if q else 0.0
        cpu = ((m - q) / b_host if b_host else float("inf")) if m - q else 0.0
        return max(fill, cpu)

    best = 0
    for q in range(m + 1):
        if step_time(q) <= step_time(best):
            best = q
    return best


def split_misses(miss_experts, b_pcie: float, b_host: float):
    """(filled, cpu): the lowest expert ids are filled first."""
    ms = sorted(int(e) for e in miss_experts)
    q = miss_split(len(ms), b_pcie, b_host)
    return ms[:q], ms[q:]
