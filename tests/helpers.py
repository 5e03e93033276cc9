"""Shared test helpers: building inputs, oracle expectations and tolerance checks."""
from __future__ import annotations

import numpy as np

import synth
from oracle import formats, moe

# Parity bar for floating-point outputs (rel-L2 and max-abs relative to the
# reference RMS); bf16 outputs also get their own final rounding (half ulp).
REL_L2 = 5e-3
MAX_ABS_RMS = 2e-2


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |ref| (the rounding of a bf16 output)."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1e-38)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def check_close(got, ref, bf16_out=False, what=""):
    """Assert rel-L2 <= 5e-3 and max |got-ref| <= 2e-2 rms(ref) (+ half ulp for bf16 outputs)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / max(nref, 1e-300)
    rms = nref / np.sqrt(max(ref.size, 1))
    bound = MAX_ABS_RMS * rms + (bf16_half_ulp(ref) if bf16_out else 0.0)
    worst = np.max(np.abs(diff) - bound) if ref.size else -1
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    assert worst <= 0, f"{what}: max-abs exceeds bound by {worst:.3e} (rms {rms:.3e}, max abs {np.max(np.abs(diff)):.3e})"
    return rel, float(np.max(np.abs(diff))) if ref.size else 0.0


class Experts:
    """Synthetic experts of one workload: storage arrays and float64 weights, on demand."""

    def __init__(self, cfg: synth.LayerConfig, layer: int = 0):
        self.cfg, self.layer = cfg, layer
        self._raw: dict[int, synth.ExpertWeights] = {}
        self._f64: dict[int, tuple] = {}

    def raw(self, e: int) -> synth.ExpertWeights:
        if e not in self._raw:
            self._raw[e] = synth.expert_weights(self.cfg, self.layer, e)
        return self._raw[e]

    def f64(self, e: int):
        if e not in self._f64:
            self._f64[e] = formats.expert_to_f64(self.cfg.wdtype, self.raw(e).arrays)
        return self._f64[e]

    def drop(self):
        self._f64.clear()


def route_oracle(cfg, x64, wr64=None, logits=None):
    if logits is None:
        logits = moe.router_logits(x64, wr64)
    ids = moe.topk(logits, cfg.k)
    w = moe.gating_weights(logits, ids, cfg.gating, cfg.renormalize)
    return logits, ids, w, moe.topk_margin(logits, cfg.k)
