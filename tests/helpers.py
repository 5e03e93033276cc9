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


def check_close(got, ref, bf16_out=False, what="", allow=None):
    """Assert rel-L2 <= 5e-3 and max |got-ref| <= 2e-2 rms(ref) (+ half ulp for bf16 outputs,
    + ``allow``, an element-wise bound on deviations the reference cannot pin down).

    Prints one line per comparison with the literal max |got-ref| beside the relative bound, so a
    run with ``-s`` (or ``-rP``) lists both readings of the max-abs tolerance."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / max(nref, 1e-300)
    rms = nref / np.sqrt(max(ref.size, 1))
    bound = MAX_ABS_RMS * rms + (bf16_half_ulp(ref) if bf16_out else 0.0) + (0.0 if allow is None else allow)
    worst = np.max(np.abs(diff) - bound) if ref.size else -1
    max_abs = float(np.max(np.abs(diff))) if ref.size else 0.0
    print(f"PARITY {what}: n={ref.size} rel-L2 {rel:.3e} (<= {REL_L2}) max-abs {max_abs:.3e} "
          f"(literal 2e-2: {'ok' if max_abs <= 2e-2 else 'over'}; bound 2e-2*rms = {MAX_ABS_RMS * rms:.3e}) "
          f"rms(ref) {rms:.3e}", flush=True)
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    assert worst <= 0, f"{what}: max-abs exceeds bound by {worst:.3e} (rms {rms:.3e}, max abs {max_abs:.3e})"
    return rel, max_abs


# Top-k margin below which the router's own fp32 logits may order two experts
# differently from the float64 oracle (the routing exactness rule).
TOPK_MARGIN = 1e-4


def check_topk_valid(got_ids, logits_ref, k, tol=TOPK_MARGIN, what=""):
    """Where several top-k results are correct (near-tied logits), check what is unique and that
    the rest is valid: per token k distinct experts in range, every picked expert's oracle logit
    within ``tol`` of the oracle's k-th largest or above it, and every expert left out within
    ``tol`` of it or below.  Returns the tokens whose ids differ from the oracle's own top-k."""
    got_ids = np.asarray(got_ids)
    l = np.asarray(logits_ref, np.float64)
    T, E = l.shape
    assert got_ids.shape == (T, k), (what, got_ids.shape)
    assert np.all((got_ids >= 0) & (got_ids < E)), f"{what}: id out of range"
    kth = -np.sort(-l, axis=1)[:, k - 1]
    differ = []
    for t in range(T):
        ids = got_ids[t].astype(np.int64)
        assert len(set(ids.tolist())) == k, f"{what}: token {t} picks an expert twice"
        assert np.all(l[t, ids] >= kth[t] - tol), f"{what}: token {t} picks an expert below the k-th logit"
        out = np.setdiff1d(np.arange(E), ids)
        assert np.all(l[t, out] <= kth[t] + tol), f"{what}: token {t} leaves out an expert above the k-th logit"
    ref_ids = moe.topk(l.astype(np.float32), k)
    for t in range(T):
        if not np.array_equal(got_ids[t], ref_ids[t]):
            differ.append(t)
    return np.array(differ, dtype=np.int64)


# Native MXFP4 mode: the GPU forms the SwiGLU hidden vector in fp32 (relative
# error well below 2^-14 here), the oracle in float64, and each side rounds it
# to bf16 and then to E4M3 codes.  A value within that error of a rounding
# boundary may get the neighbouring code on the GPU; the oracle cannot tell
# which, so the output bound admits exactly those alternatives.
MX_HIDDEN_REL_ERR = 2.0 ** -14


def mx_hidden_allowance(h64: np.ndarray, Wd: np.ndarray, eps: float = MX_HIDDEN_REL_ERR) -> np.ndarray:
    """Largest |y| change [n, H] from hidden codes that differ when h moves by eps relative."""
    from oracle import mx
    mid = mx.mxfp8_round_trip(mx.round_to_bf16(h64))
    dev = np.zeros_like(mid)
    for f in (1.0 - eps, 1.0 + eps):
        dev = np.maximum(dev, np.abs(mx.mxfp8_round_trip(mx.round_to_bf16(h64 * f)) - mid))
    return dev @ np.abs(Wd).T


def native_mx_expert(X: np.ndarray, Wg, Wu, Wd):
    """Oracle native-mode expert output [n, H] and its hidden-rounding allowance [n, H]."""
    from oracle import mx
    Xq = mx.mxfp8_round_trip(np.asarray(X, np.float64))
    G, U = Xq @ Wg.T, Xq @ Wu.T
    h64 = G * moe.sigmoid(G) * U
    return moe.swiglu_expert_mx(X, Wg, Wu, Wd), mx_hidden_allowance(h64, Wd)


def native_mx_token(x_t, ids_t, w_t, experts, shared=None):
    """One token's native-mode layer output and allowance (weighted like the output)."""
    out = np.zeros(len(x_t))
    allow = np.zeros(len(x_t))
    X = np.asarray(x_t, np.float64)[None, :]
    for e, wj in zip(ids_t, w_t):
        y, a = native_mx_expert(X, *experts(int(e)))
        out += float(wj) * y[0]
        allow += abs(float(wj)) * a[0]
    if shared is not None:
        y, a = native_mx_expert(X, *shared)
        out += y[0]
        allow += a[0]
    return out, allow


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

    def fresh(self, e: int):
        """Expert e's float64 weights decoded now and not kept (for sweeps over many experts)."""
        if e in self._f64:
            return self._f64[e]
        return formats.expert_to_f64(self.cfg.wdtype, synth.expert_weights(self.cfg, self.layer, e).arrays)

    def drop(self):
        self._f64.clear()


def route_oracle(cfg, x64, wr64=None, logits=None):
    if logits is None:
        logits = moe.router_logits(x64, wr64)
    ids = moe.topk(logits, cfg.k)
    w = moe.gating_weights(logits, ids, cfg.gating, cfg.renormalize)
    return logits, ids, w, moe.topk_margin(logits, cfg.k)
