"""Seeded synthetic inputs for the routed MoE FFN layer and its expert cache.

This module only draws data: activations, router weights, expert weights in
their storage formats, router logits and routing traces.  It holds none of the
layer's arithmetic (no routing, gating, FFN, combine or cache logic), so both
the CPU oracle and the GPU path can consume its arrays without sharing any
computation.

Storage formats produced here:

* ``f32``   -- float32 arrays.
* ``bf16``  -- uint16 arrays holding bfloat16 bit patterns, rounded from the
  float32 draw to nearest-even.
* ``mxfp4`` -- OCP Microscaling FP4: uint8 code arrays (two E2M1 nibbles per
  byte, element 2i in bits 3:0, element 2i+1 in bits 7:4) and uint8 E8M0 scale
  arrays (one scale byte per 32 consecutive elements along the contraction
  axis of each row).

Every tensor has its own seed, keyed by (config, case, tensor tag, indices),
so any single expert of any layer can be regenerated without drawing the
others.  The workload shapes follow the pages' example model (FreeToken linux
page, "Cómo gestiona FreeToken la memoria MoE": 6 of 256 routed experts per
layer) and the layer shapes the repository's design notes list.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Tensor tags used in the seed key.
TAG_X = 1
TAG_ROUTER = 2
TAG_EXPERT = 3
TAG_LOGITS = 4
TAG_TRACE = 5
TAG_EXTRA = 6


@dataclass(frozen=True)
class LayerConfig:
    """Shapes and formats of one synthetic MoE layer workload."""

    cfg_id: int
    name: str
    H: int                 # hidden size (contraction axis of gate/up)
    I: int                 # expert intermediate size (contraction axis of down)
    E: int                 # routed experts per layer
    k: int                 # experts selected per token
    wdtype: str            # 'f32' | 'bf16' | 'mxfp4' | 'nvfp4'
    xdtype: str            # 'f32' | 'bf16'
    gating: str            # 'softmax' | 'sigmoid'
    renormalize: bool
    shared: bool           # one always-active shared expert
    batches: tuple         # token counts exercised by this workload
    logits_given: bool = False   # router logits are synthetic inputs (no router GEMV)
    n_layers: int = 1
    capacity: int = 0      # expert-cache slots; 0 = every expert resident
    steps: int = 0         # decode steps of a cache trace
    zipf_s: float = 0.0    # Zipf exponent of expert popularity (0 = none)
    reuse_p: float = 0.0   # probability of reusing one of the previous token's experts
    w_std: float = 0.02
    x_std: float = 1.0
    scale_bytes: tuple = (119, 123)  # inclusive range of E8M0 scale bytes
    nv_scale_codes: tuple = (0x30, 0x40)  # inclusive range of E4M3 block-scale codes (0.5 .. 2.0)
    nv_tensor_scale: tuple = (0.01, 0.03)  # range of the per-tensor fp32 scale


CONFIGS = {
    1: LayerConfig(1, "tiny-f32", H=256, I=128, E=16, k=2, wdtype="f32", xdtype="f32",
                   gating="softmax", renormalize=False, shared=False, batches=(8,)),
    2: LayerConfig(2, "qwen3-a3b-shaped-bf16-decode", H=2048, I=768, E=128, k=8,
                   wdtype="bf16", xdtype="bf16", gating="softmax", renormalize=True,
                   shared=False, batches=(1, 16, 64)),
    3: LayerConfig(3, "dsv4-flash-shaped-mxfp4-decode", H=4096, I=2048, E=256, k=6,
                   wdtype="mxfp4", xdtype="bf16", gating="sigmoid", renormalize=False,
                   shared=True, batches=(1, 8, 32)),
    4: LayerConfig(4, "dsv4-flash-shaped-mxfp4-prefill", H=4096, I=2048, E=256, k=6,
                   wdtype="mxfp4", xdtype="bf16", gating="sigmoid", renormalize=False,
                   shared=True, batches=(8192,), logits_given=True, zipf_s=1.1),
    5: LayerConfig(5, "dsv4-flash-shaped-expert-cache-trace", H=4096, I=2048, E=256, k=6,
                   wdtype="mxfp4", xdtype="bf16", gating="sigmoid", renormalize=False,
                   shared=True, batches=(1,), logits_given=True, n_layers=8,
                   capacity=512, steps=512, zipf_s=1.1, reuse_p=0.6),
    6: LayerConfig(6, "qwen3-a3b-shaped-nvfp4-decode", H=2048, I=768, E=128, k=8,
                   wdtype="nvfp4", xdtype="bf16", gating="softmax", renormalize=True,
                   shared=False, batches=(1, 16, 64)),
    7: LayerConfig(7, "qwen3-a3b-shaped-nvfp4-prefill", H=2048, I=768, E=128, k=8,
                   wdtype="nvfp4", xdtype="bf16", gating="softmax", renormalize=True,
                   shared=False, batches=(8192,), logits_given=True, zipf_s=1.1),
}


def shrink(cfg: LayerConfig, **kw) -> LayerConfig:
    """A copy of ``cfg`` with some fields replaced (small parity cases)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return LayerConfig(**d)


def rng_for(cfg: LayerConfig, case: int, tag: int, *idx: int) -> np.random.Generator:
    """Independent PCG64 stream for one tensor of one case of one workload."""
    return np.random.default_rng(np.random.SeedSequence([0, cfg.cfg_id, case, tag, *idx]))


# ----------------------------------------------------------------------------
# storage-format helpers (data encoding only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _normal_as(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    v = (rng.standard_normal(shape) * std).astype(np.float32)
    if dtype == "f32":
        return v
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# activations and router
# ----------------------------------------------------------------------------

def tokens(cfg: LayerConfig, T: int, case: int = 0, layer: int = 0, step: int = 0) -> np.ndarray:
    """Activations x [T, H] in cfg.xdtype storage (float32 or bf16 bits)."""
    rng = rng_for(cfg, case, TAG_X, T, layer, step)
    return _normal_as(rng, (T, cfg.H), cfg.x_std, cfg.xdtype)


def router_weight(cfg: LayerConfig, layer: int = 0) -> np.ndarray:
    """Router weight W_r [E, H] in cfg.xdtype storage."""
    rng = rng_for(cfg, 0, TAG_ROUTER, layer)
    return _normal_as(rng, (cfg.E, cfg.H), cfg.w_std, cfg.xdtype)


# ----------------------------------------------------------------------------
# expert weights
# ----------------------------------------------------------------------------

@dataclass
class ExpertWeights:
    """One expert's three projections in storage format.

    Dense formats: ``wg``/``wu`` [I, H], ``wd`` [H, I] (row-major, contraction
    axis contiguous).  MXFP4: ``*_codes`` [rows, K/2] uint8 and ``*_scales``
    [rows, K/32] uint8 with K the contraction axis of that projection.
    NVFP4: the same codes, ``*_scales`` [rows, K/16] uint8 (E4M3 codes) and
    ``tensor_scales`` float32 [3] (gate, up, down).
    """

    fmt: str
    arrays: dict = field(default_factory=dict)

    def __getitem__(self, key):
        return self.arrays[key]


def expert_weights(cfg: LayerConfig, layer: int, expert: int) -> ExpertWeights:
    """Weights of routed expert ``expert`` (0..E-1) or of the shared expert (E)."""
    rng = rng_for(cfg, 0, TAG_EXPERT, layer, expert)
    H, I = cfg.H, cfg.I
    if cfg.wdtype in ("f32", "bf16"):
        return ExpertWeights(cfg.wdtype, {
            "wg": _normal_as(rng, (I, H), cfg.w_std, cfg.wdtype),
            "wu": _normal_as(rng, (I, H), cfg.w_std, cfg.wdtype),
            "wd": _normal_as(rng, (H, I), cfg.w_std, cfg.wdtype),
        })
    if cfg.wdtype == "mxfp4":
        lo, hi = cfg.scale_bytes
        a = {
            "gate_codes": rng.integers(0, 256, size=(I, H // 2), dtype=np.uint8),
            "up_codes": rng.integers(0, 256, size=(I, H // 2), dtype=np.uint8),
            "down_codes": rng.integers(0, 256, size=(H, I // 2), dtype=np.uint8),
            "gate_scales": rng.integers(lo, hi + 1, size=(I, H // 32), dtype=np.uint8),
            "up_scales": rng.integers(lo, hi + 1, size=(I, H // 32), dtype=np.uint8),
            "down_scales": rng.integers(lo, hi + 1, size=(H, I // 32), dtype=np.uint8),
        }
        return ExpertWeights("mxfp4", a)
    if cfg.wdtype == "nvfp4":
        lo, hi = cfg.nv_scale_codes
        t_lo, t_hi = cfg.nv_tensor_scale
        a = {
            "gate_codes": rng.integers(0, 256, size=(I, H // 2), dtype=np.uint8),
            "up_codes": rng.integers(0, 256, size=(I, H // 2), dtype=np.uint8),
            "down_codes": rng.integers(0, 256, size=(H, I // 2), dtype=np.uint8),
            "gate_scales": rng.integers(lo, hi + 1, size=(I, H // 16), dtype=np.uint8),
            "up_scales": rng.integers(lo, hi + 1, size=(I, H // 16), dtype=np.uint8),
            "down_scales": rng.integers(lo, hi + 1, size=(H, I // 16), dtype=np.uint8),
            "tensor_scales": rng.uniform(t_lo, t_hi, size=3).astype(np.float32),
        }
        return ExpertWeights("nvfp4", a)
    raise ValueError(cfg.wdtype)


# ----------------------------------------------------------------------------
# synthetic router logits (workloads whose logits are given)
# ----------------------------------------------------------------------------

def zipf_popularity(n: int, s: float) -> np.ndarray:
    """Finite Zipf probabilities over ranks 1..n: p_r proportional to r^-s."""
    r = np.arange(1, n + 1, dtype=np.float64)
    w = r ** (-s)
    return w / w.sum()


def rank_to_expert(cfg: LayerConfig, layer: int) -> np.ndarray:
    """Seeded permutation: popularity rank -> expert id, per layer."""
    return rng_for(cfg, 0, TAG_EXTRA, 1, layer).permutation(cfg.E)


def prefill_logits(cfg: LayerConfig, T: int, case: int = 0, layer: int = 0) -> np.ndarray:
    """Logits [T, E] float32 whose top-k follows Zipf popularity.

    Gumbel-top-k: l[t, e] = ln p(e) + G[t, e] with G standard Gumbel, so the
    top-k of each row is a draw without replacement proportional to p.
    """
    rng = rng_for(cfg, case, TAG_LOGITS, T, layer)
    p_rank = zipf_popularity(cfg.E, cfg.zipf_s)
    p = np.empty(cfg.E)
    p[rank_to_expert(cfg, layer)] = p_rank
    u = rng.random((T, cfg.E))
    u = np.clip(u, np.finfo(np.float64).tiny, None)
    g = -np.log(-np.log(u))
    return (np.log(p)[None, :] + g).astype(np.float32)


@dataclass
class CacheTrace:
    """Routing of a multi-layer decode trace.

    ``ids[s, l]`` is the ordered expert list drawn for step s, layer l (k
    entries); ``logits[s, l]`` [E] float32 realises it: the expert drawn j-th
    gets 8 - 0.25 j, every other expert N(0, 1) clipped to [-3, 3], so its
    top-k reproduces the draw with a margin of at least 3.75.
    """

    ids: np.ndarray
    logits: np.ndarray


def cache_trace(cfg: LayerConfig, steps: int | None = None, n_layers: int | None = None,
                case: int = 0) -> CacheTrace:
    """Zipf popularity with per-layer reuse of the previous token's experts."""
    steps = cfg.steps if steps is None else steps
    L = cfg.n_layers if n_layers is None else n_layers
    E, k = cfg.E, cfg.k
    ids = np.zeros((steps, L, k), dtype=np.int32)
    logits = np.zeros((steps, L, E), dtype=np.float32)
    p_rank = zipf_popularity(E, cfg.zipf_s)
    for l in range(L):
        rng = rng_for(cfg, case, TAG_TRACE, l)
        p = np.empty(E)
        p[rank_to_expert(cfg, l)] = p_rank
        prev: list[int] = []
        for s in range(steps):
            chosen: list[int] = []
            for j in range(k):
                left_prev = [e for e in prev if e not in chosen]
                if s > 0 and left_prev and rng.random() < cfg.reuse_p:
                    e = left_prev[int(rng.integers(len(left_prev)))]
                else:
                    q = p.copy()
                    q[chosen] = 0.0
                    q /= q.sum()
                    e = int(rng.choice(E, p=q))
                chosen.append(e)
            ids[s, l] = chosen
            noise = np.clip(rng.standard_normal(E), -3.0, 3.0)
            row = noise.astype(np.float32)
            for j, e in enumerate(chosen):
                row[e] = np.float32(8.0 - 0.25 * j)
            logits[s, l] = row
            prev = chosen
    return CacheTrace(ids=ids, logits=logits)


def routing_ids_uniform(cfg: LayerConfig, T: int, case: int = 0) -> np.ndarray:
    """Random distinct-per-token expert ids [T, k] (for per-call parity cases)."""
    rng = rng_for(cfg, case, TAG_EXTRA, 2, T)
    out = np.empty((T, cfg.k), dtype=np.int32)
    for t in range(T):
        out[t] = rng.choice(cfg.E, size=cfg.k, replace=False)
    return out


def gating_weights_uniform(cfg: LayerConfig, T: int, case: int = 0) -> np.ndarray:
    """Random positive per-slot weights [T, k] float32 (for per-call parity cases)."""
    rng = rng_for(cfg, case, TAG_EXTRA, 3, T)
    return rng.uniform(0.05, 1.0, size=(T, cfg.k)).astype(np.float32)
