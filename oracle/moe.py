"""The routed MoE FFN layer, written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: a router activates a small subset of the experts for each
token (6 of 256 routed experts per layer in their example; FreeToken linux
page, "Cómo gestiona FreeToken la memoria MoE"; FreeToken rtx 4090 page,
"Cómo funciona la jerarquía de memoria MoE"), and an expert runs from its
resident copy whatever tier it came from, so the layer's output never depends
on the cache state (FreeToken quantization page, "Cómo se desplazan los pesos
MoE cuantizados por la memoria").  Everything else below is the plainest
textbook reading, listed in the design notes:

* logits = x W_r^T accumulated exactly, rounded to float32;
* top-k: descending logit, lower expert index first on ties;
* gating: softmax over all E (optionally renormalised over the k picked) or
  element-wise sigmoid (optionally renormalised);
* expert FFN: SwiGLU as defined in Shazeer, "GLU Variants Improve
  Transformer" (2020): (silu(x W_g^T) * (x W_u^T)) W_d^T, silu(z) = z sigma(z),
  no biases;
* combine: out[t] = sum_j w[t, j] y[t, j] + y_shared[t].
"""
from __future__ import annotations

import numpy as np

from . import mx


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] W_r[e, h], summed in float64, stored as float32."""
    return (np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T).astype(np.float32)


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k indices with the largest logits, in order.

    Order key (-logit, index): larger logits first, the lower index first on
    equal logits (-0.0 and +0.0 are equal).
    """
    logits = np.asarray(logits)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in 1..E")
    idx = np.arange(E)
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        key = -logits[t].astype(np.float64)
        order = np.lexsort((idx, key))
        out[t] = order[:k]
    return out


def topk_margin(logits: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest logit of each row (inf if k == E)."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-z), evaluated without overflow."""
    z = np.asarray(z, np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def gating_weights(logits: np.ndarray, ids: np.ndarray, gating: str,
                   renormalize: bool) -> np.ndarray:
    """Weights w[t, j] of the experts ids[t, j].

    softmax: p = exp(l - max l) / sum_E exp(l - max l); w_j = p[id_j].
    sigmoid: w_j = sigma(l[id_j]).
    renormalize: w_j /= sum over the k picked of the same quantity.
    """
    l = np.asarray(logits, np.float64)
    ids = np.asarray(ids)
    if gating == "softmax":
        z = l - l.max(axis=1, keepdims=True)
        ez = np.exp(z)
        p = ez / ez.sum(axis=1, keepdims=True)
    elif gating == "sigmoid":
        p = sigmoid(l)
    else:
        raise ValueError(gating)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def permute(ids: np.ndarray, E: int):
    """Token-to-expert permutation of the flat rows r = t*k + j.

    Returns (offsets [E+1], sorted_rows [T*k], row_pos [T*k]):
    offsets = exclusive prefix sum of the per-expert counts; sorted_rows lists
    the rows of expert 0, then expert 1, ..., each segment in ascending row
    order; row_pos is its inverse (row_pos[sorted_rows[i]] = i).
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_rows = np.argsort(flat, kind="stable")
    row_pos = np.empty_like(sorted_rows)
    row_pos[sorted_rows] = np.arange(flat.size)
    return offsets.astype(np.int32), sorted_rows.astype(np.int32), row_pos.astype(np.int32)


def swiglu_expert(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
                  return_hidden: bool = False):
    """SwiGLU expert FFN on the rows of X [n, H]: (silu(X Wg^T) * (X Wu^T)) Wd^T.

    Wg, Wu: [I, H]; Wd: [H, I]; result [n, H].
    """
    X = np.asarray(X, np.float64)
    G = X @ Wg.T
    U = X @ Wu.T
    h = G * sigmoid(G) * U
    Y = h @ Wd.T
    if return_hidden:
        return Y, h
    return Y


def swiglu_expert_mx(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
                     return_hidden: bool = False):
    """The SwiGLU expert as a scaled matrix unit computes it (native MXFP4 mode).

    Both products take MXFP8 E4M3 activations (mx.mxfp8_round_trip): X is
    quantized as given; the hidden vector h = silu(G) * U is rounded to bf16,
    then quantized.  Weights are used exactly as decoded; sums are exact.
    """
    Xq = mx.mxfp8_round_trip(np.asarray(X, np.float64))
    G = Xq @ Wg.T
    U = Xq @ Wu.T
    h = mx.round_to_bf16(G * sigmoid(G) * U)
    Y = mx.mxfp8_round_trip(h) @ Wd.T
    if return_hidden:
        return Y, h
    return Y


def grouped_ffn(x: np.ndarray, k: int, offsets: np.ndarray, sorted_rows: np.ndarray,
                experts, expert_fn=swiglu_expert) -> np.ndarray:
    """Expert outputs in permuted order: y_rows[i] = FFN_e(x[sorted_rows[i] // k]).

    ``experts(e)`` returns (Wg, Wu, Wd) of expert e as float64.  Segment e is
    the rows offsets[e] .. offsets[e+1]-1.  ``expert_fn`` is swiglu_expert
    (exact) or swiglu_expert_mx (native MXFP4 mode).
    """
    x = np.asarray(x, np.float64)
    n = int(offsets[-1])
    y = np.zeros((n, x.shape[1]), dtype=np.float64)
    E = len(offsets) - 1
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        tok = np.asarray(sorted_rows[a:b], dtype=np.int64) // k
        y[a:b] = expert_fn(x[tok], *experts(e))
    return y


def combine(y_rows: np.ndarray, w: np.ndarray, row_pos: np.ndarray,
            y_shared: np.ndarray | None, T: int, k: int) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y_rows[row_pos[t*k + j]]  (+ y_shared[t])."""
    y_rows = np.asarray(y_rows, np.float64)
    w = np.asarray(w, np.float64)
    H = y_rows.shape[1]
    out = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            out[t] += w[t, j] * y_rows[int(row_pos[t * k + j])]
        if y_shared is not None:
            out[t] += y_shared[t]
    return out


def moe_layer(x: np.ndarray, *, k: int, E: int, gating: str, renormalize: bool,
              experts, shared=None, w_router: np.ndarray | None = None,
              logits: np.ndarray | None = None, native_mx: bool = False) -> dict:
    """The whole layer: route, permute, expert FFN, combine.

    x: [T, H] float64.  Either ``w_router`` [E, H] (logits computed) or
    ``logits`` [T, E] (given).  ``experts(e)`` -> (Wg, Wu, Wd) float64;
    ``shared`` is the shared expert's (Wg, Wu, Wd) or None.
    ``native_mx`` selects the native MXFP4 mode's expert (swiglu_expert_mx).
    Returns a dict with every intermediate.
    """
    expert_fn = swiglu_expert_mx if native_mx else swiglu_expert
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    if logits is None:
        logits = router_logits(x, w_router)
    ids = topk(logits, k)
    w = gating_weights(logits, ids, gating, renormalize)
    offsets, sorted_rows, row_pos = permute(ids, E)
    y_rows = grouped_ffn(x, k, offsets, sorted_rows, experts, expert_fn)
    y_shared = expert_fn(x, *shared) if shared is not None else None
    out = combine(y_rows, w, row_pos, y_shared, T, k)
    return dict(logits=np.asarray(logits, np.float32), ids=ids, w=w, offsets=offsets,
                sorted_rows=sorted_rows, row_pos=row_pos, y_rows=y_rows,
                y_shared=y_shared, out=out, margin=topk_margin(logits, k))


def token_output(x_t: np.ndarray, ids_t, w_t, experts, shared=None,
                 native_mx: bool = False) -> np.ndarray:
    """One token's layer output from its routing: sum_j w_j FFN_{id_j}(x) (+ shared)."""
    expert_fn = swiglu_expert_mx if native_mx else swiglu_expert
    x_t = np.asarray(x_t, np.float64)[None, :]
    out = np.zeros(x_t.shape[1])
    for e, wj in zip(ids_t, w_t):
        out += float(wj) * expert_fn(x_t, *experts(int(e)))[0]
    if shared is not None:
        out += expert_fn(x_t, *shared)[0]
    return out
