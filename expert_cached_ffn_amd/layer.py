"""Device buffers and call sequence for one MoE layer (plumbing only).

``pack_expert`` places one expert's weights into its blob at the offsets the
library's ``ft_expert_layout_init`` reports.  ``MoELayer`` owns the device
buffers of one layer shape and enqueues route -> permute -> grouped FFN ->
combine on one stream; every step runs in the HIP library.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import _lib, ops

DTYPES = {"f32": _lib.FT_F32, "bf16": _lib.FT_BF16, "mxfp4": _lib.FT_MXFP4, "nvfp4": _lib.FT_NVFP4}
GATING = {"softmax": _lib.FT_SOFTMAX, "sigmoid": _lib.FT_SIGMOID}

_DENSE_PARTS = (("wg", "off_gate"), ("wu", "off_up"), ("wd", "off_down"))
_FP4_PARTS = (("gate_codes", "off_gate"), ("up_codes", "off_up"), ("down_codes", "off_down"),
              ("gate_scales", "off_sgate"), ("up_scales", "off_sup"), ("down_scales", "off_sdown"))


def pack_expert(layout, arrays: dict, out: np.ndarray | None = None) -> np.ndarray:
    """One expert's storage arrays -> its blob bytes (uint8 [expert_bytes])."""
    eb = int(layout.expert_bytes)
    blob = np.zeros(eb, np.uint8) if out is None else out
    parts = _FP4_PARTS if layout.wdtype in (_lib.FT_MXFP4, _lib.FT_NVFP4) else _DENSE_PARTS
    if layout.wdtype == _lib.FT_NVFP4:
        parts = parts + (("tensor_scales", "off_tscale"),)
    for name, off in parts:
        a = np.ascontiguousarray(arrays[name]).view(np.uint8).ravel()
        o = int(getattr(layout, off))
        blob[o:o + a.size] = a
    return blob


def as_device_u8(blobs: list[np.ndarray], device="cuda") -> torch.Tensor:
    """Stack blobs into one contiguous uint8 device tensor (slot s = blob s)."""
    host = np.stack(blobs) if blobs else np.zeros((0, 0), np.uint8)
    return torch.from_numpy(host).to(device)


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """A storage array as a device tensor with the same bytes (bf16 bits stay int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


@dataclass
class LayerShape:
    H: int
    I: int
    E: int
    k: int
    wdtype: str
    xdtype: str
    gating: str
    renormalize: bool
    shared: bool


class MoELayer:
    """Buffers for up to ``T_max`` tokens and the four-call layer sequence."""

    def __init__(self, shape: LayerShape, T_max: int, device="cuda"):
        self.s = shape
        self.T_max = T_max
        self.layout = ops.ft_expert_layout_init(DTYPES[shape.wdtype], shape.H, shape.I)
        H, E, k = shape.H, shape.E, shape.k
        dev = torch.device(device)
        i32, f32 = torch.int32, torch.float32
        self.logits = torch.empty((T_max, E), dtype=f32, device=dev)
        self.ids = torch.empty((T_max, k), dtype=i32, device=dev)
        self.w = torch.empty((T_max, k), dtype=f32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.sorted_rows = torch.empty(max(1, T_max * k), dtype=i32, device=dev)
        self.row_pos = torch.empty(max(1, T_max * k), dtype=i32, device=dev)
        self.y_rows = torch.empty((max(1, T_max * k), H), dtype=f32, device=dev)
        self.y_shared = torch.empty((T_max, H), dtype=f32, device=dev) if shape.shared else None
        out_dt = torch.float32 if shape.xdtype == "f32" else torch.int16
        self.out = torch.empty((T_max, H), dtype=out_dt, device=dev)
        self.ws_perm_bytes = ops.ft_workspace_bytes(_lib.FT_WS_PERMUTE, T_max, k, E)
        self.ws_ffn_bytes = ops.ft_workspace_bytes(_lib.FT_WS_FFN, T_max, k, E, H, shape.I)
        self.ws_perm = torch.empty(max(256, self.ws_perm_bytes), dtype=torch.uint8, device=dev)
        self.ws_rp_bytes = ops.ft_workspace_bytes(_lib.FT_WS_ROUTE_PERMUTE, T_max, k, E)
        self.ws_rp = torch.empty(max(256, self.ws_rp_bytes), dtype=torch.uint8, device=dev)
        self.ws_ffn = torch.empty(max(256, self.ws_ffn_bytes), dtype=torch.uint8, device=dev)
        self.ws_layer_bytes = ops.ft_workspace_bytes(_lib.FT_WS_LAYER, T_max, k, E, H, shape.I)
        # zeroed: its first 8192 bytes are ft_moe_layer's wait area (the one-token kernel's grid-wide wait),
        # which must be zero before the first call; every call leaves it ready for the next
        self.ws_layer = torch.zeros(max(256, self.ws_layer_bytes), dtype=torch.uint8, device=dev)

    def route(self, T, x=None, w_router=None, logits=None, stream=None):
        s = self.s
        if logits is not None:
            self.logits[:T].copy_(logits[:T])
            x, w_router = None, None
        ops.ft_moe_route(x, DTYPES[s.xdtype], w_router, self.logits, T, s.H, s.E, s.k, GATING[s.gating],
                         s.renormalize, self.ids, self.w, stream=stream)

    def route_permute(self, T, x=None, w_router=None, logits=None, stream=None):
        """route + permute through ft_moe_route_permute (one launch in the decode regime)."""
        s = self.s
        if logits is not None:
            self.logits[:T].copy_(logits[:T])
            x, w_router = None, None
        ops.ft_moe_route_permute(x, DTYPES[s.xdtype], w_router, self.logits, T, s.H, s.E, s.k, GATING[s.gating],
                                 s.renormalize, self.ids, self.w, self.offsets, self.sorted_rows, self.row_pos,
                                 self.ws_rp, self.ws_rp_bytes, stream=stream)

    def permute(self, T, ids=None, stream=None):
        ids = self.ids if ids is None else ids
        ops.ft_moe_permute(ids, T, self.s.k, self.s.E, self.offsets, self.sorted_rows, self.row_pos,
                           self.ws_perm, self.ws_perm_bytes, stream=stream)

    def ffn(self, T, x, pool, slot_of_expert=None, shared_blob=None, stream=None, mode=0):
        s = self.s
        ops.ft_moe_grouped_ffn(self.layout, pool, slot_of_expert, shared_blob, x, DTYPES[s.xdtype], T, s.k,
                               s.E, self.offsets, self.sorted_rows, self.y_rows,
                               self.y_shared if shared_blob is not None else None, mode, self.ws_ffn,
                               self.ws_ffn_bytes, stream=stream)

    def combine(self, T, w=None, with_shared=True, stream=None):
        s = self.s
        w = self.w if w is None else w
        out_dt = _lib.FT_F32 if s.xdtype == "f32" else _lib.FT_BF16
        ys = self.y_shared if (with_shared and self.y_shared is not None) else None
        ops.ft_moe_combine(self.y_rows, w, self.row_pos, ys, T, s.k, s.H, out_dt, self.out, stream=stream)

    def stage_cpu_misses(self, cache, T, x, stream=None):
        """After the cache step, before ffn(): stage this step's inputs of the CPU misses."""
        cache.stage_cpu_misses(x, DTYPES[self.s.xdtype], T, self.s.k, self.offsets, self.sorted_rows, stream=stream)

    def run_cpu_misses(self, cache, stream=None, n_threads=0):
        """After ffn(): the CPU misses' rows on the host, copied into y_rows on the stream."""
        cache.run_cpu_misses(self.y_rows, stream=stream, n_threads=n_threads)

    def forward_layer(self, T, x, pool, w_router=None, logits=None, slot_of_expert=None, shared_blob=None,
                      stream=None, mode=0):
        """The whole layer through ft_moe_layer (three launches for a few tokens)."""
        s = self.s
        if logits is not None:
            self.logits[:T].copy_(logits[:T])
            w_router = None
        out_dt = _lib.FT_F32 if s.xdtype == "f32" else _lib.FT_BF16
        ops.ft_moe_layer(self.layout, pool, slot_of_expert, shared_blob, x, DTYPES[s.xdtype], w_router, self.logits,
                         T, s.E, s.k, GATING[s.gating], s.renormalize, self.ids, self.w, self.offsets,
                         self.sorted_rows, self.row_pos, self.y_rows,
                         self.y_shared if shared_blob is not None else None, mode, out_dt, self.out,
                         self.ws_layer, self.ws_layer_bytes, stream=stream)
        return self.out[:T]

    def forward(self, T, x, pool, w_router=None, logits=None, slot_of_expert=None, shared_blob=None,
                stream=None, mode=0):
        """route -> permute -> grouped FFN -> combine, all enqueued on one stream."""
        self.route_permute(T, x=x, w_router=w_router, logits=logits, stream=stream)
        self.ffn(T, x, pool, slot_of_expert=slot_of_expert, shared_blob=shared_blob, stream=stream,
                 mode=mode)
        self.combine(T, with_shared=shared_blob is not None, stream=stream)
        return self.out[:T]
