"""Thin Python binding of the C ABI: one function per entry point, same names.

Arguments are torch tensors (device memory, or pinned host memory for the
cache's host bank) or ``None`` for nullable pointers; the current torch stream
is used unless ``stream`` is given.  Every call only marshals arguments: all
arithmetic runs in the HIP library, and a missing library raises.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib
from ._lib import ExpertLayout, CacheStats, CacheEvent


class FtError(RuntimeError):
    def __init__(self, status: int, text: str):
        self.status = status
        super().__init__(f"{_lib.STATUS_NAMES.get(status, status)}: {text}")


def _check(status: int) -> None:
    if status != 0:
        raise FtError(status, _lib.lib().ft_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data  # numpy array (host)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def version() -> str:
    return _lib.lib().ft_version().decode()


def ft_expert_layout_init(wdtype: int, H: int, I: int) -> ExpertLayout:
    L = ExpertLayout()
    _check(_lib.lib().ft_expert_layout_init(wdtype, H, I, C.byref(L)))
    return L


def ft_workspace_bytes(which: int, T: int, k: int, E: int, H: int = 0, I: int = 0) -> int:
    return int(_lib.lib().ft_workspace_bytes(which, T, k, E, H, I))


def ft_moe_route(x, x_dtype: int, w_router, logits, T: int, H: int, E: int, k: int, gating: int,
                 renormalize: bool, topk_ids, topk_w, stream=None) -> None:
    _check(_lib.lib().ft_moe_route(_ptr(x), x_dtype, _ptr(w_router), _ptr(logits), T, H, E, k, gating,
                                   int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


def ft_moe_route_permute(x, x_dtype: int, w_router, logits, T: int, H: int, E: int, k: int, gating: int,
                         renormalize: bool, topk_ids, topk_w, expert_offsets, sorted_rows, row_pos,
                         workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    _check(_lib.lib().ft_moe_route_permute(_ptr(x), x_dtype, _ptr(w_router), _ptr(logits), T, H, E, k, gating,
                                           int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_w),
                                           _ptr(expert_offsets), _ptr(sorted_rows), _ptr(row_pos),
                                           _ptr(workspace), workspace_bytes, _stream(stream)))


def ft_moe_permute(topk_ids, T: int, k: int, E: int, expert_offsets, sorted_rows, row_pos,
                   workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    _check(_lib.lib().ft_moe_permute(_ptr(topk_ids), T, k, E, _ptr(expert_offsets), _ptr(sorted_rows),
                                     _ptr(row_pos), _ptr(workspace), workspace_bytes, _stream(stream)))


def ft_moe_grouped_ffn(layout: ExpertLayout, slot_pool, slot_of_expert, shared_blob, x, x_dtype: int,
                       T: int, k: int, E: int, expert_offsets, sorted_rows, y_rows, y_shared,
                       mode: int = 0, workspace=None, workspace_bytes: int = 0, stream=None,
                       n_slots: int | None = None) -> None:
    """n_slots: blobs in slot_pool; by default the pool tensor's size over the layout's blob size
    (E for a raw pointer)."""
    if n_slots is None:
        n_slots = slot_pool.numel() * slot_pool.element_size() // int(layout.expert_bytes) \
            if hasattr(slot_pool, "numel") else E
    _check(_lib.lib().ft_moe_grouped_ffn(C.byref(layout), _ptr(slot_pool), int(n_slots), _ptr(slot_of_expert),
                                         _ptr(shared_blob), _ptr(x), x_dtype, T, k, E, _ptr(expert_offsets),
                                         _ptr(sorted_rows), _ptr(y_rows), _ptr(y_shared), mode,
                                         _ptr(workspace), workspace_bytes, _stream(stream)))


def ft_moe_layer(layout: ExpertLayout, slot_pool, slot_of_expert, shared_blob, x, x_dtype: int, w_router, logits,
                 T: int, E: int, k: int, gating: int, renormalize: int, topk_ids, topk_w, expert_offsets,
                 sorted_rows, row_pos, y_rows, y_shared, mode: int, out_dtype: int, out, workspace,
                 workspace_bytes: int, stream=None, n_slots: int | None = None) -> None:
    if n_slots is None:
        n_slots = slot_pool.numel() * slot_pool.element_size() // int(layout.expert_bytes) \
            if hasattr(slot_pool, "numel") else E
    _check(_lib.lib().ft_moe_layer(C.byref(layout), _ptr(slot_pool), int(n_slots), _ptr(slot_of_expert),
                                   _ptr(shared_blob), _ptr(x), x_dtype, _ptr(w_router), _ptr(logits), T, E, k,
                                   gating, int(renormalize), _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets),
                                   _ptr(sorted_rows), _ptr(row_pos), _ptr(y_rows), _ptr(y_shared), mode,
                                   out_dtype, _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)))


def ft_moe_grouped_ffn_noalloc(layout: ExpertLayout, slot_pool, slot_of_expert, shared_blob, x, x_dtype: int,
                               T: int, k: int, E: int, expert_offsets, sorted_rows, y_rows, y_shared,
                               mode: int = 0, stream=None, n_slots: int | None = None) -> None:
    """ft_moe_grouped_ffn with the library's static scratch instead of a workspace."""
    if n_slots is None:
        n_slots = slot_pool.numel() * slot_pool.element_size() // int(layout.expert_bytes) \
            if hasattr(slot_pool, "numel") else E
    _check(_lib.lib().ft_moe_grouped_ffn_noalloc(C.byref(layout), _ptr(slot_pool), int(n_slots),
                                                 _ptr(slot_of_expert), _ptr(shared_blob), _ptr(x), x_dtype, T, k,
                                                 E, _ptr(expert_offsets), _ptr(sorted_rows), _ptr(y_rows),
                                                 _ptr(y_shared), mode, _stream(stream)))


def ft_noalloc_scratch_bytes() -> int:
    return int(_lib.lib().ft_noalloc_scratch_bytes())


def ft_read_checksum(buf, nbytes: int, sink, stream=None) -> None:
    _check(_lib.lib().ft_read_checksum(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))


def ft_cpu_expert_ffn(layout: ExpertLayout, blob, x, n: int, y, n_threads: int = 0) -> None:
    """Host pointers (numpy arrays or pinned tensors) for blob, x (bf16 bits) and y (float32)."""
    _check(_lib.lib().ft_cpu_expert_ffn(C.byref(layout), _ptr(blob), _ptr(x), n, _ptr(y), n_threads))


def ft_cpu_isa(request: int = -1) -> int:
    """Select the host kernel's instruction path (-1: query); returns the path in use."""
    active = C.c_int32()
    _check(_lib.lib().ft_cpu_isa(request, C.byref(active)))
    return active.value


def ft_cpu_miss_rows(layout: ExpertLayout, bank, layer: int, E: int, experts, n_experts: int, expert_offsets,
                     sorted_rows, T: int, k: int, x, y_rows, n_threads: int = 0) -> None:
    """Host rows of a step's CPU misses (all pointers host)."""
    _check(_lib.lib().ft_cpu_miss_rows(C.byref(layout), _ptr(bank), layer, E, _ptr(experts), n_experts,
                                       _ptr(expert_offsets), _ptr(sorted_rows), T, k, _ptr(x), _ptr(y_rows),
                                       n_threads))


def ft_mxfp8_quantize(x, ldx: int, n: int, K: int, codes, scales, stream=None) -> None:
    _check(_lib.lib().ft_mxfp8_quantize(_ptr(x), ldx, n, K, _ptr(codes), _ptr(scales), _stream(stream)))


def ft_moe_combine(y_rows, topk_w, row_pos, y_shared, T: int, k: int, H: int, out_dtype: int, out,
                   stream=None) -> None:
    _check(_lib.lib().ft_moe_combine(_ptr(y_rows), _ptr(topk_w), _ptr(row_pos), _ptr(y_shared), T, k, H,
                                     out_dtype, _ptr(out), _stream(stream)))


class ExpertCache:
    """Owner of one ``ft_expert_cache`` handle (create / step / stats / trace / destroy)."""

    def __init__(self, layout: ExpertLayout, n_layers: int, E: int, capacity: int, slot_pool, host_bank,
                 copy_stream, trace_events: int = 0):
        """trace_events > 0 keeps an event ring of that many records (ft_expert_cache_set_trace)."""
        self.layout = layout
        self.n_layers, self.E, self.capacity = n_layers, E, capacity
        self._keep = (slot_pool, host_bank, copy_stream)
        h = C.c_void_p()
        _check(_lib.lib().ft_expert_cache_create(C.byref(layout), n_layers, E, capacity, _ptr(slot_pool),
                                                 _ptr(host_bank), _stream(copy_stream), C.byref(h)))
        self._h = h
        if trace_events:
            self.set_trace(trace_events)

    def ft_expert_cache_set_trace(self, max_events: int) -> None:
        _check(_lib.lib().ft_expert_cache_set_trace(self._h, int(max_events)))

    set_trace = ft_expert_cache_set_trace

    def ft_expert_cache_step(self, layer: int, topk_ids, T: int, k: int, slot_of_expert, stream=None) -> None:
        _check(_lib.lib().ft_expert_cache_step(self._h, layer, _ptr(topk_ids), T, k, _ptr(slot_of_expert),
                                               _stream(stream)))

    step = ft_expert_cache_step

    def ft_expert_cache_step_split(self, layer: int, topk_ids, T: int, k: int, slot_hits, slot_misses,
                                   stream=None) -> int:
        """Hits-first step: returns the number of fills (wait for them with wait_fills)."""
        n = C.c_int32()
        _check(_lib.lib().ft_expert_cache_step_split(self._h, layer, _ptr(topk_ids), T, k, _ptr(slot_hits),
                                                     _ptr(slot_misses), C.byref(n), _stream(stream)))
        return n.value

    step_split = ft_expert_cache_step_split

    def ft_expert_cache_plan(self, layer: int, topk_ids, T: int, k: int, slot_hits, slot_misses,
                             stream=None) -> None:
        """First half of a hits-first step: enqueue the LRU update and return without waiting."""
        _check(_lib.lib().ft_expert_cache_plan(self._h, layer, _ptr(topk_ids), T, k, _ptr(slot_hits),
                                               _ptr(slot_misses), _stream(stream)))

    plan = ft_expert_cache_plan

    def ft_expert_cache_fill(self) -> int:
        """Second half: wait for the planned LRU update, enqueue the fills; returns their number."""
        n = C.c_int32()
        _check(_lib.lib().ft_expert_cache_fill(self._h, C.byref(n)))
        return n.value

    fill = ft_expert_cache_fill

    def ft_expert_cache_wait_fills(self, stream=None) -> None:
        _check(_lib.lib().ft_expert_cache_wait_fills(self._h, _stream(stream)))

    wait_fills = ft_expert_cache_wait_fills

    def ft_expert_cache_set_split(self, b_pcie: float, b_host: float, T_max: int = 0, k: int = 0) -> None:
        """T_max, k: the largest step whose CPU misses are staged (needed when b_host > 0)."""
        _check(_lib.lib().ft_expert_cache_set_split(self._h, float(b_pcie), float(b_host), int(T_max), int(k)))

    set_split = ft_expert_cache_set_split

    def ft_expert_cache_cpu_misses(self) -> list[int]:
        n = C.c_int32()
        buf = (C.c_int32 * 4096)()
        _check(_lib.lib().ft_expert_cache_cpu_misses(self._h, buf, 4096, C.byref(n)))
        return list(buf[:n.value])

    cpu_misses = ft_expert_cache_cpu_misses

    def ft_expert_cache_stage_cpu_misses(self, x, x_dtype: int, T: int, k: int, expert_offsets, sorted_rows,
                                         stream=None) -> None:
        _check(_lib.lib().ft_expert_cache_stage_cpu_misses(self._h, _ptr(x), x_dtype, T, k, _ptr(expert_offsets),
                                                           _ptr(sorted_rows), _stream(stream)))

    stage_cpu_misses = ft_expert_cache_stage_cpu_misses

    def ft_expert_cache_run_cpu_misses(self, y_rows, stream=None, n_threads: int = 0) -> None:
        _check(_lib.lib().ft_expert_cache_run_cpu_misses(self._h, _ptr(y_rows), _stream(stream), n_threads))

    run_cpu_misses = ft_expert_cache_run_cpu_misses

    def ft_expert_cache_prefetch_layer(self, layer: int, stream=None) -> None:
        _check(_lib.lib().ft_expert_cache_prefetch_layer(self._h, layer, _stream(stream)))

    prefetch_layer = ft_expert_cache_prefetch_layer

    def ft_expert_cache_resize(self, capacity: int, slot_pool, stream=None) -> None:
        _check(_lib.lib().ft_expert_cache_resize(self._h, capacity, _ptr(slot_pool), _stream(stream)))
        self.capacity = capacity
        self._keep = (slot_pool,) + tuple(self._keep[1:])

    resize = ft_expert_cache_resize

    def stats(self) -> dict:
        s = CacheStats()
        _check(_lib.lib().ft_expert_cache_stats(self._h, C.byref(s)))
        return {n: int(getattr(s, n)) for n, _ in CacheStats._fields_}

    def trace(self) -> list[tuple]:
        need = C.c_size_t()
        _check(_lib.lib().ft_expert_cache_trace(self._h, None, 0, C.byref(need)))
        n = need.value // C.sizeof(CacheEvent)
        buf = (CacheEvent * max(n, 1))()
        _check(_lib.lib().ft_expert_cache_trace(self._h, C.cast(buf, C.c_void_p), need.value, None))
        return [(e.step, e.layer, e.expert, e.hit, e.slot, e.evicted) for e in buf[:n]]

    def lookup(self, layer: int, expert: int) -> int:
        s = C.c_int32()
        _check(_lib.lib().ft_expert_cache_lookup(self._h, layer, expert, C.byref(s)))
        return s.value

    def destroy(self) -> None:
        if self._h:
            _check(_lib.lib().ft_expert_cache_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
