"""ctypes declarations of the C ABI in ``include/ft_moe.h`` (no logic here)."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# FTMOE_LIB: another build of the same library (e.g. the sanitizer build of build.py)
LIB_PATH = os.environ.get("FTMOE_LIB") or os.path.join(PKG, "libftmoe.so")

# status codes
FT_OK, FT_EINVAL, FT_ENOTSUP, FT_ECAPACITY, FT_EHIP = 0, -1, -2, -3, -4
STATUS_NAMES = {0: "FT_OK", -1: "FT_EINVAL", -2: "FT_ENOTSUP", -3: "FT_ECAPACITY", -4: "FT_EHIP"}
# dtypes / gating / workspace selectors
FT_F32, FT_BF16, FT_MXFP4, FT_NVFP4 = 0, 1, 2, 3
FT_SOFTMAX, FT_SIGMOID = 0, 1
FT_WS_PERMUTE, FT_WS_FFN, FT_WS_ROUTE_PERMUTE, FT_WS_LAYER = 1, 2, 3, 4
FT_FFN_EXACT, FT_FFN_NATIVE_MX = 0, 1
FT_SLOT_SKIP = -2
FT_CPU_ISA_QUERY, FT_CPU_ISA_BEST, FT_CPU_AVX2, FT_CPU_AVX512_BF16 = -1, 0, 1, 2
FT_FFN_GATE_UP_ONLY, FT_FFN_DOWN_ONLY = 0x100, 0x200

EXPORTS = [
    "ft_last_error", "ft_version", "ft_expert_layout_init", "ft_moe_route", "ft_moe_permute",
    "ft_moe_grouped_ffn", "ft_moe_combine", "ft_expert_cache_create", "ft_expert_cache_step",
    "ft_expert_cache_stats", "ft_expert_cache_trace", "ft_expert_cache_lookup",
    "ft_expert_cache_destroy", "ft_workspace_bytes", "ft_mxfp8_quantize", "ft_moe_route_permute",
    "ft_expert_cache_resize", "ft_expert_cache_prefetch_layer", "ft_expert_cache_set_split",
    "ft_expert_cache_cpu_misses", "ft_cpu_expert_ffn", "ft_cpu_miss_rows", "ft_cpu_isa",
    "ft_expert_cache_stage_cpu_misses", "ft_expert_cache_run_cpu_misses", "ft_expert_cache_step_split",
    "ft_expert_cache_wait_fills", "ft_expert_cache_plan", "ft_expert_cache_fill", "ft_expert_cache_set_trace",
    "ft_moe_grouped_ffn_noalloc", "ft_noalloc_scratch_bytes", "ft_moe_layer", "ft_read_checksum",
]


class ExpertLayout(C.Structure):
    _fields_ = [
        ("wdtype", C.c_int32), ("H", C.c_int32), ("I", C.c_int32), ("reserved", C.c_int32),
        ("expert_bytes", C.c_uint64),
        ("off_gate", C.c_uint64), ("off_up", C.c_uint64), ("off_down", C.c_uint64),
        ("off_sgate", C.c_uint64), ("off_sup", C.c_uint64), ("off_sdown", C.c_uint64),
        ("off_tscale", C.c_uint64),
    ]


class CacheStats(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in
                ("accesses", "hits", "misses", "evictions", "bytes_h2d", "steps", "prefetch_fills",
                 "cpu_misses", "cpu_ns", "trace_dropped")]


class CacheEvent(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("step", "layer", "expert", "hit", "slot", "evicted")]


_lib = None


class LibraryMissing(RuntimeError):
    """The HIP library has not been built (run expert_cached_ffn_amd.build)."""


def lib() -> C.CDLL:
    """Load libftmoe.so once; raise if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(f"{LIB_PATH} not found: build it with `python -m expert_cached_ffn_amd.build`")
    L = C.CDLL(LIB_PATH)
    p, i32, sz, u64 = C.c_void_p, C.c_int32, C.c_size_t, C.c_uint64
    L.ft_last_error.restype = C.c_char_p
    L.ft_last_error.argtypes = []
    L.ft_version.restype = C.c_char_p
    L.ft_version.argtypes = []
    L.ft_expert_layout_init.restype = i32
    L.ft_expert_layout_init.argtypes = [i32, i32, i32, C.POINTER(ExpertLayout)]
    L.ft_moe_route.restype = i32
    L.ft_moe_route.argtypes = [p, i32, p, p, i32, i32, i32, i32, i32, i32, p, p, p]
    L.ft_moe_permute.restype = i32
    L.ft_moe_permute.argtypes = [p, i32, i32, i32, p, p, p, p, sz, p]
    L.ft_moe_grouped_ffn.restype = i32
    L.ft_moe_grouped_ffn.argtypes = [C.POINTER(ExpertLayout), p, i32, p, p, p, i32, i32, i32, i32, p, p, p, p,
                                     i32, p, sz, p]
    L.ft_moe_layer.restype = i32
    L.ft_moe_layer.argtypes = [C.POINTER(ExpertLayout), p, i32, p, p, p, i32, p, p, i32, i32, i32, i32, i32,
                               p, p, p, p, p, p, p, i32, i32, p, p, sz, p]
    L.ft_moe_grouped_ffn_noalloc.restype = i32
    L.ft_moe_grouped_ffn_noalloc.argtypes = [C.POINTER(ExpertLayout), p, i32, p, p, p, i32, i32, i32, i32, p, p,
                                             p, p, i32, p]
    L.ft_noalloc_scratch_bytes.restype = sz
    L.ft_noalloc_scratch_bytes.argtypes = []
    L.ft_read_checksum.restype = i32
    L.ft_read_checksum.argtypes = [p, C.c_uint64, p, p]
    L.ft_cpu_expert_ffn.restype = i32
    L.ft_cpu_expert_ffn.argtypes = [C.POINTER(ExpertLayout), p, p, i32, p, i32]
    L.ft_cpu_miss_rows.restype = i32
    L.ft_cpu_isa.restype = i32
    L.ft_expert_cache_stage_cpu_misses.restype = i32
    L.ft_expert_cache_stage_cpu_misses.argtypes = [p, p, i32, i32, i32, p, p, p]
    L.ft_expert_cache_step_split.restype = i32
    L.ft_expert_cache_step_split.argtypes = [p, i32, p, i32, i32, p, p, C.POINTER(C.c_int32), p]
    L.ft_expert_cache_wait_fills.restype = i32
    L.ft_expert_cache_wait_fills.argtypes = [p, p]
    L.ft_expert_cache_plan.restype = i32
    L.ft_expert_cache_plan.argtypes = [p, i32, p, i32, i32, p, p, p]
    L.ft_expert_cache_fill.restype = i32
    L.ft_expert_cache_fill.argtypes = [p, C.POINTER(C.c_int32)]
    L.ft_expert_cache_run_cpu_misses.restype = i32
    L.ft_expert_cache_run_cpu_misses.argtypes = [p, p, p, i32]
    L.ft_cpu_isa.argtypes = [i32, p]
    L.ft_cpu_miss_rows.argtypes = [C.POINTER(ExpertLayout), p, i32, i32, p, i32, p, p, i32, i32, p, p, i32]
    L.ft_expert_cache_set_split.restype = i32
    L.ft_expert_cache_set_split.argtypes = [p, C.c_double, C.c_double, i32, i32]
    L.ft_expert_cache_set_trace.restype = i32
    L.ft_expert_cache_set_trace.argtypes = [p, C.c_int64]
    L.ft_expert_cache_cpu_misses.restype = i32
    L.ft_expert_cache_cpu_misses.argtypes = [p, p, i32, p]
    L.ft_expert_cache_prefetch_layer.restype = i32
    L.ft_expert_cache_prefetch_layer.argtypes = [p, i32, p]
    L.ft_expert_cache_resize.restype = i32
    L.ft_expert_cache_resize.argtypes = [p, i32, p, p]
    L.ft_moe_route_permute.restype = i32
    L.ft_moe_route_permute.argtypes = [p, i32, p, p, i32, i32, i32, i32, i32, i32, p, p, p, p, p, p, sz, p]
    L.ft_mxfp8_quantize.restype = i32
    L.ft_mxfp8_quantize.argtypes = [p, C.c_int64, i32, i32, p, p, p]
    L.ft_moe_combine.restype = i32
    L.ft_moe_combine.argtypes = [p, p, p, p, i32, i32, i32, i32, p, p]
    L.ft_expert_cache_create.restype = i32
    L.ft_expert_cache_create.argtypes = [C.POINTER(ExpertLayout), i32, i32, i32, p, p, p, C.POINTER(p)]
    L.ft_expert_cache_step.restype = i32
    L.ft_expert_cache_step.argtypes = [p, i32, p, i32, i32, p, p]
    L.ft_expert_cache_stats.restype = i32
    L.ft_expert_cache_stats.argtypes = [p, C.POINTER(CacheStats)]
    L.ft_expert_cache_trace.restype = i32
    L.ft_expert_cache_trace.argtypes = [p, p, sz, C.POINTER(sz)]
    L.ft_expert_cache_lookup.restype = i32
    L.ft_expert_cache_lookup.argtypes = [p, i32, i32, C.POINTER(i32)]
    L.ft_expert_cache_destroy.restype = i32
    L.ft_expert_cache_destroy.argtypes = [p]
    L.ft_workspace_bytes.restype = sz
    L.ft_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    _ = u64
    _lib = L
    return L
