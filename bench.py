#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X, with the roofline of its dominant kernel.

    python bench.py [--steps K] [--warmup W] [--workload decode-bf16|decode-mxfp4|decode-nvfp4|prefill-mxfp4|...]

A step is one pass of the whole layer -- route, permute, grouped SwiGLU FFN
(weights through the slot table), combine; plus the cache step for the
cache-trace workload -- over one batch of synthetic tokens whose inputs are
already resident in HBM.  The default workload is the Qwen3-A3B-shaped bf16
decode layer (H=2048, I=768, 128 experts, top-8 softmax renormalised) at a
decode batch of 64 tokens; batches 1 and 16 are reported beside it.  Input
sets rotate (8 different token batches, hence different routings) so the
activated experts change every step.

Prints one JSON line.  ``roofline`` is computed for the dominant kernel (the
gate/up + SwiGLU stage of the grouped FFN) from its average duration measured
with HIP events on the launch stream inside the timed region, against its
algorithmic bytes.  ``cpu_baseline`` times the CPU oracle (float64 NumPy) on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (decode, prefill) + % HBM BW / % MFMA peak, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA bf16
FP8_PEAK_TFLOPS = 5000.0       # dense MFMA fp8 (and fp8 x fp4 block-scaled)
N_INPUT_SETS = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources (and build flags) the FFN kernels are compiled from: a change to
# any of them invalidates committed counter readings of those kernels
FFN_KERNEL_SOURCES = ("csrc/ffn.hip", "csrc/ft_internal.hpp", "csrc/stream_persist.hpp", "csrc/stream_gemm.hpp",
                      "csrc/gemm_prefill.hpp", "csrc/gemm_mx.hpp", "csrc/mx.hip", "build.py")


def kernel_sources_hash():
    """Short sha256 over the FFN kernels' sources (names and contents)."""
    import hashlib
    h = hashlib.sha256()
    for rel in FFN_KERNEL_SOURCES:
        h.update(rel.encode())
        with open(os.path.join(ROOT, "expert_cached_ffn_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(profile, kernel_prefix):
    """HBM bytes per launch from a committed counter summary, if it belongs to these sources."""
    path = os.path.join(ROOT, "profiles", profile)
    try:
        with open(path) as f:
            doc = json.load(f)
    except OSError:
        return None
    if doc.get("csrc_sha256_16") != kernel_sources_hash():
        return None  # kernels changed since the counters were taken
    for name, v in doc.get("kernels", {}).items():
        if name.startswith(kernel_prefix):
            return v["traffic_bytes"]
    return None


# ----------------------------------------------------------------------------- inputs

def build_pool(L, layer, cfg, experts, n_slots, layer_idx=0):
    """All given experts packed into a device pool, expert e in slot e."""
    import torch
    import synth
    eb = int(layer.layout.expert_bytes)
    pool = torch.empty((n_slots, eb), dtype=torch.uint8, device="cuda")
    buf = np.zeros(eb, np.uint8)
    for e in experts:
        L.pack_expert(layer.layout, synth.expert_weights(cfg, layer_idx, e).arrays, buf)
        pool[e].copy_(torch.from_numpy(buf))
    return pool


def expert_weight_bytes(cfg, part):
    """Bytes of one expert's gate+up ('gate_up') or down ('down') weights incl. scales."""
    n = cfg.H * cfg.I
    if cfg.wdtype == "mxfp4":
        one = n // 2 + n // 32
    elif cfg.wdtype == "nvfp4":
        one = n // 2 + n // 16 + 4   # codes, E4M3 block scales, the fp32 tensor scale
    elif cfg.wdtype == "bf16":
        one = 2 * n
    else:
        one = 4 * n
    return 2 * one if part == "gate_up" else one


# ----------------------------------------------------------------------------- timing

class Timer:
    """HIP events on the current stream.  ``n`` events are created (and recorded once) up front, so
    that no event creation falls inside a timed region."""

    def __init__(self, n=0):
        import torch
        self.torch = torch
        self.pool = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.pool:
            e.record()
        torch.cuda.synchronize()
        self.ev = []

    def mark(self):
        i = len(self.ev)
        e = self.pool[i] if i < len(self.pool) else self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.ev.append(e)
        return e


class no_gc:
    """Python's cyclic garbage collector paused for a timed region (a collection pass would stall
    the host thread that enqueues the launches)."""

    def __enter__(self):
        self.was = gc.isenabled()
        gc.disable()

    def __exit__(self, *exc):
        if self.was:
            gc.enable()


def run_decode(args, cfg, batches, main_T):
    import torch
    import synth
    from expert_cached_ffn_amd import layer as L
    from expert_cached_ffn_amd import _lib

    torch.cuda.set_device(0)
    shape = L.LayerShape(cfg.H, cfg.I, cfg.E, cfg.k, cfg.wdtype, cfg.xdtype, cfg.gating, cfg.renormalize,
                         cfg.shared)
    probe = L.MoELayer(shape, 1)
    t0 = time.time()
    pool = build_pool(L, probe, cfg, range(cfg.E), cfg.E)
    shared = None
    if cfg.shared:
        shared = L.as_device_u8([L.pack_expert(probe.layout, synth.expert_weights(cfg, 0, cfg.E).arrays)])[0]
    wr = L.to_device(synth.router_weight(cfg))
    torch.cuda.synchronize()
    log(f"pool of {cfg.E} experts ({pool.numel() / 1e9:.2f} GB) built in {time.time() - t0:.1f}s")

    results = {}
    for T in batches:
        layer = L.MoELayer(shape, T)
        xs = [L.to_device(synth.tokens(cfg, T, case=r)) for r in range(N_INPUT_SETS)]
        # distinct routed experts of every input set (for the algorithmic bytes)
        n_act = []
        for r in range(N_INPUT_SETS):
            layer.forward(T, xs[r], pool, w_router=wr, shared_blob=shared)
            torch.cuda.synchronize()
            n_act.append(len(np.unique(layer.ids[:T].cpu().numpy())))

        def step(i, tm=None):
            x = xs[i % N_INPUT_SETS]
            if tm is not None:
                tm.mark()
            layer.route_permute(T, x=x, w_router=wr)
            if tm is not None:
                tm.mark()
            layer.ffn(T, x, pool, shared_blob=shared, mode=_lib.FT_FFN_GATE_UP_ONLY)
            if tm is not None:
                tm.mark()
            layer.ffn(T, x, pool, shared_blob=shared, mode=_lib.FT_FFN_DOWN_ONLY)
            layer.combine(T, with_shared=shared is not None)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        tm = Timer(3 * args.steps)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        with no_gc():
            start.record()
            for i in range(args.steps):
                step(i, tm)
            end.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)
        ms = total_ms / args.steps
        k_ms = [tm.ev[3 * i + 1].elapsed_time(tm.ev[3 * i + 2]) for i in range(args.steps)]
        step_ms = [tm.ev[3 * i].elapsed_time(tm.ev[3 * (i + 1)] if i + 1 < args.steps else end)
                   for i in range(args.steps)]
        k_avg = float(np.mean(k_ms))
        act = np.array([n_act[i % N_INPUT_SETS] for i in range(args.steps)], np.float64)
        bytes_gu = float(np.mean((act + (1 if cfg.shared else 0)) * expert_weight_bytes(cfg, "gate_up")))
        bytes_gu += T * cfg.H * 2 + (T * cfg.k + (T if cfg.shared else 0)) * cfg.I * 2
        layer_bytes = float(np.mean((act + (1 if cfg.shared else 0)) *
                                    (expert_weight_bytes(cfg, "gate_up") + expert_weight_bytes(cfg, "down"))))

        # HIP-graph replay of the same step (one graph per input set)
        graph_ms = None
        if not args.no_graph:
            graphs = []
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for r in range(N_INPUT_SETS):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=s):
                        step(r)
                    graphs.append(g)
            torch.cuda.current_stream().wait_stream(s)
            for i in range(args.warmup):
                graphs[i % N_INPUT_SETS].replay()
            torch.cuda.synchronize()
            with no_gc():
                start.record()
                for i in range(args.steps):
                    graphs[i % N_INPUT_SETS].replay()
                end.record()
            torch.cuda.synchronize()
            graph_ms = start.elapsed_time(end) / args.steps
        # the same layer as one ft_moe_layer call (for a few tokens: router, gate/up with the routing
        # inside, down with the combine inside), eager and from HIP graphs
        def lstep(i):
            layer.forward_layer(T, xs[i % N_INPUT_SETS], pool, w_router=wr, shared_blob=shared)

        for i in range(args.warmup):
            lstep(i)
        torch.cuda.synchronize()
        # the mean from events around the whole run; the spread from a second run with an event
        # between every two steps (those markers add a little time of their own)
        with no_gc():
            start.record()
            for i in range(args.steps):
                lstep(i)
            end.record()
        torch.cuda.synchronize()
        lms = start.elapsed_time(end) / args.steps
        lt = Timer(args.steps + 1)
        with no_gc():
            for i in range(args.steps):
                lt.mark()
                lstep(i)
            lt.mark()
        torch.cuda.synchronize()
        lstep_ms = [lt.ev[i].elapsed_time(lt.ev[i + 1]) for i in range(args.steps)]
        lgraph_ms = lgraph8_ms = lgraph48_ms = None
        if not args.no_graph:
            lgraphs = []
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for r in range(N_INPUT_SETS):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=s):
                        lstep(r)
                    lgraphs.append(g)
            torch.cuda.current_stream().wait_stream(s)
            for i in range(args.warmup):
                lgraphs[i % N_INPUT_SETS].replay()
            torch.cuda.synchronize()
            with no_gc():
                start.record()
                for i in range(args.steps):
                    lgraphs[i % N_INPUT_SETS].replay()
                end.record()
            torch.cuda.synchronize()
            lgraph_ms = start.elapsed_time(end) / args.steps
            # one graph holding G layer calls, the input sets in turn, as a decode step's graph holds
            # its model's layers one after another (48 MoE layers in the Qwen3-30B-A3B model whose
            # expert shape this is): per-replay costs spread over them
            def graph_of(G):
                gg = torch.cuda.CUDAGraph()
                with torch.cuda.stream(s):
                    with torch.cuda.graph(gg, stream=s):
                        for r in range(G):
                            lstep(r % N_INPUT_SETS)
                torch.cuda.current_stream().wait_stream(s)
                reps = max(1, args.steps // G)
                for i in range(max(1, args.warmup // G)):
                    gg.replay()
                torch.cuda.synchronize()
                with no_gc():
                    start.record()
                    for i in range(reps):
                        gg.replay()
                    end.record()
                torch.cuda.synchronize()
                return start.elapsed_time(end) / (reps * G)
            lgraph8_ms = graph_of(N_INPUT_SETS)
            lgraph48_ms = graph_of(48)
        # one layer call is the unit of work: its time gives tokens/s; the four calls (with events
        # around the gate/up launch for the roofline) are reported beside it
        results[T] = dict(ms_per_step=lms, tokens_per_s=T / (lms * 1e-3), gate_up_ms=k_avg,
                          step_ms_p10_p50_p90=[float(v) for v in np.percentile(lstep_ms, [10, 50, 90])],
                          gate_up_bytes=bytes_gu, layer_weight_bytes=layer_bytes,
                          distinct_experts=float(np.mean(n_act)), graph_ms_per_step=lgraph_ms,
                          graph_of_8_steps_ms_per_step=lgraph8_ms, graph_of_48_steps_ms_per_step=lgraph48_ms,
                          four_calls_ms_per_step=ms, four_calls_graph_ms_per_step=graph_ms,
                          four_calls_step_ms_p10_p50_p90=[float(v) for v in np.percentile(step_ms, [10, 50, 90])])
        gtxt = (f"{lgraph_ms * 1e3:.1f} us (8 / 48 steps per graph {lgraph8_ms * 1e3:.1f} / {lgraph48_ms * 1e3:.1f} us)"
                if lgraph_ms is not None else "n/a")
        g4 = f"{graph_ms * 1e3:.1f} us" if graph_ms is not None else "n/a"
        log(f"T={T}: layer call {lms * 1e3:.1f} us/step ({T / (lms * 1e-3):,.0f} tok/s), graph {gtxt}; four calls "
            f"{ms * 1e3:.1f} us, graph {g4}; gate/up {k_avg * 1e3:.1f} us = {bytes_gu / (k_avg * 1e-3) / 1e9:,.0f} GB/s, "
            f"layer weights {layer_bytes / (lms * 1e-3) / 1e9:,.0f} GB/s")
        del layer, xs
    if args.copy_calibration:
        copy_calibration()
    return results


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size, so HBM counters can be scaled."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} x {nbytes} B device copy")


def achievable_peaks():
    """What this machine reaches: a 1 GiB device copy (read + write bytes / time), a plain read of the same
    1 GiB (the library's checksum, whole 128-byte lines: the ceiling of a read-only weight stream), an
    8192^3 bf16 GEMM through torch's BLAS (hipBLASLt) and the same GEMM in FP8; best of a few runs."""
    import torch
    from expert_cached_ffn_amd import ops
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(5):
        s.record()
        b.copy_(a)
        e.record()
        torch.cuda.synchronize()
        best = max(best, 2 * n / (s.elapsed_time(e) * 1e-3) / 1e9)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.ft_read_checksum(a, n, sink)
    read = 0.0
    for _ in range(5):
        s.record()
        ops.ft_read_checksum(a, n, sink)
        e.record()
        torch.cuda.synchronize()
        read = max(read, n / (s.elapsed_time(e) * 1e-3) / 1e9)
    del a, b
    m = 8192
    x = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    y = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    x @ y
    torch.cuda.synchronize()
    tf = 0.0
    for _ in range(5):
        s.record()
        x @ y
        e.record()
        torch.cuda.synchronize()
        tf = max(tf, 2 * m ** 3 / (s.elapsed_time(e) * 1e-3) / 1e12)
    # the same GEMM in OCP FP8 E4M3 with per-tensor scales (torch._scaled_mm): the library's context for
    # the scaled FP8 x FP4 MFMA mode; None where this torch build has no FP8 GEMM for the device
    tf8 = None
    try:
        x8 = x.to(torch.float8_e4m3fn)
        y8 = y.t().contiguous().to(torch.float8_e4m3fn).t()      # column-major right operand
        one = torch.ones((), dtype=torch.float32, device="cuda")
        torch._scaled_mm(x8, y8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        tf8 = 0.0
        for _ in range(5):
            s.record()
            torch._scaled_mm(x8, y8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            e.record()
            torch.cuda.synchronize()
            tf8 = max(tf8, 2 * m ** 3 / (s.elapsed_time(e) * 1e-3) / 1e12)
        del x8, y8
    except (RuntimeError, AttributeError, TypeError) as err:
        log(f"fp8 GEMM through torch unavailable: {err}")
    del x, y
    fp8_txt = f", fp8 GEMM {tf8:,.0f} TFLOP/s" if tf8 else ""
    log(f"achievable on this box: device copy {best:,.0f} GB/s (read + write), plain read {read:,.0f} GB/s, "
        f"bf16 GEMM {tf:,.0f} TFLOP/s{fp8_txt}")
    return {"copy_GBps": best, "read_GBps": read, "bf16_gemm_TFLOPs": tf, "fp8_gemm_TFLOPs": tf8}


def run_prefill(args, cfg, T, mode=0):
    """Prefill layer: given Zipf-skewed logits, grouped MFMA GEMM over ragged segments.

    mode 0: exact (MXFP4 decoded to bf16, bf16 MFMA); mode 1: native (MXFP8 x MXFP4 scaled MFMA)."""
    import torch
    import synth
    from expert_cached_ffn_amd import layer as L
    from expert_cached_ffn_amd import _lib

    torch.cuda.set_device(0)
    shape = L.LayerShape(cfg.H, cfg.I, cfg.E, cfg.k, cfg.wdtype, cfg.xdtype, cfg.gating, cfg.renormalize,
                         cfg.shared)
    layer = L.MoELayer(shape, T)
    t0 = time.time()
    pool = build_pool(L, layer, cfg, range(cfg.E), cfg.E)
    shared = L.as_device_u8([L.pack_expert(layer.layout, synth.expert_weights(cfg, 0, cfg.E).arrays)])[0] \
        if cfg.shared else None
    n_sets = 2
    xs = [L.to_device(synth.tokens(cfg, T, case=r)) for r in range(n_sets)]
    lg = [L.to_device(synth.prefill_logits(cfg, T, case=r)) for r in range(n_sets)]
    torch.cuda.synchronize()
    log(f"prefill inputs built in {time.time() - t0:.1f}s")
    rows = T * cfg.k + (T if cfg.shared else 0)
    flops_gu = 2.0 * 2 * cfg.H * cfg.I * rows
    flops_all = 3.0 * 2 * cfg.H * cfg.I * rows

    def step(i, tm=None):
        r = i % n_sets
        layer.route(T, logits=lg[r])
        layer.permute(T)
        if tm is not None:
            tm.mark()
        layer.ffn(T, xs[r], pool, shared_blob=shared, mode=mode | _lib.FT_FFN_GATE_UP_ONLY)
        if tm is not None:
            tm.mark()
        layer.ffn(T, xs[r], pool, shared_blob=shared, mode=mode | _lib.FT_FFN_DOWN_ONLY)
        if tm is not None:
            tm.mark()
        layer.combine(T)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    tm = Timer(3 * args.steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with no_gc():
        start.record()
        for i in range(args.steps):
            step(i, tm)
        end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    gu = float(np.mean([tm.ev[3 * i].elapsed_time(tm.ev[3 * i + 1]) for i in range(args.steps)]))
    dn = float(np.mean([tm.ev[3 * i + 1].elapsed_time(tm.ev[3 * i + 2]) for i in range(args.steps)]))
    ffn_ms = [tm.ev[3 * i].elapsed_time(tm.ev[3 * i + 2]) for i in range(args.steps)]
    log(f"prefill mode {mode} T={T}: {ms:.3f} ms/step ({T / (ms * 1e-3):,.0f} tok/s); gate/up {gu:.3f} ms = "
        f"{flops_gu / (gu * 1e-3) / 1e12:.0f} TFLOP/s, down {dn:.3f} ms = "
        f"{flops_all / 3 / (dn * 1e-3) / 1e12:.0f} TFLOP/s; FFN {flops_all / ((gu + dn) * 1e-3) / 1e12:.0f} TFLOP/s")
    return dict(ms_per_step=ms, tokens_per_s=T / (ms * 1e-3), gate_up_ms=gu, down_ms=dn,
                flops_gate_up=flops_gu, flops_ffn=flops_all,
                ffn_ms_p10_p50_p90=[float(v) for v in np.percentile(ffn_ms, [10, 50, 90])])


def pinned_h2d_bandwidth(expert_bytes, n=32, n_streams=1):
    """B_p: pinned host -> device copies of one expert blob each, spread over n_streams queues."""
    import torch
    src = torch.empty((n, expert_bytes), dtype=torch.uint8, pin_memory=True)
    dst = torch.empty((n, expert_bytes), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(n_streams)]
    main = torch.cuda.current_stream()

    def go():
        for s in streams:
            s.wait_stream(main)
        for i in range(n):
            with torch.cuda.stream(streams[i % n_streams]):
                dst[i].copy_(src[i], non_blocking=True)
        for s in streams:
            main.wait_stream(s)

    go()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    go()
    b.record()
    torch.cuda.synchronize()
    return n * expert_bytes / (a.elapsed_time(b) * 1e-3) / 1e9


def run_cache_trace(args, cfg, light=False):
    """8-layer decode trace at batch 1 through the device LRU cache with pinned-host miss fills.

    light: only the timed hits-first run (no serialised, resize or hybrid passes)."""
    import concurrent.futures as cf
    import torch
    import synth
    from expert_cached_ffn_amd import layer as L
    from expert_cached_ffn_amd import ops

    torch.cuda.set_device(0)
    Lyr, E, C, S = cfg.n_layers, cfg.E, cfg.capacity, cfg.steps
    shape = L.LayerShape(cfg.H, cfg.I, cfg.E, cfg.k, cfg.wdtype, cfg.xdtype, cfg.gating, cfg.renormalize, True)
    layer = L.MoELayer(shape, 1)
    eb = int(layer.layout.expert_bytes)
    t0 = time.time()
    bank = torch.empty((Lyr * E, eb), dtype=torch.uint8, pin_memory=True)
    hb = bank.numpy()

    def fill(key):
        l, e = divmod(key, E)
        L.pack_expert(layer.layout, synth.expert_weights(cfg, l, e).arrays, hb[key])
    with cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(Lyr * E)))
    shared = torch.stack([L.as_device_u8([L.pack_expert(layer.layout, synth.expert_weights(cfg, l, E).arrays)])[0]
                          for l in range(Lyr)])
    tr = synth.cache_trace(cfg)
    logits = L.to_device(tr.logits.reshape(S * Lyr, E))
    xs = torch.stack([L.to_device(synth.tokens(cfg, 1, layer=l, step=st)) for st in range(S) for l in range(Lyr)])
    pool = torch.empty((C, eb), dtype=torch.uint8, device="cuda")
    slot_of = torch.empty(E, dtype=torch.int32, device="cuda")
    copy_stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    log(f"cache trace: host bank {bank.numel() / 1e9:.1f} GB pinned and filled in {time.time() - t0:.1f}s")
    b_p1 = pinned_h2d_bandwidth(eb)
    # B_p as the cache's own fill path achieves it: layer-steps whose k experts all miss, nothing else
    probe = ops.ExpertCache(layer.layout, Lyr, E, 64, pool, bank, copy_stream)
    n_probe = 64
    pids = torch.tensor([[(i * cfg.k + j) % E for j in range(cfg.k)] for i in range(n_probe)], dtype=torch.int32,
                        device="cuda")
    torch.cuda.synchronize()
    tp = time.perf_counter()
    for i in range(n_probe):
        probe.step((i * 7) % Lyr, pids[i], 1, cfg.k, slot_of)
    torch.cuda.synchronize()
    b_p = probe.stats()["bytes_h2d"] / (time.perf_counter() - tp) / 1e9
    assert probe.stats()["misses"] == n_probe * cfg.k
    probe.destroy()
    log(f"pinned H2D bandwidth B_p = {b_p:.1f} GB/s through the cache's fills "
        f"({b_p1:.1f} GB/s for back-to-back torch copies on one stream)")

    n_threads = min(16, len(os.sched_getaffinity(0)))

    slot_hits = torch.empty(E, dtype=torch.int32, device="cuda")

    def run(steps, cache, hybrid=False, hits_first=False):
        """hits_first: the hits' FFN (and the shared expert's) is enqueued right after the LRU update,
        before the host waits for it (ft_expert_cache_plan, then ft_expert_cache_fill) and before the
        step's fills land; the filled misses' FFN after them.  Otherwise one FFN waits for every fill."""
        for st in range(steps):
            for l in range(Lyr):
                i = st * Lyr + l
                layer.route_permute(1, logits=logits[i:i + 1])
                if hits_first:
                    cache.plan(l, layer.ids, 1, cfg.k, slot_hits, slot_of)
                    layer.ffn(1, xs[i], pool, slot_of_expert=slot_hits, shared_blob=shared[l])
                    n_fill = cache.fill()
                else:
                    cache.step(l, layer.ids, 1, cfg.k, slot_of)
                if hybrid:
                    layer.stage_cpu_misses(cache, 1, xs[i])
                if hits_first:
                    cache.wait_fills()
                    if n_fill or (hybrid and cache.cpu_misses()):
                        layer.ffn(1, xs[i], pool, slot_of_expert=slot_of)
                else:
                    layer.ffn(1, xs[i], pool, slot_of_expert=slot_of, shared_blob=shared[l])
                if hybrid:
                    layer.run_cpu_misses(cache, n_threads=n_threads)
                layer.combine(1)

    warm = ops.ExpertCache(layer.layout, Lyr, E, C, pool, bank, copy_stream)
    run(min(args.warmup, S), warm, hits_first=True)
    torch.cuda.synchronize()
    warm.destroy()
    cache = ops.ExpertCache(layer.layout, Lyr, E, C, pool, bank, copy_stream)  # cold start
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    run(S, cache, hits_first=True)  # the pages' decode order: a hit runs at once, a miss after its fill
    torch.cuda.synchronize()
    dt = time.perf_counter() - t1
    st = cache.stats()
    cache.destroy()
    hit = st["hits"] / max(1, st["accesses"])
    # lower bound of a step: resident expert reads at 8 TB/s vs fills at the measured B_p
    resident = Lyr * (cfg.k + 1) * eb
    bound = max(resident / (HBM_PEAK_GBS * 1e9), st["bytes_h2d"] / S / (b_p * 1e9))
    res = dict(tokens_per_s=S / dt, ms_per_step=dt / S * 1e3, hit_rate=hit, misses_per_step=st["misses"] / S,
               bytes_h2d=st["bytes_h2d"], h2d_GBps=st["bytes_h2d"] / dt / 1e9, b_p_GBps=b_p,
               bound_ms_per_step=bound * 1e3, frac_of_bound=bound / (dt / S), stats=st, b_p_torch_copy_GBps=b_p1)
    log(f"cache trace: {S} steps x {Lyr} layers in {dt:.2f}s = {S / dt:.1f} tok/s, hit rate {hit:.4f}, "
        f"{res['misses_per_step']:.2f} misses/step, fills {res['h2d_GBps']:.1f} GB/s (B_p {b_p:.1f}), "
        f"bound {bound * 1e3:.3f} ms/step -> {100 * res['frac_of_bound']:.0f} % of it")
    if light:
        return res
    # the same cold-start trace with one FFN that waits for every fill of its layer-step
    cache = ops.ExpertCache(layer.layout, Lyr, E, C, pool, bank, copy_stream)
    torch.cuda.synchronize()
    t5 = time.perf_counter()
    run(S, cache)
    torch.cuda.synchronize()
    dt_ser = time.perf_counter() - t5
    st_ser = cache.stats()
    assert (st_ser["hits"], st_ser["misses"]) == (st["hits"], st["misses"])  # the same LRU decisions
    log(f"hits-first step {S / dt:.1f} tok/s vs {S / dt_ser:.1f} tok/s with the FFN waiting for every fill "
        f"({dt_ser / dt:.2f}x)")
    # elastic resize at a safe point: halve the slots in place (the most recent
    # entries stay), run the first 64 steps again, grow back in the same pool
    t2 = time.perf_counter()
    cache.resize(C // 2, pool)
    shrink_ms = (time.perf_counter() - t2) * 1e3
    before = cache.stats()
    run(min(64, S), cache)
    torch.cuda.synchronize()
    after = cache.stats()
    t3 = time.perf_counter()
    cache.resize(C, pool)
    grow_ms = (time.perf_counter() - t3) * 1e3
    half_hit = (after["hits"] - before["hits"]) / max(1, after["accesses"] - before["accesses"])
    log(f"elastic resize: {C} -> {C // 2} slots in place {shrink_ms:.1f} ms, back to {C} {grow_ms:.1f} ms; "
        f"hit rate over 64 steps at {C // 2} slots {half_hit:.4f}")
    cache.destroy()
    # hybrid miss execution: B_h of the host expert kernel (one token, distinct experts,
    # so the weights stream from DRAM), then the same cold-start trace with the split on
    x1 = xs[0][:1].cpu().numpy().view(np.uint16)
    y1 = np.empty((1, cfg.H), np.float32)
    ops.ft_cpu_expert_ffn(layer.layout, hb[0], x1, 1, y1, n_threads)
    th = time.perf_counter()
    n_h = 24
    for j in range(n_h):
        ops.ft_cpu_expert_ffn(layer.layout, hb[(j * 37 + 5) % (Lyr * E)], x1, 1, y1, n_threads)
    b_h = n_h * eb / (time.perf_counter() - th) / 1e9
    cache = ops.ExpertCache(layer.layout, Lyr, E, C, pool, bank, copy_stream)
    cache.set_split(b_p, b_h, 1, cfg.k)
    run(min(args.warmup, S), cache, hybrid=True, hits_first=True)  # warm the host path
    torch.cuda.synchronize()
    cache.destroy()
    def hybrid_run(bh):
        cache = ops.ExpertCache(layer.layout, Lyr, E, C, pool, bank, copy_stream)
        cache.set_split(b_p, bh, 1, cfg.k)
        torch.cuda.synchronize()
        t4 = time.perf_counter()
        run(S, cache, hybrid=True, hits_first=True)
        torch.cuda.synchronize()
        dth = time.perf_counter() - t4
        sth = cache.stats()
        cache.destroy()
        in_loop = sth["cpu_misses"] * eb / max(1, sth["cpu_ns"])  # bytes/ns = GB/s
        out = dict(tokens_per_s=S / dth, ms_per_step=dth / S * 1e3, b_h_split_GBps=bh,
                   b_h_in_loop_GBps=in_loop, hit_rate=sth["hits"] / max(1, sth["accesses"]),
                   cpu_misses_per_step=sth["cpu_misses"] / S,
                   filled_per_step=(sth["misses"] - sth["cpu_misses"]) / S, bytes_h2d=sth["bytes_h2d"],
                   speedup=(S / dth) / (S / dt))
        log(f"hybrid miss execution, split at B_p {b_p:.1f} / B_h {bh:.1f} GB/s: {S / dth:.1f} tok/s "
            f"({out['speedup']:.2f}x the fill-only run), hit rate {out['hit_rate']:.4f}, "
            f"{out['cpu_misses_per_step']:.2f} misses/step on the CPU, {out['filled_per_step']:.2f} filled; "
            f"CPU path in the loop {in_loop:.1f} GB/s")
        return out
    # the split from the stand-alone B_h, then again from the rate the whole CPU path (staging
    # wait, expert kernel, copy back) reached in that run
    first = hybrid_run(b_h)
    second = hybrid_run(first["b_h_in_loop_GBps"])
    hybrid = dict(b_h_standalone_GBps=b_h, cpu_threads=n_threads, cpu_isa=ops.ft_cpu_isa(-1),
                  split_standalone=first, split_in_loop=second)
    res.update(serialised_step={"tokens_per_s": S / dt_ser, "ms_per_step": dt_ser / S * 1e3,
                                "hits_first_speedup": dt_ser / dt},
               hybrid=hybrid, resize={"shrink_ms": shrink_ms, "grow_ms": grow_ms, "from_slots": C, "to_slots": C // 2,
                                      "hit_rate_64_steps_at_half": half_hit})
    return res


def run_prefill_stream(args, cfg):
    """Prefill of 8 layers whose experts live in pinned host memory, through the expert cache
    (room for two layers): serial (each layer's misses filled, then compute) vs full-layer double
    buffering (layer l+1 prefetched while layer l computes), beside the compute alone."""
    import concurrent.futures as cf
    import torch
    import synth
    from expert_cached_ffn_amd import layer as L
    from expert_cached_ffn_amd import ops

    torch.cuda.set_device(0)
    Lyr, E, T = cfg.n_layers, cfg.E, cfg.batches[0]
    shape = L.LayerShape(cfg.H, cfg.I, cfg.E, cfg.k, cfg.wdtype, cfg.xdtype, cfg.gating, cfg.renormalize, True)
    layer = L.MoELayer(shape, T)
    eb = int(layer.layout.expert_bytes)
    t0 = time.time()
    bank = torch.empty((Lyr * E, eb), dtype=torch.uint8, pin_memory=True)
    hb = bank.numpy()

    def fill(key):
        l, e = divmod(key, E)
        L.pack_expert(layer.layout, synth.expert_weights(cfg, l, e).arrays, hb[key])
    with cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(Lyr * E)))
    shared = torch.stack([L.as_device_u8([L.pack_expert(layer.layout, synth.expert_weights(cfg, l, E).arrays)])[0]
                          for l in range(Lyr)])
    xs = [L.to_device(synth.tokens(cfg, T, layer=l)) for l in range(Lyr)]
    lgs = [L.to_device(synth.prefill_logits(cfg, T, layer=l)) for l in range(Lyr)]
    C = 2 * E
    pool = torch.empty((C, eb), dtype=torch.uint8, device="cuda")
    slot_of = torch.empty(E, dtype=torch.int32, device="cuda")
    copy_stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    log(f"prefill stream: host bank {bank.numel() / 1e9:.1f} GB pinned and filled in {time.time() - t0:.1f}s")

    def compute(l, table):
        layer.ffn(T, xs[l], pool, slot_of_expert=table, shared_blob=shared[l])
        layer.combine(T)

    def timed(fn):
        torch.cuda.synchronize()
        t = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t

    def serial():
        cache = ops.ExpertCache(layer.layout, Lyr, E, C, pool, bank, copy_stream)
        for l in range(Lyr):
            layer.route_permute(T, logits=lgs[l])
            cache.step(l, layer.ids, T, cfg.k, slot_of)
            compute(l, slot_of)
        torch.cuda.synchronize()
        st = cache.stats()
        cache.destroy()
        return st

    def double_buffered():
        cache = ops.ExpertCache(layer.layout, Lyr, E, C, pool, bank, copy_stream)
        cache.prefetch_layer(0)
        for l in range(Lyr):
            layer.route_permute(T, logits=lgs[l])
            cache.step(l, layer.ids, T, cfg.k, slot_of)
            if l + 1 < Lyr:
                cache.prefetch_layer(l + 1)
            compute(l, slot_of)
        torch.cuda.synchronize()
        st = cache.stats()
        cache.destroy()
        return st

    ident = torch.arange(E, dtype=torch.int32, device="cuda")

    def compute_only():  # the same 8 layer computations on resident bytes (the FFN cost does not depend on them)
        for l in range(Lyr):
            layer.route_permute(T, logits=lgs[l])
            compute(l, ident)

    def transfer_only():  # the double-buffered schedule without the FFN
        cache = ops.ExpertCache(layer.layout, Lyr, E, C, pool, bank, copy_stream)
        cache.prefetch_layer(0)
        for l in range(Lyr):
            layer.route_permute(T, logits=lgs[l])
            cache.step(l, layer.ids, T, cfg.k, slot_of)
            if l + 1 < Lyr:
                cache.prefetch_layer(l + 1)
        torch.cuda.synchronize()
        cache.destroy()

    compute_only()
    transfer_only()  # the first DMA pass over the pinned bank is slower; keep it out of the timings
    st_s, st_d = {}, {}
    t_comp = min(timed(compute_only) for _ in range(2))
    t_xfer = min(timed(transfer_only) for _ in range(2))
    t_ser = min(timed(lambda: st_s.update(serial())) for _ in range(2))
    t_db = min(timed(lambda: st_d.update(double_buffered())) for _ in range(2))
    hidden = min(1.0, max(0.0, (t_xfer + t_comp - t_db) / t_comp))  # share of the compute under the transfers
    bound = max(t_xfer, t_comp)
    moved = st_d["bytes_h2d"]
    log(f"prefill stream ({Lyr} layers x {T} tokens, experts in host memory, cache of {C} slots): "
        f"double-buffered {t_db * 1e3:.1f} ms, serial {t_ser * 1e3:.1f} ms, transfers alone {t_xfer * 1e3:.1f} ms, "
        f"compute alone {t_comp * 1e3:.1f} ms; {moved / 1e9:.1f} GB at {moved / t_db / 1e9:.1f} GB/s; "
        f"{100 * hidden:.0f} % of the compute hidden, {100 * bound / t_db:.0f} % of the max(transfer, compute) bound; "
        f"misses after prefetch {st_d['misses']}")
    return dict(tokens_per_s=T / t_db, ms_per_layer=t_db / Lyr * 1e3, serial_ms=t_ser * 1e3, double_buffered_ms=t_db * 1e3,
                transfer_ms=t_xfer * 1e3, compute_ms=t_comp * 1e3, compute_hidden_fraction=hidden,
                frac_of_bound=bound / t_db, bytes_h2d=moved, h2d_GBps=moved / t_db / 1e9,
                misses_after_prefetch=st_d["misses"], prefetch_fills=st_d["prefetch_fills"],
                serial_misses=st_s["misses"])


# ----------------------------------------------------------------------------- CPU baseline

def host_cores():
    """Host core counts the oracle timings run on: os.cpu_count(), the affinity set, BLAS threads."""
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        blas = 1
    return dict(os_cpu_count=os.cpu_count(), affinity_cpus=len(os.sched_getaffinity(0)), blas_threads=int(blas))


def time_oracle(fn, repeats):
    """Median wall time of ``repeats`` calls of fn(), all BLAS threads and (if single_too) one thread."""
    ts = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), ts


def oracle_baseline(name, fn, tokens, repeats, sample, single_thread=True):
    """The oracle timed on this host: median of ``repeats`` runs on every BLAS thread, and (decode)
    the same on one thread; tokens/s = tokens / median time."""
    cores = host_cores()
    med, ts = time_oracle(fn, repeats)
    out = dict(value=tokens / med, unit="tokens/s", cores=cores["blas_threads"], kind="oracle",
               sample=f"{sample}; median of {repeats} ({', '.join(f'{t:.2f}' for t in ts)} s)",
               median_s=med, repeats=repeats, **cores)
    if single_thread:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(1):
                med1, ts1 = time_oracle(fn, repeats)
            out["single_thread_value"] = tokens / med1
            out["single_thread_median_s"] = med1
        except Exception as err:  # threadpoolctl missing: no 1-thread figure
            log(f"{name}: no single-thread oracle run ({err})")
    log(f"oracle {name}: {out['value']:,.1f} tok/s on {cores['blas_threads']} BLAS threads "
        f"(os.cpu_count {cores['os_cpu_count']}, affinity {cores['affinity_cpus']})"
        + (f", {out['single_thread_value']:,.1f} tok/s on one" if "single_thread_value" in out else ""))
    return out


def cpu_baseline_decode(cfg, T, repeats=5):
    """The oracle on one layer call of a decode workload (input set 0): route, permute, every expert
    FFN the routing touches with its weight decode, combine."""
    import synth
    from oracle import formats, moe
    x = synth.tokens(cfg, T, case=0)
    wr = synth.router_weight(cfg)
    raw = {}
    x64 = formats.activations_to_f64(cfg.xdtype, x)
    wr64 = formats.activations_to_f64(cfg.xdtype, wr)
    ids = moe.topk(moe.router_logits(x64, wr64), cfg.k)
    for e in sorted(set(ids.ravel().tolist())) + ([cfg.E] if cfg.shared else []):
        raw[e] = synth.expert_weights(cfg, 0, e).arrays        # input generation: not timed

    def run():
        r = moe.moe_layer(x64, k=cfg.k, E=cfg.E, gating=cfg.gating, renormalize=cfg.renormalize,
                          experts=lambda e: formats.expert_to_f64(cfg.wdtype, raw[e]),
                          shared=formats.expert_to_f64(cfg.wdtype, raw[cfg.E]) if cfg.shared else None,
                          w_router=wr64)
        assert np.all(np.isfinite(r["out"]))
    return oracle_baseline(f"cfg{cfg.cfg_id} T={T}", run, T, repeats,
                           f"one {T}-token layer call (input set 0): route, permute, {len(raw)} expert FFNs "
                           f"with weight decode, combine")


def cpu_baseline_prefill(cfg, T_sample=32):
    """The oracle on the first T_sample tokens of the prefill batch (given logits): permute, every
    expert those tokens touch with its weight decode, the shared expert, combine.  One run."""
    import synth
    from oracle import formats, moe
    T = cfg.batches[0]
    x = synth.tokens(cfg, T, case=0)[:T_sample]
    logits = synth.prefill_logits(cfg, T, case=0)[:T_sample]
    ids = moe.topk(logits, cfg.k)
    raw = {e: synth.expert_weights(cfg, 0, e).arrays for e in sorted(set(ids.ravel().tolist())) + [cfg.E]}
    x64 = formats.activations_to_f64(cfg.xdtype, x)

    def run():
        r = moe.moe_layer(x64, k=cfg.k, E=cfg.E, gating=cfg.gating, renormalize=cfg.renormalize,
                          experts=lambda e: formats.expert_to_f64(cfg.wdtype, raw[e]),
                          shared=formats.expert_to_f64(cfg.wdtype, raw[cfg.E]), logits=logits)
        assert np.all(np.isfinite(r["out"]))
    return oracle_baseline("prefill", run, T_sample, 1,
                           f"the first {T_sample} of the {T} prefill tokens (given logits): permute, "
                           f"{len(raw)} expert FFNs with weight decode, combine", single_thread=False)


def cpu_baseline_cache(cfg, steps_sample=1):
    """The cache-trace oracle: the LRU simulator over every access of the trace, plus the layer
    computation of the first ``steps_sample`` steps (all layers), scaled to the whole trace."""
    import synth
    from oracle import formats, moe
    from oracle.lru import ExpertLRU
    tr = synth.cache_trace(cfg)
    t0 = time.perf_counter()
    sim = ExpertLRU(cfg.n_layers, cfg.E, cfg.capacity)
    for st in range(cfg.steps):
        for l in range(cfg.n_layers):
            sim.step(l, tr.ids[st, l])
    t_sim = time.perf_counter() - t0
    work = []
    for st in range(steps_sample):
        for l in range(cfg.n_layers):
            raw = {e: synth.expert_weights(cfg, l, e).arrays for e in tr.ids[st, l].tolist() + [cfg.E]}
            work.append((synth.tokens(cfg, 1, layer=l, step=st), tr.logits[st, l][None, :], raw))
    t1 = time.perf_counter()
    for x, lg, raw in work:
        r = moe.moe_layer(formats.activations_to_f64(cfg.xdtype, x), k=cfg.k, E=cfg.E, gating=cfg.gating,
                          renormalize=cfg.renormalize, experts=lambda e: formats.expert_to_f64(cfg.wdtype, raw[e]),
                          shared=formats.expert_to_f64(cfg.wdtype, raw[cfg.E]), logits=lg)
        assert np.all(np.isfinite(r["out"]))
    t_step = (time.perf_counter() - t1) / steps_sample
    total = t_sim + cfg.steps * t_step
    cores = host_cores()
    out = dict(value=cfg.steps / total, unit="tokens/s", cores=cores["blas_threads"], kind="oracle",
               sample=f"LRU simulator over all {cfg.steps * cfg.n_layers * cfg.k} accesses ({t_sim:.2f} s) + the "
                      f"{cfg.n_layers}-layer computation of {steps_sample} step(s) with weight decode "
                      f"({t_step:.2f} s per step), scaled to {cfg.steps} steps",
               hit_rate=sim.hits / max(1, sim.accesses), **cores)
    log(f"oracle cache trace: {out['value']:.3f} tok/s (simulator {t_sim:.2f} s, {t_step:.2f} s per step)")
    return out


# ----------------------------------------------------------------------------- main

WORKLOADS = {
    "cache-trace": (5, "dsv4-flash-shaped expert-cache decode trace (8 layers x 256 MXFP4 experts + shared, "
                       "512 cache slots = 25 %, 512 steps of batch 1, Zipf(1.1) + 60 % reuse routing)"),
    "prefill-mxfp4": (4, "dsv4-flash-shaped MXFP4 prefill MoE layer (8192 tokens, H=4096, I=2048, 256 experts "
                         "top-6 sigmoid with Zipf(1.1) popularity + 1 shared, SwiGLU)"),
    "prefill-stream": (4, "dsv4-flash-shaped MXFP4 prefill, 8 layers x 8192 tokens with every routed expert in "
                          "pinned host memory, expert cache of two layers, full-layer double buffering"),
    "prefill-mxfp4-native": (4, "dsv4-flash-shaped MXFP4 prefill MoE layer (8192 tokens, H=4096, I=2048, 256 "
                                "experts top-6 sigmoid with Zipf(1.1) popularity + 1 shared, SwiGLU), native "
                                "MXFP8 x MXFP4 scaled-MFMA mode"),
    "decode-bf16": (2, "qwen3-a3b-shaped bf16 decode MoE layer (H=2048, I=768, 128 experts, top-8 softmax "
                       "renormalised, SwiGLU)"),
    "decode-mxfp4": (3, "dsv4-flash-shaped MXFP4 decode MoE layer (H=4096, I=2048, 256 experts top-6 sigmoid "
                        "+ 1 shared, SwiGLU)"),
    "decode-nvfp4": (6, "qwen3-a3b-shaped NVFP4 decode MoE layer (H=2048, I=768, 128 experts, top-8 softmax "
                        "renormalised, SwiGLU)"),
    "prefill-nvfp4": (7, "qwen3-a3b-shaped NVFP4 prefill MoE layer (8192 tokens, H=2048, I=768, 128 experts "
                         "top-8 softmax renormalised with Zipf(1.1) popularity, SwiGLU)"),
}


def decode_summary(cfg, res, main_T, peaks, traffic=None):
    """The decode part of a JSON line: throughput of the main batch, the roofline of its gate/up
    kernel (HIP events), the layer-level activated-byte rate and every batch."""
    m = res[main_T]
    ach = m["gate_up_bytes"] / (m["gate_up_ms"] * 1e-3) / 1e9
    kname = "ffn_persist_kernel<bf16, gate_up>" if cfg.wdtype == "bf16" else \
        f"ffn_persist_xs_kernel<{cfg.wdtype}, gate_up>"
    layer_gbps = m["layer_weight_bytes"] / (m["ms_per_step"] * 1e-3) / 1e9
    return {
        "tokens_per_s": m["tokens_per_s"], "ms_per_step": m["ms_per_step"], "batch_tokens": main_T,
        "distinct_experts_per_step": m["distinct_experts"],
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": traffic, "avg_launch_us": m["gate_up_ms"] * 1e3,
                     "algorithmic_bytes_per_launch": m["gate_up_bytes"],
                     "frac_of_achievable_copy": ach / peaks["copy_GBps"] if peaks else None,
                     "frac_of_achievable_read": ach / peaks["read_GBps"] if peaks else None},
        "layer_weight_GBps": layer_gbps, "layer_frac_of_hbm_peak": layer_gbps / HBM_PEAK_GBS,
        "step_ms_p10_p50_p90": m["step_ms_p10_p50_p90"], "graph_ms_per_step": m["graph_ms_per_step"],
        "batches": {str(T): {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                             "graph_ms_per_step": r["graph_ms_per_step"],
                             "graph_of_8_steps_ms_per_step": r["graph_of_8_steps_ms_per_step"],
                             "graph_of_48_steps_ms_per_step": r["graph_of_48_steps_ms_per_step"],
                             "four_calls_ms_per_step": r["four_calls_ms_per_step"],
                             "four_calls_graph_ms_per_step": r["four_calls_graph_ms_per_step"],
                             "step_ms_p10_p50_p90": r["step_ms_p10_p50_p90"],
                             "gate_up_GBps": r["gate_up_bytes"] / (r["gate_up_ms"] * 1e-3) / 1e9,
                             "layer_weight_GBps": r["layer_weight_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9,
                             "layer_frac_of_hbm_peak": r["layer_weight_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
                             / HBM_PEAK_GBS}
                    for T, r in sorted(res.items())},
    }


def prefill_summary(cfg, p, native, peaks):
    ach = p["flops_gate_up"] / (p["gate_up_ms"] * 1e-3) / 1e12
    peak = FP8_PEAK_TFLOPS if native else BF16_PEAK_TFLOPS
    layer_tf = p["flops_ffn"] / (p["ms_per_step"] * 1e-3) / 1e12
    return {
        "tokens_per_s": p["tokens_per_s"], "ms_per_step": p["ms_per_step"], "batch_tokens": cfg.batches[0],
        "roofline": {"bound": "mfma",
                     "kernel": "ffn_mx_gemm_kernel<gate_up>" if native else f"ffn_gemm_kernel<{cfg.wdtype}, gate_up>",
                     "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak, "traffic": None,
                     "avg_launch_us": p["gate_up_ms"] * 1e3, "algorithmic_flops_per_launch": p["flops_gate_up"],
                     "frac_of_achievable_bf16_gemm": (ach / peaks["bf16_gemm_TFLOPs"] if peaks and not native else None),
                     "frac_of_achievable_fp8_gemm": (ach / peaks["fp8_gemm_TFLOPs"]
                                                     if peaks and native and peaks["fp8_gemm_TFLOPs"] else None)},
        "layer_TFLOPs": layer_tf, "layer_frac_of_peak": layer_tf / peak,
        "ffn_TFLOPs": p["flops_ffn"] / ((p["gate_up_ms"] + p["down_ms"]) * 1e-3) / 1e12,
        "gate_up_ms": p["gate_up_ms"], "down_ms": p["down_ms"], "ffn_ms_p10_p50_p90": p["ffn_ms_p10_p50_p90"],
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOADS),
                    help="all (default): the bf16 decode line with the MXFP4 decode, prefill and cache-trace "
                         "workloads beside it")
    ap.add_argument("--batch", type=int, default=None, help="main decode batch (default: largest of the workload)")
    ap.add_argument("--only-main-batch", action="store_true",
                    help="time only the main batch (profiling runs: one kernel shape per kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak probes (device copy, bf16 GEMM); implied by --only-main-batch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import synth
    everything = args.workload == "all"
    workload = "decode-bf16" if everything else args.workload
    cfg_id, desc = WORKLOADS[workload]
    cfg = synth.CONFIGS[cfg_id]
    batches = list(cfg.batches)
    main_T = args.batch or max(batches)
    if main_T not in batches:
        batches.append(main_T)
    if args.only_main_batch:
        batches = [main_T]
    base = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "data": "synthetic"}
    if workload == "cache-trace":
        c = run_cache_trace(args, cfg)
        out = dict(base, value=c["tokens_per_s"], steps=cfg.steps, warmup=min(args.warmup, cfg.steps),
                   ms_per_step=c["ms_per_step"], dtype="mxfp4-w/bf16",
                   config={"workload": desc, "batch_tokens": 1},
                   cache={k: v for k, v in c.items() if k not in ("tokens_per_s", "ms_per_step")})
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_cache(cfg)
        print(json.dumps(out), flush=True)
        return
    if workload == "prefill-stream":
        scfg = synth.shrink(cfg, n_layers=8, capacity=2 * cfg.E)
        p = run_prefill_stream(args, scfg)
        out = dict(base, value=p["tokens_per_s"], steps=1, warmup=1, ms_per_step=p["double_buffered_ms"],
                   dtype="mxfp4-w/bf16", config={"workload": desc, "batch_tokens": scfg.batches[0],
                                                 "layers": scfg.n_layers}, stream=p)
        print(json.dumps(out), flush=True)
        return
    if workload.startswith("prefill"):
        native = workload.endswith("native")
        p = run_prefill(args, cfg, cfg.batches[0], mode=1 if native else 0)
        peaks = None if args.no_peaks else achievable_peaks()
        ps = prefill_summary(cfg, p, native, peaks)
        out = dict(base, value=p["tokens_per_s"], steps=args.steps, warmup=args.warmup, ms_per_step=p["ms_per_step"],
                   dtype="mxfp8-a/mxfp4-w" if native else f"{cfg.wdtype}-w/bf16",
                   config={"workload": desc, "batch_tokens": cfg.batches[0]}, roofline=ps["roofline"],
                   layer_TFLOPs=ps["layer_TFLOPs"], ffn_TFLOPs=ps["ffn_TFLOPs"],
                   ffn_ms_p10_p50_p90=ps["ffn_ms_p10_p50_p90"], achievable=peaks)
        if not args.no_cpu_baseline and not native:
            out["cpu_baseline"] = cpu_baseline_prefill(cfg)
        print(json.dumps(out), flush=True)
        return
    t_start = time.time()
    res = run_decode(args, cfg, batches, main_T)
    peaks = None if (args.no_peaks or args.only_main_batch) else achievable_peaks()
    traffic = None
    if workload == "decode-bf16" and main_T == 64:
        traffic = measured_traffic("decode-bf16-T64_hbm_traffic.json", "void ft::ffn_persist_kernel<0, true,")
    d = decode_summary(cfg, res, main_T, peaks, traffic)
    out = dict(base, value=d["tokens_per_s"], steps=args.steps, warmup=args.warmup, ms_per_step=d["ms_per_step"],
               dtype="bf16" if cfg.wdtype == "bf16" else f"{cfg.wdtype}-w/bf16",
               config={"workload": desc, "batch_tokens": main_T, "input_sets": N_INPUT_SETS,
                       "distinct_experts_per_step": d["distinct_experts_per_step"]},
               roofline=d["roofline"], achievable=peaks, step_ms_p10_p50_p90=d["step_ms_p10_p50_p90"],
               layer_weight_GBps=d["layer_weight_GBps"], layer_frac_of_hbm_peak=d["layer_frac_of_hbm_peak"],
               graph_ms_per_step=d["graph_ms_per_step"], batches=d["batches"])
    if everything:
        # the other workloads of the metric, each with its own roofline and oracle baseline
        c3 = synth.CONFIGS[3]
        r3 = run_decode(args, c3, list(c3.batches), max(c3.batches))
        out["decode_mxfp4"] = dict(workload=WORKLOADS["decode-mxfp4"][1],
                                   **decode_summary(c3, r3, max(c3.batches), peaks))
        c4 = synth.CONFIGS[4]
        pargs = argparse.Namespace(**vars(args))
        pargs.steps, pargs.warmup = min(args.steps, 20), min(args.warmup, 3)
        out["prefill"] = dict(workload=WORKLOADS["prefill-mxfp4"][1],
                              **prefill_summary(c4, run_prefill(pargs, c4, c4.batches[0], mode=0), False, peaks))
        c5 = synth.CONFIGS[5]
        cr = run_cache_trace(args, c5, light=True)
        out["cache_trace"] = dict(workload=WORKLOADS["cache-trace"][1], **cr)
        log(f"GPU part of the run: {time.time() - t_start:.0f} s")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(cfg, main_T)
        if everything:
            out["decode_mxfp4"]["cpu_baseline"] = cpu_baseline_decode(synth.CONFIGS[3], 1)
            out["prefill"]["cpu_baseline"] = cpu_baseline_prefill(synth.CONFIGS[4])
            out["cache_trace"]["cpu_baseline"] = cpu_baseline_cache(synth.CONFIGS[5])
    log(f"whole run: {time.time() - t_start:.0f} s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
