#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

Headline step: one fmoe_forward call (router top-k -> grouping -> gate/up GEMM with
SiLU-and-mul -> down GEMM -> weighted combine) on the bf16 layer H=2048, I=768, E=128,
top-8 (the 30B-total / 3B-active expert shape) at T=256 tokens with uniform routing from
N(0,1) logits.  Inputs and weights are resident in HBM before timing starts.  Every step
uses another seeded batch, and the weights rotate over several copies in HBM, so a step
cannot find the expert weights it needs in the 256 MB Infinity Cache left over from the
previous step (each call reads them from HBM, as in a model where other layers run between
two calls of this one).

value = HBM TB/s on the touched expert weights (bytes of the experts the routing used /
wall time per step).  ms_per_step is the wall time per call.  Stage times come from HIP
events the library records on its stream between the stages (fmoe_forward_profiled).

Also reported: a sweep over T = 1..4096 (uniform and concentrated routing), the FP8 w8a8
layer at T = 64/128/256, and the FP8 expert-parallel shard (T=288, top-6 of 400 slots, the
50 local experts of rank 0) uniform and concentrated; the roofline of the dominant kernel;
and the CPU oracle timed on a bounded sample of the headline batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused-MoE µs/call + HBM TB/s on touched weights (T=1..4096), uniform & skewed"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
CACHE_BYTES = 256 << 20  # Infinity Cache (MALL)
PROFILE_DIR = os.path.join(ROOT, "profiles")


class Workload:
    def __init__(self, name, *, config, T, H, I, E, k, fp8=False, routing="uniform", ep_size=1, ep_rank=0,
                 weight_config=None):
        self.name, self.config, self.T, self.H, self.I, self.E, self.k = name, config, T, H, I, E, k
        self.fp8, self.routing, self.ep_size, self.ep_rank = fp8, routing, ep_size, ep_rank
        self.weight_config = config if weight_config is None else weight_config
        self.El = E // ep_size

    @property
    def dtype(self):
        return "fp8" if self.fp8 else "bf16"

    def expert_bytes(self):
        """Weight bytes of one expert (gate + up + down, plus fp32 block scales for FP8)."""
        elems = 3 * self.H * self.I
        if self.fp8:
            return elems + 3 * (self.H // 128) * (self.I // 128) * 4
        return 2 * elems

    def gemm1_bytes_per_expert(self):
        elems = 2 * self.H * self.I
        return elems + 2 * (self.H // 128) * (self.I // 128) * 4 if self.fp8 else 2 * elems

    def describe(self):
        return dict(workload=self.name, tokens=self.T, hidden=self.H, inter=self.I, experts=self.E, top_k=self.k,
                    ep_size=self.ep_size, ep_rank=self.ep_rank, local_experts=self.El, weights=self.dtype,
                    routing=self.routing)


def build_inputs(wl: Workload, n_batches: int, n_copies: int):
    import torch

    import mixture_experts_layer_sigmoid_amd as fm
    from mixture_experts_layer_sigmoid_amd import synth

    dev = torch.device("cuda:0")
    if wl.fp8:
        base = [t.to(dev) for t in synth.expert_weights_fp8(wl.weight_config, wl.El, wl.H, wl.I, wl.ep_rank * wl.El)]
    else:
        base = [t.to(dev) for t in synth.expert_weights_bf16(wl.weight_config, wl.El, wl.H, wl.I, wl.ep_rank * wl.El)]
    copies = [fm.ExpertWeights(*base)] + [fm.ExpertWeights(*[t.clone() for t in base]) for _ in range(n_copies - 1)]
    batches = []
    for b in range(n_batches):
        x = synth.activations(wl.config, wl.T, wl.H, seed=b).to(dev)
        lg = synth.routed_logits(wl.config, wl.T, wl.E, wl.k, wl.routing, seed=b).to(dev)
        batches.append((x, lg))
    shape = fm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.k, wl.ep_size, wl.ep_rank, wl.fp8)
    ws = fm.workspace(shape, dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
    return shape, copies, batches, ws, out


class HipEvent:
    """A HIP timing event created without the system-scope fence (hipEventDisableSystemFence):
    recording it does not write back and invalidate the caches, so an event between two kernels
    costs about a microsecond instead of several and does not slow the kernel after it.  Passed
    to the library by handle (`cuda_event`), like a torch.cuda.Event."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = hip
        h = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), HipEvent.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = h.value

    def record(self):
        """Record on torch's current stream."""
        import ctypes

        import torch
        HipEvent._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        if HipEvent._hip.hipEventRecord(ctypes.c_void_p(self.cuda_event),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end: "HipEvent") -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        import ctypes
        f = ctypes.c_float()
        if HipEvent._hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(self.cuda_event),
                                             ctypes.c_void_p(end.cuda_event)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def __del__(self):
        hip = type(self)._hip  # not the module global, which is gone at interpreter exit
        if self.cuda_event and hip is not None:
            hip.hipEventDestroy(self.cuda_event)


def pct(v, q):
    s = sorted(v)
    i = min(len(s) - 1, max(0, int(math.ceil(q / 100.0 * len(s))) - 1))
    return s[i]


def measure(wl: Workload, steps: int, warmup: int, dominant: str | None = None, every: int = 1):
    """warmup + steps timed calls, back to back; returns the wall time per call, per-call times
    from a start/end event pair (or, with `dominant`, the live duration of that stage from the
    event pair around it, on every `every`-th timed call: each event record makes the stream
    drain before the next kernel, so the other calls run as they do without instrumentation),
    a separate untimed pass with every stage event, and the routing counters of every batch."""
    import torch

    import mixture_experts_layer_sigmoid_amd as fm

    touched_guess = wl.El * (1 - (1 - wl.k / wl.E) ** wl.T) * wl.expert_bytes()
    n_copies = max(2, min(8, int(math.ceil(2 * CACHE_BYTES / max(touched_guess, 1))) + 1))
    n_batches = max(4, n_copies)
    shape, copies, batches, ws, out = build_inputs(wl, n_batches, n_copies)

    # routing counters of each batch (read once, outside the timed region)
    stats = []
    for b in range(n_batches):
        fm.fmoe_forward(shape, batches[b][0], batches[b][1], copies[0], ws=ws, out=out)
        stats.append(fm.fmoe_read_stats(ws))

    NS = fm.FMOE_NUM_STAGES
    if dominant is None:
        pair = (0, NS)
    else:
        s = fm.STAGES.index(dominant)
        pair = (s, s + 1)
    ev = []
    for i in range(steps):
        e = None
        if i % every == 0:
            e = [None] * (NS + 1)
            e[pair[0]] = HipEvent()
            e[pair[1]] = HipEvent()
        ev.append(e)

    def call(j, events=None):
        x, lg = batches[j % n_batches]
        fm.fmoe_forward(shape, x, lg, copies[j % n_copies], ws=ws, out=out, stage_events=events)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(warmup + i, ev[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    pair_us = [ev[i][pair[0]].elapsed_time(ev[i][pair[1]]) * 1e3 for i in range(steps) if ev[i] is not None]

    # warm secondary figure: the same weight copy and batch every call (weights stay in the
    # caches between calls), timed back to back between one event pair
    wa, wb = HipEvent(), HipEvent()
    for i in range(3):
        call(0)
    wa.record()
    for i in range(steps):
        x, lg = batches[0]
        fm.fmoe_forward(shape, x, lg, copies[0], ws=ws, out=out)
    wb.record()
    torch.cuda.synchronize()
    warm_us = wa.elapsed_time(wb) * 1e3 / steps

    # stage breakdown: a separate pass with every event (each record adds about a microsecond)
    full = [[HipEvent() for _ in range(NS + 1)] for _ in range(steps)]
    for i in range(steps):
        call(warmup + steps + i, full[i])
    torch.cuda.synchronize()
    stage_us = {name: sum(full[i][s].elapsed_time(full[i][s + 1]) for i in range(steps)) * 1e3 / steps
                for s, name in enumerate(fm.STAGES)}

    used = [stats[(warmup + i) % n_batches] for i in range(steps)]
    touched = sum(wl.El - u["empty_experts"] for u in used) / steps
    rows = sum(u["local_rows"] for u in used) / steps
    max_rows = max(u["max_rows"] for u in used)
    del copies, batches, ws, out
    torch.cuda.empty_cache()
    return dict(wall_s=wall, pair_us=pair_us, dominant=dominant, stage_us=stage_us, touched=touched, rows=rows,
                warm_us=warm_us,
                max_rows=max_rows, rows_estimate=used[0]["rows_estimate"], tile_rows=used[0]["tile_rows"],
                copies=n_copies)


def summarize(wl: Workload, m: dict) -> dict:
    call_us = m["pair_us"] if m["dominant"] is None else [m["wall_s"] * 1e6]
    p50 = pct(call_us, 50)
    tb = m["touched"] * wl.expert_bytes()
    flops = 6.0 * m["rows"] * wl.H * wl.I
    return dict(**wl.describe(), us_p20=round(pct(call_us, 20), 2), us_p50=round(p50, 2),
                us_p80=round(pct(call_us, 80), 2), us_wall=round(m["wall_s"] * 1e6, 2),
                us_warm=round(m["warm_us"], 2),
                touched_experts=round(m["touched"], 2), touched_MB=round(tb / 1e6, 1),
                hbm_TBps=round(tb / (p50 * 1e-6) / 1e12, 3), tokens_per_s=round(wl.T / (p50 * 1e-6), 1),
                mfma_util=round(flops / (p50 * 1e-6) / (MFMA_PEAK_TFLOPS[wl.dtype] * 1e12), 4),
                rows_estimate=m["rows_estimate"], tile_rows=m["tile_rows"], max_rows=m["max_rows"],
                stages_us={k: round(v, 2) for k, v in m["stage_us"].items()})


DOMINANT_SOURCE = "gemm_stream.hip"  # the gate/up GEMM of the headline workload (light row tiles)


def kernel_hash():
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "mixture_experts_layer_sigmoid_amd", "csrc", DOMINANT_SOURCE), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload_name: str, stage: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        ent = rec.get(workload_name, {}).get(stage)
        if not ent or ent.get("kernel_sha") != kernel_hash():
            return None
        return ent.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None


CALIBRATION_KERNEL = "CUDAFunctorOnSelf_add<float>"  # the 256 MiB copy of --calibrate
HEADLINE_GATE_UP_KERNEL = "k_grouped_gemm_stream<true, false, 0,"  # bf16 gate/up, bf16 output


def traffic_from_counters(fetch_csv: str, write_csv: str, workload_name: str, stage: str = "gemm1") -> dict:
    """HBM bytes per launch of the headline gate/up kernel from two rocprofv3 --pmc runs of
    `bench.py --no-sweep --no-cpu --calibrate` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).
    Each counter is scaled by what it reads for the calibration copy (256 MiB read, 256 MiB
    written), so the result is in bytes whatever the counter's unit; the mean over the
    kernel's dispatches is written to profiles/traffic.json with the kernel source hash."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        vals = per_kernel(path, counter)
        cal = [v for k, vs in vals.items() if CALIBRATION_KERNEL in k for v in vs]
        ker = [(k, v) for k, vs in vals.items() if HEADLINE_GATE_UP_KERNEL in k for v in vs]
        if not cal or not ker:
            raise SystemExit(f"{path}: calibration or gate/up kernel dispatches not found")
        factor = (256 << 20) / (sum(cal) / len(cal) * 1024)
        out[key] = dict(kib=sum(v for _, v in ker) / len(ker), factor=factor, cal_kib=sum(cal) / len(cal),
                        kernel=ker[0][0], launches=len(ker))
    hbm = out["fetch"]["kib"] * 1024 * out["fetch"]["factor"] + out["write"]["kib"] * 1024 * out["write"]["factor"]
    ent = dict(kernel=out["fetch"]["kernel"], fetch_kib_per_launch=round(out["fetch"]["kib"], 1),
               write_kib_per_launch=round(out["write"]["kib"], 1),
               calibration=dict(kernel=CALIBRATION_KERNEL, bytes_read=256 << 20, bytes_written=256 << 20,
                                fetch_kib=round(out["fetch"]["cal_kib"], 1), write_kib=round(out["write"]["cal_kib"], 1),
                                fetch_factor=round(out["fetch"]["factor"], 4),
                                write_factor=round(out["write"]["factor"], 4)),
               hbm_bytes_per_launch=int(hbm), launches=out["fetch"]["launches"], kernel_sha=kernel_hash())
    rec = {workload_name: {stage: ent}}
    with open(os.path.join(PROFILE_DIR, "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return ent


def cpu_baseline(wl: Workload, target_s: float = 12.0, threads: int = 0) -> dict:
    """The CPU oracle (as it stands) on a bounded token sample of batch 0 of the workload, on
    `threads` OpenMP threads (0: all of them)."""
    import numpy as np

    import oracle
    from mixture_experts_layer_sigmoid_amd import synth

    all_threads = oracle.num_threads()  # OpenMP's default: OMP_NUM_THREADS, else every core
    oracle.set_num_threads(threads if threads > 0 else all_threads)

    x = synth.activations(wl.config, wl.T, wl.H, seed=0)
    lg = synth.routed_logits(wl.config, wl.T, wl.E, wl.k, wl.routing, seed=0)
    t0 = time.perf_counter()
    ids, w = oracle.router_topk(synth.bf16_bits(lg), wl.k)
    route_s = time.perf_counter() - t0
    wg, wu, wd = (synth.bf16_bits(t) for t in synth.expert_weights_bf16(wl.weight_config, wl.El, wl.H, wl.I))
    xb = synth.bf16_bits(x)
    threads = oracle.num_threads()
    done, spent, n = 0, 0.0, max(threads, 1)
    while spent < target_s and done < wl.T:
        tok = np.arange(done, min(wl.T, done + n), dtype=np.int32)
        t0 = time.perf_counter()
        oracle.moe_tokens(xb, ids, w, wg, wu, wd, E=wl.E, tokens=tok)
        spent += time.perf_counter() - t0
        done += len(tok)
        n *= 2
    per_call = spent / done * wl.T + route_s
    oracle.set_num_threads(all_threads)
    touched = len(np.unique(ids)) * wl.expert_bytes()
    return dict(value=round(touched / per_call / 1e12, 6), unit="TB/s", cores=threads, kind="oracle",
                us_per_call=round(per_call * 1e6, 1),
                sample=f"{done} of {wl.T} tokens of batch 0 ({spent:.1f} s of expert work, router on all "
                       f"{wl.T} tokens), extrapolated to the whole call; double-precision C oracle, "
                       f"OpenMP over tokens, {threads} threads on {platform.processor() or platform.machine()}")


def cpu_oracle_sample(wl: Workload, cache: dict) -> dict:
    """The CPU oracle (as it stands) on one token sample of a sweep workload's batch 0: the first
    max(threads, 8) tokens (all of them below that), the router on all T tokens.  Only the local
    experts those tokens pick are generated, from the same per-expert streams as the GPU's
    weights (FP8: quantised with the same offline routine), and handed to the oracle as a compact
    expert set; generated experts are kept in `cache` for the next workloads.  The expert time is
    extrapolated to the call by OpenMP rounds of `threads` tokens."""
    import numpy as np

    import oracle
    from mixture_experts_layer_sigmoid_amd import synth

    x = synth.activations(wl.config, wl.T, wl.H, seed=0)
    lg = synth.routed_logits(wl.config, wl.T, wl.E, wl.k, wl.routing, seed=0)
    t0 = time.perf_counter()
    ids, w = oracle.router_topk(synth.bf16_bits(lg), wl.k)
    route_s = time.perf_counter() - t0
    threads = oracle.num_threads()
    n = min(wl.T, max(threads, 8))
    lo = wl.ep_rank * wl.El
    local = sorted({int(e) for e in ids[:n].ravel() if lo <= e < lo + wl.El})

    def expert(gid):
        key = (wl.weight_config, wl.H, wl.I, gid, wl.fp8)
        if key not in cache:
            ws = synth.expert_weights_bf16(wl.weight_config, 1, wl.H, wl.I, gid)
            if wl.fp8:
                q = [synth.block_quantize_fp8(t) for t in ws]
                cache[key] = tuple(c.numpy() for c, _ in q) + tuple(s.numpy() for _, s in q)
            else:
                cache[key] = tuple(synth.bf16_bits(t) for t in ws)
        return cache[key]

    parts = [expert(g) for g in local]
    spent = 0.0
    if parts:
        cat = [np.ascontiguousarray(np.concatenate([p[i] for p in parts])) for i in range(len(parts[0]))]
        ids_c = np.full(ids.shape, -1, np.int32)
        for i, g in enumerate(local):
            ids_c[ids == g] = i
        sc = dict(sg=cat[3], su=cat[4], sd=cat[5]) if wl.fp8 else {}
        t0 = time.perf_counter()
        oracle.moe_tokens(synth.bf16_bits(x), ids_c, w, cat[0], cat[1], cat[2], E=len(local),
                          tokens=np.arange(n, dtype=np.int32), **sc)
        spent = time.perf_counter() - t0
    per_call = spent / math.ceil(n / threads) * math.ceil(wl.T / threads) + route_s
    return dict(cpu_oracle_us=round(per_call * 1e6, 1),
                cpu_sample=f"{n} of {wl.T} tokens of batch 0 ({len(local)} local experts, {spent:.2f} s), router on "
                           f"all tokens, {threads} threads")


def router_microbench(samples: int = 24, warmup: int = 5, batch_calls: int = 200) -> dict:
    """The router alone on the pages' micro-benchmark batch: 128 tokens x 128 experts bf16 logits,
    top-8, 10% NaN plus 4 all-NaN rows, softmax and sigmoid (renormalised).  Per call: an event
    pair around one call, with a device fill enqueued before the pair so the GPU is still busy
    while the host enqueues (the interval is device time only); p20/p50/p80 over `samples` calls
    after `warmup`.  Also the mean over `batch_calls` calls back to back."""
    import ctypes

    import torch

    import mixture_experts_layer_sigmoid_amd as fm
    from mixture_experts_layer_sigmoid_amd import synth

    lib = fm.load_library()
    T, E, k = 128, 128, 8
    lg = synth.router_batch(T, E, k).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    busy = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for name, sc in (("softmax", fm.FMOE_SOFTMAX), ("sigmoid", fm.FMOE_SIGMOID)):
        def call():
            rc = lib.fmoe_router_topk(ctypes.c_void_p(lg.data_ptr()), fm.FMOE_BF16, T, E, k, sc, 1,
                                      ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(wts.data_ptr()), st)
            if rc != fm.FMOE_OK:
                raise RuntimeError(f"fmoe_router_topk: status {rc}")
        for _ in range(warmup):
            call()
        us = []
        for _ in range(samples):
            a, b = HipEvent(), HipEvent()
            busy.fill_(1.0)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            us.append(a.elapsed_time(b) * 1e3)
        a, b = HipEvent(), HipEvent()
        busy.fill_(1.0)
        a.record()
        for _ in range(batch_calls):
            call()
        b.record()
        torch.cuda.synchronize()
        res[name] = dict(us_p20=round(pct(us, 20), 2), us_p50=round(pct(us, 50), 2), us_p80=round(pct(us, 80), 2),
                         us_back_to_back=round(a.elapsed_time(b) * 1e3 / batch_calls, 2))
    del busy
    return dict(workload="router only: 128 tokens x 128 experts bf16, top-8, 10% NaN + 4 all-NaN rows, renormalised",
                samples=samples, warmup=warmup, **res,
                pages_context="topk_softmax p50 10.24 us, topk_sigmoid p50 12.16 us with the NaN check fused, on B200 "
                              "(another GPU and another kernel: context only)")


def tile_sweep(workloads, steps: int = 10) -> list:
    """Tile-space sweep: every tile plan the library can run (light tile rows 16/32 x gate/up
    reduction split 1/2/4 x down split 1/2/4 x light tiles per expert 1/8, and the heuristic's
    plan with the heavy-tile cut forced to 256 or 320 rows) against the host heuristic, per
    workload.  Each
    variant: 2 warmup calls, then `steps` back-to-back calls timed between two events (GPU
    time per call), weights rotating over the workload's copies."""
    import torch

    import mixture_experts_layer_sigmoid_amd as fm

    # the heuristic runs first and last (the faster of the two counts), after a warmup of its own;
    # two more plans keep the heuristic's choices but force the heavy-tile cut (256 rows, or one
    # tile for an expert of 257..320 rows: bf16 only, an FP8 layer rejects it)
    plans = [None] + [(tr, s1, s2, lt) for tr in (16, 32) for s1 in (1, 2, 4) for s2 in (1, 2, 4)
                      for lt in (1, 8)] + [(0, 0, 0, 0, 256), (0, 0, 0, 0, 320)] + [None]
    out = []
    for wl in workloads:
        print(f"[bench] tile sweep: {wl.name}", file=sys.stderr, flush=True)
        touched_guess = wl.El * (1 - (1 - wl.k / wl.E) ** wl.T) * wl.expert_bytes()
        n_copies = max(2, min(8, int(math.ceil(2 * CACHE_BYTES / max(touched_guess, 1))) + 1))
        shape, copies, batches, ws, o = build_inputs(wl, max(4, n_copies), n_copies)
        times = {}
        for j in range(20):  # warmup: clocks, caches, the library's first-launch queries
            x, lg = batches[j % len(batches)]
            fm.fmoe_forward(shape, x, lg, copies[j % n_copies], ws=ws, out=o)
        for plan in plans:
            fp = None if plan is None else fm.fmoe_plan(*plan)

            def call(j):
                x, lg = batches[j % len(batches)]
                try:
                    fm.fmoe_forward(shape, x, lg, copies[j % n_copies], ws=ws, out=o, plan=fp)
                    return True
                except RuntimeError:  # a plan this shape cannot take (FP8 LDS limit)
                    return False
            if not (call(0) and call(1)):
                continue
            a, b = HipEvent(), HipEvent()
            torch.cuda.synchronize()
            a.record()
            for j in range(steps):
                call(2 + j)
            b.record()
            torch.cuda.synchronize()
            if plan is None:
                key = "heuristic"
            elif len(plan) == 5:
                key = "heuristic, heavy tiles of %d rows" % plan[4]
            else:
                key = "tile %d, split %d/%d, light tiles %d" % plan
            t = a.elapsed_time(b) * 1e3 / steps
            times[key] = min(t, times.get(key, t))
        best = min((v, k) for k, v in times.items() if k != "heuristic")
        rec = dict(workload=wl.name, heuristic_us=round(times["heuristic"], 1), best_plan=best[1],
                   best_us=round(best[0], 1), heuristic_over_best=round(times["heuristic"] / best[0], 3),
                   worst_us=round(max(times.values()), 1), plans_us={k: round(v, 1) for k, v in times.items()})
        print(f"[bench]   heuristic {rec['heuristic_us']} us, best {rec['best_plan']} {rec['best_us']} us "
              f"(x{rec['heuristic_over_best']})", file=sys.stderr, flush=True)
        out.append(rec)
        del copies, batches, ws, o
        torch.cuda.empty_cache()
    return out


def sweep_workloads(B3, synth):
    """The T sweep of the bf16 layer (uniform and concentrated), the FP8 w8a8 layer, and the FP8
    expert-parallel shard; the headline workload is not repeated."""
    work = []
    for T in (1, 8, 32, 128, 256, 512, 1024, 4096):
        for routing in ("uniform", "concentrated"):
            if (T == 256 and routing == "uniform") or (T == 1 and routing == "concentrated"):
                continue
            work.append(Workload(f"bf16 H2048 I768 E128 top8, T={T}, {routing}", config=B3, T=T, H=2048, I=768,
                                 E=128, k=8, routing=routing))
    for T in (64, 128, 256):
        for routing in ("uniform", "concentrated"):
            if T == 64 and routing == "concentrated":
                continue
            work.append(Workload(f"fp8 w8a8 H2048 I768 E128 top8, T={T}, {routing}", config=synth.FP8_LAYER,
                                 weight_config=B3, T=T, H=2048, I=768, E=128, k=8, fp8=True, routing=routing))
    for routing in ("uniform", "concentrated"):
        work.append(Workload(f"fp8 shard H7168 I2048 top6 of 400 (ep 8, 50 local), T=288, {routing}",
                             config=synth.EP_SHARD, T=288, H=7168, I=2048, E=400, k=6, fp8=True, routing=routing,
                             ep_size=8, ep_rank=0))
    return work


def host_cpu():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true", help="headline step only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sweep-steps", type=int, default=12)
    ap.add_argument("--roofline-every", type=int, default=3,
                    help="time the dominant kernel with an event pair on every N-th timed step (3: the "
                         "sampled steps run through every batch and both weight copies in turn)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn the counter CSVs of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --no-sweep --no-cpu --calibrate` into profiles/traffic.json")
    ap.add_argument("--calibrate", action="store_true",
                    help="first run a plain 256 MiB device copy (torch elementwise kernel): the reference launch "
                         "for scaling hardware byte counters")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="time every tile plan against the heuristic on the sweep workloads (tuning report; "
                         "prints one JSON line, no headline)")
    ap.add_argument("--workload", default=None,
                    help="run only the sweep workloads whose name contains this text (profiling); no headline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this layer runs on a single MI355X (no collectives); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        ent = traffic_from_counters(*args.traffic_from, "bf16 H2048 I768 E128 top8, T=256, uniform")
        print(json.dumps(ent))
        return

    import torch

    import mixture_experts_layer_sigmoid_amd as fm
    from mixture_experts_layer_sigmoid_amd import synth

    fm.load_library()
    torch.cuda.init()
    if args.calibrate:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.add(src, 0.0, out=dst)  # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del src, dst
    B3 = synth.BF16_LAYER
    head = Workload("bf16 H2048 I768 E128 top8, T=256, uniform", config=B3, T=256, H=2048, I=768, E=128, k=8)
    if args.tile_sweep:
        wls = [head] + sweep_workloads(B3, synth)
        if args.workload is not None:
            wls = [wl for wl in wls if args.workload in wl.name]
        print(json.dumps(dict(metric="tile-space sweep: µs/call per tile plan vs the heuristic",
                              results=tile_sweep(wls))))
        return
    if args.workload is not None:
        picked = [wl for wl in [head] + sweep_workloads(B3, synth) if args.workload in wl.name]
        rows = []
        for wl in picked:
            print(f"[bench] workload: {wl.name}", file=sys.stderr, flush=True)
            rows.append(summarize(wl, measure(wl, args.steps, args.warmup)))
        print(json.dumps(dict(metric=METRIC, workloads=rows)))
        return
    print(f"[bench] headline: {head.name}", file=sys.stderr, flush=True)
    # the gate/up GEMM streams two thirds of the touched weight bytes: the dominant kernel
    dom = "gemm1"
    m = measure(head, args.steps, args.warmup, dominant=dom, every=max(1, args.roofline_every))
    hs = summarize(head, m)
    touched_bytes = m["touched"] * head.expert_bytes()
    value = touched_bytes / m["wall_s"] / 1e12

    # algorithmic bytes of one gate/up launch: the touched experts' gate and up weights, the
    # gathered activation rows it reads and the activation it writes
    alg = m["touched"] * head.gemm1_bytes_per_expert() + m["rows"] * (head.H + head.I) * 2
    dom_us = sum(m["pair_us"]) / len(m["pair_us"])
    achieved = alg / (dom_us * 1e-6) / 1e9
    roof = dict(kernel="k_grouped_gemm_stream (gate/up, SiLU-and-mul)", bound="hbm", achieved=round(achieved, 1),
                peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                traffic=traffic_from_profile(head.name, dom), algorithmic_bytes_per_launch=int(alg),
                avg_launch_us=round(dom_us, 2), timed_launches=len(m["pair_us"]),
                launch_us=[round(u, 2) for u in m["pair_us"]],
                stage_breakdown_us={k: round(v, 2) for k, v in m["stage_us"].items()})

    sweep = [hs]
    if not args.no_sweep:
        for wl in sweep_workloads(B3, synth):
            print(f"[bench] sweep: {wl.name}", file=sys.stderr, flush=True)
            sweep.append(summarize(wl, measure(wl, args.sweep_steps, 3)))
            print(f"[bench]   p50 {sweep[-1]['us_p50']} us, {sweep[-1]['hbm_TBps']} TB/s", file=sys.stderr, flush=True)

    print("[bench] router micro-benchmark (128 x 128, top-8, 10% NaN)", file=sys.stderr, flush=True)
    router = router_microbench()

    cpu = None
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle, all cores)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(head)
        print("[bench] cpu baseline (oracle, 1 core)", file=sys.stderr, flush=True)
        one = cpu_baseline(head, threads=1)
        cpu["one_core"] = dict(value=one["value"], us_per_call=one["us_per_call"], cores=1, sample=one["sample"])
        hs.update(cpu_oracle_us=cpu["us_per_call"], cpu_sample=cpu["sample"])
        if not args.no_sweep:
            cache = {}
            for wl, rec in zip(sweep_workloads(B3, synth), sweep[1:]):
                print(f"[bench] cpu oracle sample: {wl.name}", file=sys.stderr, flush=True)
                try:
                    rec.update(cpu_oracle_sample(wl, cache))
                except Exception as e:  # the GPU figures stand without it
                    rec.update(cpu_oracle_us=None, cpu_sample=f"failed: {e!r}")
            del cache

    line = dict(metric=METRIC, value=round(value, 4), unit="TB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=round(m["wall_s"] * 1e3, 5), higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="bf16", data="synthetic",
                config=dict(**head.describe(), us_per_call=round(m["wall_s"] * 1e6, 2),
                            tokens_per_s=round(head.T / m["wall_s"], 1),
                            warm_us_per_call=round(m["warm_us"], 2),
                            mfma_util=round(6.0 * m["rows"] * head.H * head.I / m["wall_s"] / 2.5e15, 4),
                            weight_copies=m["copies"]),
                roofline=roof, cpu_baseline=cpu, router_microbench=router, host_cpu=host_cpu(),
                host_cores=os.cpu_count(), kernel_sha=kernel_hash(),
                sweep=sweep)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
