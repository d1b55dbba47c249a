#!/usr/bin/env python3
"""Benchmark of quantized-KV attention on one MI355X.

A step is one pass of the hot path over one batch of the workload: the step's
new token(s) are quantized and appended to the cache and the read runs.  Decode
workloads take the fused step (kvq_decode_step; kvq_decode_step_shared for the
KV-shared groups), which does both in one read launch; prefill, verify and
mixed workloads append (kvq_append_quantize, or one kvq_append_quantize_multi
launch for several caches) and then read (kvq_attn_prefill_chunk /
kvq_attn_mixed).  Inputs are resident in HBM before timing starts.

To read HBM rather than the 256 MB last-level cache, every timed step reads one
of several identical cache replicas in rotation, so that the rotation covers at
least --rotate-gib of memory, and a 1 GiB buffer is read before each timed
region.

Timing, all with HIP events on the launch stream:
  * steps: K steps captured in one HIP graph and replayed (no host gaps between
    launches); median, p10 and p90 over --reps replays of the per-step time;
  * the attention call alone (main kernel + combine), the same way;
  * the dominant kernel alone: K attention calls launched eagerly behind a GPU
    sleep that holds the stream until all K are queued, each call asked
    (kvq_mark_next_read) to record two events around its main kernel; median,
    p10 and p90 over the K launches.  `roofline.achieved` uses this median.

Output: one JSON line.  `value` is the headline workload's throughput per step
(algorithmic bytes, or FLOPs for prefill, per step time); `roofline` is its
dominant kernel against the published peak (8 TB/s HBM3E; 2.5 PFLOP/s dense bf16)
and against the ceilings the probes measure on the same GPU (a stream read and
an MFMA loop, include/kvq_probes.h); `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload; `configs` holds the same figures for every
other workload.

Algorithmic bytes per visible (key, KV head): K and V codes plus one bf16
scale and one bf16 bias per 64-group for K and for V (an unquantized bf16
cache: its 2-byte K and V values, no scale or bias); a donor cache read by
several layers counts once; plus the bf16 queries read and outputs written.
Prefill is reported in TFLOP/s: 4*head_dim FLOPs per visible (query, key) pair.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# the largest configuration: three layers over a sliding donor plus a full
# 16384-token head_dim-512 layer, batch 32, in one launch (581 MB per read)
HEADLINE = "shared_decode_b32"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "decode attention effective KV GB/s (% of HBM peak); prefill TFLOP/s"


PROFILES = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_sources_sha() -> str:
    """Hash of the kernel sources, recorded next to the HBM counters they were taken with."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "decode_attention_group_amd", "csrc", "*"))):
        if p.endswith((".hip", ".h")):
            h.update(os.path.basename(p).encode())
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per launch of the workload's dominant kernel from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE runs, or None when there are none or the
    kernel sources changed since they were taken."""
    try:
        with open(PROFILES) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256_16") != kernel_sources_sha():
        return None
    w = t.get("workloads", {}).get(name)
    return None if w is None else int(w["bytes_per_launch"])


def visible(spec, p):
    lo = max(0, p - spec.window + 1) if spec.window else 0
    return p - lo + 1


def algorithmic(wl):
    """(bytes, flops) of one read of the workload, per the formula in the module docstring."""
    byts, flops = 0, 0
    for spec in wl.caches:
        per_key = spec.D * (spec.k_bits + spec.v_bits) // 8 + (0 if spec.k_bits == 16 else (spec.D // 64) * 8)
        qs = [q for q in wl.queries if q.cache == spec.name]
        C = max(q.C for q in qs)
        first = spec.length - C
        lo = max(0, first - spec.window + 1) if spec.window else 0
        keys = spec.length - lo                          # distinct keys read
        byts += spec.B * spec.Hkv * keys * per_key
        for q in qs:
            byts += 2 * q.layers * spec.B * q.Hq * q.C * spec.D * 2
            pairs = sum(visible(spec, spec.length - C + i) for i in range(q.C))
            flops += 4 * spec.D * q.layers * spec.B * q.Hq * pairs
    return byts, flops


class Runner:
    """GPU state of one workload: cache replicas, queries, the step's new tokens."""

    def __init__(self, wl, rotate_bytes: float, keep_oracle: bool = False):
        import torch
        import decode_attention_group_amd as kvq
        import synth
        self.wl, self.kvq, self.torch = wl, kvq, torch
        gen = synth.Generator(wl)
        cache_bytes = 0
        for spec in wl.caches:
            G = spec.D // 64
            cache_bytes += spec.B * spec.Hkv * spec.R * (spec.D * (spec.k_bits + spec.v_bits) // 8 + 8 * G)
        self.nrep = max(1, int(np.ceil(rotate_bytes / cache_bytes)))
        self.C = max(q.C for q in wl.queries)
        # tokens each cache's step appends: the chunk of the queries that read it
        self.C_of = {spec.name: max(q.C for q in wl.queries if q.cache == spec.name) for spec in wl.caches}
        dev = "cuda"
        self.caches = {spec.name: [kvq.KVCache(spec.B, spec.Hkv, spec.D, spec.k_bits, spec.v_bits, spec.R, spec.window)]
                       for spec in wl.caches}
        self.step_kv = {}
        self.oracle_chunks = {} if keep_oracle else None
        for spec in wl.caches:
            new0 = spec.length - self.C_of[spec.name]
            for pos, k, v in gen.kv_chunks(spec):
                if keep_oracle:
                    self.oracle_chunks.setdefault(spec.name, []).append((pos, k, v))
                T = k.shape[2]
                kt, vt = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
                # positions >= new0 are the step's own tokens: held back, appended by each step
                keep = min(T, max(0, new0 - pos))
                if keep < T:
                    self.step_kv[spec.name] = (kt[:, :, keep:].contiguous(), vt[:, :, keep:].contiguous())
                if keep > 0:
                    pos0 = torch.full((spec.B,), pos, dtype=torch.int32, device=dev)
                    a, b = kt[:, :, :keep].contiguous(), vt[:, :, :keep].contiguous()
                    for g in self.caches[spec.name]:
                        kvq.kvq_append_quantize(g, a, b, pos0)
                del kt, vt
        for spec in wl.caches:                   # identical replicas, to rotate through
            g0 = self.caches[spec.name][0]
            for _ in range(self.nrep - 1):
                g = kvq.KVCache(spec.B, spec.Hkv, spec.D, spec.k_bits, spec.v_bits, spec.R, spec.window, zero=False)
                for a, b in ((g.k_codes, g0.k_codes), (g.v_codes, g0.v_codes), (g.k_sb, g0.k_sb), (g.v_sb, g0.v_sb)):
                    if a is not None:
                        a.copy_(b)
                self.caches[spec.name].append(g)
        self.q = {}
        for qs, layers in zip(wl.queries, gen.q):
            t = [torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) for x in layers]
            if qs.C == 1 and wl.kind != "mixed":         # mixed reads take [B][Hq][C][D] queries
                t = [x[:, :, 0].contiguous() for x in t]
            self.q[qs.cache] = t
        self.q_draws = gen.q
        self.len = {spec.name: torch.full((spec.B,), spec.length, dtype=torch.int32, device=dev) for spec in wl.caches}
        self.pos_new = {spec.name: torch.full((spec.B,), spec.length - self.C_of[spec.name], dtype=torch.int32,
                                              device=dev)
                        for spec in wl.caches}
        self.out = {name: [torch.empty_like(x) for x in qs] for name, qs in self.q.items()}
        if wl.kind == "shared":
            self.groups = [[kvq.SharedGroup(self.caches[qs.cache][r], self.q[qs.cache], self.len[qs.cache],
                                            wl.cache(qs.cache).length, 1.0, self.out[qs.cache])
                            for qs in wl.queries] for r in range(self.nrep)]
            nbytes = kvq.kvq_decode_workspace_bytes(
                [(g.cache, g.q, g.out, g.len, g.max_len, g.scale) for g in self.groups[0]])
            keep: list = []
            arr = (kvq.SharedGroupStruct * len(self.groups[0]))(
                *[kvq._group_struct(g.cache, g.q, g.out, g.len, g.max_len, g.scale, keep=keep)
                  for g in self.groups[0]])
            nbytes = max(nbytes, kvq.load_library().kvq_decode_step_shared_workspace_bytes(arr, len(self.groups[0])))
            self.step_k = [self.step_kv[qs.cache][0].reshape(spec.B, spec.Hkv, spec.D)
                           for qs in wl.queries for spec in [wl.cache(qs.cache)]]
            self.step_v = [self.step_kv[qs.cache][1].reshape(spec.B, spec.Hkv, spec.D)
                           for qs in wl.queries for spec in [wl.cache(qs.cache)]]
        elif wl.kind == "mixed":
            self.reads = [[kvq.Read(self.caches[qs.cache][r], self.q[qs.cache], self.len[qs.cache],
                                    wl.cache(qs.cache).length, 1.0, self.out[qs.cache])
                           for qs in wl.queries] for r in range(self.nrep)]
            nbytes = kvq.kvq_mixed_workspace_bytes(self.reads[0])
        elif wl.kind in ("prefill", "verify"):
            spec = wl.caches[0]
            nbytes = kvq.kvq_prefill_workspace_bytes(self.caches["kv"][0], wl.queries[0].Hq, self.C, spec.length)
        else:
            spec = wl.caches[0]
            g = self.caches["kv"][0]
            nbytes = kvq.kvq_decode_workspace_bytes([(g, self.q["kv"], self.out["kv"], self.len["kv"], spec.length, 1.0)])
            nbytes = max(nbytes, kvq.kvq_decode_step_workspace_bytes(g, wl.queries[0].Hq, spec.length))
            k, v = self.step_kv["kv"]
            self.step_k1 = k.reshape(spec.B, spec.Hkv, spec.D)
            self.step_v1 = v.reshape(spec.B, spec.Hkv, spec.D)
        # decode steps (one cache or KV-shared groups) run as one fused call
        # (append + read); prefill, verify and mixed reads as append, then read
        self.fused = wl.kind in ("decode", "shared")
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def append(self, r):
        """The step's tokens into every cache: one launch for several caches."""
        items = [(self.caches[s.name][r], *self.step_kv[s.name], self.pos_new[s.name]) for s in self.wl.caches]
        if len(items) > 1:
            self.kvq.kvq_append_quantize_multi(items)
        else:
            self.kvq.kvq_append_quantize(*items[0])

    def attend(self, r):
        kvq, wl = self.kvq, self.wl
        if wl.kind == "shared":
            kvq.kvq_attn_decode_shared(self.groups[r], workspace=self.ws)
        elif wl.kind == "mixed":
            kvq.kvq_attn_mixed(self.reads[r], workspace=self.ws)
        elif wl.kind in ("prefill", "verify"):
            kvq.kvq_attn_prefill_chunk(self.caches["kv"][r], self.q["kv"][0], self.len["kv"], wl.caches[0].length,
                                       1.0, out=self.out["kv"][0], workspace=self.ws)
        else:
            kvq.kvq_attn_decode(self.caches["kv"][r], self.q["kv"][0], self.len["kv"], wl.caches[0].length,
                                1.0, out=self.out["kv"][0], workspace=self.ws)

    def step(self, r):
        """One decode step as the fused call: the tokens' appends and the read."""
        if self.wl.kind == "shared":
            self.kvq.kvq_decode_step_shared(self.groups[r], self.step_k, self.step_v, workspace=self.ws)
            return
        self.kvq.kvq_decode_step(self.caches["kv"][r], self.step_k1, self.step_v1, self.q["kv"][0],
                                 self.len["kv"], self.wl.caches[0].length, 1.0, out=self.out["kv"][0],
                                 workspace=self.ws)

    def _graph(self, steps, first, mode):
        """mode: "step" (fused where the workload has it), "two" (append, then
        read), "attn" (the read alone)."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                r = (first + i) % self.nrep
                if mode == "step" and self.fused:
                    self.step(r)
                    continue
                if mode != "attn":
                    self.append(r)
                self.attend(r)
        return g

    def run(self, steps, warmup, reps=7):
        """Time `steps` steps replayed from a HIP graph (no host gaps between
        launches), after flushing the last-level cache; also time the attention
        calls alone the same way.  Per-step time of each of `reps` replays."""
        torch = self.torch
        for i in range(warmup):
            self.append(i % self.nrep)
            self.attend(i % self.nrep)
            if self.fused:
                self.step(i % self.nrep)
        torch.cuda.synchronize()
        g_step = self._graph(steps, warmup, "step")
        g_two = self._graph(steps, warmup, "two") if self.fused else None
        g_attn = self._graph(steps, warmup, "attn")
        stream = torch.cuda.current_stream()

        def timed(graph):
            flush_llc()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps

        self.step_ms = [timed(g_step) for _ in range(reps)]
        self.attn_ms = [timed(g_attn) for _ in range(reps)]
        self.two_ms = [timed(g_two) for _ in range(reps)] if g_two else None
        del g_step, g_attn, g_two
        self.kernel_ms = self.kernel_events(steps)

    def kernel_events(self, steps):
        """Duration of each of `steps` launches of the read's main kernel, from the
        two events the library records around it (kvq_mark_next_read).  The calls
        are queued behind a GPU sleep, so no host gap falls inside a launch's pair."""
        torch, kvq = self.torch, self.kvq
        stream = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:                              # create the handles
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        flush_llc()
        torch.cuda._sleep(gate_cycles(steps * 0.3))   # ~0.3 ms of host time per queued call
        for i, (a, b) in enumerate(evs):
            kvq.kvq_mark_next_read(a, b)
            self.attend(i % self.nrep)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]


_FLUSH = {}
_GATE = {}


def flush_llc():
    """Evict the last-level cache by reading 1 GiB: a read leaves clean lines,
    whereas a write fill would leave dirty ones whose write-back would be charged
    to the first timed launches."""
    import torch
    if "buf" not in _FLUSH:
        _FLUSH["buf"] = torch.ones(1 << 28, dtype=torch.float32, device="cuda")    # 1 GiB
        _FLUSH["sink"] = torch.empty(1, dtype=torch.float32, device="cuda")
    torch.sum(_FLUSH["buf"], dim=0, out=_FLUSH["sink"][0])


def gate_cycles(ms: float) -> int:
    """Argument of torch.cuda._sleep that keeps the GPU busy for about `ms` ms
    (its spin counts the GPU's clock, calibrated once)."""
    import torch
    if "per_ms" not in _GATE:
        torch.cuda.synchronize()
        n = 1 << 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        torch.cuda.synchronize()
        _GATE["per_ms"] = n / max(e0.elapsed_time(e1), 1e-3)
    return int(_GATE["per_ms"] * max(ms, 1.0))


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(wl, runner, budget_s):
    """Time the CPU oracle on the same workload: quantize-and-append of the step's
    tokens plus the fp64 read of every query row, repeated for about `budget_s`
    seconds.  Batch rows are sampled (row 0 only, time scaled by the batch) when
    the whole batch would be too slow for a short run."""
    import oracle
    nthreads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    byts, flops = algorithmic(wl)
    B = wl.caches[0].B
    work = sum(s.B * min(s.length, s.window or s.length) * s.D for s in wl.caches)
    nb = B if work <= 64e6 else 1
    caches = {}
    for spec in wl.caches:
        o = oracle.Cache(nb, spec.Hkv, spec.D, spec.R, spec.k_bits, spec.v_bits, spec.window)
        for pos, k, v in runner.oracle_chunks[spec.name]:
            o.append(k[:nb], v[:nb], np.full(nb, pos, np.int32))
        caches[spec.name] = (o, spec)
    n, t_total = 0, 0.0
    while t_total < budget_s:
        t = time.perf_counter()
        for spec in wl.caches:
            o, _ = caches[spec.name]
            pos, k, v = runner.oracle_chunks[spec.name][-1]
            T, C = k.shape[2], runner.C_of[spec.name]
            o.append(k[:nb, :, T - C:], v[:nb, :, T - C:], np.full(nb, spec.length - C, np.int32))
        for qs, layers in zip(wl.queries, runner.q_draws):
            o, spec = caches[qs.cache]
            for x in layers:
                o.attend(x[:nb], np.full(nb, spec.length, np.int32), 1.0, nthreads)
        t_total += time.perf_counter() - t
        n += 1
    step_s = t_total / n * (B / nb)
    model, affinity = host_cpu()
    rows = "all %d batch rows" % B if nb == B else "batch row 0 of %d, time scaled x%d" % (B, B)
    if wl.kind == "prefill":
        value, unit = flops / step_s / 1e12, "TFLOP/s"
    else:
        value, unit = byts / step_s / 1e9, "GB/s"
    return {"value": round(value, 6), "unit": unit, "cores": nthreads, "kind": "oracle",
            "sample": f"{n} full oracle steps ({t_total:.1f} s) on {rows}: fp32 quantize-append of the "
                      f"step's tokens + fp64 attention of every query row",
            "s_per_step": round(step_s, 6), "cpu_model": model, "affinity_cpus": affinity}


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def probe_ceilings():
    """Attainable HBM read rate and dense bf16 MFMA rate on this GPU, from the
    probes of include/kvq_probes.h (best over a few launch shapes, 3 runs each)."""
    import torch
    from decode_attention_group_amd import probes
    stream = torch.cuda.current_stream()

    def time_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    nbytes = 4 << 30                                  # 16x the last-level cache
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")
    best_read, read_cfg, read_sweep = 0.0, None, []
    for blocks in (512, 1024, 2048, 4096, 8192):
        for nt in (0, 1):
            probes.stream_read(src, blocks, bool(nt), sink)          # warm-up
            ms = min(time_ms(lambda: probes.stream_read(src, blocks, bool(nt), sink)) for _ in range(3))
            gbs = nbytes / (ms * 1e-3) / 1e9
            read_sweep.append([blocks, nt, round(gbs, 1)])
            if gbs > best_read:
                best_read, read_cfg = gbs, {"blocks": blocks, "nontemporal": nt}
    # workgroups that each stream their own run (a split-KV read's shape): the rate
    # such a read can reach with 16 KB in flight per 256-thread workgroup
    seg_sweep = []
    for blocks, seg in ((460, 310 << 10), (512, 1 << 20), (1024, 1 << 20), (2048, 512 << 10)):
        for nt in (0, 1):
            probes.segment_read(src, seg, blocks, bool(nt), sink)
            ms = min(time_ms(lambda: probes.segment_read(src, seg, blocks, bool(nt), sink)) for _ in range(3))
            seg_sweep.append([blocks, seg >> 10, nt, round(blocks * seg / (ms * 1e-3) / 1e9, 1)])
    del src
    fsink = torch.empty(4096 * 256, dtype=torch.float32, device="cuda")
    best_mfma, mfma_cfg, mfma_sweep = 0.0, None, []
    for shape in (0, 1):
        for blocks in (1024, 2048, 4096):
            iters = 2000
            probes.mfma_bf16(shape, 10, blocks, fsink)
            flops = 0.0

            def run():
                nonlocal flops
                flops = probes.mfma_bf16(shape, iters, blocks, fsink)
            ms = min(time_ms(run) for _ in range(3))
            tf = flops / (ms * 1e-3) / 1e12
            mfma_sweep.append([shape, blocks, round(tf, 1)])
            if tf > best_mfma:
                best_mfma, mfma_cfg = tf, {"mfma": "16x16x32" if shape == 0 else "32x32x16", "blocks": blocks}
    torch.cuda.synchronize()
    return {"hbm_read_gbs": round(best_read, 1), "hbm_read_probe": read_cfg,
            "mfma_bf16_tflops": round(best_mfma, 1), "mfma_probe": mfma_cfg,
            "hbm_read_sweep [blocks, nontemporal, GB/s]": read_sweep,
            "hbm_segment_read_sweep [blocks, KiB per block, nontemporal, GB/s]": seg_sweep,
            "mfma_sweep [shape 0=16x16x32 1=32x32x16, blocks, TFLOP/s]": mfma_sweep}


def measure(name, steps, warmup, rotate_gib, cpu_s, ceilings):
    import synth
    wl = synth.WORKLOADS[name]
    runner = Runner(wl, rotate_gib * (1 << 30), keep_oracle=cpu_s > 0)
    runner.run(steps, warmup)
    byts, flops = algorithmic(wl)
    step_ms, attn_ms, kern_ms = (float(np.median(x)) for x in (runner.step_ms, runner.attn_ms, runner.kernel_ms))
    res = {"workload": name, "ms_per_step": step_ms,
           "step_p10_ms": pct(runner.step_ms, 10), "step_p90_ms": pct(runner.step_ms, 90),
           "attn_ms": attn_ms, "bytes": byts, "flops": flops, "replicas": runner.nrep, "fused_step": runner.fused,
           "two_call_ms_per_step": None if runner.two_ms is None else round(float(np.median(runner.two_ms)), 5)}
    if wl.kind == "prefill":
        work, scale, unit, peak, ceil, bound = flops, 1e12, "TFLOP/s", BF16_PEAK_TFLOPS, ceilings.get(
            "mfma_bf16_tflops"), "mfma"
    else:
        work, scale, unit, peak, ceil, bound = byts, 1e9, "GB/s", HBM_PEAK_GBS, ceilings.get("hbm_read_gbs"), "hbm"
    rate = lambda ms: work / (ms * 1e-3) / scale  # noqa: E731
    achieved = rate(kern_ms)
    res.update(value=rate(step_ms), unit=unit)
    res["roofline"] = {
        "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
        "frac": round(achieved / peak, 5), "traffic": measured_traffic(name),
        "kernel": dominant_kernel_name(name), "kernel_ms": round(kern_ms, 6),
        "kernel_p10_ms": round(pct(runner.kernel_ms, 10), 6), "kernel_p90_ms": round(pct(runner.kernel_ms, 90), 6),
        "kernel_launches": len(runner.kernel_ms),
        "measured_ceiling": ceil, "frac_of_measured_ceiling": round(achieved / ceil, 5) if ceil else None,
        "call_achieved": round(rate(attn_ms), 3), "call_frac": round(rate(attn_ms) / peak, 5),
        "call_frac_of_measured_ceiling": round(rate(attn_ms) / ceil, 5) if ceil else None,
    }
    if cpu_s > 0:
        res["cpu_baseline"] = cpu_baseline(wl, runner, cpu_s)
    del runner
    import torch
    torch.cuda.empty_cache()
    return res


def dominant_kernel_name(name):
    try:
        with open(PROFILES) as f:
            return json.load(f)["workloads"][name]["kernel"]
    except (OSError, ValueError, KeyError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="measure only --workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-probes", action="store_true", help="skip the ceiling probes")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget for the headline")
    ap.add_argument("--cpu-seconds-other", type=float, default=3.0, help="oracle time budget for other configs")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, 5 times (reference kernel for "
                         "scaling the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        n = args.copy_probe << 18                       # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4}))
        return
    ceilings = {} if args.no_probes else probe_ceilings()
    if ceilings:
        print(f"# probes: {json.dumps(ceilings)}", file=sys.stderr, flush=True)
    cpu_head = 0.0 if args.no_cpu else args.cpu_seconds
    cpu_other = 0.0 if args.no_cpu else args.cpu_seconds_other

    def summary(r):
        rf = r["roofline"]
        print(f"# {r['workload']}: {r['value']:.2f} {r['unit']} step {r['ms_per_step'] * 1e3:.1f} us, call "
              f"{r['attn_ms'] * 1e3:.1f} us, kernel {rf['kernel_ms'] * 1e3:.1f} us = {rf['achieved']} {rf['unit']} "
              f"({100 * rf['frac']:.1f}% of peak, "
              f"{'-' if rf['frac_of_measured_ceiling'] is None else round(100 * rf['frac_of_measured_ceiling'], 1)}"
              f"% of measured)", file=sys.stderr, flush=True)

    head = measure(args.workload, args.steps, args.warmup, args.rotate_gib, cpu_head, ceilings)
    summary(head)
    others = {}
    if not args.only:
        for name in synth.WORKLOADS:
            if name == args.workload:
                continue
            r = measure(name, args.steps, args.warmup, args.rotate_gib, cpu_other, ceilings)
            summary(r)
            others[name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "step_p10_ms", "step_p90_ms",
                                              "attn_ms", "replicas", "two_call_ms_per_step", "roofline")
                            if k in r}
            if "cpu_baseline" in r:
                others[name]["cpu_baseline"] = r["cpu_baseline"]
    wl = synth.WORKLOADS[args.workload]
    config = {"workload": args.workload, "description": wl.description, "batch": wl.caches[0].B,
              "caches": [{"name": c.name, "head_dim": c.D, "kv_heads": c.Hkv, "k_bits": c.k_bits,
                          "v_bits": c.v_bits, "window": c.window, "capacity": c.R, "cached_tokens": c.length}
                         for c in wl.caches],
              "queries": [{"cache": q.cache, "layers": q.layers, "q_heads": q.Hq, "chunk": q.C} for q in wl.queries],
              "replicas": head["replicas"],
              "step": ("kvq_decode_step: the token's append and the attention read in one call"
                       if head["fused_step"] else "append the step's token(s) + attention read"),
              "compute": "4/8-bit codes -> fp16 MFMA, fp32 accumulate, bf16 out"}
    line = {
        "metric": METRIC,
        "value": round(head["value"], 3),
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "step_p10_ms": round(head["step_p10_ms"], 6),
        "step_p90_ms": round(head["step_p90_ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": config,
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "ceilings": ceilings,
        "attn_ms": round(head["attn_ms"], 6),
        "two_call_ms_per_step": head["two_call_ms_per_step"],
        "configs": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
