#!/usr/bin/env python3
"""Benchmark of quantized-KV attention on one MI355X.

A step is one pass of the hot path over one batch of the workload: the step's
new token(s) are quantized and appended to the cache (kvq_append_quantize),
then the read runs (kvq_attn_decode / kvq_attn_prefill_chunk /
kvq_attn_decode_shared).  Inputs are resident in HBM before timing starts.

To read HBM rather than the 256 MB last-level cache, every timed step reads
one of several identical cache replicas in rotation, so that the rotation
covers at least --rotate-gib of memory, and a 1 GiB buffer is read before
each timed region.  The K timed steps are replayed from one HIP graph,
so host launch overhead does not sit between them.

Output: one JSON line.  `value` is the headline workload's effective KV
bandwidth (algorithmic bytes per step / time per step); `roofline` measures the
attention call alone (split kernel + combine kernel, HIP events on the launch
stream) against the 8 TB/s HBM peak; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload; `configs` holds the same figures for
every workload.

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

HEADLINE = "sliding_decode_b8_w512"
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
        # decode steps run as one fused call (append + read); the others as two
        self.fused = wl.kind == "decode"
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def append(self, r):
        for spec in self.wl.caches:
            k, v = self.step_kv[spec.name]
            self.kvq.kvq_append_quantize(self.caches[spec.name][r], k, v, self.pos_new[spec.name])

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
        """One decode step as the fused call: the token's append and the read."""
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

    def run(self, steps, warmup, reps=3):
        """Time `steps` steps replayed from a HIP graph (no host gaps between
        launches), after flushing the last-level cache; also time the attention
        calls alone the same way.  Median over `reps` replays of each."""
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
        # Evict the last-level cache by reading 1 GiB: a read leaves clean lines,
        # whereas a write fill would leave dirty ones whose write-back would be
        # charged to the first timed steps.
        flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")    # 1 GiB
        sink = torch.empty(1, dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()

        def timed(graph, k):
            torch.sum(flush, dim=0, out=sink[0])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps

        step_ms = float(np.median([timed(g_step, k) for k in range(reps)]))
        attn_ms = float(np.median([timed(g_attn, k) for k in range(reps)]))
        self.two_call_ms = float(np.median([timed(g_two, k) for k in range(reps)])) if g_two else None
        del flush, g_step, g_attn, g_two
        return step_ms, attn_ms


def cpu_baseline(wl, runner, budget_s=10.0):
    """Time the CPU oracle on the same workload: quantize-and-append of the step's
    tokens plus the fp64 read of every query row.  Batch rows are sampled only
    when the whole batch would be too slow for a short run; the time is then
    scaled to the full batch."""
    import oracle
    nthreads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    byts, _ = algorithmic(wl)
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
    rows = "all %d batch rows" % B if nb == B else "batch row 0 of %d, time scaled x%d" % (B, B)
    return {"value": round(byts / step_s / 1e9, 4), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{n} full oracle steps ({t_total:.1f} s) on {rows}: fp32 quantize-append of the "
                      f"step's tokens + fp64 attention of every query row"}


def measure(name, steps, warmup, rotate_gib, with_cpu):
    import synth
    wl = synth.WORKLOADS[name]
    runner = Runner(wl, rotate_gib * (1 << 30), keep_oracle=with_cpu)
    step_ms, attn_ms = runner.run(steps, warmup)
    byts, flops = algorithmic(wl)
    res = {"workload": name, "ms_per_step": step_ms, "attn_ms": attn_ms, "bytes": byts, "flops": flops,
           "replicas": runner.nrep, "fused_step": runner.fused,
           "two_call_ms_per_step": None if runner.two_call_ms is None else round(runner.two_call_ms, 5)}
    if wl.kind == "prefill":
        res.update(value=flops / (step_ms * 1e-3) / 1e12, unit="TFLOP/s",
                   roofline={"bound": "mfma", "achieved": round(flops / (attn_ms * 1e-3) / 1e12, 3),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(flops / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5)})
    else:
        res.update(value=byts / (step_ms * 1e-3) / 1e9, unit="GB/s",
                   roofline={"bound": "hbm", "achieved": round(byts / (attn_ms * 1e-3) / 1e9, 2),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(byts / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5)})
    res["roofline"]["traffic"] = measured_traffic(name)
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, runner)
    del runner
    import torch
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="measure only --workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
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
    head = measure(args.workload, args.steps, args.warmup, args.rotate_gib, not args.no_cpu)
    others = {}
    if not args.only:
        for name in synth.WORKLOADS:
            if name == args.workload:
                continue
            r = measure(name, args.steps, args.warmup, args.rotate_gib, False)
            others[name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "attn_ms", "replicas",
                                              "two_call_ms_per_step")}
            others[name]["roofline_frac"] = r["roofline"]["frac"]
            others[name]["achieved"] = r["roofline"]["achieved"]
            print(f"# {name}: {r['value']:.2f} {r['unit']} step {r['ms_per_step'] * 1e3:.1f} us, "
                  f"attention {r['attn_ms'] * 1e3:.1f} us = {r['roofline']['achieved']} {r['roofline']['unit']} "
                  f"({100 * r['roofline']['frac']:.1f}% of peak)", file=sys.stderr, flush=True)
    wl = synth.WORKLOADS[args.workload]
    spec = wl.caches[0]
    line = {
        "metric": METRIC,
        "value": round(head["value"], 3),
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": spec.B, "head_dim": spec.D, "q_heads": wl.queries[0].Hq,
                   "kv_heads": spec.Hkv, "k_bits": spec.k_bits, "v_bits": spec.v_bits, "window": spec.window,
                   "cached_tokens": spec.length, "replicas": head["replicas"],
                   "step": ("kvq_decode_step: the token's append and the attention read in one call"
                            if head["fused_step"] else "append the step's token(s) + attention read"),
                   "compute": "4/8-bit codes -> fp16 MFMA, fp32 accumulate, bf16 out"},
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "attn_ms": round(head["attn_ms"], 5),
        "two_call_ms_per_step": head["two_call_ms_per_step"],
        "configs": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
