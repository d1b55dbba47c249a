"""Seeded synthetic inputs for quantized-KV attention.

This module only draws numbers and names shapes; it holds none of the
method's arithmetic.  Both the GPU path's tests/bench and the CPU oracle read
the tensors it returns.

Recipe (every workload):
  * one ``torch.Generator('cpu')`` seeded with the workload's seed (0);
  * queries first, in the order the workload lists them, each drawn as fp32
    ``torch.randn(shape) * D**-0.25`` and rounded to bf16 (round-half-even);
    the same bf16 values feed both sides;
  * then each cache in turn, keys and values drawn in position chunks of at
    most ``CHUNK`` tokens starting at position 0: for every chunk, K as fp32
    ``randn([B, Hkv, T, D]) * D**-0.25`` and then V the same way.  These fp32
    values are what gets quantized.
D**-0.25 is a standard deviation, so q.k has unit variance at SDPA scale 1.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Iterator, List, Tuple

import numpy as np
import torch

CHUNK = 4096


@dataclass(frozen=True)
class CacheSpec:
    """One layer's quantized cache: R slots (a ring when window > 0)."""
    name: str
    B: int
    Hkv: int
    D: int
    k_bits: int
    v_bits: int
    R: int
    window: int          # 0: full attention
    length: int          # tokens appended in total, the current step's included


@dataclass(frozen=True)
class QuerySpec:
    """Queries of ``layers`` layers reading cache ``cache``; C queries per sequence."""
    cache: str
    layers: int
    Hq: int
    C: int = 1


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "decode" | "prefill" | "verify" (a few queries per sequence) | "shared" | "mixed"
    caches: Tuple[CacheSpec, ...]
    queries: Tuple[QuerySpec, ...]
    seed: int = 0
    description: str = ""

    def cache(self, name: str) -> CacheSpec:
        for c in self.caches:
            if c.name == name:
                return c
        raise KeyError(name)


def _wl(name, kind, caches, queries, description):
    return Workload(name, kind, tuple(caches), tuple(queries), 0, description)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        _wl("decode_b1_l128", "decode",
            [CacheSpec("kv", 1, 2, 256, 4, 4, 128, 0, 128)],
            [QuerySpec("kv", 1, 8)],
            "single decode step, B1, 8 q / 2 kv heads, D256, cached length 128, K4/V4"),
        _wl("sliding_decode_b8_w512", "decode",
            [CacheSpec("kv", 8, 2, 256, 4, 8, 512, 512, 4096)],
            [QuerySpec("kv", 1, 8)],
            "sliding-window decode, B8, 8 q / 2 kv heads, D256, 4096 tokens through a ring of 512, K4/V8"),
        _wl("full_decode_b4_l32768", "decode",
            [CacheSpec("kv", 4, 1, 512, 8, 8, 32768, 0, 32768)],
            [QuerySpec("kv", 1, 8)],
            "full-attention decode, B4, 8 q heads / 1 kv head, D512, cached length 32768, K8/V8"),
        _wl("prefill_b2_c512_w512", "prefill",
            [CacheSpec("kv", 2, 2, 256, 4, 4, 1024, 512, 8192 + 512)],
            [QuerySpec("kv", 1, 8, 512)],
            "chunked prefill, B2, 512-query chunk after 8192 cached tokens, 8 q / 2 kv heads, "
            "D256, K4/V4, window 512 (ring of 1024)"),
        _wl("verify_b8_c5_w512", "verify",
            [CacheSpec("kv", 8, 2, 256, 4, 8, 520, 512, 4096)],
            [QuerySpec("kv", 1, 8, 5)],
            "speculative verify window, B8, 5 queries per sequence (4 drafted + 1), 8 q / 2 kv heads, "
            "D256, K4/V8, window 512 (ring of 520)"),
        _wl("verify_b4_c5_l32768", "verify",
            [CacheSpec("kv", 4, 1, 512, 8, 8, 32768, 0, 32768)],
            [QuerySpec("kv", 1, 8, 5)],
            "speculative verify window on a full layer, B4, 5 queries per sequence, 8 q / 1 kv head, "
            "D512, K8/V8, cached length 32768"),
        _wl("mixed_b8_decode_verify", "mixed",
            [CacheSpec("donor", 8, 2, 256, 4, 8, 520, 512, 4096),
             CacheSpec("full", 8, 1, 512, 8, 8, 16384, 0, 16384)],
            [QuerySpec("donor", 3, 8), QuerySpec("full", 1, 8, 5)],
            "mixed launch, B8: three layers decoding over a sliding cache (D256, K4/V8, window 512) "
            "and a 5-token verify chunk over a full layer (D512, K8/V8, 16384 tokens), one attention launch"),
        _wl("sliding_decode_bf16_b8_w512", "decode",
            [CacheSpec("kv", 8, 2, 256, 16, 16, 512, 512, 4096)],
            [QuerySpec("kv", 1, 8)],
            "sliding-window decode over an unquantized bf16 cache (the pages' bf16 sliding layers), B8, "
            "8 q / 2 kv heads, D256, 4096 tokens through a ring of 512"),
        _wl("prefill_bf16_b2_c512_w512", "prefill",
            [CacheSpec("kv", 2, 2, 256, 16, 16, 1024, 512, 8192 + 512)],
            [QuerySpec("kv", 1, 8, 512)],
            "chunked prefill over an unquantized bf16 cache (the pages' bf16 sliding layers), B2, 512-query "
            "chunk after 8192 cached tokens, 8 q / 2 kv heads, D256, window 512 (ring of 1024)"),
        _wl("shared_decode_b32", "shared",
            [CacheSpec("donor", 32, 2, 256, 4, 4, 512, 512, 16384),
             CacheSpec("full", 32, 1, 512, 8, 8, 16384, 0, 16384)],
            [QuerySpec("donor", 3, 8), QuerySpec("full", 1, 8)],
            "KV-shared decode, B32: three layers over one 4-bit sliding donor (window 512, D256) "
            "plus one full layer (8 q / 1 kv, D512, 8-bit, length 16384), one launch"),
    ]
}


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """Round fp32 to bf16 (round-half-even) and return the bit patterns as uint16."""
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclass
class Draws:
    """Queries (bf16 bit patterns) per QuerySpec: list over layers of [B][Hq][C][D]."""
    q: List[List[np.ndarray]] = field(default_factory=list)


class Generator:
    """Replays one workload's draws in the fixed order of the module docstring."""

    def __init__(self, workload: Workload):
        self.w = workload
        self.gen = torch.Generator(device="cpu")
        self.gen.manual_seed(workload.seed)
        self.q: List[List[np.ndarray]] = []
        for qs in workload.queries:
            c = workload.cache(qs.cache)
            sigma = c.D ** -0.25
            layers = []
            for _ in range(qs.layers):
                x = torch.randn((c.B, qs.Hq, qs.C, c.D), generator=self.gen, dtype=torch.float32) * sigma
                layers.append(bf16_bits(x))
            self.q.append(layers)
        self._cache_pos = 0

    def kv_chunks(self, cache: CacheSpec, chunk: int = CHUNK) -> Iterator[Tuple[int, np.ndarray, np.ndarray]]:
        """Yield (pos0, K, V) for positions [pos0, pos0+T), T <= chunk, K/V fp32 [B][Hkv][T][D].

        Caches must be consumed in the workload's order, each to the end."""
        sigma = cache.D ** -0.25
        pos = 0
        while pos < cache.length:
            T = min(chunk, cache.length - pos)
            shape = (cache.B, cache.Hkv, T, cache.D)
            k = (torch.randn(shape, generator=self.gen, dtype=torch.float32) * sigma).numpy()
            v = (torch.randn(shape, generator=self.gen, dtype=torch.float32) * sigma).numpy()
            yield pos, k, v
            pos += T


def small_randn(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """Independent seeded fp32 draws for small test cases."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.randn(tuple(shape), generator=g, dtype=torch.float32) * sigma).numpy()


def small_q_bits(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return bf16_bits(torch.randn(tuple(shape), generator=g, dtype=torch.float32) * sigma)
