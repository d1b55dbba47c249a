"""Quantized-KV attention for AMD MI355X (gfx950): Python binding of libkvq.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/kvq.h``; PyTorch supplies device memory
and the current stream.  There is no CPU fallback -- calls fail with
``KvqUnavailable`` when the library is not built or no GPU tensor is given.

Functions (same names as the C entry points):
  kvq_append_quantize(cache, k, v, pos0)
  kvq_append_norm_quantize(cache, k, v, pos0, k_weight, eps, rope=None, k_out=None, v_out=None)
  kvq_attn_decode(cache, q, len, max_len, scale=1.0, out=None, workspace=None)
  kvq_attn_prefill_chunk(cache, q, len, max_len, scale=1.0, out=None, workspace=None)
  kvq_decode_step(cache, k, v, q, len, max_len, scale=1.0, out=None, workspace=None)
  kvq_attn_decode_shared(groups, workspace=None)
  kvq_decode_step_shared(groups, k, v, workspace=None)
  kvq_attn_mixed(reads, workspace=None)
  kvq_decode_workspace_bytes(groups), kvq_decode_step_workspace_bytes(...),
  kvq_mixed_workspace_bytes(reads), kvq_prefill_workspace_bytes(...)
  kvq_mark_next_read(before, after)   (measurement: events around the next read's main kernel)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK = 0
STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "CAPACITY", 4: "WORKSPACE", 5: "HIP"}
GROUP_SIZE = 64
V_BLOCK = 8
MAX_SHARED_LAYERS = 16
MAX_SHARED_GROUPS = 4
SIZE_MAX = (1 << 64) - 1

# Symbols include/kvq.h declares.
EXPORTS = ("kvq_append_quantize", "kvq_append_quantize_multi", "kvq_append_norm_quantize", "kvq_attn_decode", "kvq_decode_step", "kvq_attn_prefill_chunk",
           "kvq_attn_decode_shared", "kvq_decode_step_shared", "kvq_attn_mixed", "kvq_decode_workspace_bytes",
           "kvq_decode_step_workspace_bytes", "kvq_decode_step_shared_workspace_bytes",
           "kvq_mixed_workspace_bytes", "kvq_prefill_workspace_bytes",
           "kvq_last_error", "kvq_mark_next_read", "kvq_attn_decode_static")
STATIC_SCRATCH_BYTES = 32 << 20


class KvqUnavailable(RuntimeError):
    pass


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class CacheStruct(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_sb", ctypes.c_void_p), ("v_sb", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("window", ctypes.c_int32)]


class SharedGroupStruct(ctypes.Structure):
    _fields_ = [("cache", ctypes.POINTER(CacheStruct)), ("n_layers", ctypes.c_int32),
                ("q", ctypes.POINTER(ctypes.c_void_p)), ("out", ctypes.POINTER(ctypes.c_void_p)),
                ("n_q_heads", ctypes.c_int32), ("scale", ctypes.c_float),
                ("len", ctypes.c_void_p), ("max_len", ctypes.c_int32)]


class AppendItemStruct(ctypes.Structure):
    _fields_ = [("cache", ctypes.POINTER(CacheStruct)), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("T", ctypes.c_int32), ("pos0", ctypes.c_void_p)]


class ReadStruct(ctypes.Structure):
    _fields_ = [("cache", ctypes.POINTER(CacheStruct)), ("n_layers", ctypes.c_int32),
                ("q", ctypes.POINTER(ctypes.c_void_p)), ("out", ctypes.POINTER(ctypes.c_void_p)),
                ("n_q_heads", ctypes.c_int32), ("chunk", ctypes.c_int32), ("scale", ctypes.c_float),
                ("len", ctypes.c_void_p), ("max_len", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkvq.so (raises KvqUnavailable if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise KvqUnavailable(f"{path} is not built; run __graft_entry__.build() or "
                             "python -m decode_attention_group_amd.build")
    lib = ctypes.CDLL(path)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    CP = ctypes.POINTER(CacheStruct)
    GP = ctypes.POINTER(SharedGroupStruct)
    lib.kvq_append_quantize.argtypes = [CP, P, P, i32, P, P]
    lib.kvq_append_quantize_multi.argtypes = [ctypes.POINTER(AppendItemStruct), i32, P]
    lib.kvq_append_norm_quantize.argtypes = [CP, P, P, i32, P, P, ctypes.c_float, P, P, i32, i32, P, P, P]
    lib.kvq_attn_decode.argtypes = [CP, P, i32, P, i32, ctypes.c_float, P, P, sz, P]
    lib.kvq_decode_step.argtypes = [CP, P, P, P, i32, P, i32, ctypes.c_float, P, P, sz, P]
    lib.kvq_decode_step_workspace_bytes.argtypes = [CP, i32, i32]
    lib.kvq_decode_step_workspace_bytes.restype = sz
    lib.kvq_attn_prefill_chunk.argtypes = [CP, P, i32, i32, P, i32, ctypes.c_float, P, P, sz, P]
    lib.kvq_attn_decode_shared.argtypes = [GP, i32, P, sz, P]
    lib.kvq_decode_step_shared.argtypes = [GP, i32, P, P, P, sz, P]
    lib.kvq_decode_step_shared_workspace_bytes.argtypes = [GP, i32]
    lib.kvq_decode_step_shared_workspace_bytes.restype = sz
    RP = ctypes.POINTER(ReadStruct)
    lib.kvq_attn_mixed.argtypes = [RP, i32, P, sz, P]
    lib.kvq_mixed_workspace_bytes.argtypes = [RP, i32]
    lib.kvq_mixed_workspace_bytes.restype = sz
    lib.kvq_decode_workspace_bytes.argtypes = [GP, i32]
    lib.kvq_decode_workspace_bytes.restype = sz
    lib.kvq_prefill_workspace_bytes.argtypes = [CP, i32, i32, i32]
    lib.kvq_prefill_workspace_bytes.restype = sz
    lib.kvq_attn_decode_static.argtypes = [CP, P, i32, P, i32, ctypes.c_float, P, P]
    lib.kvq_attn_decode_static.restype = ctypes.c_int
    lib.kvq_mark_next_read.argtypes = [P, P]
    lib.kvq_mark_next_read.restype = ctypes.c_int
    lib.kvq_last_error.argtypes = []
    lib.kvq_last_error.restype = ctypes.c_char_p
    for name in ("kvq_append_quantize", "kvq_append_quantize_multi", "kvq_append_norm_quantize", "kvq_attn_decode", "kvq_decode_step", "kvq_attn_prefill_chunk",
                 "kvq_attn_decode_shared", "kvq_decode_step_shared", "kvq_attn_mixed"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != KVQ_OK:
        raise KvqError(status, load_library().kvq_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _gpu(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise KvqUnavailable(f"{name} must be a GPU tensor (no CPU path exists)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class KVCache:
    """Device memory of one layer's quantized cache, in the layouts of include/kvq.h.

    k_codes int32 [B][H][R][D*k_bits/32]     (uint32 words)
    v_codes int32 [B][H][R/8][D][v_bits/4]   (uint32 words)
    k_sb, v_sb int32 [B][H][R][D/64]         (bf16 scale | bf16 bias << 16)
    k_bits == v_bits == 16: an unquantized bf16 cache, the same layouts holding
    bf16 values; no k_sb / v_sb (None).
    """

    def __init__(self, batch: int, n_kv_heads: int, head_dim: int, k_bits: int, v_bits: int,
                 capacity: int, window: int = 0, device="cuda", zero: bool = True):
        self.batch, self.n_kv_heads, self.head_dim = batch, n_kv_heads, head_dim
        self.k_bits, self.v_bits, self.capacity, self.window = k_bits, v_bits, capacity, window
        B, H, D, R = batch, n_kv_heads, head_dim, capacity
        alloc = torch.zeros if zero else torch.empty
        self.k_codes = alloc((B, H, R, D * k_bits // 32), dtype=torch.int32, device=device)
        self.v_codes = alloc((B, H, R // V_BLOCK, D, v_bits // 4), dtype=torch.int32, device=device)
        if k_bits == 16:
            self.k_sb = self.v_sb = None
        else:
            self.k_sb = alloc((B, H, R, D // GROUP_SIZE), dtype=torch.int32, device=device)
            self.v_sb = alloc((B, H, R, D // GROUP_SIZE), dtype=torch.int32, device=device)
        self._struct = None

    @property
    def struct(self) -> CacheStruct:
        if self._struct is None:
            self._struct = CacheStruct(self.k_codes.data_ptr(), self.v_codes.data_ptr(),
                                       _ptr(self.k_sb) or 0, _ptr(self.v_sb) or 0,
                                       self.batch, self.n_kv_heads, self.head_dim, GROUP_SIZE,
                                       self.k_bits, self.v_bits, self.capacity, self.window)
        return self._struct

    def nbytes(self) -> int:
        return sum(t.numel() * 4 for t in (self.k_codes, self.v_codes, self.k_sb, self.v_sb) if t is not None)


def kvq_mark_next_read(before: Optional["torch.cuda.Event"], after: Optional["torch.cuda.Event"]):
    """Arm two torch.cuda.Events (already recorded once, so that they exist) for the next
    attention call on this thread: it records them around its main kernel."""
    def handle(ev):
        if ev is None:
            return None
        h = ev.cuda_event
        if not h:
            raise ValueError("record the event once before arming it")
        return h
    _check(load_library().kvq_mark_next_read(handle(before), handle(after)))


def kvq_append_quantize(cache: KVCache, k: torch.Tensor, v: torch.Tensor, pos0: torch.Tensor):
    """Quantize fp32 k, v [B][H][T][D] and write them at slots (pos0[b] + t) mod R."""
    lib = load_library()
    _gpu(k, "k", torch.float32)
    _gpu(v, "v", torch.float32)
    _gpu(pos0, "pos0", torch.int32)
    B, H, T, D = k.shape
    if tuple(v.shape) != tuple(k.shape) or (B, H, D) != (cache.batch, cache.n_kv_heads, cache.head_dim):
        raise ValueError("k/v shape does not match the cache")
    _check(lib.kvq_append_quantize(ctypes.byref(cache.struct), _ptr(k), _ptr(v), T, _ptr(pos0), _stream()))


def kvq_append_quantize_multi(items):
    """Several appends in one launch: items = [(cache, k, v, pos0), ...], each as
    kvq_append_quantize takes them; every item names its own cache."""
    lib = load_library()
    arr = (AppendItemStruct * max(1, len(items)))()
    for i, (cache, k, v, pos0) in enumerate(items):
        _gpu(k, "k", torch.float32)
        _gpu(v, "v", torch.float32)
        _gpu(pos0, "pos0", torch.int32)
        B, H, T, D = k.shape
        if tuple(v.shape) != tuple(k.shape) or (B, H, D) != (cache.batch, cache.n_kv_heads, cache.head_dim):
            raise ValueError(f"item {i}: k/v shape does not match the cache")
        arr[i] = AppendItemStruct(ctypes.pointer(cache.struct), _ptr(k), _ptr(v), T, _ptr(pos0))
    _check(lib.kvq_append_quantize_multi(arr, len(items), _stream()))


def kvq_append_norm_quantize(cache: KVCache, k: torch.Tensor, v: torch.Tensor, pos0: torch.Tensor,
                             k_weight: Optional[torch.Tensor], eps: float, rope=None,
                             k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None):
    """Norm (keys weighted by k_weight [D], values un-scaled), rotate the keys with
    rope = (cos, sin) fp32 [positions][rope_dims/2] at absolute positions, then
    quantize and append as kvq_append_quantize; k_out / v_out receive the normed rows."""
    lib = load_library()
    _gpu(k, "k", torch.float32)
    _gpu(v, "v", torch.float32)
    _gpu(pos0, "pos0", torch.int32)
    B, H, T, D = k.shape
    if tuple(v.shape) != tuple(k.shape) or (B, H, D) != (cache.batch, cache.n_kv_heads, cache.head_dim):
        raise ValueError("k/v shape does not match the cache")
    if k_weight is not None:
        _gpu(k_weight, "k_weight", torch.float32)
        if k_weight.numel() != D:
            raise ValueError("k_weight must hold head_dim values")
    cos_t = sin_t = None
    rope_dims = rope_positions = 0
    if rope is not None:
        cos_t, sin_t = rope
        _gpu(cos_t, "rope cos", torch.float32)
        _gpu(sin_t, "rope sin", torch.float32)
        if cos_t.dim() != 2 or tuple(sin_t.shape) != tuple(cos_t.shape):
            raise ValueError("rope tables must both be [positions][rope_dims/2]")
        rope_positions, rope_dims = cos_t.shape[0], 2 * cos_t.shape[1]
    for name, o in (("k_out", k_out), ("v_out", v_out)):
        if o is not None:
            _gpu(o, name, torch.float32)
            if tuple(o.shape) != tuple(k.shape):
                raise ValueError(f"{name} must have k's shape")
    _check(lib.kvq_append_norm_quantize(ctypes.byref(cache.struct), _ptr(k), _ptr(v), T, _ptr(pos0),
                                        _ptr(k_weight), float(eps), _ptr(cos_t), _ptr(sin_t), rope_dims,
                                        rope_positions, _ptr(k_out), _ptr(v_out), _stream()))


def _group_struct(cache: KVCache, qs: Sequence[torch.Tensor], outs: Sequence[torch.Tensor],
                  len_: torch.Tensor, max_len: int, scale: float, keep: list) -> SharedGroupStruct:
    qa = (ctypes.c_void_p * len(qs))(*[_ptr(q) for q in qs])
    oa = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
    cs = cache.struct
    keep.extend([qa, oa, cs])
    n_q_heads = qs[0].shape[1] if len(qs) else 0
    return SharedGroupStruct(ctypes.pointer(cs), len(qs), qa, oa, n_q_heads, float(scale), _ptr(len_), int(max_len))


def kvq_decode_workspace_bytes(groups) -> int:
    keep: list = []
    arr = (SharedGroupStruct * len(groups))(*[_group_struct(*g, keep=keep) for g in groups])
    n = load_library().kvq_decode_workspace_bytes(arr, len(groups))
    if n == SIZE_MAX:
        raise KvqError(1, "invalid arguments for kvq_decode_workspace_bytes")
    return n


def kvq_prefill_workspace_bytes(cache: KVCache, n_q_heads: int, chunk: int, max_len: int) -> int:
    n = load_library().kvq_prefill_workspace_bytes(ctypes.byref(cache.struct), n_q_heads, chunk, max_len)
    if n == SIZE_MAX:
        raise KvqError(1, "invalid arguments for kvq_prefill_workspace_bytes")
    return n


def _workspace(nbytes: int, workspace: Optional[torch.Tensor], device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return workspace
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise KvqError(4, f"workspace of {workspace.numel() * workspace.element_size()} bytes given, "
                              f"{nbytes} needed")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def kvq_attn_decode(cache: KVCache, q: torch.Tensor, len_: torch.Tensor, max_len: int, scale: float = 1.0,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q bf16 [B][Hq][D] -> out bf16 [B][Hq][D]."""
    lib = load_library()
    _gpu(q, "q", torch.bfloat16)
    _gpu(len_, "len", torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _gpu(out, "out", torch.bfloat16)
    nbytes = kvq_decode_workspace_bytes([(cache, [q], [out], len_, max_len, scale)])
    ws = _workspace(nbytes, workspace, q.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.kvq_attn_decode(ctypes.byref(cache.struct), _ptr(q), q.shape[1], _ptr(len_), int(max_len),
                               float(scale), _ptr(out), _ptr(ws), wsb, _stream()))
    return out


def kvq_attn_decode_static(cache: KVCache, q: torch.Tensor, len_: torch.Tensor, max_len: int,
                           scale: float = 1.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kvq_attn_decode with the library's static device scratch instead of a workspace
    (no allocation inside the call; `out` must be given by callers that cannot allocate)."""
    lib = load_library()
    _gpu(q, "q", torch.bfloat16)
    _gpu(len_, "len", torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _gpu(out, "out", torch.bfloat16)
    _check(lib.kvq_attn_decode_static(ctypes.byref(cache.struct), _ptr(q), q.shape[1], _ptr(len_), int(max_len),
                                      float(scale), _ptr(out), _stream()))
    return out


def kvq_decode_step_workspace_bytes(cache: KVCache, n_q_heads: int, max_len: int) -> int:
    n = load_library().kvq_decode_step_workspace_bytes(ctypes.byref(cache.struct), n_q_heads, max_len)
    if n == SIZE_MAX:
        raise KvqError(1, "invalid arguments for kvq_decode_step_workspace_bytes")
    return n


def kvq_decode_step(cache: KVCache, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, len_: torch.Tensor,
                    max_len: int, scale: float = 1.0, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Append k, v fp32 [B][H][D] at position len-1 and read: q bf16 [B][Hq][D] -> out bf16 [B][Hq][D]."""
    lib = load_library()
    _gpu(k, "k", torch.float32)
    _gpu(v, "v", torch.float32)
    _gpu(q, "q", torch.bfloat16)
    _gpu(len_, "len", torch.int32)
    B, H, D = k.shape
    if tuple(v.shape) != tuple(k.shape) or (B, H, D) != (cache.batch, cache.n_kv_heads, cache.head_dim):
        raise ValueError("k/v shape does not match the cache")
    if out is None:
        out = torch.empty_like(q)
    _gpu(out, "out", torch.bfloat16)
    nbytes = lib.kvq_decode_step_workspace_bytes(ctypes.byref(cache.struct), q.shape[1], max_len)
    if nbytes == SIZE_MAX:      # invalid or unsupported: the call itself reports why
        _check(lib.kvq_decode_step(ctypes.byref(cache.struct), _ptr(k), _ptr(v), _ptr(q), q.shape[1], _ptr(len_),
                                   int(max_len), float(scale), _ptr(out), None, 0, _stream()))
        raise KvqError(1, "invalid arguments for kvq_decode_step")
    ws = _workspace(nbytes, workspace, q.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.kvq_decode_step(ctypes.byref(cache.struct), _ptr(k), _ptr(v), _ptr(q), q.shape[1], _ptr(len_),
                               int(max_len), float(scale), _ptr(out), _ptr(ws), wsb, _stream()))
    return out


def kvq_attn_prefill_chunk(cache: KVCache, q: torch.Tensor, len_: torch.Tensor, max_len: int, scale: float = 1.0,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q bf16 [B][Hq][C][D] (queries at len-C .. len-1) -> out bf16 [B][Hq][C][D]."""
    lib = load_library()
    _gpu(q, "q", torch.bfloat16)
    _gpu(len_, "len", torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _gpu(out, "out", torch.bfloat16)
    B, Hq, C, D = q.shape
    nbytes = kvq_prefill_workspace_bytes(cache, Hq, C, max_len)
    ws = _workspace(nbytes, workspace, q.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.kvq_attn_prefill_chunk(ctypes.byref(cache.struct), _ptr(q), Hq, C, _ptr(len_), int(max_len),
                                      float(scale), _ptr(out), _ptr(ws), wsb, _stream()))
    return out


@dataclass
class SharedGroup:
    """One cache read by several KV-sharing layers' queries (each bf16 [B][Hq][D])."""
    cache: KVCache
    q: List[torch.Tensor]
    len: torch.Tensor
    max_len: int
    scale: float = 1.0
    out: Optional[List[torch.Tensor]] = None


def kvq_attn_decode_shared(groups: Sequence[SharedGroup], workspace: Optional[torch.Tensor] = None):
    """All groups in one attention launch; returns the list of per-group output lists."""
    lib = load_library()
    specs = []
    for g in groups:
        for i, q in enumerate(g.q):
            _gpu(q, f"q[{i}]", torch.bfloat16)
        _gpu(g.len, "len", torch.int32)
        if g.out is None:
            g.out = [torch.empty_like(q) for q in g.q]
        for i, o in enumerate(g.out):
            _gpu(o, f"out[{i}]", torch.bfloat16)
        specs.append((g.cache, g.q, g.out, g.len, g.max_len, g.scale))
    keep: list = []
    arr = (SharedGroupStruct * len(specs))(*[_group_struct(*s, keep=keep) for s in specs])
    nbytes = lib.kvq_decode_workspace_bytes(arr, len(specs))
    if nbytes == SIZE_MAX:
        _check(lib.kvq_attn_decode_shared(arr, len(specs), None, 0, _stream()))
    device = groups[0].q[0].device
    ws = _workspace(nbytes, workspace, device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.kvq_attn_decode_shared(arr, len(specs), _ptr(ws), wsb, _stream()))
    return [g.out for g in groups]


def kvq_decode_step_shared(groups: Sequence[SharedGroup], k: Sequence[torch.Tensor], v: Sequence[torch.Tensor],
                           workspace: Optional[torch.Tensor] = None):
    """Append k[i], v[i] fp32 [B][H][D] to group i's cache at position len-1 and run
    the shared read of every group in one launch; returns the per-group output lists."""
    lib = load_library()
    if len(k) != len(groups) or len(v) != len(groups):
        raise ValueError("one k and one v per group")
    specs = []
    for gi, g in enumerate(groups):
        for i, q in enumerate(g.q):
            _gpu(q, f"q[{i}]", torch.bfloat16)
        _gpu(g.len, "len", torch.int32)
        _gpu(k[gi], f"k[{gi}]", torch.float32)
        _gpu(v[gi], f"v[{gi}]", torch.float32)
        c = g.cache
        if tuple(k[gi].shape) != (c.batch, c.n_kv_heads, c.head_dim) or tuple(v[gi].shape) != tuple(k[gi].shape):
            raise ValueError(f"k[{gi}]/v[{gi}] shape does not match the cache")
        if g.out is None:
            g.out = [torch.empty_like(q) for q in g.q]
        for i, o in enumerate(g.out):
            _gpu(o, f"out[{i}]", torch.bfloat16)
        specs.append((g.cache, g.q, g.out, g.len, g.max_len, g.scale))
    keep: list = []
    arr = (SharedGroupStruct * len(specs))(*[_group_struct(*s, keep=keep) for s in specs])
    ka = (ctypes.c_void_p * len(k))(*[_ptr(t) for t in k])
    va = (ctypes.c_void_p * len(v))(*[_ptr(t) for t in v])
    nbytes = lib.kvq_decode_step_shared_workspace_bytes(arr, len(specs))
    if nbytes == SIZE_MAX:
        _check(lib.kvq_decode_step_shared(arr, len(specs), ka, va, None, 0, _stream()))
        raise KvqError(1, "invalid arguments for kvq_decode_step_shared")
    device = groups[0].q[0].device
    ws = _workspace(nbytes, workspace, device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.kvq_decode_step_shared(arr, len(specs), ka, va, _ptr(ws), wsb, _stream()))
    return [g.out for g in groups]


@dataclass
class Read:
    """One read of a mixed launch: queries bf16 [B][Hq][chunk][D] per layer (chunk > 1: one layer)."""
    cache: KVCache
    q: List[torch.Tensor]
    len: torch.Tensor
    max_len: int
    scale: float = 1.0
    out: Optional[List[torch.Tensor]] = None


def kvq_mixed_workspace_bytes(reads: Sequence[Read]) -> int:
    """Workspace bytes kvq_attn_mixed needs for these reads."""
    keep: list = []
    arr = _read_structs(reads, keep)
    n = load_library().kvq_mixed_workspace_bytes(arr, len(reads))
    if n == SIZE_MAX:
        raise KvqError(1, "invalid arguments for kvq_mixed_workspace_bytes")
    return n


def _read_structs(reads: Sequence["Read"], keep: list):
    structs = []
    for r in reads:
        outs = r.out if r.out is not None else r.q
        qa = (ctypes.c_void_p * len(r.q))(*[_ptr(q) for q in r.q])
        oa = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
        cs = r.cache.struct
        keep.extend([qa, oa, cs])
        structs.append(ReadStruct(ctypes.pointer(cs), len(r.q), qa, oa, r.q[0].shape[1], r.q[0].shape[2],
                                  float(r.scale), _ptr(r.len), int(r.max_len)))
    return (ReadStruct * len(structs))(*structs)


def kvq_attn_mixed(reads: Sequence[Read], workspace: Optional[torch.Tensor] = None):
    """Decode reads and short chunks in one attention launch; returns the per-read output lists."""
    lib = load_library()
    keep: list = []
    for r in reads:
        for i, q in enumerate(r.q):
            _gpu(q, f"q[{i}]", torch.bfloat16)
            if q.dim() != 4:
                raise ValueError("kvq_attn_mixed queries are [B][Hq][chunk][D]")
        _gpu(r.len, "len", torch.int32)
        if r.out is None:
            r.out = [torch.empty_like(q) for q in r.q]
        for i, o in enumerate(r.out):
            _gpu(o, f"out[{i}]", torch.bfloat16)
    arr = _read_structs(reads, keep)
    nbytes = lib.kvq_mixed_workspace_bytes(arr, len(reads))
    if nbytes == SIZE_MAX:
        raise KvqError(1, "invalid arguments for kvq_mixed_workspace_bytes")
    ws = _workspace(nbytes, workspace, reads[0].q[0].device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.kvq_attn_mixed(arr, len(reads), _ptr(ws), wsb, _stream()))
    return [r.out for r in reads]
