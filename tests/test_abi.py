"""The C ABI library: it loads, exports every entry point include/kvq.h declares, and
its host-side validation returns the documented statuses.  No GPU is needed: every
call here fails validation before anything reaches the HIP runtime."""
import ctypes
import os
import re

import pytest

import decode_attention_group_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

FAKE = 0x100000  # a non-null address; validation fails before it is used


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return kvq.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:kvq_status|size_t|const char \*)\s*(kvq_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(kvq.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_every_declared_symbol():
    """include/kvq_probes.h (the measurement probes) against libkvq_probes.so."""
    from decode_attention_group_amd import probes
    if not os.path.exists(probes.LIB_PATH):
        pytest.skip("libkvq_probes.so not built")
    text = open(os.path.join(ROOT, "include", "kvq_probes.h")).read()
    names = set(re.findall(r"^\s*(?:int|double)\s*(kvq_\w+)\s*\(", text, re.M))
    assert names == set(probes.EXPORTS)
    so = probes.load_library()
    for n in names:
        assert hasattr(so, n), n
    # argument checks need no GPU: nothing is launched on a bad argument
    assert so.kvq_probe_stream_read(None, 16, 1, 0, FAKE, None) == 1
    assert so.kvq_probe_stream_read(FAKE + 4, 16, 1, 0, FAKE, None) == 1
    assert so.kvq_probe_mfma_bf16(2, 1, 1, FAKE, None) == 1
    assert so.kvq_probe_mfma_flops_per_iter(0, 2) == 8 * 2 * 16 * 16 * 32 * 4 * 2


def test_mark_next_read_needs_no_gpu(lib):
    """Arming NULL events is valid; the next (failing) call drops the marks."""
    assert lib.kvq_mark_next_read(None, None) == 0
    assert decode(lib, cache(head_dim=100)) == 2


def cache(**kw):
    c = dict(k_codes=FAKE, v_codes=FAKE, k_sb=FAKE, v_sb=FAKE, batch=2, n_kv_heads=2, head_dim=256,
             group_size=64, k_bits=4, v_bits=8, capacity=512, window=512)
    c.update(kw)
    return kvq.CacheStruct(**c)


def decode(lib, c, Hq=8, max_len=4096, scale=1.0, ws=0, q=FAKE, out=FAKE, ln=FAKE, ws_ptr=None):
    return lib.kvq_attn_decode(ctypes.byref(c), q, Hq, ln, max_len, scale, out, ws_ptr, ws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=100), 2), (dict(head_dim=576), 2), (dict(head_dim=32), 2), (dict(group_size=32), 2),
    (dict(k_bits=16, v_bits=16, head_dim=320), 2), (dict(k_bits=5), 2),
    (dict(v_bits=2), 2), (dict(capacity=12), 1), (dict(capacity=0), 1), (dict(window=1024), 3),
    (dict(window=-1), 1), (dict(capacity=1 << 24, window=0, head_dim=512, k_bits=8, v_bits=8), 1),
    (dict(capacity=1 << 23, window=0, head_dim=512, k_bits=16, v_bits=16), 1), (dict(batch=0), 1), (dict(n_kv_heads=0), 1), (dict(k_codes=0), 1),
    (dict(v_sb=0), 1), (dict(capacity=24, window=0), 1), (dict(k_bits=16), 2), (dict(v_bits=16), 2),
    (dict(k_bits=16, v_bits=16, v_codes=0), 1), (dict(k_codes=FAKE + 8), 1), (dict(v_sb=FAKE + 4), 1),
    (dict(batch=40000), 1), (dict(n_kv_heads=70000), 1),
])
def test_decode_cache_validation(lib, kw, status):
    assert decode(lib, cache(**kw)) == status
    assert lib.kvq_last_error().decode()


def test_decode_argument_validation(lib):
    assert decode(lib, cache(), Hq=7) == 1            # Hq % Hkv
    assert decode(lib, cache(), q=FAKE + 2) == 1      # q not 16-byte aligned
    assert decode(lib, cache(), out=FAKE + 4) == 1    # out not 8-byte aligned
    assert "aligned" in lib.kvq_last_error().decode()
    assert decode(lib, cache(), q=0) == 1
    assert decode(lib, cache(), out=0) == 1
    assert decode(lib, cache(), ln=0) == 1
    assert decode(lib, cache(), max_len=0) == 1
    assert decode(lib, cache(), scale=float("inf")) == 1
    full = cache(window=0, capacity=1024)
    assert decode(lib, full, max_len=2048) == 3       # full cache cannot hold max_len
    big = cache(window=0, capacity=32768, head_dim=512, n_kv_heads=1, k_bits=8, v_bits=8, batch=4)
    assert decode(lib, big, max_len=32768, ws=0) == 4  # split partials need a workspace
    assert "workspace" in lib.kvq_last_error().decode()
    assert decode(lib, big, max_len=32768, ws=1 << 30, ws_ptr=FAKE + 8) == 1   # misaligned workspace
    assert "16-byte" in lib.kvq_last_error().decode()


@pytest.mark.parametrize("C", [8, 512])
def test_prefill_workspace_alignment(lib, C):
    """The short-chunk (8 queries: 64 rows over 32768 keys) and band (512 queries)
    paths refuse a workspace that is not 16-byte aligned, before any launch."""
    c = cache(window=0, capacity=32768, head_dim=512, n_kv_heads=1, k_bits=8, v_bits=8, batch=4)
    st = lib.kvq_attn_prefill_chunk(ctypes.byref(c), FAKE, 8, C, FAKE, 32768, 1.0, FAKE, FAKE + 4, 1 << 34, None)
    assert st == 1 and "16-byte" in lib.kvq_last_error().decode()


def test_prefill_validation(lib):
    c = cache(window=512, capacity=1024)
    f = lib.kvq_attn_prefill_chunk
    assert f(ctypes.byref(c), FAKE, 8, 600, FAKE, 9000, 1.0, FAKE, None, 0, None) == 3   # W + C - 1 > R
    assert f(ctypes.byref(c), FAKE, 8, 0, FAKE, 9000, 1.0, FAKE, None, 0, None) == 1     # chunk 0
    assert f(ctypes.byref(c), FAKE, 8, 512, FAKE, 100, 1.0, FAKE, None, 0, None) == 1    # max_len < chunk


def test_append_validation(lib):
    c = cache()
    f = lib.kvq_append_quantize
    assert f(ctypes.byref(c), FAKE, FAKE, -1, FAKE, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, 0, FAKE, None) == 0        # T == 0 is a no-op
    assert f(ctypes.byref(c), 0, FAKE, 4, FAKE, None) == 1
    assert f(ctypes.byref(c), FAKE + 4, FAKE, 4, FAKE, None) == 1    # k not 16-byte aligned
    assert f(ctypes.byref(cache(head_dim=96)), FAKE, FAKE, 4, FAKE, None) == 2


def test_multi_append_validation(lib):
    """Items are checked in order and nothing launches on an error, so every call
    here returns before the HIP runtime is reached."""
    a, b, c96 = cache(head_dim=128), cache(head_dim=256), cache(head_dim=96)
    b.k_codes, b.v_codes = FAKE + 0x10000, FAKE + 0x20000
    f = lib.kvq_append_quantize_multi

    def items(*specs):
        arr = (kvq.AppendItemStruct * max(1, len(specs)))()
        for i, (c, T, k) in enumerate(specs):
            arr[i] = kvq.AppendItemStruct(ctypes.pointer(c), k, FAKE, T, FAKE)
        return arr
    assert f(None, 1, None) == 1
    assert f(items((a, 0, FAKE)), 0, None) == 1                     # n_items < 1
    assert f(items(*[(a, 0, FAKE)] * 5), 5, None) == 1              # n_items > 4
    assert f(items((a, 0, FAKE), (b, 0, FAKE)), 2, None) == 0        # nothing to write: no launch
    assert f(items((a, 0, FAKE), (a, 0, FAKE)), 2, None) == 1        # one cache twice
    assert f(items((a, 0, FAKE), (b, -1, FAKE)), 2, None) == 1       # T < 0
    assert f(items((a, 4, FAKE), (b, 4, 0)), 2, None) == 1           # k NULL in the second item
    assert f(items((a, 4, FAKE), (b, 4, FAKE + 4)), 2, None) == 1    # k not 16-byte aligned
    assert f(items((a, 4, FAKE), (c96, 4, FAKE)), 2, None) == 2      # unsupported head_dim


def test_normed_append_validation(lib):
    c = cache(head_dim=128)
    f = lib.kvq_append_norm_quantize
    ok = dict(w=FAKE, eps=1e-6, cos=FAKE, sin=FAKE, n=64, P=100, ko=None, vo=None)

    def call(T=4, k=FAKE, **kw):
        a = dict(ok, **kw)
        return f(ctypes.byref(c), k, FAKE, T, FAKE, a["w"], a["eps"], a["cos"], a["sin"], a["n"], a["P"],
                 a["ko"], a["vo"], None)
    assert call(T=-1) == 1
    assert call(T=0) == 0                                            # a no-op once the arguments check out
    assert call(k=0) == 1
    assert call(eps=-1e-6) == 1
    assert call(eps=float("nan")) == 1
    assert call(eps=float("inf")) == 1
    assert call(n=3) == 1                                            # odd rope_dims
    assert call(n=130) == 1                                          # rope_dims > head_dim
    assert call(n=-2) == 1
    assert call(cos=None) == 1 and call(sin=None) == 1
    assert call(P=0) == 1
    assert call(ko=FAKE + 8) == 1                                    # outputs 16-byte aligned
    assert call(T=0, n=0, cos=None, sin=None, P=0, w=None) == 0      # no rotation, no weight
    assert f(ctypes.byref(cache(head_dim=96)), FAKE, FAKE, 4, FAKE, None, 1e-6, None, None, 0, 0, None, None,
             None) == 2


def _group(c, n_layers=1, Hq=8, max_len=4096):
    qa = (ctypes.c_void_p * max(n_layers, 1))(*([FAKE] * max(n_layers, 1)))
    oa = (ctypes.c_void_p * max(n_layers, 1))(*([FAKE] * max(n_layers, 1)))
    return kvq.SharedGroupStruct(ctypes.pointer(c), n_layers, qa, oa, Hq, 1.0, FAKE, max_len), (qa, oa)


def test_shared_validation_and_workspace_query(lib):
    c = cache()
    g, keep = _group(c, 3)
    arr = (kvq.SharedGroupStruct * 1)(g)
    assert lib.kvq_attn_decode_shared(arr, 0, None, 0, None) == 1
    assert lib.kvq_attn_decode_shared(arr, 5, None, 0, None) == 1
    bad, keep2 = _group(c, 17)
    assert lib.kvq_attn_decode_shared((kvq.SharedGroupStruct * 1)(bad), 1, None, 0, None) == 1
    assert lib.kvq_decode_workspace_bytes((kvq.SharedGroupStruct * 1)(bad), 1) == kvq.SIZE_MAX
    n = lib.kvq_decode_workspace_bytes(arr, 1)
    assert n != kvq.SIZE_MAX
    big = cache(window=0, capacity=32768, head_dim=512, n_kv_heads=1, k_bits=8, v_bits=8, batch=4)
    gb, keep3 = _group(big, 1, 8, 32768)
    need = lib.kvq_decode_workspace_bytes((kvq.SharedGroupStruct * 1)(gb), 1)
    assert 0 < need < (1 << 30)
    # a workspace one byte short is refused
    assert lib.kvq_attn_decode_shared((kvq.SharedGroupStruct * 1)(gb), 1, FAKE, need - 1, None) == 4


def test_prefill_workspace_query(lib):
    c = cache(window=512, capacity=1024)
    assert lib.kvq_prefill_workspace_bytes(ctypes.byref(c), 8, 512, 8704) != kvq.SIZE_MAX
    assert lib.kvq_prefill_workspace_bytes(ctypes.byref(c), 7, 512, 8704) == kvq.SIZE_MAX


def test_bf16_prefill_workspace_needs_no_band(lib, monkeypatch):
    """Long chunks are read in place: a quantized cache's prefill kernel reads the
    codes itself and a bf16 cache's reads the stored values, so neither workspace
    holds a band (the 512-query chunk of 2 sequences x 2 KV heads fills 256 work
    items with no split, so it needs none at all), unless a bf16 cache is too
    large for 32-bit DMA offsets within one (sequence, KV head) (capacity *
    head_dim * 2 >= 2^31) or the band copy is forced with KVQ_BF16_BAND=1."""
    monkeypatch.delenv("KVQ_BF16_BAND", raising=False)
    q = dict(k_bits=16, v_bits=16, k_sb=0, v_sb=0)
    sliding = cache(window=512, capacity=1024, **q)
    quant = cache(window=512, capacity=1024)
    n_bf16 = lib.kvq_prefill_workspace_bytes(ctypes.byref(sliding), 8, 512, 8704)
    n_quant = lib.kvq_prefill_workspace_bytes(ctypes.byref(quant), 8, 512, 8704)
    band = 2 * 2 * (512 + 511 + 32) * 256 * 2 * 2          # at least the band's K and V tiles
    assert n_bf16 != kvq.SIZE_MAX and n_bf16 < band and n_quant == 0
    monkeypatch.setenv("KVQ_BF16_BAND", "1")
    assert lib.kvq_prefill_workspace_bytes(ctypes.byref(sliding), 8, 512, 8704) >= band
    monkeypatch.delenv("KVQ_BF16_BAND")
    D = 512
    small = cache(batch=1, n_kv_heads=1, head_dim=D, window=0, capacity=(1 << 30) // D - 8, **q)
    large = cache(batch=1, n_kv_heads=1, head_dim=D, window=0, capacity=(1 << 30) // D, **q)
    n_small = lib.kvq_prefill_workspace_bytes(ctypes.byref(small), 8, 512, 4096)
    n_large = lib.kvq_prefill_workspace_bytes(ctypes.byref(large), 8, 512, 4096)
    assert n_large - n_small >= 4096 * D * 2 * 2


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    c = kvq.KVCache.__new__(kvq.KVCache)
    with pytest.raises(kvq.KvqUnavailable):
        kvq.kvq_append_quantize(c, torch.zeros(1, 1, 1, 128), torch.zeros(1, 1, 1, 128), torch.zeros(1, dtype=torch.int32))


def mixed(lib, c, n_layers=1, chunk=1, Hq=8, max_len=600, n=1, ws=0):
    qa = (ctypes.c_void_p * max(n_layers, 1))(*([FAKE] * max(n_layers, 1)))
    r = kvq.ReadStruct(ctypes.pointer(c), n_layers, qa, qa, Hq, chunk, 1.0, FAKE, max_len)
    arr = (kvq.ReadStruct * max(n, 1))(*([r] * max(n, 1)))
    return lib.kvq_attn_mixed(arr, n, None, ws, None), lib.kvq_mixed_workspace_bytes(arr, n)


def test_mixed_validation_and_workspace_query(lib):
    st, nb = mixed(lib, cache(), n=0)
    assert st == 1 and nb == kvq.SIZE_MAX
    st, nb = mixed(lib, cache(), n=kvq.MAX_SHARED_GROUPS + 1)
    assert st == 1 and nb == kvq.SIZE_MAX
    st, nb = mixed(lib, cache(), chunk=0)                          # chunk < 1
    assert st == 1 and nb == kvq.SIZE_MAX
    st, nb = mixed(lib, cache(), chunk=4, n_layers=2)              # a chunk reads one layer
    assert st == 1 and nb == kvq.SIZE_MAX
    st, _ = mixed(lib, cache(), chunk=4)                           # window 512 + 4 - 1 > capacity 512
    assert st == 3
    st, nb = mixed(lib, cache(capacity=520), chunk=4)              # valid: needs a workspace
    assert nb not in (0, kvq.SIZE_MAX) and st == 4
    st, nb = mixed(lib, cache(capacity=520), n_layers=3)           # decode by three layers
    assert nb not in (0, kvq.SIZE_MAX) and st == 4
    assert lib.kvq_last_error().decode()


def test_decode_step_validation(lib):
    c = cache()
    step = lambda k, v, Hq=8, ws=0: lib.kvq_decode_step(ctypes.byref(c), k, v, FAKE, Hq, FAKE, 600, 1.0, FAKE,
                                                        None, ws, None)
    assert step(None, FAKE) == 1                                   # k NULL
    assert step(FAKE, FAKE + 4) == 1                               # v not 16-byte aligned
    assert step(FAKE, FAKE, Hq=7) == 1                             # Hq % Hkv
    assert step(FAKE, FAKE) == 4                                   # workspace too small
    nb = lib.kvq_decode_step_workspace_bytes(ctypes.byref(c), 8, 600)
    assert nb not in (0, kvq.SIZE_MAX)
    assert lib.kvq_decode_step_workspace_bytes(ctypes.byref(c), 7, 600) == kvq.SIZE_MAX


def test_bf16_cache_validation(lib):
    """A bf16 cache (both widths 16) needs no scale/bias arrays and is taken by
    every call.  Only host-side checks run here (no launch)."""
    c = cache(k_bits=16, v_bits=16, k_sb=0, v_sb=0)
    g, keep = _group(c, n_layers=3)
    assert lib.kvq_decode_workspace_bytes(ctypes.byref(g), 1) != kvq.SIZE_MAX
    assert lib.kvq_prefill_workspace_bytes(ctypes.byref(c), 8, 5, 4096) != kvq.SIZE_MAX
    assert lib.kvq_decode_step_workspace_bytes(ctypes.byref(c), 8, 4096) != kvq.SIZE_MAX
    st = lib.kvq_decode_step(ctypes.byref(c), FAKE + 4, FAKE, FAKE, 8, FAKE, 4096, 1.0, FAKE, None, 0, None)
    assert st == 1 and "aligned" in lib.kvq_last_error().decode()     # refused before any launch
    mixed = cache(k_bits=16, v_bits=8, k_sb=0, v_sb=0)
    g2, keep2 = _group(mixed)
    assert lib.kvq_decode_workspace_bytes(ctypes.byref(g2), 1) == kvq.SIZE_MAX


@pytest.mark.parametrize("bits", [(4, 4), (4, 8), (8, 4), (8, 8), (16, 16)])
def test_binding_buffers_follow_the_header_layouts(bits):
    """KVCache allocates exactly the layouts include/kvq.h documents (host only:
    the buffers live on the CPU here)."""
    kb, vb = bits
    B, H, D, R = 3, 2, 256, 96
    c = kvq.KVCache(B, H, D, kb, vb, R, window=64, device="cpu")
    assert tuple(c.k_codes.shape) == (B, H, R, D * kb // 32)
    assert tuple(c.v_codes.shape) == (B, H, R // 8, D, vb // 4)
    if kb == 16:
        assert c.k_sb is None and c.v_sb is None
        assert c.nbytes() == B * H * R * D * 2 * 2
    else:
        assert tuple(c.k_sb.shape) == (B, H, R, D // 64) == tuple(c.v_sb.shape)
        assert c.nbytes() == B * H * R * (D * (kb + vb) // 8 + 2 * 4 * D // 64)
    s = c.struct
    assert (s.k_bits, s.v_bits, s.capacity, s.window, s.group_size) == (kb, vb, R, 64, 64)
    assert (not s.k_sb) == (kb == 16)               # NULL (ctypes reads it back as None) for bf16


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says so,
    before touching a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_static_decode_validation(lib, monkeypatch):
    """The allocation-free decode read validates like kvq_attn_decode and refuses a
    read whose partials exceed its static scratch, before touching the GPU."""
    c = cache(head_dim=100)
    assert lib.kvq_attn_decode_static(ctypes.byref(c), FAKE, 8, FAKE, 4096, 1.0, FAKE, None) == 2
    c = cache()
    assert lib.kvq_attn_decode_static(ctypes.byref(c), None, 8, FAKE, 4096, 1.0, FAKE, None) == 1
    monkeypatch.setenv("KVQ_SPLITS", "128")
    c = cache(batch=64, n_kv_heads=1, head_dim=512, k_bits=8, v_bits=8, capacity=32768, window=0)
    assert lib.kvq_attn_decode_static(ctypes.byref(c), FAKE, 8, FAKE, 32768, 1.0, FAKE, None) == 4
    assert "static scratch" in lib.kvq_last_error().decode()
