"""GPU normed append (kvq_append_norm_quantize) against the oracle's normed
append: the normed rows (k_out, v_out) and the cache's codes, scales and biases
bit for bit [page 80, gemma4/model.ts attentionTraining: kNorm, the rotation at
cache positions, vNorm, appendWindow]."""
import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
import oracle
from kvq_testutil import assert_cache_equal
from synth import small_randn

pytestmark = pytest.mark.gpu

F32 = np.float32


def _table(seed, positions, rope_dims):
    rng = np.random.default_rng(seed)
    inv = 10000.0 ** (-np.arange(rope_dims // 2) / max(rope_dims // 2, 1))
    ang = np.arange(positions)[:, None] * inv[None, :] + rng.uniform(0, 0.1, (1, rope_dims // 2))
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def _rows(seed, shape):
    """Rows of mixed magnitudes (each row its own scale over 12 decades)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * 10.0 ** rng.uniform(-6, 6, shape[:-1] + (1,))
    return x.astype(F32)


def _run(g, o, k, v, pos0, w, eps, rope, same_kv=False):
    B, H, T, D = k.shape
    print(f"normed append D={D} T={T} pos0={list(pos0)} rope={None if rope is None else 2 * rope[0].shape[1]} "
          f"bits={g.k_bits}/{g.v_bits}", flush=True)
    kt = torch.from_numpy(k).cuda()
    vt = kt if same_kv else torch.from_numpy(v).cuda()
    ko = torch.full_like(kt, float("nan"))
    vo = torch.full_like(kt, float("nan"))
    rt = None if rope is None else (torch.from_numpy(rope[0]).cuda(), torch.from_numpy(rope[1]).cuda())
    wt = None if w is None else torch.from_numpy(w).cuda()
    p = np.asarray(pos0, np.int32)
    kvq.kvq_append_norm_quantize(g, kt, vt, torch.from_numpy(p).cuda(), wt, eps, rope=rt, k_out=ko, v_out=vo)
    kn, vn = oracle.append_normed(o, k, k if same_kv else v, p, w, eps, rope=rope)
    torch.cuda.synchronize()
    n = min(T, g.capacity)
    kg, vg = ko.cpu().numpy(), vo.cpu().numpy()
    for what, got, want in (("keys", kg, kn), ("values", vg, vn)):
        bad = np.argwhere(got[:, :, T - n:].view(np.uint32) != want[:, :, T - n:].view(np.uint32))
        assert len(bad) == 0, (f"normed {what} differ at {len(bad)} places, first {bad[:4].tolist()}: "
                               f"{[float(got[tuple(i[:2]) + (i[2] + T - n, i[3])]) for i in bad[:4]]} vs "
                               f"{[float(want[tuple(i[:2]) + (i[2] + T - n, i[3])]) for i in bad[:4]]}")
    assert np.isnan(kg[:, :, :T - n]).all() and np.isnan(vg[:, :, :T - n]).all(), "rows past the ring were written"
    assert_cache_equal(g, o)


HEAD_DIMS = [64, 128, 192, 256, 320, 384, 448, 512]


@pytest.mark.parametrize("D", HEAD_DIMS)
@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4), (4, 8), (8, 8), (16, 16)])
def test_normed_append_bitexact(D, kb, vb):
    if kb == 16 and D % 128:
        pytest.skip("bf16 caches take head_dim multiples of 128")
    B, H, R = 2, 2, 64
    g = kvq.KVCache(B, H, D, kb, vb, R, window=R)
    o = oracle.Cache(B, H, D, R, kb, vb, window=R)
    rng = np.random.default_rng(D * 10 + kb)
    w = (rng.standard_normal(D) * 0.5 + 1.0).astype(F32)
    pos = np.array([0, 5], np.int32)
    for i, (T, rope_dims) in enumerate([(1, D), (7, D // 4), (37, 2), (1, 0), (70, D - 2), (9, D // 2 + 6)]):
        rope = None if rope_dims == 0 else _table(i, 512, rope_dims)
        k = _rows(100 * D + i, (B, H, T, D))
        v = _rows(200 * D + i, (B, H, T, D))
        _run(g, o, k, v, pos, w if i % 3 else None, [1e-6, 0.0, 1e-2][i % 3], rope)
        pos = pos + T


def test_normed_append_shared_projection_and_windowed_ring():
    """Keys and values from one tensor (the shared-projection case), a windowed
    ring that wraps, and T > R (only the last R tokens are normed and written)."""
    B, H, D, R = 3, 2, 256, 40
    g = kvq.KVCache(B, H, D, 4, 8, R, window=32)
    o = oracle.Cache(B, H, D, R, 4, 8, window=32)
    w = (np.random.default_rng(1).standard_normal(D) + 1.0).astype(F32)
    rope = _table(3, 400, D)
    pos = np.array([3, 17, 33], np.int32)
    for i, T in enumerate([1, 29, R + 11, 1, 8]):
        k = _rows(50 + i, (B, H, T, D))
        _run(g, o, k, None, pos, w, 1e-6, rope, same_kv=True)
        pos = pos + T


def test_normed_append_special_rows():
    """Constant rows, a row with one nonzero value, a row near the bottom of the
    normal range (about a third of it subnormal) with eps 0, and rows near the
    input limit."""
    B, H, D, R = 1, 1, 512, 32
    rows = [np.full(D, 0.125, F32), np.full(D, -3.0, F32), np.eye(1, D, 7, dtype=F32)[0] * F32(-2.5),
            (small_randn(1, (D,), 1.0) * 3e-38).astype(F32), (small_randn(2, (D,), 1.0) * 1e37).astype(F32),
            np.linspace(-1e38, 1e38, D).astype(F32), small_randn(3, (D,), 1e-20), np.arange(D, dtype=F32) - 255.5]
    k = np.stack(rows)[None, None]
    v = np.ascontiguousarray(k[:, :, ::-1])
    rope = _table(9, 16, 128)
    g = kvq.KVCache(B, H, D, 8, 4, R)
    o = oracle.Cache(B, H, D, R, 8, 4)
    _run(g, o, k, v, [2], np.linspace(0.5, 1.5, D).astype(F32), 0.0, rope)


def test_normed_append_matches_norm_then_plain_append():
    """The fused call writes the same cache as the plain append of rows normed and
    rotated elsewhere (the oracle's), on a model-sized step: 16 sequences, 1 token."""
    B, H, D, R = 16, 1, 512, 4096
    g1 = kvq.KVCache(B, H, D, 4, 4, R)
    g2 = kvq.KVCache(B, H, D, 4, 4, R)
    k = _rows(5, (B, H, 1, D))
    v = _rows(6, (B, H, 1, D))
    w = (np.random.default_rng(2).standard_normal(D) + 1.0).astype(F32)
    rope = _table(4, R, 128)
    pos0 = np.random.default_rng(7).integers(0, R, B).astype(np.int32)
    kn = oracle.norm_rows(k, w, 1e-6, rope, (pos0[:, None, None] + np.zeros((1, H, 1), np.int64)).astype(np.int32))
    vn = oracle.norm_rows(v, None, 1e-6)
    p = torch.from_numpy(pos0).cuda()
    kvq.kvq_append_norm_quantize(g1, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), p,
                                 torch.from_numpy(w).cuda(), 1e-6,
                                 rope=(torch.from_numpy(rope[0]).cuda(), torch.from_numpy(rope[1]).cuda()))
    kvq.kvq_append_quantize(g2, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), p)
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes", "k_sb", "v_sb"):
        assert torch.equal(getattr(g1, name), getattr(g2, name)), name


def test_normed_append_argument_errors():
    g = kvq.KVCache(1, 1, 128, 4, 4, 32)
    k = torch.zeros(1, 1, 1, 128, device="cuda")
    p = torch.zeros(1, dtype=torch.int32, device="cuda")
    cos = torch.ones(4, 3, device="cuda")
    with pytest.raises(kvq.KvqError):
        kvq.kvq_append_norm_quantize(g, k, k, p, None, -1.0)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_append_norm_quantize(g, k, k, p, None, float("inf"))
    with pytest.raises(kvq.KvqError):                      # rope_dims 6 fine, but 130 > head_dim
        kvq.kvq_append_norm_quantize(g, k, k, p, None, 1e-6, rope=(torch.ones(4, 65, device="cuda"),) * 2)
    kvq.kvq_append_norm_quantize(g, k, k, p, None, 1e-6, rope=(cos, cos))
    torch.cuda.synchronize()
