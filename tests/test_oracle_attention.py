"""Pins for the oracle's attention, independent of the oracle's own code.

The pages (@mlx-bun/inference 0.0.0-stage -> 1.0.0 diff, page 80, model.ts header
notes and attentionTraining) fix: SDPA with scale 1.0 over the layer's cache,
GQA (several query heads per KV head; full layers have one KV head of width 512),
causal reads, sliding layers reading a rotating cache that owns the window, and
KV-sharing layers reading a donor's cache.  Pins used here:
  * grid-exact caches (quantization is lossless) must reproduce torch's
    scaled_dot_product_attention in float64 on the original values (a library
    routine), for decode and chunked prefill, full and windowed, with ring wrap;
  * closed forms: a window of 1 returns the current value row; identical keys or
    q = 0 give the plain mean of the visible values; a dominant logit returns
    its value row;
  * invariants: GQA == MHA with repeated KV heads; a window >= length == full;
    decode at p == row p of a prefill; ring storage == linear storage;
    shared layers == separate reads;
  * the 8-bit error bound: |o_q - o| <= (exp(2*delta) - 1) max|v| + max s_v/2.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import small_q_bits, small_randn


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def grid_values(rng, shape, bits, sigma):
    """fp32 values on an exact per-group grid c*s + b with bf16 s and b."""
    n = (1 << bits) - 1
    B, H, T, D = shape
    G = D // 64
    E = 8 if bits == 8 else 5
    s_int = rng.integers(160, 256, (B, H, T, G, 1))
    s = s_int * 2.0 ** -(E + int(np.round(-np.log2(sigma))) + 2)
    b = -(rng.integers(100, 256, (B, H, T, G, 1)) * 2.0 ** -(8 + int(np.round(-np.log2(sigma)))))
    codes = rng.integers(0, n + 1, (B, H, T, G, 64))
    codes[..., 0] = 0
    codes[..., 1] = n
    x = (codes * s + b).reshape(B, H, T, D)
    x32 = x.astype(np.float32)
    assert (x32.astype(np.float64) == x).all()
    return x32


def dense_reference(q64, k64, v64, len_, C, W, scale):
    """torch SDPA (float64, CPU) over linear K/V [B][Hkv][L][D] with the causal/window mask."""
    B, Hq, _, D = q64.shape
    Hkv = k64.shape[1]
    L = k64.shape[2]
    out = np.zeros(q64.shape)
    for b in range(B):
        n = int(len_[b])
        p = np.arange(n - C, n)[:, None]
        j = np.arange(n)[None, :]
        mask = j <= p
        if W:
            mask &= j > p - W
        kk = torch.from_numpy(np.repeat(k64[b:b + 1, :, :n], Hq // Hkv, axis=1))
        vv = torch.from_numpy(np.repeat(v64[b:b + 1, :, :n], Hq // Hkv, axis=1))
        qq = torch.from_numpy(q64[b:b + 1])
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=torch.from_numpy(mask)[None, None], scale=scale)
        out[b] = o[0].numpy()
        assert L >= n
    return out


CASES = [
    # B, Hq, Hkv, D, kb, vb, R, W, L(len), C
    (1, 8, 2, 256, 4, 4, 128, 0, 128, 1),
    (2, 8, 2, 128, 4, 8, 64, 64, 300, 1),      # ring wrap, window == R
    (2, 8, 1, 512, 8, 8, 96, 0, 90, 1),
    (2, 4, 2, 64, 8, 4, 64, 24, 100, 17),      # prefill, window, ring
    (1, 6, 3, 192, 4, 4, 80, 0, 80, 9),        # prefill, full
]


@pytest.mark.parametrize("case", CASES)
def test_grid_exact_matches_torch_sdpa(case):
    B, Hq, Hkv, D, kb, vb, R, W, L, C = case
    rng = np.random.default_rng(sum(case))
    sigma = D ** -0.25
    k = grid_values(rng, (B, Hkv, L, D), kb, sigma)
    v = grid_values(rng, (B, Hkv, L, D), vb, sigma)
    q = small_q_bits(sum(case), (B, Hq, C, D), sigma)
    cache = oracle.Cache(B, Hkv, D, R, kb, vb, window=W)
    for t0 in range(0, L, 37):                 # uneven append chunks
        t1 = min(L, t0 + 37)
        cache.append(k[:, :, t0:t1], v[:, :, t0:t1], np.full(B, t0, np.int32))
    len_ = np.full(B, L, np.int32)
    got = cache.attend(q, len_, 1.0)
    ref = dense_reference(bf16_to_f64(q), k.astype(np.float64), v.astype(np.float64), len_, C, W, 1.0)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_scale_argument():
    B, Hq, Hkv, D, L = 1, 2, 1, 64, 20
    rng = np.random.default_rng(3)
    k = grid_values(rng, (B, Hkv, L, D), 8, 0.5)
    v = grid_values(rng, (B, Hkv, L, D), 8, 0.5)
    q = small_q_bits(3, (B, Hq, 1, D), 0.5)
    cache = oracle.Cache(B, Hkv, D, 32, 8, 8)
    cache.append(k, v, np.zeros(B, np.int32))
    len_ = np.array([L], np.int32)
    got = cache.attend(q, len_, 0.37)
    ref = dense_reference(bf16_to_f64(q), k.astype(np.float64), v.astype(np.float64), len_, 1, 0, 0.37)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _random_cache(seed, B, Hkv, D, R, W, L, kb=4, vb=8):
    k = small_randn(seed, (B, Hkv, L, D), D ** -0.25)
    v = small_randn(seed + 1, (B, Hkv, L, D), D ** -0.25)
    c = oracle.Cache(B, Hkv, D, R, kb, vb, window=W)
    c.append(k, v, np.zeros(B, np.int32))
    return c, k, v


def test_window_one_returns_current_value():
    c, _, _ = _random_cache(11, 2, 2, 128, 16, 1, 40)
    q = small_q_bits(12, (2, 4, 1, 128), 0.3)
    out = c.attend(q, np.array([40, 40], np.int32))
    vh = c.dequant_v()
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[b, h, 0], vh[b, h // 2, 39 % 16])


def test_zero_query_is_window_mean():
    B, Hkv, D, R, W, L = 2, 1, 64, 48, 20, 100
    c, _, _ = _random_cache(21, B, Hkv, D, R, W, L)
    q = np.zeros((B, 3, 1, D), np.uint16)
    len_ = np.array([L, L - 7], np.int32)      # b=1 queries an earlier position
    out = c.attend(q, len_)
    vh = c.dequant_v()
    for b in range(B):
        p = int(len_[b]) - 1
        slots = [j % R for j in range(max(0, p - W + 1), p + 1)]
        np.testing.assert_allclose(out[b, :, 0], np.broadcast_to(vh[b, 0, slots].mean(0), (3, D)), atol=1e-13)


def test_identical_keys_give_mean():
    B, Hkv, D, R, L = 1, 1, 128, 64, 50
    k = np.broadcast_to(small_randn(31, (1, 1, 1, D), 0.3), (B, Hkv, L, D)).copy()
    v = small_randn(32, (B, Hkv, L, D), 0.3)
    c = oracle.Cache(B, Hkv, D, R, 8, 4)
    c.append(k, v, np.zeros(B, np.int32))
    q = small_q_bits(33, (B, 2, 1, D), 0.3)
    out = c.attend(q, np.array([L], np.int32))
    vh = c.dequant_v()
    np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(vh[0, 0, :L].mean(0), (2, D)), atol=1e-13)


def test_dominant_logit_selects_row():
    B, Hkv, D, R, L = 1, 1, 64, 32, 20
    k = np.zeros((B, Hkv, L, D), np.float32)
    k[0, 0, 7, :] = 4.0                       # q.k = 64*4*0.25 = 64 for key 7, 0 for others
    v = small_randn(41, (B, Hkv, L, D), 0.5)
    c = oracle.Cache(B, Hkv, D, R, 8, 8)
    c.append(k, v, np.zeros(B, np.int32))
    q = np.full((B, 1, 1, D), 0x3E80, np.uint16)  # bf16 0.25
    out = c.attend(q, np.array([L], np.int32))
    vh = c.dequant_v()
    np.testing.assert_allclose(out[0, 0, 0], vh[0, 0, 7], atol=1e-20)


def test_gqa_equals_repeated_mha():
    B, Hkv, rep, D, R, W, L = 2, 2, 4, 128, 64, 40, 90
    k = small_randn(51, (B, Hkv, L, D), 0.3)
    v = small_randn(52, (B, Hkv, L, D), 0.3)
    q = small_q_bits(53, (B, Hkv * rep, 3, D), 0.3)
    g = oracle.Cache(B, Hkv, D, R, 4, 8, window=W)
    g.append(k, v, np.zeros(B, np.int32))
    m = oracle.Cache(B, Hkv * rep, D, R, 4, 8, window=W)
    m.append(np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), np.zeros(B, np.int32))
    len_ = np.array([L, L - 5], np.int32)
    # b=1 shares the cache contents of 90 positions; its len 85 only moves p back
    np.testing.assert_array_equal(g.attend(q, len_), m.attend(q, len_))


def test_big_window_equals_full():
    B, Hkv, D, L = 1, 2, 64, 70
    k = small_randn(61, (B, Hkv, L, D), 0.4)
    v = small_randn(62, (B, Hkv, L, D), 0.4)
    q = small_q_bits(63, (B, 4, 5, D), 0.4)
    a = oracle.Cache(B, Hkv, D, 128, 8, 4, window=0)
    w = oracle.Cache(B, Hkv, D, 128, 8, 4, window=L)
    for c in (a, w):
        c.append(k, v, np.zeros(B, np.int32))
    len_ = np.array([L], np.int32)
    np.testing.assert_array_equal(a.attend(q, len_), w.attend(q, len_))


def test_decode_equals_prefill_rows():
    B, Hkv, D, R, W, L, C = 2, 1, 128, 64, 32, 60, 12
    c, _, _ = _random_cache(71, B, Hkv, D, R, W, L)
    q = small_q_bits(72, (B, 3, C, D), 0.3)
    pre = c.attend(q, np.full(B, L, np.int32))
    for i in range(C):
        dec = c.attend(q[:, :, i:i + 1], np.full(B, L - C + i + 1, np.int32))
        np.testing.assert_array_equal(dec[:, :, 0], pre[:, :, i])


def test_ring_equals_linear():
    B, Hkv, D, W, L = 2, 2, 128, 48, 400
    k = small_randn(81, (B, Hkv, L, D), 0.3)
    v = small_randn(82, (B, Hkv, L, D), 0.3)
    ring = oracle.Cache(B, Hkv, D, W, 4, 4, window=W)
    lin = oracle.Cache(B, Hkv, D, 512, 4, 4, window=W)
    for t0 in range(0, L, 64):
        ring.append(k[:, :, t0:t0 + 64], v[:, :, t0:t0 + 64], np.full(B, t0, np.int32))
    lin.append(k, v, np.zeros(B, np.int32))
    q = small_q_bits(83, (B, 4, 1, D), 0.3)
    len_ = np.full(B, L, np.int32)
    np.testing.assert_array_equal(ring.attend(q, len_), lin.attend(q, len_))


def test_shared_equals_separate():
    c, _, _ = _random_cache(91, 2, 2, 128, 64, 64, 150)
    qs = [small_q_bits(92 + i, (2, 4, 1, 128), 0.3) for i in range(3)]
    len_ = np.full(2, 150, np.int32)
    shared = oracle.attend_shared(c, qs, len_)
    for q, o in zip(qs, shared):
        np.testing.assert_array_equal(o, c.attend(q, len_))


def test_capacity_errors():
    c = oracle.Cache(1, 1, 64, 32, 4, 4, window=24)
    x = np.zeros((1, 1, 40, 64), np.float32)
    c.append(x, x, np.zeros(1, np.int32))
    q = np.zeros((1, 1, 10, 64), np.uint16)
    with pytest.raises(oracle.OracleError) as e:       # needs R >= W - 1 + C = 33
        c.attend(q, np.array([40], np.int32))
    assert e.value.status == 2
    full = oracle.Cache(1, 1, 64, 32, 4, 4, window=0)
    with pytest.raises(oracle.OracleError):            # full cache holds only 32
        full.attend(np.zeros((1, 1, 1, 64), np.uint16), np.array([33], np.int32))


@pytest.mark.parametrize("D", [256, 512])
def test_8bit_error_bound(D):
    """Random (off-grid) 8-bit K/V: the oracle stays within the bound implied by
    |x - xhat| <= s/2 of dense attention on the original values."""
    B, Hkv, Hq, L = 1, 1, 4, 200
    sigma = D ** -0.25
    k = small_randn(101, (B, Hkv, L, D), sigma)
    v = small_randn(102, (B, Hkv, L, D), sigma)
    q = small_q_bits(103, (B, Hq, 1, D), sigma)
    c = oracle.Cache(B, Hkv, D, 256, 8, 8)
    c.append(k, v, np.zeros(B, np.int32))
    len_ = np.array([L], np.int32)
    got = c.attend(q, len_)
    ref = dense_reference(bf16_to_f64(q), k.astype(np.float64), v.astype(np.float64), len_, 1, 0, 1.0)
    ks = bf16_to_f64(c.k_scales[0, 0, :L])            # [L][G]
    vs = bf16_to_f64(c.v_scales[0, 0, :L])
    qa = np.abs(bf16_to_f64(q[0, :, 0]))              # [Hq][D]
    qg = qa.reshape(Hq, D // 64, 64).sum(-1)          # [Hq][G]
    for h in range(Hq):
        delta = (ks * qg[h][None, :] / 2).sum(-1).max()
        bound = (np.exp(2 * delta) - 1) * np.abs(v[0, 0, :L]).max() + vs.max() / 2
        err = np.abs(got[0, h, 0] - ref[0, h, 0]).max()
        assert err <= bound, (err, bound)
    # and the bound is not vacuous: 8-bit attention is close to dense attention
    assert np.abs(got - ref).max() < 0.02
