"""Degenerate and extreme inputs through the GPU reads, against the oracle.

  * q = 0: every visible key gets the same weight (the plain mean of the values);
  * a large SDPA scale (30): logits spread over hundreds, so the running max of
    the online softmax moves many times and the lazy rescale must follow;
  * identical keys: equal logits, the mean of the visible values;
  * a window of 1: each query sees only its own key;
  * a window of 1 on a chunk (3 and 100 queries): every row sees only itself;
  * the large scale on chunks of 8 and 96 queries (every chunk path).
Each on 4/8-bit and bf16 caches; outputs within the attention tolerance of the
fp64 oracle (max-abs 1e-2, mean-abs 1e-3)."""
import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
import oracle
from kvq_testutil import assert_close, torch_bf16_to_f64
from synth import small_q_bits, small_randn
from test_gpu_attention import q_dev

pytestmark = pytest.mark.gpu

BITS = [(4, 8), (8, 8), (16, 16)]


def build(B, H, D, kb, vb, R, W, k, v):
    g = kvq.KVCache(B, H, D, kb, vb, R, window=W)
    o = oracle.Cache(B, H, D, R, kb, vb, window=W)
    L = k.shape[2]
    for t0 in range(0, L, 200):
        t1 = min(L, t0 + 200)
        pos0 = np.full(B, t0, np.int32)
        kvq.kvq_append_quantize(g, torch.from_numpy(k[:, :, t0:t1].copy()).cuda(),
                                torch.from_numpy(v[:, :, t0:t1].copy()).cuda(), torch.from_numpy(pos0).cuda())
        o.append(k[:, :, t0:t1], v[:, :, t0:t1], pos0)
    return g, o



def decode_check(g, o, q_bits, L, scale, what):
    B = q_bits.shape[0]
    lens = np.full(B, L, np.int32)
    out = kvq.kvq_attn_decode(g, q_dev(q_bits[:, :, 0].copy()), torch.from_numpy(lens).cuda(), L, scale=scale)
    torch.cuda.synchronize()
    ref = o.attend(q_bits, lens, scale=scale)[:, :, 0]
    assert_close(torch_bf16_to_f64(out), ref, what)
    return ref


@pytest.mark.parametrize("bits", BITS)
def test_zero_query_is_the_mean(bits):
    kb, vb = bits
    B, Hq, H, D, R, L = 2, 8, 2, 256, 1024, 700
    k = small_randn(901, (B, H, L, D), 0.25)
    v = small_randn(902, (B, H, L, D), 0.25)
    g, o = build(B, H, D, kb, vb, R, 0, k, v)
    q = np.zeros((B, Hq, 1, D), np.uint16)
    ref = decode_check(g, o, q, L, 1.0, f"q = 0 bits={bits}")
    mean = o.dequant_v()[:, :, :L].mean(axis=2)                  # [B][H][D]
    np.testing.assert_allclose(ref, np.repeat(mean, Hq // H, axis=1), atol=1e-12)


@pytest.mark.parametrize("window", [512, 0])
@pytest.mark.parametrize("bits", BITS)
def test_large_scale_moves_the_running_max(bits, window):
    kb, vb = bits
    B, Hq, H, D, L = 2, 8, 2, 256, 2600
    R = 640 if window else 2688
    # logits grow along the positions, so later keys keep raising the max
    ramp = np.linspace(0.0, 1.0, L, dtype=np.float32)[None, None, :, None]
    k = small_randn(903, (B, H, L, D), 0.25) + 0.3 * ramp
    v = small_randn(904, (B, H, L, D), 0.25)
    g, o = build(B, H, D, kb, vb, R, window, k, v)
    q = small_q_bits(905, (B, Hq, 1, D), 0.25)
    decode_check(g, o, q, L, 30.0, f"scale 30 W={window} bits={bits}")
    lens = np.full(B, L, np.int32)
    # 8 queries (32 rows: the short-chunk kernel on the full cache, the split read
    # on the window) and 96 (384 rows: the prefill kernel), all against the exact
    # oracle.
    for C in (8, 96):
        qc = small_q_bits(913 + C, (B, Hq, C, D), 0.25)
        out = kvq.kvq_attn_prefill_chunk(g, q_dev(qc), torch.from_numpy(lens).cuda(), L, scale=30.0)
        torch.cuda.synchronize()
        assert_close(torch_bf16_to_f64(out), o.attend(qc, lens, scale=30.0), f"scale 30 chunk C={C} W={window} bits={bits}")



@pytest.mark.parametrize("bits", BITS)
def test_identical_keys(bits):
    kb, vb = bits
    B, Hq, H, D, R, L = 1, 8, 1, 512, 512, 400
    k = np.repeat(small_randn(906, (B, H, 1, D), 0.21), L, axis=2)
    v = small_randn(907, (B, H, L, D), 0.21)
    g, o = build(B, H, D, kb, vb, R, 0, k, v)
    q = small_q_bits(908, (B, Hq, 1, D), 0.21)
    decode_check(g, o, q, L, 1.0, f"identical keys bits={bits}")


@pytest.mark.parametrize("bits", BITS)
def test_window_of_one(bits):
    kb, vb = bits
    B, Hq, H, D, R, L = 2, 8, 2, 256, 128, 300
    k = small_randn(909, (B, H, L, D), 0.25)
    v = small_randn(910, (B, H, L, D), 0.25)
    g, o = build(B, H, D, kb, vb, R, 1, k, v)
    q = small_q_bits(911, (B, Hq, 1, D), 0.25)
    ref = decode_check(g, o, q, L, 1.0, f"window 1 bits={bits}")
    np.testing.assert_allclose(ref, np.repeat(o.dequant_v()[:, :, (L - 1) % R], Hq // H, axis=1), atol=1e-12)
    lens = np.full(B, L, np.int32)
    for C in (3, 100):                                         # 12 rows: the split read; 400: the band path
        qc = small_q_bits(912 + C, (B, Hq, C, D), 0.25)
        out = kvq.kvq_attn_prefill_chunk(g, q_dev(qc), torch.from_numpy(lens).cuda(), L)
        torch.cuda.synchronize()
        assert_close(torch_bf16_to_f64(out), o.attend(qc, lens), f"window 1 chunk C={C} bits={bits}")
