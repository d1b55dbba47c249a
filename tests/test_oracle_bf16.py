"""Pins for the oracle's unquantized bf16 caches.

The pages (@mlx-bun/inference 0.0.0-stage -> 1.0.0 diff, page 80,
gemma4/model.ts, note on cacheLayers) keep the sliding layers' caches in bf16
under the model's other KV scheme: a ring of the window, read by the same SDPA.
Such a cache stores each fp32 key and value rounded to the nearest bf16.  Pins,
none of them the oracle's own code:
  * the rounding: hand-worked examples (tests/golden/bf16_rounding_examples.txt:
    ties to even, carries into the exponent, subnormals, signs) and torch's own
    float32 -> bfloat16 conversion (round to nearest even) on random and
    tie-heavy values;
  * the append: ring storage equals linear storage, and T > R keeps the last R;
  * the read: torch's scaled_dot_product_attention in float64 on the rounded
    values (a library routine; the read adds no rounding of its own), decode and
    chunks, full and windowed, GQA, with ring wrap; a cache with bf16 keys and
    8-bit values against the same routine on the 8-bit values' exact
    dequantization.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import small_q_bits, small_randn
from test_oracle_attention import bf16_to_f64, dense_reference

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rounding_examples.txt")


def golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        x, h, _ = [p.strip() for p in line.split("|", 2)]
        rows.append((int(x, 16), int(h, 16)))
    return rows


def test_bf16_rounding_worked_examples():
    rows = golden_rows()
    assert len(rows) >= 10
    for xbits, hbits in rows:
        x = np.array([xbits], np.uint32).view(np.float32)[0]
        assert oracle.bf16(x) == hbits, f"{xbits:#010x}: got {oracle.bf16(x):#06x}, expected {hbits:#06x}"


def torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy()
    return t.view(np.uint16)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 0.25,
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        (rng.standard_normal(5000) * 1e-30).astype(np.float32),
        # exact ties: a random bf16 value plus half its last place
        ((rng.integers(0, 1 << 15, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
        ((rng.integers(0, 1 << 15, 5000).astype(np.uint32) << 16) | 0x80008000).view(np.float32),
    ])
    x = x[np.isfinite(x) & (np.abs(x) <= 1e38)]
    B, H, D, R = 1, 1, 64, 1
    want = torch_bf16_bits(x)
    # through the cache append (one token per 64 values)
    n = (x.size // D) * D
    c = oracle.Cache(1, 1, D, n // D, 16, 16)
    k = x[:n].reshape(1, 1, n // D, D)
    c.append(k, k, np.zeros(1, np.int32))
    assert (c.k_vals.reshape(-1) == want[:n]).all()
    assert (c.v_vals.reshape(-1) == want[:n]).all()
    for i in range(0, x.size, 997):
        assert oracle.bf16(x[i]) == want[i]


def test_bf16_append_ring_and_overflow():
    B, H, D, R = 2, 2, 64, 16
    rng_k = small_randn(11, (B, H, 40, D), 0.25)
    rng_v = small_randn(12, (B, H, 40, D), 0.25)
    ring = oracle.Cache(B, H, D, R, 16, 16, window=R)
    pos = 0
    for T in (5, 9, 3, 7, 16):
        ring.append(rng_k[:, :, pos:pos + T], rng_v[:, :, pos:pos + T], np.full(B, pos, np.int32))
        pos += T
    # linear storage of the same 40 tokens: slot j mod R holds the last write of position j
    want_k = torch_bf16_bits(rng_k.reshape(-1)).reshape(rng_k.shape)
    want_v = torch_bf16_bits(rng_v.reshape(-1)).reshape(rng_v.shape)
    for j in range(pos - R, pos):
        assert (ring.k_vals[:, :, j % R] == want_k[:, :, j]).all()
        assert (ring.v_vals[:, :, j % R] == want_v[:, :, j]).all()
    # T > R in one call keeps the last R tokens
    one = oracle.Cache(B, H, D, R, 16, 16, window=R)
    one.append(rng_k, rng_v, np.zeros(B, np.int32))
    assert (one.k_vals == ring.k_vals).all() and (one.v_vals == ring.v_vals).all()
    # an input outside the domain is rejected before anything is written
    bad = rng_k[:, :, :2].copy()
    bad[1, 1, 1, 3] = np.inf
    fresh = oracle.Cache(B, H, D, R, 16, 16)
    with pytest.raises(oracle.OracleError):
        fresh.append(bad, bad, np.zeros(B, np.int32))
    assert not fresh.k_vals.any()


CASES = [
    # B, Hq, Hkv, D, R, W, len, C
    (2, 8, 2, 256, 512, 512, 1300, 1),    # sliding decode, ring wrap
    (1, 8, 1, 128, 200, 0, 200, 1),       # full decode
    (2, 4, 2, 64, 64, 24, 100, 17),       # chunk, window, ring
    (1, 6, 3, 192, 80, 0, 80, 9),         # chunk, full
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_bf16_attention_equals_sdpa_on_rounded_values(case):
    B, Hq, Hkv, D, R, W, L, C = case
    k = small_randn(sum(case), (B, Hkv, L, D), D ** -0.25)
    v = small_randn(sum(case) + 1, (B, Hkv, L, D), D ** -0.25)
    q = small_q_bits(sum(case) + 2, (B, Hq, C, D), D ** -0.25)
    c = oracle.Cache(B, Hkv, D, R, 16, 16, window=W)
    for t0 in range(0, L, 37):
        t1 = min(L, t0 + 37)
        c.append(k[:, :, t0:t1], v[:, :, t0:t1], np.full(B, t0, np.int32))
    # ragged lengths only where no slot a shorter sequence reads was rewritten
    ragged = W == 0 and R >= L
    lens = np.array([L - (b % 2) * 3 * ragged for b in range(B)], np.int32)
    got = c.attend(q, lens)
    k64 = bf16_to_f64(torch_bf16_bits(k.reshape(-1)).reshape(k.shape))
    v64 = bf16_to_f64(torch_bf16_bits(v.reshape(-1)).reshape(v.shape))
    ref = dense_reference(bf16_to_f64(q), k64, v64, lens, C, W, 1.0)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_bf16_keys_with_8bit_values():
    B, Hq, Hkv, D, R, L = 1, 4, 1, 128, 96, 90
    k = small_randn(31, (B, Hkv, L, D), D ** -0.25)
    v = small_randn(32, (B, Hkv, L, D), D ** -0.25)
    q = small_q_bits(33, (B, Hq, 1, D), D ** -0.25)
    c = oracle.Cache(B, Hkv, D, R, 16, 8)
    c.append(k, v, np.zeros(B, np.int32))
    lens = np.array([L], np.int32)
    k64 = bf16_to_f64(torch_bf16_bits(k.reshape(-1)).reshape(k.shape))
    v64 = c.dequant_v()[:, :, :L]
    ref = dense_reference(bf16_to_f64(q), k64, v64, lens, 1, 0, 1.0)
    np.testing.assert_allclose(c.attend(q, lens), ref, rtol=0, atol=1e-12)
