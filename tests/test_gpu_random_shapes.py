"""Seeded random shapes through every read against the fp64 oracle.

Each case draws, from its own seed: head_dim (any multiple of 64 up to 512;
a bf16 cache a multiple of 128), K and V widths (4 or 8 each, or a bf16 cache), KV heads and query heads per KV head, batch,
window (full or a random width) and ring capacity (a multiple of 8, at least
32, large enough for the read), a length, and the call: decode, fused decode
step, or a chunk of 2..80 queries.  The GPU appends its own cache (codes
bit-exact with the oracle's, checked here too) and every output must be
within the attention tolerance (max-abs 1e-2, mean-abs 1e-3) of the oracle."""
import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
import oracle
from kvq_testutil import assert_cache_equal, assert_close, torch_bf16_to_f64
from synth import small_q_bits, small_randn
from test_gpu_attention import q_dev

pytestmark = pytest.mark.gpu

N_CASES = 128


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128, 192, 256, 320, 384, 448, 512]))
    if rng.random() < 0.2 and D % 128 == 0:
        kb = vb = 16
    else:
        kb, vb = int(rng.choice([4, 8])), int(rng.choice([4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    hpk = int(rng.choice([1, 2, 4, 8, 12]))
    B = int(rng.integers(1, 4))
    call = str(rng.choice(["decode", "step", "chunk"]))
    C = int(rng.choice([2, 5, 17, 33, 80])) if call == "chunk" else 1
    L = int(rng.integers(C, 1400))
    if rng.random() < 0.5:
        W = 0
        R = int(np.ceil((L + 1) / 8)) * 8 + 8 * int(rng.integers(0, 4))
    else:
        W = int(rng.integers(1, 700))
        R = max(32, int(np.ceil((W + C - 1) / 8)) * 8 + 8 * int(rng.integers(0, 3)))
    R = max(R, 32)
    return dict(D=D, kb=kb, vb=vb, Hkv=Hkv, Hq=Hkv * hpk, B=B, call=call, C=C, L=L, W=W, R=R)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    c = draw(seed)
    print(f"random case {seed}: {c}", flush=True)
    B, Hkv, Hq, D, kb, vb, R, W, L, C = (c[k] for k in ("B", "Hkv", "Hq", "D", "kb", "vb", "R", "W", "L", "C"))
    g = kvq.KVCache(B, Hkv, D, kb, vb, R, window=W)
    o = oracle.Cache(B, Hkv, D, R, kb, vb, window=W)
    hist = L - 1 if c["call"] == "step" else L
    k = small_randn(7 * seed + 1, (B, Hkv, max(hist, 1), D), D ** -0.25)
    v = small_randn(7 * seed + 2, (B, Hkv, max(hist, 1), D), D ** -0.25)
    for t0 in range(0, hist, 257):
        t1 = min(hist, t0 + 257)
        pos0 = np.full(B, t0, np.int32)
        kvq.kvq_append_quantize(g, torch.from_numpy(k[:, :, t0:t1].copy()).cuda(),
                                torch.from_numpy(v[:, :, t0:t1].copy()).cuda(), torch.from_numpy(pos0).cuda())
        o.append(k[:, :, t0:t1], v[:, :, t0:t1], pos0)
    lens = np.full(B, L, np.int32)
    lens_d = torch.from_numpy(lens).cuda()
    if c["call"] == "step":
        kn = small_randn(7 * seed + 3, (B, Hkv, D), D ** -0.25)
        vn = small_randn(7 * seed + 4, (B, Hkv, D), D ** -0.25)
        qb = small_q_bits(7 * seed + 5, (B, Hq, D), D ** -0.25)
        out = kvq.kvq_decode_step(g, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), q_dev(qb), lens_d, L)
        torch.cuda.synchronize()
        o.append(kn[:, :, None], vn[:, :, None], lens - 1)
        ref = o.attend(qb[:, :, None], lens)[:, :, 0]
    elif c["call"] == "decode":
        qb = small_q_bits(7 * seed + 5, (B, Hq, 1, D), D ** -0.25)
        out = kvq.kvq_attn_decode(g, q_dev(qb[:, :, 0].copy()), lens_d, L)
        torch.cuda.synchronize()
        ref = o.attend(qb, lens)[:, :, 0]
    else:
        qb = small_q_bits(7 * seed + 5, (B, Hq, C, D), D ** -0.25)
        out = kvq.kvq_attn_prefill_chunk(g, q_dev(qb), lens_d, L)
        torch.cuda.synchronize()
        ref = o.attend(qb, lens)
    assert_cache_equal(g, o)              # codes (or bf16 values) written by the GPU, bit for bit
    assert_close(torch_bf16_to_f64(out), ref, f"random case {seed} {c}")


@pytest.mark.parametrize("dims", [(64, 192), (320, 448), (384, 256)])
def test_shared_launch_mixed_head_dims(dims):
    """One shared call over two caches of other head_dims (two layers on the first,
    one on the second), each layer against the oracle."""
    B, L = 2, 900
    groups, refs = [], []
    lens = np.full(B, L, np.int32)
    lens_d = torch.from_numpy(lens).cuda()
    for i, D in enumerate(dims):
        H, W = (2, 256) if i == 0 else (1, 0)
        R = W + 8 if W else (L + 7) // 8 * 8
        kb, vb = (4, 8) if i == 0 else (8, 4)
        k = small_randn(5000 + D, (B, H, L, D), D ** -0.25)
        v = small_randn(5001 + D, (B, H, L, D), D ** -0.25)
        g = kvq.KVCache(B, H, D, kb, vb, R, window=W)
        o = oracle.Cache(B, H, D, R, kb, vb, window=W)
        kvq.kvq_append_quantize(g, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                                torch.zeros(B, dtype=torch.int32, device="cuda"))
        o.append(k, v, np.zeros(B, np.int32))
        qs = [small_q_bits(5002 + D + j, (B, 4 * H, 1, D), D ** -0.25) for j in range(2 - i)]
        groups.append(kvq.SharedGroup(g, [q_dev(x[:, :, 0].copy()) for x in qs], lens_d, L))
        refs.append([o.attend(x, lens)[:, :, 0] for x in qs])
    print(f"shared head_dims {dims}", flush=True)
    outs = kvq.kvq_attn_decode_shared(groups)
    torch.cuda.synchronize()
    for res, ref in zip(outs, refs):
        for out, r in zip(res, ref):
            assert_close(torch_bf16_to_f64(out), r, f"shared {dims}")
