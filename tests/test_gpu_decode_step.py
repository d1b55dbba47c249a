"""Fused decode step (kvq_decode_step): append the step's token and attend, in one launch.

Checked two ways: the cache it leaves equals, word for word, the cache that
kvq_append_quantize writes for the same token (itself bit-exact with the
oracle, see test_gpu_append); the output is within the attention tolerance
(max-abs 1e-2, mean-abs 1e-3) of the fp64 oracle after the oracle's append."""
import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
import oracle
from kvq_testutil import assert_close, build_workload, torch_bf16_to_f64
from synth import WORKLOADS, small_q_bits, small_randn

pytestmark = pytest.mark.gpu


def q_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def clone_cache(g: kvq.KVCache) -> kvq.KVCache:
    c = kvq.KVCache(g.batch, g.n_kv_heads, g.head_dim, g.k_bits, g.v_bits, g.capacity, window=g.window)
    for src, dst in ((g.k_codes, c.k_codes), (g.v_codes, c.v_codes), (g.k_sb, c.k_sb), (g.v_sb, c.v_sb)):
        dst.copy_(src)
    return c


def assert_same_cache(a: kvq.KVCache, b: kvq.KVCache, what: str):
    for name in ("k_codes", "v_codes", "k_sb", "v_sb"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x, y), f"{what}: {name} differs in {(x != y).sum().item()} words"


def history(B, H, D, kb, vb, R, W, L, seed):
    """GPU and oracle caches holding positions 0 .. L-1 of every sequence."""
    g = kvq.KVCache(B, H, D, kb, vb, R, window=W)
    o = oracle.Cache(B, H, D, R, kb, vb, window=W)
    if L > 0:
        k = small_randn(seed, (B, H, L, D), D ** -0.25)
        v = small_randn(seed + 1, (B, H, L, D), D ** -0.25)
        for t0 in range(0, L, 300):
            t1 = min(L, t0 + 300)
            pos0 = np.full(B, t0, np.int32)
            kvq.kvq_append_quantize(g, torch.from_numpy(k[:, :, t0:t1].copy()).cuda(),
                                    torch.from_numpy(v[:, :, t0:t1].copy()).cuda(), torch.from_numpy(pos0).cuda())
            o.append(k[:, :, t0:t1], v[:, :, t0:t1], pos0)
    return g, o


def one_step(g, o, lens, seed, Hq, what):
    """Run one fused step at positions lens-1; check the cache and the output."""
    B, H, D = g.batch, g.n_kv_heads, g.head_dim
    k = small_randn(seed, (B, H, D), D ** -0.25)
    v = small_randn(seed + 1, (B, H, D), D ** -0.25)
    qb = small_q_bits(seed + 2, (B, Hq, D), D ** -0.25)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    lens_d = torch.from_numpy(lens).cuda()
    ref_cache = clone_cache(g)
    kvq.kvq_append_quantize(ref_cache, kd[:, :, None].contiguous(), vd[:, :, None].contiguous(), lens_d - 1)
    out = kvq.kvq_decode_step(g, kd, vd, q_dev(qb), lens_d, int(lens.max()))
    torch.cuda.synchronize()
    assert_same_cache(g, ref_cache, what)
    o.append(k[:, :, None], v[:, :, None], lens - 1)
    ref = o.attend(qb[:, :, None], lens)[:, :, 0]
    assert_close(torch_bf16_to_f64(out), ref, what)
    return out


STEP_CASES = [
    # B, Hq, Hkv, D, kb, vb, R, W, history length
    (1, 8, 2, 256, 4, 4, 128, 0, 127),
    (2, 8, 2, 256, 4, 8, 512, 512, 1499),     # ring wrap, window = capacity
    (2, 8, 1, 512, 8, 8, 2048, 0, 1999),      # full layer, D512
    (3, 4, 4, 128, 8, 4, 256, 100, 699),      # MHA, window < capacity
    (1, 16, 1, 512, 4, 8, 64, 0, 0),          # the new token is the only key
    (2, 24, 2, 128, 4, 4, 96, 40, 332),       # 12 rows per KV head
    (1, 40, 2, 256, 8, 8, 160, 0, 149),       # 20 rows: two row tiles
    (2, 8, 2, 256, 8, 4, 64, 64, 7),          # short history, ring
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_step_small(case):
    B, Hq, Hkv, D, kb, vb, R, W, L = case
    print(f"decode step {case}", flush=True)
    g, o = history(B, Hkv, D, kb, vb, R, W, L, seed=sum(case))
    # ragged: odd sequences one or two positions behind (their token overwrites a slot)
    lens = np.array([L + 1 - (b % 2) * min(2, L) for b in range(B)], np.int32)
    one_step(g, o, lens, sum(case) + 11, Hq, f"decode step {case}")


def test_decode_step_sequence():
    """Consecutive steps across the ring's wrap, each checked against the oracle."""
    B, Hq, Hkv, D, kb, vb, R, W, L = 2, 8, 2, 256, 4, 8, 64, 48, 50
    print("decode step sequence", flush=True)
    g, o = history(B, Hkv, D, kb, vb, R, W, L, seed=21)
    for t in range(24):
        lens = np.full(B, L + 1 + t, np.int32)
        one_step(g, o, lens, 100 + 3 * t, Hq, f"sequence step {t}")


def test_decode_step_matches_two_calls():
    """The output agrees with append + kvq_attn_decode to the attention tolerance."""
    B, Hq, Hkv, D, R, L = 2, 8, 1, 512, 4096, 3000
    print("decode step vs two calls", flush=True)
    g, _ = history(B, Hkv, D, 8, 8, R, 0, L, seed=31)
    g2 = clone_cache(g)
    k = torch.from_numpy(small_randn(32, (B, Hkv, D), 0.21)).cuda()
    v = torch.from_numpy(small_randn(33, (B, Hkv, D), 0.21)).cuda()
    q = q_dev(small_q_bits(34, (B, Hq, D), 0.21))
    lens = torch.full((B,), L + 1, dtype=torch.int32, device="cuda")
    out = kvq.kvq_decode_step(g, k, v, q, lens, L + 1)
    kvq.kvq_append_quantize(g2, k[:, :, None].contiguous(), v[:, :, None].contiguous(), lens - 1)
    out2 = kvq.kvq_attn_decode(g2, q, lens, L + 1)
    torch.cuda.synchronize()
    assert_same_cache(g, g2, "two calls")
    d = (torch_bf16_to_f64(out) - torch_bf16_to_f64(out2))
    assert np.abs(d).max() <= 1e-2 and np.abs(d).mean() <= 1e-3


@pytest.mark.parametrize("name", ["sliding_decode_b8_w512", "decode_b1_l128"])
def test_decode_step_workload(name):
    wl = WORKLOADS[name]
    print(f"decode step workload {name}", flush=True)
    gpu, orc, _, _ = build_workload(wl)
    spec = wl.caches[0]
    o, _ = orc["kv"]
    # the step's token is the last position of the workload (it rewrites that slot)
    lens = np.full(spec.B, spec.length, np.int32)
    one_step(gpu["kv"], o, lens, 77, wl.queries[0].Hq, name)


def test_decode_step_rejects_bad_arguments():
    g = kvq.KVCache(1, 2, 256, 4, 4, 64)
    k = torch.zeros(1, 2, 256, device="cuda")
    q = torch.zeros(1, 8, 256, dtype=torch.bfloat16, device="cuda")
    lens = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError):
        kvq.kvq_decode_step(g, k, k, q, lens, 65)               # full layer cannot hold 65
    with pytest.raises(kvq.KvqError):
        kvq.kvq_decode_step(g, k, k, torch.zeros(1, 3, 256, dtype=torch.bfloat16, device="cuda"), lens, 1)
