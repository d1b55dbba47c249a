"""Unquantized bf16 caches on the GPU against the oracle.

The pages (@mlx-bun/inference 0.0.0-stage -> 1.0.0 diff, page 80,
gemma4/model.ts, note on cacheLayers) keep the sliding layers' caches in bf16
under the model's other KV scheme.  Checked here:
  * the append writes, word for word, the oracle's nearest-even bf16 values in
    the cache layouts (K token-major pairs, V blocked by 8 slots);
  * decode, chunk, KV-shared and mixed reads over bf16 caches are within the
    attention tolerance (max-abs 1e-2, mean-abs 1e-3) of the fp64 oracle, with
    ring wrap, ragged lengths, several row tiles and forced split counts;
  * the fused decode step writes the same cache words as the append and reads
    within the same tolerance.
"""
import os

import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
import oracle
from kvq_testutil import assert_close, torch_bf16_to_f64
from synth import small_q_bits, small_randn
from test_gpu_attention import make_pair, q_dev

pytestmark = pytest.mark.gpu


def words_u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def expected_k_words(vals: np.ndarray) -> np.ndarray:
    """Oracle bf16 values [B][H][R][D] -> K words [B][H][R][D/2] (element 2w low)."""
    v = vals.astype(np.uint32)
    return v[..., 0::2] | (v[..., 1::2] << 16)


def expected_v_words(vals: np.ndarray) -> np.ndarray:
    """Oracle bf16 values [B][H][R][D] -> blocked V words [B][H][R/8][D][4]."""
    B, H, R, D = vals.shape
    blk = vals.reshape(B, H, R // 8, 8, D).transpose(0, 1, 2, 4, 3).astype(np.uint32)   # [.., n, d, t]
    return blk[..., 0::2] | (blk[..., 1::2] << 16)


def assert_bf16_cache_equal(g: kvq.KVCache, o: oracle.Cache, what: str):
    np.testing.assert_array_equal(words_u32(g.k_codes), expected_k_words(o.k_vals), err_msg=f"{what}: K")
    np.testing.assert_array_equal(words_u32(g.v_codes), expected_v_words(o.v_vals), err_msg=f"{what}: V")


@pytest.mark.parametrize("D", [128, 256, 512])
def test_bf16_append_bit_exact(D):
    B, H, R = 2, 2, 64
    print(f"bf16 append D={D}", flush=True)
    g = kvq.KVCache(B, H, D, 16, 16, R, window=R)
    o = oracle.Cache(B, H, D, R, 16, 16, window=R)
    k = small_randn(D, (B, H, 150, D), D ** -0.25)
    v = small_randn(D + 1, (B, H, 150, D), D ** -0.25)
    pos = 0
    for T in (5, 11, 1, 37, 96):              # ring wrap; the last call has T > R
        pos0 = np.full(B, pos, np.int32)
        kvq.kvq_append_quantize(g, torch.from_numpy(k[:, :, pos:pos + T].copy()).cuda(),
                                torch.from_numpy(v[:, :, pos:pos + T].copy()).cuda(), torch.from_numpy(pos0).cuda())
        o.append(k[:, :, pos:pos + T], v[:, :, pos:pos + T], pos0)
        torch.cuda.synchronize()
        assert_bf16_cache_equal(g, o, f"D={D} after T={T}")
        pos += T


DECODE_CASES = [
    # B, Hq, Hkv, D, R, W, L, splits (None: the planner's)
    (2, 8, 2, 256, 512, 512, 1500, None),     # sliding decode with ring wrap
    (8, 8, 2, 256, 512, 512, 4096, None),     # the sliding-decode workload's shape
    (2, 8, 1, 512, 2048, 0, 2000, None),      # full layer, head_dim 512, GQA 8:1
    (3, 4, 4, 128, 256, 100, 700, None),      # MHA, head_dim 128, window < R
    (2, 24, 2, 128, 96, 40, 333, 3),          # 12 rows per KV head
    (1, 40, 2, 256, 160, 0, 150, 1),          # 20 rows: two row tiles, no split
    (2, 8, 2, 256, 1024, 0, 900, 17),         # many splits
    (1, 16, 1, 512, 64, 0, 1, None),          # a single key
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bf16_decode(case):
    B, Hq, Hkv, D, R, W, L, splits = case
    print(f"bf16 decode {case}", flush=True)
    g, o = make_pair(B, Hkv, D, 16, 16, R, W, L, seed=sum(c for c in case if c) + 5)
    q = small_q_bits(sum(c for c in case if c) + 6, (B, Hq, 1, D), D ** -0.25)
    ragged = W == 0 and R >= L
    lens = np.array([L - (b % 2) * min(3, L - 1) * ragged for b in range(B)], np.int32)
    if splits:
        os.environ["KVQ_SPLITS"] = str(splits)
    try:
        out = kvq.kvq_attn_decode(g, q_dev(q[:, :, 0].copy()), torch.from_numpy(lens).cuda(), int(lens.max()))
        torch.cuda.synchronize()
    finally:
        os.environ.pop("KVQ_SPLITS", None)
    assert_close(torch_bf16_to_f64(out), o.attend(q, lens)[:, :, 0], f"bf16 decode {case}")


CHUNK_CASES = [
    # B, Hq, Hkv, D, R, W, L, C
    (2, 8, 2, 256, 520, 512, 1500, 5),        # verify window on a sliding ring (split kernel)
    (2, 8, 2, 256, 1024, 512, 1200, 64),      # prefill chunk, window (band: 256 rows per KV head)
    (1, 8, 1, 512, 4096, 0, 3000, 5),         # verify on a full layer
    (2, 4, 2, 128, 256, 0, 200, 17),          # head_dim 128, full
    (1, 8, 1, 512, 2048, 0, 1500, 40),        # head_dim 512 band, full layer
    (2, 8, 2, 256, 200, 64, 400, 96),         # band over a ring whose capacity is not a multiple of 32
]


PATH_ENV = {
    "auto": {},
    "band": {"KVQ_PREFILL_PATH": "band"},                          # attention reads the cache in place
    "band_copy": {"KVQ_PREFILL_PATH": "band", "KVQ_BF16_BAND": "1"},   # band copy kernel first
    "decode": {"KVQ_PREFILL_PATH": "decode"},
}


def chunk_read(g, q, lens, L, path):
    env = PATH_ENV[path]
    os.environ.update(env)
    try:
        out = kvq.kvq_attn_prefill_chunk(g, q_dev(q), torch.from_numpy(lens).cuda(), L)
        torch.cuda.synchronize()
    finally:
        for k in env:
            os.environ.pop(k, None)
    return out


@pytest.mark.parametrize("path", list(PATH_ENV))
@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bf16_chunk(case, path):
    """Every case on the path the library picks and on each path forced (the
    band exists for head_dim 256 and 512; on a bf16 cache the attention kernel
    reads the cache in place unless the band copy is forced)."""
    B, Hq, Hkv, D, R, W, L, C = case
    print(f"bf16 chunk {case} path={path}", flush=True)
    g, o = make_pair(B, Hkv, D, 16, 16, R, W, L, seed=sum(case) + 9)
    q = small_q_bits(sum(case) + 10, (B, Hq, C, D), D ** -0.25)
    lens = np.full(B, L, np.int32)
    out = chunk_read(g, q, lens, L, path)
    assert_close(torch_bf16_to_f64(out), o.attend(q, lens), f"bf16 chunk {case} path={path}")


@pytest.mark.parametrize("path", ["band", "band_copy", "decode"])
@pytest.mark.parametrize("W", [0, 256])
def test_bf16_chunk_unwritten_slots_hold_nan(path, W):
    """Slots that no append wrote hold NaN bit patterns (the library does not
    ask for zeroed caches).  The reads fetch whole 32-key steps, so the last
    step reaches slots past len; those keys get weight 0 and their values must
    not reach the output."""
    B, Hq, Hkv, D, R, L, C = 2, 8, 2, 256, 1024, 333, 80
    g = kvq.KVCache(B, Hkv, D, 16, 16, R, window=W)
    g.k_codes.fill_(-1)                       # 0xFFFF halves: bf16 NaN
    g.v_codes.fill_(-1)
    o = oracle.Cache(B, Hkv, D, R, 16, 16, window=W)
    k = small_randn(31, (B, Hkv, L, D), D ** -0.25)
    v = small_randn(32, (B, Hkv, L, D), D ** -0.25)
    pos0 = np.zeros(B, np.int32)
    kvq.kvq_append_quantize(g, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(pos0).cuda())
    o.append(k, v, pos0)
    q = small_q_bits(33, (B, Hq, C, D), D ** -0.25)
    lens = np.full(B, L, np.int32)
    out = chunk_read(g, q, lens, L, path)
    assert_close(torch_bf16_to_f64(out), o.attend(q, lens), f"bf16 chunk over NaN slots W={W} path={path}")


def test_bf16_shared_with_quantized_group():
    """Three sharers of a bf16 sliding cache and one reader of an 8-bit full cache
    in one call (a bf16 read launches on its own kernel)."""
    print("bf16 shared + quantized", flush=True)
    B, L = 4, 1000
    g, o = make_pair(B, 2, 256, 16, 16, 512, 512, L, seed=71)
    g2, o2 = make_pair(B, 1, 512, 8, 8, 1024, 0, L, seed=72)
    lens_np = np.array([L, L, L - 2, L - 5], np.int32)
    # the sliding ring holds the last 512 of L for every sequence: shorter lengths
    # read slots already rewritten, so the bf16 group reads at full length
    lens_a = torch.full((B,), L, dtype=torch.int32, device="cuda")
    lens_b = torch.from_numpy(lens_np).cuda()
    qa = [small_q_bits(73 + i, (B, 8, 1, 256), 0.25) for i in range(3)]
    qb = small_q_bits(76, (B, 8, 1, 512), 0.21)
    res = kvq.kvq_attn_decode_shared([
        kvq.SharedGroup(g, [q_dev(x[:, :, 0].copy()) for x in qa], lens_a, L),
        kvq.SharedGroup(g2, [q_dev(qb[:, :, 0].copy())], lens_b, L)])
    torch.cuda.synchronize()
    full = np.full(B, L, np.int32)
    for i, x in enumerate(qa):
        assert_close(torch_bf16_to_f64(res[0][i]), o.attend(x, full)[:, :, 0], f"bf16 sharer {i}")
    assert_close(torch_bf16_to_f64(res[1][0]), o2.attend(qb, lens_np)[:, :, 0], "8-bit full reader")


def test_bf16_two_groups_one_launch():
    """Two bf16 caches of one head_dim: one launch of the bf16 kernel over both."""
    print("bf16 two groups", flush=True)
    B, L = 2, 700
    g, o = make_pair(B, 2, 256, 16, 16, 512, 512, L, seed=81)
    g2, o2 = make_pair(B, 2, 256, 16, 16, 1024, 0, L, seed=82)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    qa = small_q_bits(83, (B, 8, 1, 256), 0.25)
    qb = small_q_bits(84, (B, 8, 1, 256), 0.25)
    res = kvq.kvq_attn_decode_shared([kvq.SharedGroup(g, [q_dev(qa[:, :, 0].copy())], lens, L),
                                      kvq.SharedGroup(g2, [q_dev(qb[:, :, 0].copy())], lens, L)])
    torch.cuda.synchronize()
    full = np.full(B, L, np.int32)
    assert_close(torch_bf16_to_f64(res[0][0]), o.attend(qa, full)[:, :, 0], "bf16 group 0")
    assert_close(torch_bf16_to_f64(res[1][0]), o2.attend(qb, full)[:, :, 0], "bf16 group 1")


STEP_CASES = [
    # B, Hq, Hkv, D, R, W, history length
    (2, 8, 2, 256, 512, 512, 1499),           # sliding ring wrap, the token replaces the oldest slot
    (2, 8, 1, 512, 2048, 0, 1999),            # full layer, head_dim 512
    (3, 4, 4, 128, 256, 100, 699),            # MHA, head_dim 128, window < R
    (1, 40, 2, 256, 160, 0, 149),             # 20 rows: two row tiles
    (1, 16, 1, 512, 64, 0, 0),                # the token is the only key
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bf16_decode_step(case):
    """kvq_decode_step on a bf16 cache: the cache it leaves equals the one the
    append writes for the same token, word for word, and the output is within
    the attention tolerance of the oracle after its own append."""
    B, Hq, Hkv, D, R, W, L = case
    print(f"bf16 decode step {case}", flush=True)
    if L > 0:
        g, o = make_pair(B, Hkv, D, 16, 16, R, W, L, seed=sum(case) + 31)
    else:
        g, o = kvq.KVCache(B, Hkv, D, 16, 16, R, window=W), oracle.Cache(B, Hkv, D, R, 16, 16, window=W)
    k = small_randn(sum(case) + 32, (B, Hkv, D), D ** -0.25)
    v = small_randn(sum(case) + 33, (B, Hkv, D), D ** -0.25)
    qb = small_q_bits(sum(case) + 34, (B, Hq, D), D ** -0.25)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    lens = np.full(B, L + 1, np.int32)
    lens_d = torch.from_numpy(lens).cuda()
    ref_cache = kvq.KVCache(B, Hkv, D, 16, 16, R, window=W)
    ref_cache.k_codes.copy_(g.k_codes)
    ref_cache.v_codes.copy_(g.v_codes)
    kvq.kvq_append_quantize(ref_cache, kd[:, :, None].contiguous(), vd[:, :, None].contiguous(), lens_d - 1)
    out = kvq.kvq_decode_step(g, kd, vd, q_dev(qb), lens_d, L + 1)
    torch.cuda.synchronize()
    assert torch.equal(g.k_codes, ref_cache.k_codes) and torch.equal(g.v_codes, ref_cache.v_codes), "cache"
    o.append(k[:, :, None], v[:, :, None], lens - 1)
    assert_bf16_cache_equal(g, o, f"step {case}")
    assert_close(torch_bf16_to_f64(out), o.attend(qb[:, :, None], lens)[:, :, 0], f"bf16 step {case}")
