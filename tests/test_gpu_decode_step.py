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
        if src is not None:                   # (a bf16 cache has no scale|bias arrays)
            dst.copy_(src)
    return c


def assert_same_cache(a: kvq.KVCache, b: kvq.KVCache, what: str):
    for name in ("k_codes", "v_codes", "k_sb", "v_sb"):
        x, y = getattr(a, name), getattr(b, name)
        if x is None and y is None:
            continue
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


# ---- fused step of several shared groups (kvq_decode_step_shared)

SHARED_STEP_GROUPS = [
    # Hkv, D, kb, vb, R, W, layers, Hq
    (2, 256, 4, 4, 512, 300, 3, 8),     # sliding donor with three sharing layers (ring)
    (1, 512, 8, 8, 1024, 0, 1, 8),      # full donor, head_dim 512
    (2, 128, 8, 4, 256, 200, 2, 4),     # a head_dim outside the two-configuration launch
    (1, 256, 16, 16, 512, 512, 2, 4),   # a bf16 cache
]


# groups of one configuration (one launch of the same kernel), the first with
# 24 rows per KV head (two row tiles, both taking the token; tile 0 writes it)
SHARED_SAME_CONFIG = [
    (2, 256, 4, 4, 512, 300, 3, 16),
    (2, 256, 4, 4, 1024, 0, 1, 8),
]


@pytest.mark.parametrize("groups", [SHARED_STEP_GROUPS[:1], SHARED_STEP_GROUPS[:2], SHARED_STEP_GROUPS[:3],
                                    SHARED_STEP_GROUPS, SHARED_SAME_CONFIG],
                         ids=["1", "2", "3", "4", "same-config"])
def test_decode_step_shared_small(groups):
    """Each group's cache equals kvq_append_quantize's for the same token; every
    layer's output is within tolerance of the oracle after the oracle's append.
    Ragged lengths: the second sequence is one position behind.  One group
    launches alone (the token a split of its own); several groups share a launch
    (the last split of each item takes the token), of two configurations, of
    one, or per read where a configuration has no shared kernel."""
    n_groups = len(groups)
    B, L = 2, 600
    lens_np = np.array([L + 1, L], np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    groups_, refs, caches, ks, vs = [], [], [], [], []
    for gi, (Hkv, D, kb, vb, R, W, layers, Hq) in enumerate(groups):
        g, o = history(B, Hkv, D, kb, vb, R, W, L, seed=500 + 10 * gi)
        k = small_randn(600 + gi, (B, Hkv, D), D ** -0.25)
        v = small_randn(700 + gi, (B, Hkv, D), D ** -0.25)
        ref_cache = clone_cache(g)
        kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        kvq.kvq_append_quantize(ref_cache, kd[:, :, None].contiguous(), vd[:, :, None].contiguous(), lens - 1)
        o.append(k[:, :, None], v[:, :, None], lens_np - 1)
        qs = [small_q_bits(800 + 10 * gi + l, (B, Hq, 1, D), D ** -0.25) for l in range(layers)]
        groups_.append(kvq.SharedGroup(g, [q_dev(x[:, :, 0].copy()) for x in qs], lens, L + 1))
        refs.append([o.attend(x, lens_np)[:, :, 0] for x in qs])
        caches.append((g, ref_cache))
        ks.append(kd)
        vs.append(vd)
    print(f"shared decode step, {n_groups} groups {groups}", flush=True)
    outs = kvq.kvq_decode_step_shared(groups_, ks, vs)
    torch.cuda.synchronize()
    for gi, (g, ref_cache) in enumerate(caches):
        assert_same_cache(g, ref_cache, f"group {gi}")
        for l, ref in enumerate(refs[gi]):
            assert_close(torch_bf16_to_f64(outs[gi][l]), ref, f"group {gi} layer {l}")


def test_decode_step_shared_many_small_items():
    """The fused step over a small donor read with many items (16 sequences x 4
    KV heads, window 64, three layers) and a large full layer: both take their
    token in their last split (the donor's only one).  Caches word for word
    against the plain append, outputs against the oracle, ragged lengths (the
    donor's tokens rewrite ring slots)."""
    B, L = 16, 1999
    lens_np = np.array([L + 1 - (b % 3) for b in range(B)], np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    specs = [(4, 256, 4, 4, 64, 64, 3, 16), (1, 512, 8, 8, 2048, 0, 1, 8)]
    groups, refs, caches, ks, vs = [], [], [], [], []
    for gi, (Hkv, D, kb, vb, R, W, layers, Hq) in enumerate(specs):
        g, o = history(B, Hkv, D, kb, vb, R, W, L, seed=1500 + 10 * gi)
        k = small_randn(1600 + gi, (B, Hkv, D), D ** -0.25)
        v = small_randn(1700 + gi, (B, Hkv, D), D ** -0.25)
        ref_cache = clone_cache(g)
        kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        kvq.kvq_append_quantize(ref_cache, kd[:, :, None].contiguous(), vd[:, :, None].contiguous(), lens - 1)
        o.append(k[:, :, None], v[:, :, None], lens_np - 1)
        qs = [small_q_bits(1800 + 10 * gi + l, (B, Hq, 1, D), D ** -0.25) for l in range(layers)]
        groups.append(kvq.SharedGroup(g, [q_dev(x[:, :, 0].copy()) for x in qs], lens, L + 1))
        refs.append([o.attend(x, lens_np)[:, :, 0] for x in qs])
        caches.append((g, ref_cache))
        ks.append(kd)
        vs.append(vd)
    print("shared decode step, many small items", flush=True)
    outs = kvq.kvq_decode_step_shared(groups, ks, vs)
    torch.cuda.synchronize()
    for gi, (g, ref_cache) in enumerate(caches):
        assert_same_cache(g, ref_cache, f"group {gi}")
        for l, ref in enumerate(refs[gi]):
            assert_close(torch_bf16_to_f64(outs[gi][l]), ref, f"group {gi} layer {l}")


def test_decode_step_shared_matches_two_calls():
    """Against appends followed by kvq_attn_decode_shared on copies of the caches:
    the same caches word for word, outputs within the attention tolerance."""
    B, L = 3, 900
    lens = torch.full((B,), L + 1, dtype=torch.int32, device="cuda")
    specs = SHARED_STEP_GROUPS[:2]
    ga, gb, ks, vs, qss = [], [], [], [], []
    for gi, (Hkv, D, kb, vb, R, W, layers, Hq) in enumerate(specs):
        g, _ = history(B, Hkv, D, kb, vb, R, W, L, seed=900 + gi)
        ga.append(g)
        gb.append(clone_cache(g))
        ks.append(torch.from_numpy(small_randn(910 + gi, (B, Hkv, D), 0.25)).cuda())
        vs.append(torch.from_numpy(small_randn(920 + gi, (B, Hkv, D), 0.25)).cuda())
        qss.append([q_dev(small_q_bits(930 + 10 * gi + l, (B, Hq, D), 0.25)) for l in range(layers)])
    print("shared decode step vs two calls", flush=True)
    outs = kvq.kvq_decode_step_shared([kvq.SharedGroup(g, qs, lens, L + 1) for g, qs in zip(ga, qss)], ks, vs)
    for g, k, v in zip(gb, ks, vs):
        kvq.kvq_append_quantize(g, k[:, :, None].contiguous(), v[:, :, None].contiguous(), lens - 1)
    outs2 = kvq.kvq_attn_decode_shared([kvq.SharedGroup(g, qs, lens, L + 1) for g, qs in zip(gb, qss)])
    torch.cuda.synchronize()
    for gi in range(len(specs)):
        assert_same_cache(ga[gi], gb[gi], f"group {gi}")
        for x, y in zip(outs[gi], outs2[gi]):
            d = torch_bf16_to_f64(x) - torch_bf16_to_f64(y)
            assert np.abs(d).max() <= 1e-2 and np.abs(d).mean() <= 1e-3


def test_decode_step_shared_workload():
    """The KV-shared decode workload as a fused step: its last position is the
    step's token (appended by the step), every batch row checked."""
    wl = WORKLOADS["shared_decode_b32"]
    print("shared decode step workload shared_decode_b32", flush=True)
    gpu, orc, qd, last = build_workload(wl, hold_last=True)
    donor, full = wl.cache("donor"), wl.cache("full")
    lens_np = np.full(donor.B, donor.length, np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    refs = {}
    for name in ("donor", "full"):
        ref_cache = clone_cache(gpu[name])
        kvq.kvq_append_quantize(ref_cache, last[name][0], last[name][1], lens - 1)
        refs[name] = ref_cache
    qa = [q_dev(x[:, :, 0].copy()) for x in qd[0]]
    qb = [q_dev(x[:, :, 0].copy()) for x in qd[1]]
    outs = kvq.kvq_decode_step_shared(
        [kvq.SharedGroup(gpu["donor"], qa, lens, donor.length), kvq.SharedGroup(gpu["full"], qb, lens, full.length)],
        [last["donor"][0][:, :, 0].contiguous(), last["full"][0][:, :, 0].contiguous()],
        [last["donor"][1][:, :, 0].contiguous(), last["full"][1][:, :, 0].contiguous()])
    torch.cuda.synchronize()
    for name in ("donor", "full"):
        assert_same_cache(gpu[name], refs[name], name)
    od, _ = orc["donor"]
    for i, x in enumerate(qd[0]):
        assert_close(torch_bf16_to_f64(outs[0][i]), od.attend(x, lens_np)[:, :, 0], f"donor layer {i}")
    of, _ = orc["full"]
    assert_close(torch_bf16_to_f64(outs[1][0]), of.attend(qd[1][0], lens_np)[:, :, 0], "full layer")


def test_decode_step_shared_rejects_bad_arguments():
    g = kvq.KVCache(1, 2, 256, 4, 4, 64)
    k = torch.zeros(1, 2, 256, device="cuda")
    q = torch.zeros(1, 8, 256, dtype=torch.bfloat16, device="cuda")
    lens = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError):                     # two groups on one cache
        kvq.kvq_decode_step_shared([kvq.SharedGroup(g, [q], lens, 1), kvq.SharedGroup(g, [q], lens, 1)],
                                   [k, k], [k, k])
    with pytest.raises(kvq.KvqError):                     # k not 16-byte aligned
        kb = torch.zeros(1 * 2 * 256 + 1, device="cuda")[1:].view(1, 2, 256)
        kvq.kvq_decode_step_shared([kvq.SharedGroup(g, [q], lens, 1)], [kb], [k])
