"""GPU attention (decode, KV-shared decode, chunked prefill) against the fp64 oracle.

Tolerance: bf16 outputs within max-abs 1e-2 and mean-abs 1e-3 of the oracle.
The GPU appends its own cache (bit-exact with the oracle's, see test_gpu_append)
and the oracle attends its own cache; the two share only the seeded draws."""
import os

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


def make_pair(B, H, D, kb, vb, R, W, L, seed, zero=True):
    g = kvq.KVCache(B, H, D, kb, vb, R, window=W, zero=zero)
    o = oracle.Cache(B, H, D, R, kb, vb, window=W)
    k = small_randn(seed, (B, H, L, D), D ** -0.25)
    v = small_randn(seed + 1, (B, H, L, D), D ** -0.25)
    for t0 in range(0, L, 300):
        t1 = min(L, t0 + 300)
        pos0 = np.full(B, t0, np.int32)
        kvq.kvq_append_quantize(g, torch.from_numpy(k[:, :, t0:t1].copy()).cuda(),
                                torch.from_numpy(v[:, :, t0:t1].copy()).cuda(), torch.from_numpy(pos0).cuda())
        o.append(k[:, :, t0:t1], v[:, :, t0:t1], pos0)
    return g, o


DECODE_CASES = [
    # B, Hq, Hkv, D, kb, vb, R, W, L
    (1, 8, 2, 256, 4, 4, 128, 0, 128),
    (2, 8, 2, 256, 4, 8, 512, 512, 1500),     # ring wrap
    (2, 8, 1, 512, 8, 8, 2048, 0, 2000),      # full, cache not full (garbage-free zeros)
    (3, 4, 4, 128, 8, 4, 256, 100, 700),      # MHA, window < R
    (1, 16, 1, 512, 4, 8, 64, 0, 1),          # a single key
    (2, 24, 2, 128, 4, 4, 96, 40, 333),       # 12 rows per KV head
    (1, 40, 2, 256, 8, 8, 160, 0, 150),       # 20 rows: two row tiles
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_small(case):
    B, Hq, Hkv, D, kb, vb, R, W, L = case
    print(f"decode {case}", flush=True)
    g, o = make_pair(B, Hkv, D, kb, vb, R, W, L, seed=sum(case))
    q = small_q_bits(sum(case) + 7, (B, Hq, 1, D), D ** -0.25)
    lens = np.array([L - (b % 2) * min(3, L - 1) for b in range(B)], np.int32)
    out = kvq.kvq_attn_decode(g, q_dev(q[:, :, 0].copy()), torch.from_numpy(lens).cuda(), int(lens.max()))
    torch.cuda.synchronize()
    ref = o.attend(q, lens)[:, :, 0]
    assert_close(torch_bf16_to_f64(out), ref, f"decode {case}")


def test_decode_garbage_slots():
    """Slots beyond len hold arbitrary bits (torch.empty); they must not leak into the output."""
    B, Hq, Hkv, D, R, L = 2, 8, 1, 512, 256, 77
    g = kvq.KVCache(B, Hkv, D, 8, 8, R, window=0, zero=False)
    for t in (g.k_codes, g.v_codes, g.k_sb, g.v_sb):
        t.copy_(torch.randint(-2 ** 31, 2 ** 31 - 1, t.shape, dtype=torch.int32, device="cuda"))
    o = oracle.Cache(B, Hkv, D, R, 8, 8)
    k = small_randn(1, (B, Hkv, L, D), 0.21)
    v = small_randn(2, (B, Hkv, L, D), 0.21)
    kvq.kvq_append_quantize(g, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                            torch.zeros(B, dtype=torch.int32, device="cuda"))
    o.append(k, v, np.zeros(B, np.int32))
    q = small_q_bits(3, (B, Hq, 1, D), 0.21)
    lens = np.array([L, 40], np.int32)
    out = kvq.kvq_attn_decode(g, q_dev(q[:, :, 0].copy()), torch.from_numpy(lens).cuda(), 256)
    torch.cuda.synchronize()
    assert_close(torch_bf16_to_f64(out), o.attend(q, lens)[:, :, 0], "garbage slots")


def test_decode_split_invariance_and_determinism():
    B, Hq, Hkv, D, R, L = 2, 8, 1, 512, 4096, 4000
    g, o = make_pair(B, Hkv, D, 8, 8, R, 0, L, seed=5)
    q = q_dev(small_q_bits(6, (B, Hq, D), 0.21))
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    outs = []
    try:
        for s in ("1", "3", "16", "64", "128"):
            os.environ["KVQ_SPLITS"] = s
            outs.append(kvq.kvq_attn_decode(g, q, lens, L).clone())
        again = kvq.kvq_attn_decode(g, q, lens, L)
    finally:
        os.environ.pop("KVQ_SPLITS", None)
    torch.cuda.synchronize()
    assert torch.equal(outs[-1], again)                      # same plan: bitwise
    os.environ["KVQ_SPLITS"] = "3"
    try:
        again3 = kvq.kvq_attn_decode(g, q, lens, L)
    finally:
        os.environ.pop("KVQ_SPLITS", None)
    assert torch.equal(outs[1], again3)
    ref = o.attend(small_q_bits(6, (B, Hq, D), 0.21)[:, :, None], np.full(B, L, np.int32))[:, :, 0]
    for x in outs:
        assert_close(torch_bf16_to_f64(x), ref, "split")


@pytest.mark.parametrize("name", ["decode_b1_l128", "sliding_decode_b8_w512", "full_decode_b4_l32768",
                                  "sliding_decode_bf16_b8_w512"])
def test_decode_workload(name):
    wl = WORKLOADS[name]
    print(f"workload {name}", flush=True)
    gpu, orc, qd, _ = build_workload(wl)
    spec = wl.caches[0]
    q = qd[0][0]                                             # [B][Hq][1][D]
    lens = np.full(spec.B, spec.length, np.int32)
    out = kvq.kvq_attn_decode(gpu["kv"], q_dev(q[:, :, 0].copy()), torch.from_numpy(lens).cuda(), spec.length)
    torch.cuda.synchronize()
    o, _ = orc["kv"]
    ref = o.attend(q, lens)[:, :, 0]
    mx, mean = assert_close(torch_bf16_to_f64(out), ref, name)
    print(f"{name}: max-abs {mx:.2e} mean-abs {mean:.2e}", flush=True)


def test_workspace_reuse_across_calls():
    """One workspace, never cleared, through split decodes, split prefills and
    shared decodes of different plans: every result matches the oracle."""
    B, Hkv, D, R, W, L = 2, 2, 256, 1024, 512, 900
    g, o = make_pair(B, Hkv, D, 4, 8, R, W, L, seed=91)
    lens_np = np.full(B, L, np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    ws = torch.full((64 << 20,), 0xA5, dtype=torch.uint8, device="cuda")   # stale bytes, never cleared
    qd = small_q_bits(92, (B, 8, 1, D), 0.25)
    qp = small_q_bits(93, (B, 8, 64, D), 0.25)
    ref_d = o.attend(qd, lens_np)[:, :, 0]
    ref_p = o.attend(qp, lens_np)
    try:
        for splits in ("4", "17", "2", "9"):
            os.environ["KVQ_SPLITS"] = splits
            print(f"reuse splits={splits}", flush=True)
            out = kvq.kvq_attn_decode(g, q_dev(qd[:, :, 0].copy()), lens, L, workspace=ws)
            torch.cuda.synchronize()
            assert_close(torch_bf16_to_f64(out), ref_d, f"decode splits={splits}")
            out = kvq.kvq_attn_prefill_chunk(g, q_dev(qp), lens, L, workspace=ws)
            torch.cuda.synchronize()
            assert_close(torch_bf16_to_f64(out), ref_p, f"prefill splits={splits}")
            outs = kvq.kvq_attn_decode_shared([kvq.SharedGroup(g, [q_dev(qd[:, :, 0].copy())] * 2, lens, L)],
                                              workspace=ws)
            torch.cuda.synchronize()
            for x in outs[0]:
                assert_close(torch_bf16_to_f64(x), ref_d, f"shared splits={splits}")
    finally:
        os.environ.pop("KVQ_SPLITS", None)


def test_shared_equals_separate_small():
    B, Hkv, D, R, W, L = 2, 2, 256, 512, 512, 1000
    g, o = make_pair(B, Hkv, D, 4, 4, R, W, L, seed=40)
    g2, o2 = make_pair(B, 1, 512, 8, 8, 1024, 0, L, seed=41)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    qa = [q_dev(small_q_bits(50 + i, (B, 8, D), 0.25)) for i in range(3)]
    qb = [q_dev(small_q_bits(60, (B, 8, 512), 0.21))]
    try:
        os.environ["KVQ_SPLITS"] = "2"
        outs = kvq.kvq_attn_decode_shared([kvq.SharedGroup(g, qa, lens, L), kvq.SharedGroup(g2, qb, lens, L)])
        sep_a = [kvq.kvq_attn_decode(g, q, lens, L) for q in qa]
        sep_b = [kvq.kvq_attn_decode(g2, q, lens, L) for q in qb]
    finally:
        os.environ.pop("KVQ_SPLITS", None)
    torch.cuda.synchronize()
    for x, y in zip(outs[0] + outs[1], sep_a + sep_b):
        assert torch.equal(x, y)
    lens_np = np.full(B, L, np.int32)
    for i in range(3):
        ref = o.attend(small_q_bits(50 + i, (B, 8, D), 0.25)[:, :, None], lens_np)[:, :, 0]
        assert_close(torch_bf16_to_f64(outs[0][i]), ref, f"shared layer {i}")


def test_shared_limits_four_groups_sixteen_layers():
    """KVQ_MAX_SHARED_GROUPS groups in one call, one of them with
    KVQ_MAX_SHARED_LAYERS layers (64 rows per KV head: four row tiles), mixed
    head_dims (128 among them: one launch per descriptor), ragged lengths."""
    B, L = 2, 700
    specs = [  # Hkv, D, kb, vb, R, W, layers, Hq
        (2, 256, 4, 4, 512, 300, kvq.MAX_SHARED_LAYERS, 8),
        (1, 512, 8, 8, 1024, 0, 2, 8),
        (2, 128, 8, 4, 256, 200, 3, 4),
        (1, 256, 8, 8, 768, 0, 1, 4),
    ]
    assert len(specs) == kvq.MAX_SHARED_GROUPS
    lens_np = np.array([L, L - 37], np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    groups, refs = [], []
    for gi, (Hkv, D, kb, vb, R, W, layers, Hq) in enumerate(specs):
        g, o = make_pair(B, Hkv, D, kb, vb, R, W, L, seed=200 + 10 * gi)
        qs = [small_q_bits(300 + 10 * gi + l, (B, Hq, 1, D), D ** -0.25) for l in range(layers)]
        groups.append(kvq.SharedGroup(g, [q_dev(x[:, :, 0].copy()) for x in qs], lens, L))
        refs.append([o.attend(x, lens_np)[:, :, 0] for x in qs])
    print("shared limits", flush=True)
    outs = kvq.kvq_attn_decode_shared(groups)
    torch.cuda.synchronize()
    for gi in range(len(specs)):
        for l, ref in enumerate(refs[gi]):
            assert_close(torch_bf16_to_f64(outs[gi][l]), ref, f"group {gi} layer {l}")


def test_shared_workload():
    wl = WORKLOADS["shared_decode_b32"]
    print("workload shared_decode_b32 (every batch row of both caches)", flush=True)
    gpu, orc, qd, _ = build_workload(wl)
    donor, full = wl.cache("donor"), wl.cache("full")
    lens = torch.full((donor.B,), donor.length, dtype=torch.int32, device="cuda")
    qa = [q_dev(x[:, :, 0].copy()) for x in qd[0]]
    qb = [q_dev(x[:, :, 0].copy()) for x in qd[1]]
    outs = kvq.kvq_attn_decode_shared([kvq.SharedGroup(gpu["donor"], qa, lens, donor.length),
                                       kvq.SharedGroup(gpu["full"], qb, lens, full.length)])
    torch.cuda.synchronize()
    od, _ = orc["donor"]
    lens_np = np.full(donor.B, donor.length, np.int32)
    for i, x in enumerate(qd[0]):
        assert_close(torch_bf16_to_f64(outs[0][i]), od.attend(x, lens_np)[:, :, 0], f"donor layer {i}")
    of, sel = orc["full"]
    assert sel == list(range(full.B))
    ref = of.attend(qd[1][0], lens_np)[:, :, 0]
    assert_close(torch_bf16_to_f64(outs[1][0]), ref, "full layer")


def test_mixed_workload():
    """Three decoding layers over a sliding cache and a 5-token verify chunk over a
    full D512 layer in one kvq_attn_mixed launch, against the oracle on every
    batch row."""
    wl = WORKLOADS["mixed_b8_decode_verify"]
    print("workload mixed_b8_decode_verify", flush=True)
    gpu, orc, qd, _ = build_workload(wl)
    donor, full = wl.cache("donor"), wl.cache("full")
    ld = torch.full((donor.B,), donor.length, dtype=torch.int32, device="cuda")
    lf = torch.full((full.B,), full.length, dtype=torch.int32, device="cuda")
    reads = [kvq.Read(gpu["donor"], [q_dev(x) for x in qd[0]], ld, donor.length),
             kvq.Read(gpu["full"], [q_dev(x) for x in qd[1]], lf, full.length)]
    kvq.kvq_attn_mixed(reads)
    torch.cuda.synchronize()
    od, _ = orc["donor"]
    for i, x in enumerate(qd[0]):
        assert_close(torch_bf16_to_f64(reads[0].out[i]), od.attend(x, np.full(donor.B, donor.length, np.int32)),
                     f"donor layer {i}")
    of, sel = orc["full"]
    ref = of.attend(qd[1][0], np.full(full.B, full.length, np.int32))
    mx, mean = assert_close(torch_bf16_to_f64(reads[1].out[0]), ref, "full layer, 5-token chunk")
    print(f"mixed full layer: max-abs {mx:.2e} mean-abs {mean:.2e}", flush=True)


PREFILL_CASES = [
    # B, Hq, Hkv, D, kb, vb, R, W, L, C
    (1, 8, 2, 256, 4, 4, 128, 100, 300, 29),
    (2, 4, 1, 128, 8, 8, 256, 0, 200, 64),
    (1, 8, 2, 256, 4, 8, 1024, 512, 2000, 512),
    (2, 2, 2, 512, 8, 4, 96, 48, 150, 17),
    (1, 4, 4, 256, 8, 8, 256, 0, 130, 33),      # MHA: 33 rows, last wave of the block idle
    (3, 16, 2, 512, 4, 8, 512, 256, 700, 70),   # 560 rows per KV head: 9 row blocks, ragged
    (2, 8, 2, 256, 8, 4, 200, 64, 400, 96),     # ring capacity not a multiple of 32
    (1, 8, 1, 512, 8, 8, 64, 0, 40, 40),        # whole cache is the chunk, single step
]


@pytest.mark.parametrize("path", ["auto", "band", "codes", "decode"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_small(case, path):
    """Every case on the path the library picks and on each path forced
    (the band and short-chunk kernels exist for head_dim 256 and 512 only)."""
    B, Hq, Hkv, D, kb, vb, R, W, L, C = case
    print(f"prefill {case} path={path}", flush=True)
    g, o = make_pair(B, Hkv, D, kb, vb, R, W, L, seed=sum(case))
    q = small_q_bits(sum(case) + 1, (B, Hq, C, D), D ** -0.25)
    lens = np.full(B, L, np.int32)
    if path != "auto":
        os.environ["KVQ_PREFILL_PATH"] = path
    try:
        out = kvq.kvq_attn_prefill_chunk(g, q_dev(q), torch.from_numpy(lens).cuda(), L)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("KVQ_PREFILL_PATH", None)
    assert_close(torch_bf16_to_f64(out), o.attend(q, lens), f"prefill {case} path={path}")


VERIFY_CASES = [
    # B, Hq, Hkv, D, kb, vb, R, W, L, C: a few queries per sequence (draft tokens + 1)
    (2, 8, 2, 256, 4, 8, 520, 512, 1500, 5),     # ring wrap, window 512
    (1, 8, 1, 512, 8, 8, 2048, 0, 1000, 2),      # full layer, two rows per head: one tile
    (3, 4, 4, 128, 8, 4, 256, 100, 700, 8),      # MHA, head_dim 128
    (2, 16, 2, 256, 8, 4, 136, 128, 333, 8),     # 64 rows per KV head: four row tiles
    (1, 8, 2, 512, 4, 4, 64, 60, 64, 5),         # window + chunk fill the ring exactly
    (2, 8, 1, 512, 8, 8, 4096, 0, 3000, 5),      # full layer, > 2048 keys: the short-chunk kernel
    (1, 16, 2, 256, 4, 8, 4096, 0, 2500, 4),     # the same at head_dim 256, 32 rows per KV head
]


@pytest.mark.parametrize("case", VERIFY_CASES, ids=lambda c: "-".join(map(str, c)))
def test_verify_window(case):
    """Short causal chunks (speculative verify): ragged lengths, against the oracle."""
    B, Hq, Hkv, D, kb, vb, R, W, L, C = case
    print(f"verify {case}", flush=True)
    g, o = make_pair(B, Hkv, D, kb, vb, R, W, L, seed=sum(case) + 3)
    q = small_q_bits(sum(case) + 4, (B, Hq, C, D), D ** -0.25)
    lens = np.array([L - (b % 2) * min(7, L - C) for b in range(B)], np.int32)
    out = kvq.kvq_attn_prefill_chunk(g, q_dev(q), torch.from_numpy(lens).cuda(), L)
    torch.cuda.synchronize()
    assert_close(torch_bf16_to_f64(out), o.attend(q, lens), f"verify {case}")


@pytest.mark.parametrize("name", ["verify_b8_c5_w512", "verify_b4_c5_l32768"])
def test_verify_workload(name):
    wl = WORKLOADS[name]
    print(f"workload {name}", flush=True)
    gpu, orc, qd, _ = build_workload(wl)
    spec = wl.caches[0]
    q = qd[0][0]
    lens = np.full(spec.B, spec.length, np.int32)
    out = kvq.kvq_attn_prefill_chunk(gpu["kv"], q_dev(q), torch.from_numpy(lens).cuda(), spec.length)
    torch.cuda.synchronize()
    o, _ = orc["kv"]
    mx, mean = assert_close(torch_bf16_to_f64(out), o.attend(q, lens), name)
    print(f"{name}: max-abs {mx:.2e} mean-abs {mean:.2e}", flush=True)


@pytest.mark.parametrize("splits", ["1", "3", "7"])
def test_prefill_split_invariance(splits):
    B, Hq, Hkv, D, kb, vb, R, W, L, C = (2, 8, 2, 256, 4, 4, 1024, 0, 900, 100)
    print(f"prefill splits={splits}", flush=True)
    g, o = make_pair(B, Hkv, D, kb, vb, R, W, L, seed=77)
    q = small_q_bits(78, (B, Hq, C, D), D ** -0.25)
    lens = np.array([900, 700], np.int32)            # ragged: batch 1 sees a shorter prefix
    os.environ["KVQ_SPLITS"] = splits
    try:
        out = kvq.kvq_attn_prefill_chunk(g, q_dev(q), torch.from_numpy(lens).cuda(), L)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("KVQ_SPLITS", None)
    assert_close(torch_bf16_to_f64(out), o.attend(q, lens), f"prefill splits={splits}")


@pytest.mark.parametrize("name", ["prefill_b2_c512_w512", "prefill_bf16_b2_c512_w512"])
def test_prefill_workload(name):
    wl = WORKLOADS[name]
    print(f"workload {name}", flush=True)
    gpu, orc, qd, _ = build_workload(wl)
    spec = wl.caches[0]
    q = qd[0][0]
    lens = np.full(spec.B, spec.length, np.int32)
    out = kvq.kvq_attn_prefill_chunk(gpu["kv"], q_dev(q), torch.from_numpy(lens).cuda(), spec.length)
    torch.cuda.synchronize()
    o, _ = orc["kv"]
    mx, mean = assert_close(torch_bf16_to_f64(out), o.attend(q, lens), name)
    print(f"{name}: max-abs {mx:.2e} mean-abs {mean:.2e}", flush=True)


@pytest.mark.parametrize("extra", [None, "d128", "bf16"])
def test_mixed_decode_and_verify_reads(extra):
    """Decode reads (several layers) and short chunks of other caches in one
    kvq_attn_mixed call, ragged lengths; with a head_dim 128 read or a bf16 cache
    the call falls back to one launch per read, without them all reads share one
    launch."""
    B, L = 2, 900
    lens_np = np.array([L, L - 11], np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    specs = [  # Hkv, D, kb, vb, R, W, layers, Hq, chunk
        (2, 256, 4, 8, 520, 512, 3, 8, 1),
        (1, 512, 8, 8, 1024, 0, 1, 8, 5),
        (2, 256, 8, 4, 136, 128, 1, 16, 8),
    ]
    if extra == "d128":
        specs.append((2, 128, 8, 4, 256, 200, 1, 4, 3))
    if extra == "bf16":                                         # at most four reads per call
        specs[2] = (2, 256, 16, 16, 520, 512, 1, 8, 5)        # a verify chunk on a bf16 ring
        specs.append((1, 512, 16, 16, 1024, 0, 2, 8, 1))      # two layers decoding a bf16 full cache
    reads, refs = [], []
    for i, (Hkv, D, kb, vb, R, W, layers, Hq, C) in enumerate(specs):
        g, o = make_pair(B, Hkv, D, kb, vb, R, W, L, seed=400 + 10 * i)
        qs = [small_q_bits(500 + 10 * i + l, (B, Hq, C, D), D ** -0.25) for l in range(layers)]
        reads.append(kvq.Read(g, [q_dev(x) for x in qs], lens, L))
        refs.append([o.attend(x, lens_np) for x in qs])
    print(f"mixed extra={extra}", flush=True)
    outs = kvq.kvq_attn_mixed(reads)
    torch.cuda.synchronize()
    for i in range(len(specs)):
        for l, ref in enumerate(refs[i]):
            assert_close(torch_bf16_to_f64(outs[i][l]), ref, f"read {i} layer {l}")


def test_mixed_with_chunk_in_its_own_launch():
    """A verify chunk long enough for the short-chunk kernel (40 rows over more
    than 2048 keys) beside decode reads: the chunk runs in a launch of its own,
    the decode reads share the other launch, one combine serves both; against
    the oracle, ragged lengths, two calls in a row."""
    B, L = 2, 3000
    lens_np = np.array([L, L - 11], np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    specs = [  # Hkv, D, kb, vb, R, W, layers, Hq, chunk
        (2, 256, 4, 8, 520, 512, 3, 8, 1),
        (1, 512, 8, 8, 4096, 0, 1, 8, 5),
    ]
    reads, refs = [], []
    for i, (Hkv, D, kb, vb, R, W, layers, Hq, C) in enumerate(specs):
        g, o = make_pair(B, Hkv, D, kb, vb, R, W, L, seed=420 + 10 * i)
        qs = [small_q_bits(520 + 10 * i + l, (B, Hq, C, D), D ** -0.25) for l in range(layers)]
        reads.append(kvq.Read(g, [q_dev(x) for x in qs], lens, L))
        refs.append([o.attend(x, lens_np) for x in qs])
    print("mixed with an own-launch chunk", flush=True)
    for rep in range(2):
        outs = kvq.kvq_attn_mixed(reads)
        torch.cuda.synchronize()
        for i in range(len(specs)):
            for l, ref in enumerate(refs[i]):
                assert_close(torch_bf16_to_f64(outs[i][l]), ref, f"call {rep} read {i} layer {l}")


def test_mixed_rejects_multi_layer_chunk():
    g = kvq.KVCache(1, 1, 256, 4, 4, 64)
    q = torch.zeros(1, 8, 2, 256, dtype=torch.bfloat16, device="cuda")
    lens = torch.full((1,), 10, dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError):
        kvq.kvq_attn_mixed([kvq.Read(g, [q, q], lens, 10)])


@pytest.mark.parametrize("bits", [(4, 8), (8, 4), (16, 16)])
def test_minimum_capacity_ring(bits):
    """The smallest cache (32 slots) as a ring: every read step wraps inside it.
    Decode at W = R and a chunk with W + C - 1 = R, against the oracle."""
    kb, vb = bits
    B, Hq, Hkv, D, R = 2, 8, 2, 256, 32
    print(f"minimum capacity bits={bits}", flush=True)
    g, o = make_pair(B, Hkv, D, kb, vb, R, R, 101, seed=17 + kb)
    q = small_q_bits(18 + kb, (B, Hq, 1, D), D ** -0.25)
    lens = np.full(B, 101, np.int32)
    out = kvq.kvq_attn_decode(g, q_dev(q[:, :, 0].copy()), torch.from_numpy(lens).cuda(), 101)
    torch.cuda.synchronize()
    assert_close(torch_bf16_to_f64(out), o.attend(q, lens)[:, :, 0], f"decode R=32 bits={bits}")
    g2, o2 = make_pair(B, Hkv, D, kb, vb, R, 16, 77, seed=19 + kb)
    qc = small_q_bits(20 + kb, (B, Hq, 17, D), D ** -0.25)
    lens2 = np.full(B, 77, np.int32)
    out2 = kvq.kvq_attn_prefill_chunk(g2, q_dev(qc), torch.from_numpy(lens2).cuda(), 77)
    torch.cuda.synchronize()
    assert_close(torch_bf16_to_f64(out2), o2.attend(qc, lens2), f"chunk R=32 W=16 bits={bits}")


def test_shared_many_small_items():
    """A small donor read with many work items (16 sequences x 4 KV heads,
    window 64, three layers) beside a large full-layer read in one launch (the
    donor's items need no split, the full layer's many).  Outputs against the
    oracle, ragged lengths; also as kvq_attn_mixed."""
    B, L = 16, 2000
    lens_np = np.array([L - (b % 3) for b in range(B)], np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    g, o = make_pair(B, 4, 256, 4, 4, 64, 64, L, seed=120)
    g2, o2 = make_pair(B, 1, 512, 8, 8, 2048, 0, L, seed=121)
    qa = [small_q_bits(130 + i, (B, 16, 1, 256), 0.25) for i in range(3)]
    qb = [small_q_bits(140, (B, 8, 1, 512), 0.21)]
    print("shared, many small items", flush=True)
    outs = kvq.kvq_attn_decode_shared([kvq.SharedGroup(g, [q_dev(x[:, :, 0].copy()) for x in qa], lens, L),
                                       kvq.SharedGroup(g2, [q_dev(qb[0][:, :, 0].copy())], lens, L)])
    reads = [kvq.Read(g, [q_dev(x.copy()) for x in qa], lens, L),
             kvq.Read(g2, [q_dev(qb[0].copy())], lens, L)]
    outs_m = kvq.kvq_attn_mixed(reads)
    torch.cuda.synchronize()
    for i in range(3):
        ref = o.attend(qa[i], lens_np)[:, :, 0]
        assert_close(torch_bf16_to_f64(outs[0][i]), ref, f"donor layer {i}")
        assert_close(torch_bf16_to_f64(outs_m[0][i])[:, :, 0], ref, f"mixed donor layer {i}")
    ref = o2.attend(qb[0], lens_np)[:, :, 0]
    assert_close(torch_bf16_to_f64(outs[1][0]), ref, "full layer")
    assert_close(torch_bf16_to_f64(outs_m[1][0])[:, :, 0], ref, "mixed full layer")
