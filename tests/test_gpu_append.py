"""GPU quantize-and-append against the oracle: codes, scales and biases bit-exact."""
import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
import oracle
from kvq_testutil import assert_cache_equal, build_workload
from synth import WORKLOADS, small_randn

pytestmark = pytest.mark.gpu


def _append_both(g, o, k, v, pos0):
    print(f"append T={k.shape[2]} pos0={list(pos0)}", flush=True)
    kvq.kvq_append_quantize(g, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                            torch.from_numpy(np.asarray(pos0, np.int32)).cuda())
    o.append(k, v, np.asarray(pos0, np.int32))


@pytest.mark.parametrize("D,kb,vb", [(128, 4, 4), (128, 8, 8), (256, 4, 8), (256, 8, 4), (512, 8, 8), (512, 4, 4)])
def test_append_sequence_bitexact(D, kb, vb):
    B, H, R = 2, 2, 64
    g = kvq.KVCache(B, H, D, kb, vb, R, window=R)
    o = oracle.Cache(B, H, D, R, kb, vb, window=R)
    pos = np.array([0, 3], np.int32)
    for i, T in enumerate([1, 5, 37, 1, 130, 3, 64, 9]):
        k = small_randn(100 + i, (B, H, T, D), D ** -0.25)
        v = small_randn(200 + i, (B, H, T, D), D ** -0.25)
        _append_both(g, o, k, v, pos)
        pos = pos + T
        torch.cuda.synchronize()
        assert_cache_equal(g, o)


def test_append_ring_offsets():
    """A T=1 append at every offset of a ring, then a wrap of T=R+5 from an odd start."""
    B, H, D, R = 1, 1, 128, 40                    # not a multiple of the 32-key read step
    g = kvq.KVCache(B, H, D, 4, 8, R, window=R)
    o = oracle.Cache(B, H, D, R, 4, 8, window=R)
    for p in range(0, 2 * R + 3):
        k = small_randn(300 + p, (B, H, 1, D), 0.3)
        _append_both(g, o, k, -k, [p])
    k = small_randn(999, (B, H, R + 5, D), 0.3)
    _append_both(g, o, k, 2 * k, [57])
    torch.cuda.synchronize()
    assert_cache_equal(g, o)


def test_append_adversarial_groups():
    B, H, D, R = 1, 1, 128, 32
    vals = [
        np.full(64, 0.75, np.float32), np.full(64, -0.0, np.float32), np.full(64, 1e-30, np.float32),
        np.linspace(-1e30, 1e30, 64).astype(np.float32), np.array([-0.0] * 63 + [2.0 ** -20], np.float32),
        np.array([1e38, -1e38] + [0.0] * 62, np.float32), np.float32(np.arange(64) * 0.25 - 8.0),
        np.array([1.0 + 2.0 ** -23] * 64, np.float32),
    ]
    rows = [np.concatenate([vals[i % len(vals)], vals[(i + 3) % len(vals)]]) for i in range(8)]
    k = np.stack(rows)[None, None]                 # [1][1][8][128]
    v = k[:, :, ::-1].copy()
    g = kvq.KVCache(B, H, D, 8, 4, R)
    o = oracle.Cache(B, H, D, R, 8, 4)
    _append_both(g, o, np.ascontiguousarray(k), v, [0])
    torch.cuda.synchronize()
    assert_cache_equal(g, o)


def test_append_denormal_inputs():
    B, H, D, R = 1, 1, 128, 32
    k = (small_randn(7, (B, H, 8, D), 1.0) * 1e-39).astype(np.float32)   # fp32 subnormals
    g = kvq.KVCache(B, H, D, 4, 8, R)
    o = oracle.Cache(B, H, D, R, 4, 8)
    _append_both(g, o, k, k * 3, [0])
    torch.cuda.synchronize()
    assert_cache_equal(g, o)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_append_workload_caches(name):
    """Every cache of every benchmark workload, built at full size, bit-exact."""
    wl = WORKLOADS[name]
    print(f"workload {name}", flush=True)
    gpu, orc, _, _ = build_workload(wl)
    torch.cuda.synchronize()
    for cname, g in gpu.items():
        o, sel = orc[cname]
        assert_cache_equal(g, o, batches=sel if len(sel) != g.batch else None)


@pytest.mark.parametrize("kb,vb", [(4, 8), (8, 4)])
def test_append_exact_ties(kb, vb):
    """Groups whose code ratios land exactly on k + 1/2 (and one fp32 step off):
    codes round half to even, bit-exact with the oracle."""
    import quant_reference as qref
    B, H, D, R = 1, 2, 256, 64
    per = D // 64
    Xk, _ = qref.tie_groups(np.random.default_rng(40 + kb), kb, B * H * R * per)
    Xv, _ = qref.tie_groups(np.random.default_rng(50 + vb), vb, B * H * R * per)
    k = np.ascontiguousarray(Xk.reshape(B, H, R, D))
    v = np.ascontiguousarray(Xv.reshape(B, H, R, D))
    g = kvq.KVCache(B, H, D, kb, vb, R)
    o = oracle.Cache(B, H, D, R, kb, vb)
    _append_both(g, o, k, v, [0])
    torch.cuda.synchronize()
    assert_cache_equal(g, o)


def test_append_golden_groups():
    """The hand-worked groups (exact ties included) through the GPU append: K at
    4 bits holds the 4-bit examples, V at 8 bits the 8-bit ones, each group at
    every position of a 128-wide row, so every lane position meets every example."""
    from test_oracle_quant import _golden_rows
    rows = _golden_rows()
    g4 = [r[2] for r in rows if r[1] == 4]
    g8 = [r[2] for r in rows if r[1] == 8]
    B, H, D, R = 1, 1, 128, 32
    T = max(len(g4), len(g8)) * 2
    k = np.zeros((B, H, T, D), np.float32)
    v = np.zeros((B, H, T, D), np.float32)
    for t in range(T):
        for grp in range(2):
            k[0, 0, t, grp * 64:(grp + 1) * 64] = g4[(t + grp) % len(g4)]
            v[0, 0, t, grp * 64:(grp + 1) * 64] = g8[(t + grp) % len(g8)]
    g = kvq.KVCache(B, H, D, 4, 8, R)
    o = oracle.Cache(B, H, D, R, 4, 8)
    _append_both(g, o, k, v, [0])
    torch.cuda.synchronize()
    assert_cache_equal(g, o)
    for name, bits, x, codes, s, b in rows:       # and the oracle holds the hand values
        c, sb, bb = oracle.quantize_group(x, bits)
        assert (c == codes).all() and sb == s and bb == b, name


# (D, k_bits, v_bits, R, batch, heads) of the caches one multi-append writes
MULTI_CACHES = [(256, 4, 8, 64, 2, 2), (512, 8, 8, 48, 2, 1), (128, 16, 16, 64, 2, 2), (64, 4, 4, 32, 2, 3)]


@pytest.mark.parametrize("n", [1, 2, 4])
def test_append_multi_matches_oracle_and_single_calls(n):
    """One launch over n caches of different head_dim, bits (bf16 among them),
    capacity and T writes what n separate appends and the oracle write, call
    after call, through ring wraps and a T > R call."""
    specs = MULTI_CACHES[:n]
    gm = [kvq.KVCache(B, H, D, kb, vb, R, window=R) for D, kb, vb, R, B, H in specs]
    gs = [kvq.KVCache(B, H, D, kb, vb, R, window=R) for D, kb, vb, R, B, H in specs]
    os_ = [oracle.Cache(B, H, D, R, kb, vb, window=R) for D, kb, vb, R, B, H in specs]
    pos = [np.array([0, 5], np.int32) for _ in specs]
    for step, Ts in enumerate([(1, 3, 1, 7), (37, 0, 70, 1), (1, 1, 1, 1), (5, 60, 2, 33)]):
        items, dev = [], []
        for i, (D, kb, vb, R, B, H) in enumerate(specs):
            T = Ts[i]
            k = small_randn(1000 * step + 10 * i, (B, H, T, D), D ** -0.25)
            v = small_randn(1000 * step + 10 * i + 1, (B, H, T, D), D ** -0.25)
            kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
            pd = torch.from_numpy(pos[i].copy()).cuda()
            dev.append((kd, vd, pd))
            items.append((gm[i], kd, vd, pd))
            if T:
                os_[i].append(k, v, pos[i])
        print(f"multi append n={n} step={step} T={Ts[:n]}", flush=True)
        kvq.kvq_append_quantize_multi(items)
        for i in range(n):
            kvq.kvq_append_quantize(gs[i], *dev[i])
            pos[i] = pos[i] + Ts[i]
        torch.cuda.synchronize()
        for i in range(n):
            assert_cache_equal(gm[i], os_[i])
            for name in ("k_codes", "v_codes", "k_sb", "v_sb"):
                a, b = getattr(gm[i], name), getattr(gs[i], name)
                if a is not None:
                    assert torch.equal(a, b), f"cache {i} {name} step {step}"


def test_append_multi_workload_step():
    """The decode step of the KV-shared workload at full size: every position but
    the last appended one call at a time, then the last token of the donor
    (D=256, 4/4-bit ring) and of the full layer (D=512, 8/8-bit) in one launch."""
    wl = WORKLOADS["shared_decode_b32"]
    print(f"multi append {wl.name}", flush=True)
    sel = {c.name: [0, 7, 19, c.B - 1] for c in wl.caches}
    gpu, orc, _, last = build_workload(wl, oracle_batches=sel, hold_last=True)
    items = []
    for spec in wl.caches:
        k, v = last[spec.name]
        pos0 = torch.full((spec.B,), spec.length - 1, dtype=torch.int32, device="cuda")
        items.append((gpu[spec.name], k, v, pos0))
    kvq.kvq_append_quantize_multi(items)
    torch.cuda.synchronize()
    for spec in wl.caches:
        o, rows = orc[spec.name]
        assert_cache_equal(gpu[spec.name], o, batches=rows)


def test_append_multi_rejects_one_cache_twice():
    g = kvq.KVCache(1, 1, 128, 4, 4, 32)
    k = torch.zeros((1, 1, 1, 128), dtype=torch.float32, device="cuda")
    pos0 = torch.zeros((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError):
        kvq.kvq_append_quantize_multi([(g, k, k, pos0), (g, k, k, pos0)])
