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
    sample = {"full": [0, 13, 31]} if name == "shared_decode_b32" else None
    print(f"workload {name}", flush=True)
    gpu, orc, _, _ = build_workload(wl, oracle_batches=sample)
    torch.cuda.synchronize()
    for cname, g in gpu.items():
        o, sel = orc[cname]
        assert_cache_equal(g, o, batches=sel if len(sel) != g.batch else None)
