"""kvq_attn_decode_static (the allocation-free decode read over the library's static
device scratch) against kvq_attn_decode with a caller workspace: two calls in a
row on the same device, the second smaller and of another cache shape, each
output equal to the workspace call's (same plan, same kernels), and both within
the attention tolerance of the oracle."""
import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
import oracle
from synth import small_q_bits, small_randn

pytestmark = pytest.mark.gpu


def _case(seed, B, Hq, Hkv, D, kb, vb, R, W, L):
    print(f"static-scratch case B={B} Hq={Hq} Hkv={Hkv} D={D} K{kb}/V{vb} R={R} W={W} len={L}", flush=True)
    k = small_randn(seed, (B, Hkv, L, D), D ** -0.25)
    v = small_randn(seed + 1, (B, Hkv, L, D), D ** -0.25)
    q = small_q_bits(seed + 2, (B, Hq, 1, D), D ** -0.25)
    g = kvq.KVCache(B, Hkv, D, kb, vb, R, window=W)
    kvq.kvq_append_quantize(g, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                            torch.zeros(B, dtype=torch.int32, device="cuda"))
    qt = torch.from_numpy(q[:, :, 0].copy().view(np.int16)).cuda().view(torch.bfloat16)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o = oracle.Cache(B, Hkv, D, R, kb, vb, window=W)
    o.append(k, v, np.zeros(B, np.int32))
    ref = o.attend(q, np.full(B, L, np.int32))[:, :, 0]
    return g, qt, lens, L, ref


def _bf16_to_f64(t):
    return (t.cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_static_scratch_matches_workspace_call():
    big = _case(10, 4, 8, 1, 512, 8, 8, 8192, 0, 8192)       # many splits: partials in the scratch
    small = _case(20, 2, 8, 2, 256, 4, 8, 512, 512, 1500)    # a smaller read after it
    torch.cuda.synchronize()
    nbytes = kvq.kvq_decode_workspace_bytes([(big[0], [big[1]], [big[1]], big[2], big[3], 1.0)])
    assert 0 < nbytes <= kvq.STATIC_SCRATCH_BYTES
    for g, qt, lens, L, ref in (big, small):
        out_ws = kvq.kvq_attn_decode(g, qt, lens, L)
        out_static = torch.full_like(qt, float("nan"))
        kvq.kvq_attn_decode_static(g, qt, lens, L, out=out_static)
        torch.cuda.synchronize()
        assert torch.equal(out_static.view(torch.int16), out_ws.view(torch.int16))
        err = np.abs(_bf16_to_f64(out_static) - ref)
        assert err.max() <= 1e-2 and err.mean() <= 1e-3, (err.max(), err.mean())
    # and the first shape again, after the smaller call left its partials behind
    g, qt, lens, L, ref = big
    out2 = kvq.kvq_attn_decode_static(g, qt, lens, L)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), kvq.kvq_attn_decode(g, qt, lens, L).view(torch.int16))
