"""Caches whose never-written slots hold garbage, against the oracle.

The library does not ask callers to clear a cache before its first append.
Every read fetches whole 32-key steps, so the last step of a read reaches slots
past len that no append wrote; there the codes and the scale/bias words are
whatever the memory held.  Here those words are all-ones: bf16 NaN scales and
biases, and maximal codes.  Such keys get weight 0 and must not reach the
output on any path: the split read, the fused decode step, the short-chunk
kernel (more than 16 and at most 64 rows per KV head over more than 2048 keys)
and the band path; on a bf16 cache the unwritten values themselves are NaN.
Outputs within the attention tolerance of the oracle."""
import os

import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
import oracle
from kvq_testutil import assert_close, torch_bf16_to_f64
from synth import small_q_bits, small_randn
from test_gpu_attention import q_dev

pytestmark = pytest.mark.gpu


def garbage_pair(B, H, D, kb, vb, R, W, L, seed):
    g = kvq.KVCache(B, H, D, kb, vb, R, window=W, zero=False)
    for t in (g.k_codes, g.v_codes, g.k_sb, g.v_sb):
        if t is not None:                     # bf16 caches have no scale/bias arrays
            t.fill_(-1)
    o = oracle.Cache(B, H, D, R, kb, vb, window=W)
    k = small_randn(seed, (B, H, L, D), D ** -0.25)
    v = small_randn(seed + 1, (B, H, L, D), D ** -0.25)
    pos0 = np.zeros(B, np.int32)
    kvq.kvq_append_quantize(g, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(pos0).cuda())
    o.append(k, v, pos0)
    return g, o


def chunk(g, q, lens, max_len, path):
    if path != "auto":
        os.environ["KVQ_PREFILL_PATH"] = path
    try:
        out = kvq.kvq_attn_prefill_chunk(g, q_dev(q), torch.from_numpy(lens).cuda(), max_len)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("KVQ_PREFILL_PATH", None)
    return out


CASES = [
    # B, Hq, Hkv, D, kb, vb, R, W, L
    (1, 8, 1, 512, 8, 8, 4096, 0, 3000),      # full layer: 5-query chunks take the short-chunk kernel
    (2, 8, 2, 256, 4, 8, 1024, 512, 700),     # sliding ring, not yet wrapped
    (2, 8, 2, 256, 4, 4, 4096, 0, 2500),      # full layer, head_dim 256
    (2, 8, 2, 256, 16, 16, 1024, 0, 700),     # bf16 cache, full layer (NaN values past len)
]


@pytest.mark.parametrize("slack", [0, 300])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_reads_ignore_unwritten_slots(case, slack):
    """max_len = len + slack: with slack the launches are sized past every
    sequence's length, so more steps reach unwritten slots."""
    B, Hq, Hkv, D, kb, vb, R, W, L = case
    M = L + slack
    print(f"unwritten slots {case} max_len={M}", flush=True)
    g, o = garbage_pair(B, Hkv, D, kb, vb, R, W, L, seed=sum(case))
    lens = np.full(B, L, np.int32)
    qd = small_q_bits(sum(case) + 2, (B, Hq, 1, D), D ** -0.25)
    out = kvq.kvq_attn_decode(g, q_dev(qd[:, :, 0].copy()), torch.from_numpy(lens).cuda(), M)
    torch.cuda.synchronize()
    assert_close(torch_bf16_to_f64(out), o.attend(qd, lens)[:, :, 0], f"decode {case}")
    for C, paths in ((5, ("auto", "codes", "band", "decode")), (100, ("auto", "band", "decode"))):
        qc = small_q_bits(sum(case) + 3 + C, (B, Hq, C, D), D ** -0.25)
        ref = o.attend(qc, lens)
        for path in paths:
            out = chunk(g, qc, lens, M, path)
            assert_close(torch_bf16_to_f64(out), ref, f"chunk C={C} path={path} {case}")


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_step_ignores_unwritten_slots(case):
    B, Hq, Hkv, D, kb, vb, R, W, L = case
    g, o = garbage_pair(B, Hkv, D, kb, vb, R, W, L - 1, seed=sum(case) + 7)
    kn = small_randn(sum(case) + 8, (B, Hkv, D), D ** -0.25)
    vn = small_randn(sum(case) + 9, (B, Hkv, D), D ** -0.25)
    qb = small_q_bits(sum(case) + 10, (B, Hq, D), D ** -0.25)
    lens = np.full(B, L, np.int32)
    out = kvq.kvq_decode_step(g, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), q_dev(qb),
                              torch.from_numpy(lens).cuda(), L)
    torch.cuda.synchronize()
    o.append(kn[:, :, None], vn[:, :, None], lens - 1)
    assert_close(torch_bf16_to_f64(out), o.attend(qb[:, :, None], lens)[:, :, 0], f"decode step {case}")
