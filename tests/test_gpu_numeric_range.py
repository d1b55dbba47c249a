"""Magnitudes past the fp16 range that some kernel operands use, against the oracle.

The decode kernel (decode reads, the fused step, shared and mixed reads, chunks of
up to 16 rows per KV head) takes any finite bf16 q and any V the append accepts:
  * V times 2^16 (V scales up to thousands, biases past 2^15): the steps whose
    scale or bias leave the fp16 range run on bf16 operands;
  * q times 2^17 (|q| past 65504) with SDPA scale 2^-17, and q times 2^-26 (|q|
    near 1e-8, below the fp16 normal range) with scale 2^26: q enters the fp16
    MFMA after a power of 2 per row and group.
The short-chunk kernel (17..64 rows over more than 2048 keys) normalizes q per row
the same way; its dequantized K and V are fp16, so it is tested with V times 2^12
(values to about 3e3, scales near 20) inside that range.  The band path (more than
64 rows) is bf16 throughout.
Powers of 2 leave the quantizer's codes unchanged and scale the outputs exactly,
so every output is compared after dividing by the V factor, at the attention
tolerance (max-abs 1e-2, mean-abs 1e-3).
"""
import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
import oracle
from kvq_testutil import assert_close, torch_bf16_to_f64
from synth import small_q_bits, small_randn
from test_gpu_attention import q_dev
from test_gpu_edge_cases import build

pytestmark = pytest.mark.gpu


def scaled_q(seed, shape, sigma, factor):
    """bf16 bit patterns of factor * q (an exact power-of-2 scaling of bf16 q)."""
    q = small_q_bits(seed, shape, sigma)
    f = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * factor
    return (np.asarray(f, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def check(out, ref, vfac, what):
    assert_close(torch_bf16_to_f64(out) / vfac, ref / vfac, what)


def decode_paths(D, kb, vb, W, L, vfac, qfac, seed):
    B, Hq, H = 2, 8, 2 if D == 256 else 1
    R = W + 8 if W else (L + 64 + 7) // 8 * 8
    k = small_randn(seed, (B, H, L, D), D ** -0.25)
    v = small_randn(seed + 1, (B, H, L, D), D ** -0.25) * np.float32(vfac)
    g, o = build(B, H, D, kb, vb, R, W, k, v)
    q = scaled_q(seed + 2, (B, Hq, 1, D), D ** -0.25, qfac)
    scale = 1.0 / qfac
    lens = np.full(B, L, np.int32)
    tag = f"D={D} K{kb}/V{vb} W={W} vfac={vfac} qfac={qfac}"
    print(tag, flush=True)
    out = kvq.kvq_attn_decode(g, q_dev(q[:, :, 0].copy()), torch.from_numpy(lens).cuda(), L, scale=scale)
    torch.cuda.synchronize()
    check(out, o.attend(q, lens, scale=scale)[:, :, 0], vfac, "decode " + tag)
    # two queries per sequence (16 rows per KV head): the decode kernel with per-row positions
    Hq2 = 8 * H
    qc = scaled_q(seed + 3, (B, Hq2, 2, D), D ** -0.25, qfac)
    if Hq2 // H * 2 <= 16:
        out = kvq.kvq_attn_prefill_chunk(g, q_dev(qc), torch.from_numpy(lens).cuda(), L, scale=scale)
        torch.cuda.synchronize()
        check(out, o.attend(qc, lens, scale=scale), vfac, "chunk C=2 " + tag)
    # the fused step: one more token appended and attended
    kn = small_randn(seed + 4, (B, H, D), D ** -0.25)
    vn = small_randn(seed + 5, (B, H, D), D ** -0.25) * np.float32(vfac)
    lens1 = lens + 1
    out = kvq.kvq_decode_step(g, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), q_dev(q[:, :, 0].copy()),
                              torch.from_numpy(lens1).cuda(), L + 1, scale=scale)
    torch.cuda.synchronize()
    o.append(kn[:, :, None], vn[:, :, None], lens1 - 1)
    check(out, o.attend(q, lens1, scale=scale)[:, :, 0], vfac, "fused step " + tag)
    return g, o, q, lens1


@pytest.mark.parametrize("D,kb,vb,W", [(256, 4, 8, 512), (512, 8, 8, 0), (256, 4, 4, 0), (256, 16, 16, 512)])
def test_large_values(D, kb, vb, W):
    decode_paths(D, kb, vb, W, 1500, 2.0 ** 16, 1.0, 4000 + D + kb)


@pytest.mark.parametrize("qfac", [2.0 ** 17, 2.0 ** -26])
@pytest.mark.parametrize("D,kb,vb,W", [(256, 4, 8, 512), (512, 8, 8, 0)])
def test_query_magnitudes(D, kb, vb, W, qfac):
    decode_paths(D, kb, vb, W, 1500, 1.0, qfac, 4100 + D + kb)


def test_shared_launch_with_large_values_and_queries():
    """A sliding donor read by two layers and a full layer in one launch (the
    multi-configuration kernel), V times 2^16 and q times 2^17."""
    vfac, qfac = 2.0 ** 16, 2.0 ** 17
    B, L = 2, 1200
    k1 = small_randn(4201, (B, 2, L, 256), 0.25)
    v1 = small_randn(4202, (B, 2, L, 256), 0.25) * np.float32(vfac)
    k2 = small_randn(4203, (B, 1, L, 512), 0.21)
    v2 = small_randn(4204, (B, 1, L, 512), 0.21) * np.float32(vfac)
    g1, o1 = build(B, 2, 256, 4, 4, 512, 512, k1, v1)
    g2, o2 = build(B, 1, 512, 8, 8, L + 64, 0, k2, v2)
    qa = [scaled_q(4205 + i, (B, 8, 1, 256), 0.25, qfac) for i in range(2)]
    qb = [scaled_q(4208, (B, 8, 1, 512), 0.21, qfac)]
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    groups = [kvq.SharedGroup(g1, [q_dev(x[:, :, 0].copy()) for x in qa], lens, L, 1.0 / qfac),
              kvq.SharedGroup(g2, [q_dev(x[:, :, 0].copy()) for x in qb], lens, L, 1.0 / qfac)]
    outs = kvq.kvq_attn_decode_shared(groups)
    torch.cuda.synchronize()
    ln = np.full(B, L, np.int32)
    for o, qs, res in ((o1, qa, outs[0]), (o2, qb, outs[1])):
        for x, out in zip(qs, res):
            check(out, o.attend(x, ln, scale=1.0 / qfac)[:, :, 0], vfac, "shared")


@pytest.mark.parametrize("vexp", [12, 14])
@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 8), (16, 16)])
def test_chunk_kernels_inside_their_range(kb, vb, vexp):
    """The short-chunk kernel (8 queries: 64 rows over 2600 keys, 128 splits whose
    partials hold o / l in fp16) with q times 2^17 and V times 2^12 or 2^14 (values
    to about 1.3e4, inside its 2^15 bound), and the band path (96 queries) with the
    same inputs."""
    vfac, qfac = 2.0 ** vexp, 2.0 ** 17
    B, Hq, H, D, L = 2, 8, 1, 512, 2600
    k = small_randn(4301, (B, H, L, D), 0.21)
    v = small_randn(4302, (B, H, L, D), 0.21) * np.float32(vfac)
    g, o = build(B, H, D, kb, vb, L + 64, 0, k, v)
    lens = np.full(B, L, np.int32)
    for C in (8, 96):
        qc = scaled_q(4303 + C, (B, Hq, C, D), 0.21, qfac)
        print(f"chunk C={C} K{kb}/V{vb} V x 2^{vexp}", flush=True)
        out = kvq.kvq_attn_prefill_chunk(g, q_dev(qc), torch.from_numpy(lens).cuda(), L, scale=1.0 / qfac)
        torch.cuda.synchronize()
        check(out, o.attend(qc, lens, scale=1.0 / qfac), vfac, f"chunk C={C} K{kb}/V{vb}")
