"""Helpers shared by the tests: layout conversions between the GPU cache and the
oracle's plain cache, and comparison utilities.  Test code only."""
from __future__ import annotations

import numpy as np


def u32(t):
    """A torch int32 tensor (any device) as a numpy uint32 array."""
    return t.detach().cpu().numpy().view(np.uint32)


def unpack_v_blocked(v_codes_u32: np.ndarray, v_bits: int) -> np.ndarray:
    """GPU V layout [B][H][R/8][D][v_bits/4] words -> plain codes uint8 [B][H][R][D]."""
    B, H, NB, D, W = v_codes_u32.shape
    assert W == v_bits // 4
    t = np.arange(8)
    if v_bits == 4:
        codes = (v_codes_u32[..., 0][..., None] >> (4 * t)) & 0xF          # [B][H][NB][D][8]
    else:
        words = v_codes_u32[..., t // 4]                                    # [B][H][NB][D][8]
        codes = (words >> (8 * (t % 4))) & 0xFF
    return codes.transpose(0, 1, 2, 4, 3).reshape(B, H, NB * 8, D).astype(np.uint8)


def sb_words(scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """Oracle bf16 scale/bias bit patterns -> the GPU's packed scale | bias << 16 words."""
    return scales.astype(np.uint32) | (biases.astype(np.uint32) << 16)


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_bf16_to_f64(t) -> np.ndarray:
    return bf16_to_f64(t.detach().cpu().view(__import__("torch").int16).numpy().view(np.uint16))


def assert_cache_equal(gpu_cache, ocache, batches=None):
    """Bit-exact comparison of a GPU KVCache against an oracle Cache (optionally a
    subset of GPU batch rows matching the oracle's batch axis)."""
    import oracle
    sel = slice(None) if batches is None else list(batches)
    if ocache.k_vals is not None:           # bf16 cache: the values in the cache layouts
        kv = ocache.k_vals.astype(np.uint32)
        np.testing.assert_array_equal(u32(gpu_cache.k_codes)[sel], kv[..., 0::2] | (kv[..., 1::2] << 16),
                                      err_msg="K bf16")
        B, H, R, D = ocache.v_vals.shape
        vb = ocache.v_vals.reshape(B, H, R // 8, 8, D).transpose(0, 1, 2, 4, 3).astype(np.uint32)
        np.testing.assert_array_equal(u32(gpu_cache.v_codes)[sel], vb[..., 0::2] | (vb[..., 1::2] << 16),
                                      err_msg="V bf16")
        return
    k_words = u32(gpu_cache.k_codes)[sel]
    np.testing.assert_array_equal(k_words, oracle.pack_words(ocache.k_codes, ocache.k_bits), err_msg="K codes")
    np.testing.assert_array_equal(u32(gpu_cache.k_sb)[sel], sb_words(ocache.k_scales, ocache.k_biases),
                                  err_msg="K scale/bias")
    v = unpack_v_blocked(u32(gpu_cache.v_codes)[sel], ocache.v_bits)
    np.testing.assert_array_equal(v, ocache.v_codes, err_msg="V codes")
    np.testing.assert_array_equal(u32(gpu_cache.v_sb)[sel], sb_words(ocache.v_scales, ocache.v_biases),
                                  err_msg="V scale/bias")


# Output tolerances for bf16 attention outputs against the fp64 oracle.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def assert_close(got_f64: np.ndarray, ref_f64: np.ndarray, what: str = ""):
    err = np.abs(got_f64 - ref_f64)
    assert np.isfinite(got_f64).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}"
    return mx, mean


def build_workload(wl, oracle_batches=None, with_oracle=True, hold_last=False):
    """Draw a workload's inputs (synth), append them to GPU caches through the C ABI
    and, independently, to oracle caches.

    oracle_batches: {cache name: list of batch rows the oracle keeps} (default: all).
    hold_last: append every position but the last on the GPU and return the last
    token's K/V (device tensors) so a caller can append it as a decode step does.
    Returns (gpu caches, oracle caches, q draws per QuerySpec, last tokens)."""
    import torch
    import decode_attention_group_amd as kvq
    import oracle
    import synth

    gen = synth.Generator(wl)
    gpu, orc, last = {}, {}, {}
    for spec in wl.caches:
        g = kvq.KVCache(spec.B, spec.Hkv, spec.D, spec.k_bits, spec.v_bits, spec.R, spec.window)
        sel = list(range(spec.B)) if not oracle_batches or spec.name not in oracle_batches else list(oracle_batches[spec.name])
        o = oracle.Cache(len(sel), spec.Hkv, spec.D, spec.R, spec.k_bits, spec.v_bits, spec.window) if with_oracle else None
        for pos, k, v in gen.kv_chunks(spec):
            T = k.shape[2]
            kt = torch.from_numpy(k).cuda()
            vt = torch.from_numpy(v).cuda()
            if hold_last and pos + T == spec.length:
                last[spec.name] = (kt[:, :, T - 1:T].contiguous(), vt[:, :, T - 1:T].contiguous())
                kt, vt, T = kt[:, :, :T - 1].contiguous(), vt[:, :, :T - 1].contiguous(), T - 1
            if T > 0:
                kvq.kvq_append_quantize(g, kt, vt, torch.full((spec.B,), pos, dtype=torch.int32, device="cuda"))
            if o is not None:
                o.append(k[sel], v[sel], np.full(len(sel), pos, np.int32))
        gpu[spec.name] = g
        orc[spec.name] = (o, sel)
    return gpu, orc, gen.q, last
