"""Pins for the oracle's norm and rotation before the append (kvq_oracle.c
kvqo_norm_rows): the keys' weighted RMS norm and rotation and the values'
un-scaled RMS norm [page 80 of the @mlx-bun/inference 0.0.0-stage -> 1.0.0 diff,
gemma4/model.ts attentionTraining (kNorm, RoPE through the cache, vNorm, then
appendWindow) and header notes (the value norm has no learned scale)].

  * closed forms: a constant row c = +-2^k with eps 0 normalizes to exactly +-1
    (times the weight); a quarter-turn table maps (a, b) to (-b, a) exactly; an
    identity table (cos 1, sin 0) changes nothing;
  * exact invariances: scaling a row by a power of 2 (eps 0) leaves the result
    bit for bit; columns at and past rope_dims are untouched by the rotation;
  * bit for bit against an independent numpy statement of the same definition
    (fp64 pairwise tree, one fp32 rounding per step), random rows of every head
    dim, weights, epsilons and tables;
  * within a few fp32 ulps of the textbook RMS norm in fp64 (any summation order);
  * planted mistakes in a copy of the oracle each fail one of these.

The fp64 summation order is a reading (the pages name the norm, not its
arithmetic): any order of the fp64 sum changes the fp32 factor only when that
factor lies within about 2^-53 (relative) of an fp32 rounding boundary, so the
order is fixed for bit-exact comparison but no random test can tell orders apart.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

F32 = np.float32
SRC = os.path.join(os.path.dirname(__file__), "..", "oracle", "kvq_oracle.c")


def np_tree_sumsq(x):
    """Complete binary tree over the zero-padded row, pairs (2i, 2i+1), fp64."""
    n = x.shape[-1]
    P = 1 << (n - 1).bit_length()
    b = np.zeros(x.shape[:-1] + (P,), np.float64)
    b[..., :n] = x.astype(np.float64) ** 2
    while b.shape[-1] > 1:
        b = b[..., 0::2] + b[..., 1::2]
    return b[..., 0]


def np_norm_rows(x, w, eps, rope=None, pos=None):
    x = x.astype(F32)
    D = x.shape[-1]
    r = (1.0 / np.sqrt(np_tree_sumsq(x) / D + np.float64(F32(eps)))).astype(F32)
    y = x * r[..., None]
    if w is not None:
        y = y * w.astype(F32)
    if rope is not None:
        c = rope[0][pos].astype(F32)
        s = rope[1][pos].astype(F32)
        h = c.shape[-1]
        a, b = y[..., :h].copy(), y[..., h:2 * h].copy()
        y[..., :h] = a * c - b * s
        y[..., h:2 * h] = b * c + a * s
    return y


def rope_table(rng, P, n):
    ang = rng.uniform(-np.pi, np.pi, (P, n // 2))
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def test_constant_rows_normalize_to_one():
    for D in (64, 192, 512):
        for k in (-20, -3, 0, 7):
            for sign in (1.0, -1.0):
                x = np.full((1, D), sign * 2.0 ** k, F32)
                assert (oracle.norm_rows(x, eps=0.0) == F32(sign)).all()
                w = np.random.default_rng(D).standard_normal(D).astype(F32)
                assert (oracle.norm_rows(x, w, eps=0.0) == F32(sign) * w).all()


def test_power_of_two_scale_invariance():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((50, 256)) * 0.3).astype(F32)
    w = rng.standard_normal(256).astype(F32)
    base = oracle.norm_rows(x, w, eps=0.0)
    for k in (-12, -1, 5, 30):
        assert (oracle.norm_rows(x * F32(2.0 ** k), w, eps=0.0) == base).all()


def test_rotation_closed_forms():
    rng = np.random.default_rng(4)
    D, n, P = 256, 128, 8
    x = rng.standard_normal((3, D)).astype(F32)
    pos = np.array([0, 3, 7], np.int32)
    ident = (np.ones((P, n // 2), F32), np.zeros((P, n // 2), F32))
    assert (oracle.norm_rows(x, eps=1e-6, rope=ident, pos=pos) == oracle.norm_rows(x, eps=1e-6)).all()
    quarter = (np.zeros((P, n // 2), F32), np.ones((P, n // 2), F32))
    y0 = oracle.norm_rows(x, eps=1e-6)
    y1 = oracle.norm_rows(x, eps=1e-6, rope=quarter, pos=pos)
    h = n // 2
    assert (y1[:, :h] == -y0[:, h:n]).all() and (y1[:, h:n] == y0[:, :h]).all()
    assert (y1[:, n:] == y0[:, n:]).all()


@pytest.mark.parametrize("D", [64, 128, 192, 256, 320, 384, 448, 512])
def test_bit_for_bit_against_numpy(D):
    rng = np.random.default_rng(100 + D)
    rows, P = 300, 64
    x = (rng.standard_normal((rows, D)) * 10.0 ** rng.uniform(-3, 3, (rows, 1))).astype(F32)
    w = (rng.standard_normal(D) * 0.5 + 1.0).astype(F32)
    n = 2 * int(rng.integers(1, D // 2 + 1))
    rope = rope_table(rng, P, n)
    pos = rng.integers(0, P, rows).astype(np.int32)
    for eps in (0.0, 1e-6, 1e-2):
        assert (oracle.norm_rows(x, None, eps) == np_norm_rows(x, None, eps)).all()
        assert (oracle.norm_rows(x, w, eps, rope, pos) == np_norm_rows(x, w, eps, rope, pos)).all()


def test_close_to_textbook_rms_norm():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((200, 512)).astype(F32)
    ref = x.astype(np.float64) / np.sqrt((x.astype(np.float64) ** 2).mean(axis=1, keepdims=True) + 1e-6)
    got = oracle.norm_rows(x, eps=1e-6).astype(np.float64)
    assert np.abs(got - ref).max() <= 4 * 2.0 ** -24 * np.abs(ref).max()


def test_rejects_bad_arguments():
    x = np.ones((2, 64), F32)
    with pytest.raises(oracle.OracleError):
        oracle.norm_rows(x, eps=-1.0)
    bad = x.copy()
    bad[1, 5] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.norm_rows(bad, eps=1e-6)
    table = (np.ones((4, 8), F32), np.zeros((4, 8), F32))
    with pytest.raises(oracle.OracleError):                  # position outside the table
        oracle.norm_rows(x, eps=1e-6, rope=table, pos=np.array([0, 4], np.int32))


MUTANTS = {
    "control": [],
    "no_eps": [("(double)n + (double)eps", "(double)n")],
    "interleaved_pairs": [("const float a = yr[j], b = yr[j + h];", "const float a = yr[2 * (j % (h / 2 > 0 ? h / 2 : 1))], b = yr[j + h];")],
    "sine_sign": [("yr[j] = ac - bs;", "yr[j] = ac + bs;")],
    "weight_first": [("const float t = xr[d] * f;\n            yr[d] = w ? t * w[d] : t;",
                      "const float t = w ? xr[d] * w[d] : xr[d];\n            yr[d] = t * f;")],
    "fp32_sum": [("double buf[512];", "float buf[512];")],
    "rotation_reads_rotated": [("const float a = yr[j], b = yr[j + h];\n                const float ac = a * c[j], bs = b * s[j], bc = b * c[j], as = a * s[j];\n                yr[j] = ac - bs;\n                yr[j + h] = bc + as;",
                                "const float a = yr[j], b = yr[j + h];\n                yr[j] = a * c[j] - b * s[j];\n                yr[j + h] = b * c[j] + yr[j] * s[j];")],
}


def _build(tmp, name, edits):
    text = open(SRC).read()
    for old, new in edits:
        assert text.count(old) == 1, f"mutation site not found: {old!r}"
        text = text.replace(old, new)
    src, lib = os.path.join(tmp, f"{name}.c"), os.path.join(tmp, f"lib{name}.so")
    open(src, "w").write(text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           "-fno-fast-math", "-w", src, "-o", lib, "-lm"])
    so = ctypes.CDLL(lib)
    P, i32 = ctypes.c_void_p, ctypes.c_int
    so.kvqo_norm_rows.argtypes = [P, ctypes.c_int64, i32, P, ctypes.c_float, P, P, i32, i32, P, P]
    so.kvqo_norm_rows.restype = i32
    return so


@pytest.mark.parametrize("name", list(MUTANTS))
def test_norm_mutant_is_caught(name, tmp_path):
    so = _build(str(tmp_path), name, MUTANTS[name])
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    rng = np.random.default_rng(11)
    caught = False
    for D in (192, 256):
        x = rng.standard_normal((64, D)).astype(F32)
        w = (rng.standard_normal(D) + 1.0).astype(F32)
        rope = rope_table(rng, 16, 64)
        pos = rng.integers(0, 16, 64).astype(np.int32)
        y = np.zeros_like(x)
        st = so.kvqo_norm_rows(p(x), 64, D, p(w), F32(1e-2), p(rope[0]), p(rope[1]), 64, 16, p(pos), p(y))
        caught |= st != 0 or not (y == np_norm_rows(x, w, 1e-2, rope, pos)).all()
    assert caught == (name != "control"), name


def test_append_normed_rotates_at_absolute_positions():
    """Token t of batch row b sits at pos0[b] + t: an alternating table (identity at
    even positions, quarter turn at odd ones) shows which position each row took;
    the values take the un-scaled norm and no rotation; the cache then holds the
    plain append of those rows."""
    rng = np.random.default_rng(21)
    B, H, T, D, n, R = 2, 3, 5, 128, 64, 16
    k = rng.standard_normal((B, H, T, D)).astype(F32)
    v = rng.standard_normal((B, H, T, D)).astype(F32)
    w = (rng.standard_normal(D) + 1.0).astype(F32)
    P = 16
    odd = (np.arange(P) % 2 == 1)[:, None] * np.ones((1, n // 2))
    table = ((1.0 - odd).astype(F32), odd.astype(F32))
    pos0 = np.array([5, 2], np.int32)
    cache = oracle.Cache(B, H, D, R, 4, 8)
    kn, vn = oracle.append_normed(cache, k, v, pos0, w, 1e-6, rope=table)
    plain = oracle.norm_rows(k, w, 1e-6)
    h = n // 2
    for b in range(B):
        for t in range(T):
            if (pos0[b] + t) % 2:
                assert (kn[b, :, t, :h] == -plain[b, :, t, h:n]).all()
                assert (kn[b, :, t, h:n] == plain[b, :, t, :h]).all()
                assert (kn[b, :, t, n:] == plain[b, :, t, n:]).all()
            else:
                assert (kn[b, :, t] == plain[b, :, t]).all()
    assert (vn == oracle.norm_rows(v, None, 1e-6)).all()
    ref = oracle.Cache(B, H, D, R, 4, 8)
    ref.append(kn, vn, pos0)
    for f in ("k_codes", "k_scales", "k_biases", "v_codes", "v_scales", "v_biases"):
        assert (getattr(cache, f) == getattr(ref, f)).all(), f
