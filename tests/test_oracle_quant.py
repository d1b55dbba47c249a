"""Pins for the oracle's quantizer and packing, independent of the oracle's own code.

The pages (@mlx-bun/inference 0.0.0-stage -> 1.0.0 diff, page 78, gemma4-e4b.ts
Gemma4Layer / LAYERS) fix only "affine, 4 or 8 bits, group 64".  What pins the
oracle here:
  * hand-worked examples (tests/golden/quantizer_worked_examples.txt);
  * grid-exact groups x = c*s + b (s, b bf16) must come back as exactly (c, s, b);
  * the bias is the greatest bf16 <= min and the scale the least bf16 >= the fp32
    step, found by searching bf16 neighbours (not by the oracle's bit formula);
  * every code is the best code (brute force over all 2^bits codes) and the
    round-trip error is at most half a step;
  * packing matches a hand-built word.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_worked_examples.txt")


def bf16_value(bits: int) -> float:
    return float(np.array([bits << 16], np.uint32).view(np.float32)[0])


def _expand(spec: str, kind):
    if spec.startswith("pattern:"):
        expr = spec[len("pattern:"):]
        return np.array([eval(expr, {"i": i}) for i in range(64)], kind)  # noqa: S307 - fixed fixture text
    items = spec.split(",")
    out, fill = [], None
    for it in items:
        if it.startswith("fill:"):
            fill = it[len("fill:"):]
        else:
            out.append(it)
    vals = out + [fill] * (64 - len(out))
    return np.array([kind(v) for v in vals], dtype=kind)


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, bits, xs, cs, s, b = [p.strip() for p in line.split("|")]
            rows.append((name, int(bits), _expand(xs, np.float32), _expand(cs, np.int64), int(s, 16), int(b, 16)))
    return rows


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_worked_examples(row):
    name, bits, x, codes, s, b = row
    c, sb, bb = oracle.quantize_group(x, bits)
    assert (c.astype(np.int64) == codes).all(), name
    assert sb == s and bb == b, (name, hex(sb), hex(bb))


def _grid_group(rng, bits):
    """A group whose values sit exactly on the grid c*s + b with bf16 s and b."""
    n = (1 << bits) - 1
    E = int(rng.integers(6, 14))                  # scale exponent
    s_int = int(rng.integers(128, 256))           # 8 significant bits
    s = s_int * 2.0 ** -E
    Eb = E - int(rng.integers(0, 8))              # bias grid no finer than the scale's
    b_int = -int(rng.integers(1, 256))
    b = b_int * 2.0 ** -Eb
    codes = rng.integers(0, n + 1, 64)
    codes[rng.integers(0, 64)] = 0
    codes[rng.integers(0, 64)] = n
    codes[0] = 0 if codes[0] != n else codes[0]
    if (codes == 0).sum() == 0:
        codes[1] = 0
    if (codes == n).sum() == 0:
        codes[2] = n
    x = codes * s + b
    x32 = x.astype(np.float32)
    assert (x32.astype(np.float64) == x).all()    # exact in fp32 by construction
    return x32, codes, s, b


@pytest.mark.parametrize("bits", [4, 8])
def test_grid_exact_round_trip(bits):
    rng = np.random.default_rng(1234 + bits)
    for _ in range(300):
        x, codes, s, b = _grid_group(rng, bits)
        c, sb, bb = oracle.quantize_group(x, bits)
        assert (c == codes).all()
        assert bf16_value(sb) == s and bf16_value(bb) == b


def _bf16_neighbours(v: float):
    """All bf16 values within a few bf16 steps of v (both signs), by enumeration."""
    u = int(np.array([v], np.float32).view(np.uint32)[0]) >> 16
    cands = set()
    for base in (u, u ^ 0x8000):
        for d in range(-3, 4):
            h = (base + d) & 0xFFFF
            f = bf16_value(h)
            if np.isfinite(f):
                cands.add(f)
    cands.add(0.0)
    return sorted(cands)


def _check_group(x, bits):
    n = (1 << bits) - 1
    c, sb, bb = oracle.quantize_group(x, bits)
    s, b = bf16_value(sb), bf16_value(bb)
    mn, mx = float(x.min()), float(x.max())
    # bias: greatest bf16 <= min
    below = [f for f in _bf16_neighbours(mn) if f <= mn]
    assert b == max(below)
    # scale: least bf16 >= fp32((max - bias) / n)
    step = float((np.float32(mx) - np.float32(b)) / np.float32(n))
    above = [f for f in _bf16_neighbours(step) if f >= step]
    assert s == min(above)
    assert c.min() >= 0 and c.max() <= n
    if s == 0:
        assert (c == 0).all() and mn == mx == b
        return c, s, b
    # best code by brute force over every code, in exact rational arithmetic
    xs = [Fraction(float(v)) for v in x]
    S, Bf = Fraction(s), Fraction(b)
    half = S / 2
    for v, code in zip(xs, c):
        err = abs(v - (code * S + Bf))
        best = min(abs(v - (k * S + Bf)) for k in range(n + 1))
        # the fp32 quotient may break a near-tie either way; otherwise optimal
        assert err <= best + S * Fraction(1, 1 << 20)
        assert err <= half * (1 + Fraction(1, 1 << 20))
    return c, s, b


@pytest.mark.parametrize("bits", [4, 8])
def test_random_groups_properties(bits):
    rng = np.random.default_rng(77 + bits)
    for trial in range(120):
        scale = 10.0 ** rng.uniform(-6, 6)
        x = (rng.standard_normal(64) * scale).astype(np.float32)
        if trial % 5 == 0:
            x = np.abs(x)           # all-positive groups: bias near a positive min
        if trial % 7 == 0:
            x = -np.abs(x)
        _check_group(x, bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_adversarial_groups(bits):
    cases = [
        np.full(64, 1e-30, np.float32),
        np.full(64, -1e30, np.float32),
        np.linspace(-1e30, 1e30, 64).astype(np.float32),
        np.linspace(1e-30, 3e-30, 64).astype(np.float32),
        np.array([0.0] * 63 + [1.0], np.float32),
        np.array([-1.0] + [0.0] * 63, np.float32),
        np.array([-0.0] * 32 + [0.0] * 32, np.float32),
        np.array([-0.0] * 63 + [2.0 ** -20], np.float32),
        np.array([1.0 + 2.0 ** -23] * 64, np.float32),       # constant, not a bf16 value
        np.array([3.0, 3.0] + [1.0] * 62, np.float32),         # repeated extrema
        np.float32(np.arange(64) * 0.25 - 8.0),
        np.array([1e38, -1e38] + [0.0] * 62, np.float32),       # domain edges
    ]
    for x in cases:
        _check_group(np.ascontiguousarray(x, np.float32), bits)


def test_negative_zero_is_canonical():
    c, s, b = oracle.quantize_group(np.array([-0.0] * 64, np.float32), 4)
    assert s == 0 and b == 0 and (c == 0).all()
    c, s, b = oracle.quantize_group(np.array([-0.0] * 63 + [1.0], np.float32), 8)
    assert b == 0                                   # +0, not 0x8000


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf, 2e38, -2e38])
def test_rejects_out_of_domain(bad):
    x = np.zeros(64, np.float32)
    x[5] = bad
    with pytest.raises(oracle.OracleError):
        oracle.quantize_group(x, 8)


def test_rejects_bad_bits():
    with pytest.raises(oracle.OracleError):
        oracle.quantize_group(np.zeros(64, np.float32), 5)


def test_pack_hand_examples():
    # 4-bit codes 0..7 -> element e at bits [4e, 4e+4): 0x76543210
    w = oracle.pack_words(np.arange(8, dtype=np.uint8).reshape(1, 8), 4)
    assert int(w[0, 0]) == 0x76543210
    # 8-bit codes 0x10,0x32,0x54,0x76 -> byte e at bits [8e, 8e+8)
    w = oracle.pack_words(np.array([[0x10, 0x32, 0x54, 0x76]], np.uint8), 8)
    assert int(w[0, 0]) == 0x76543210
    # 4-bit, two words: 15,0,...,0 | 0,...,0,9
    row = np.zeros(16, np.uint8)
    row[0] = 15
    row[15] = 9
    w = oracle.pack_words(row.reshape(1, 16), 4)
    assert [int(v) for v in w[0]] == [0x0000000F, 0x90000000]


def test_append_ring_and_last_r():
    """Token t of sequence b lands in slot (pos0[b]+t) mod R; with T > R only the
    last R tokens are written (equivalent to appending them one by one)."""
    B, H, D, R = 2, 3, 128, 8
    rng = np.random.default_rng(5)
    T = 21
    x = rng.standard_normal((B, H, T, D)).astype(np.float32)
    pos0 = np.array([5, 13], np.int32)
    c1 = oracle.Cache(B, H, D, R, 4, 8, window=R)
    c1.append(x, x, pos0)
    c2 = oracle.Cache(B, H, D, R, 4, 8, window=R)
    for t in range(T):
        c2.append(x[:, :, t:t + 1], x[:, :, t:t + 1], pos0 + t)
    for a in ("k_codes", "v_codes", "k_scales", "k_biases", "v_scales", "v_biases"):
        assert (getattr(c1, a) == getattr(c2, a)).all(), a
    # slot check against single-group quantization
    for b in range(B):
        for t in range(T - R, T):
            slot = (pos0[b] + t) % R
            codes, s, bb = oracle.quantize_group(x[b, 1, t, 64:128], 8)
            assert (c1.v_codes[b, 1, slot, 64:128] == codes).all()
            assert c1.v_scales[b, 1, slot, 1] == s and c1.v_biases[b, 1, slot, 1] == bb


def test_append_validates_before_writing():
    c = oracle.Cache(1, 1, 64, 4, 4, 4)
    x = np.ones((1, 1, 2, 64), np.float32)
    x[0, 0, 1, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        c.append(x, np.ones_like(x), np.array([0], np.int32))
    assert (c.k_codes == 0).all() and (c.k_scales == 0).all()


# ---------------------------------------------------------------------------
# Bit-for-bit pins against the independent numpy-float32 statement
# (tests/quant_reference.py), with no slack, and exact ties.

import quant_reference as qref  # noqa: E402


def _oracle_groups(X, bits):
    """The oracle's quantizer over many groups at once (one append of N tokens)."""
    N = X.shape[0]
    c = oracle.Cache(1, 1, 64, N, bits, bits)
    x = np.ascontiguousarray(X.reshape(1, 1, N, 64), np.float32)
    c.append(x, x, np.zeros(1, np.int32))
    return c.k_codes[0, 0, :, :], c.k_scales[0, 0, :, 0], c.k_biases[0, 0, :, 0]


def random_groups(rng, count):
    """Groups over many magnitudes and shapes: normal, one-signed, constant, near-constant."""
    X = np.empty((count, 64), np.float32)
    for i in range(count):
        sc = 10.0 ** rng.uniform(-30, 30) if i % 11 == 0 else 10.0 ** rng.uniform(-4, 4)
        x = rng.standard_normal(64) * sc
        kind = i % 9
        if kind == 1:
            x = np.abs(x)
        elif kind == 2:
            x = -np.abs(x)
        elif kind == 3:
            x = np.full(64, x[0])
        elif kind == 4:
            x = x[0] + x * 1e-7
        elif kind == 5:
            x[rng.integers(0, 64, 8)] = x.max()
        X[i] = np.clip(x, -1e38, 1e38).astype(np.float32)
    return X


@pytest.mark.parametrize("bits", [4, 8])
def test_bit_for_bit_against_numpy_float32(bits):
    """20,000 random groups: codes, scales and biases identical, no tolerance."""
    rng = np.random.default_rng(2024 + bits)
    X = random_groups(rng, 20000)
    oc, os_, ob = _oracle_groups(X, bits)
    nc, ns, nb = qref.quantize_groups(X, bits)
    assert (os_ == ns).all() and (ob == nb).all()
    bad = np.nonzero((oc != nc).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} groups differ, first {bad[:5]}"


@pytest.mark.parametrize("bits", [4, 8])
def test_exact_ties_round_half_even(bits):
    """Constructed groups with exact k + 1/2 ratios: the oracle rounds each to the
    even neighbour (a closed form), and agrees bit for bit with the numpy statement
    on the ties and their one-ulp neighbours."""
    rng = np.random.default_rng(31 + bits)
    X, E = qref.tie_groups(rng, bits, 2000)
    oc, os_, ob = _oracle_groups(X, bits)
    nc, ns, nb = qref.quantize_groups(X, bits)
    known = E >= 0
    assert known.sum() > 2000 * 40
    assert (oc.astype(np.int64)[known] == E[known]).all()
    assert (oc == nc).all() and (os_ == ns).all() and (ob == nb).all()
