"""An independent float32 statement of the affine group quantizer, for pinning the oracle.

It is written from the definition, not from the oracle's C: numpy float32
arithmetic (each operation one IEEE fp32 operation, round-to-nearest-even) and
np.rint (round half to even).  The two directed bf16 roundings are found by
searching the bf16 values next to the input, not by the oracle's bit formula:
  bias  = the greatest bf16 value <= min(group)      (min read with -0 as +0)
  scale = the least bf16 value >= fp32((max - bias) / (2^bits - 1))
  code  = clip(rint(fp32(fp32(x - bias) / scale)), 0, 2^bits - 1), 0 when scale == 0
(page 78 of the @mlx-bun/inference 0.0.0-stage -> 1.0.0 diff, gemma4-e4b.ts
Gemma4Layer.kv: affine, 4 or 8 bits, group 64; the pages print no formula and the
reading above is this library's).
"""
import numpy as np

F32 = np.float32


def _bf16_keys(x):
    """Monotone integer key of the bf16 value obtained by dropping x's low 16 bits."""
    h = (x.view(np.uint32) >> 16).astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


def _key_values(key):
    """float32 value of a bf16 key (key 0 is +0)."""
    h = np.where(key < 0, 0x8000 | (-key), key).astype(np.uint32)
    return (h << 16).view(np.float32)


def _bf16_candidates(x):
    """[N, 5] float32: the bf16 values two keys either side of x's truncation."""
    k = _bf16_keys(np.ascontiguousarray(x, F32))
    return np.stack([_key_values(k + d) for d in (-2, -1, 0, 1, 2)], axis=1)


def bf16_floor(x):
    c = _bf16_candidates(x)
    return np.where(c <= x[:, None], c, F32(-np.inf)).max(axis=1).astype(F32)


def bf16_ceil(x):
    c = _bf16_candidates(x)
    return np.where(c >= x[:, None], c, F32(np.inf)).min(axis=1).astype(F32)


def quantize_groups(X, bits):
    """X float32 [N, 64] -> (codes uint8 [N, 64], scale bf16 bits [N], bias bf16 bits [N])."""
    X = np.ascontiguousarray(X, F32)
    n = F32((1 << bits) - 1)
    mn = X.min(axis=1) + F32(0.0)
    mx = X.max(axis=1) + F32(0.0)
    b = bf16_floor(mn)
    step = (mx - b) / n
    s = bf16_ceil(step)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint((X - b[:, None]) / s[:, None])
    r = np.clip(r, F32(0.0), n)
    codes = np.where(s[:, None] == 0, 0, r).astype(np.uint8)
    assert r.dtype == np.float32 and step.dtype == np.float32
    return codes, (s.view(np.uint32) >> 16).astype(np.uint16), (b.view(np.uint32) >> 16).astype(np.uint16)


def tie_groups(rng, bits, count):
    """Groups whose code ratios include exact ties k + 1/2 (and their fp32 neighbours).

    bias b and scale s are bf16 values with few significant bits, min = b and
    max = b + n*s, so (max - b)/n = s exactly; every other entry is b + (k + 1/2)*s
    kept only where that sum is an fp32 value, so (x - b)/s = k + 1/2 exactly.
    Returns (X [count, 64] float32, expected codes [count, 64] or -1 where an entry
    is a perturbed neighbour whose code is not a closed form)."""
    n = (1 << bits) - 1
    X = np.zeros((count, 64), F32)
    E = np.full((count, 64), -1, np.int64)
    made = 0
    while made < count:
        s = float(rng.integers(129, 256) * 2.0 ** -int(rng.integers(2, 12)))
        b = -float(rng.integers(0, 64)) * 2.0 ** -int(rng.integers(0, 6))
        if np.float64(F32(b)) != b or F32(s) != s or float(F32(b + n * s)) != b + n * s:
            continue
        if float((F32(b + n * s) - F32(b)) / F32(n)) != s:
            continue
        x = np.full(64, b, np.float64)
        e = np.zeros(64, np.int64)
        x[1], e[1] = b + n * s, n
        for i in range(2, 64):
            k = int(rng.integers(0, n))
            v = b + (k + 0.5) * s
            if float(F32(v)) != v or float(F32(F32(v) - F32(b))) != (k + 0.5) * s:
                x[i], e[i] = b, 0
                continue
            x[i] = v
            e[i] = k if k % 2 == 0 else k + 1          # half to even
            if i % 5 == 0:                            # one fp32 step either side: a near tie
                x[i] = float(np.nextafter(F32(v), F32(np.inf if i % 10 else -np.inf)))
                e[i] = -1
        X[made] = x.astype(F32)
        E[made] = e
        made += 1
    return X, E
