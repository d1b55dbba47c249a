"""The quantizer pins have teeth: each plausible mistake planted in a copy of the
oracle's C source (built here on the CPU, never loaded by anything else) must
fail at least one pin, and the unchanged source must pass all of them.

Pins run against each build: the hand-worked golden groups (exact ties
included), bit-for-bit agreement with the numpy-float32 statement on random
groups, and the closed form of exact ties (k + 1/2 rounds to the even one).
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import quant_reference as qref
from test_oracle_quant import _golden_rows, random_groups

SRC = os.path.join(os.path.dirname(__file__), "..", "oracle", "kvq_oracle.c")

MUTANTS = {
    "control": [],
    "ties_away_from_zero": [("float r = rintf(ratio);", "float r = roundf(ratio);")],
    "reciprocal_multiply": [("const float ratio = (x[i] - bias) / scale;",
                             "const float ratio = (x[i] - bias) * (1.0f / scale);")],
    "bias_toward_zero": [("if (u & 0x80000000u) return float_of(toward_zero + 0x10000u);\n    return float_of(toward_zero);\n}\n\n/* Smallest",
                          "return float_of(toward_zero);\n}\n\n/* Smallest")],
    "scale_truncated": [("if (u & 0x80000000u) return float_of(toward_zero);\n    return float_of(toward_zero + 0x10000u);",
                         "return float_of(toward_zero);")],
    "negative_zero_kept": [("mn = mn + 0.0f;", "mn = mn;")],
    "step_over_levels": [("const float step = (mx - bias) / (float)top;",
                          "const float step = (mx - bias) / (float)(top + 1);")],
    "step_from_min": [("const float step = (mx - bias) / (float)top;",
                       "const float step = (mx - mn) / (float)top;")],
}


def _build(tmp, name, edits):
    with open(SRC) as f:
        text = f.read()
    for old, new in edits:
        assert text.count(old) == 1, f"mutation site not found: {old!r}"
        text = text.replace(old, new)
    src = os.path.join(tmp, f"{name}.c")
    lib = os.path.join(tmp, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           "-fno-fast-math", "-w", src, "-o", lib, "-lm"])
    so = ctypes.CDLL(lib)
    P, i32 = ctypes.c_void_p, ctypes.c_int
    so.kvqo_append.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P]
    so.kvqo_append.restype = i32
    return so


def _quantize(so, X, bits):
    N = X.shape[0]
    x = np.ascontiguousarray(X, np.float32)
    codes = np.zeros((N, 64), np.uint8)
    s = np.zeros(N, np.uint16)
    b = np.zeros(N, np.uint16)
    pos0 = np.zeros(1, np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    st = so.kvqo_append(p(x), 1, 1, N, 64, bits, N, p(pos0), p(codes), p(s), p(b))
    assert st == 0
    return codes, s, b


def _failed_pins(so):
    failed = []
    for name, bits, x, codes, s, b in _golden_rows():
        c, sb, bb = _quantize(so, x[None], bits)
        if not ((c[0] == codes).all() and sb[0] == s and bb[0] == b):
            failed.append(f"golden:{name}")
    for bits in (4, 8):
        rng = np.random.default_rng(5 + bits)
        X = random_groups(rng, 4000)
        got = _quantize(so, X, bits)
        ref = qref.quantize_groups(X, bits)
        if not all((g == r).all() for g, r in zip(got, ref)):
            failed.append(f"numpy_bit_for_bit:{bits}")
        X, E = qref.tie_groups(np.random.default_rng(9 + bits), bits, 300)
        c, _, _ = _quantize(so, X, bits)
        known = E >= 0
        if not (c.astype(np.int64)[known] == E[known]).all():
            failed.append(f"tie_closed_form:{bits}")
    return failed


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    failed = _failed_pins(_build(str(tmp_path), name, MUTANTS[name]))
    if name == "control":
        assert failed == []
    else:
        assert failed, f"mutant {name} passes every quantizer pin"
        print(name, "caught by", failed)
