"""CPU oracle for quantized-KV attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The GPU library (``decode_attention_group_amd``)
never imports, loads or calls it, and the two share no code.

The arithmetic lives in ``kvq_oracle.c`` (fp32 quantizer, fp64 dequantization
and attention); this module builds it with gcc and wraps it with ctypes over
numpy arrays.  Citations refer to pages 78, 80 and 81 of the
@mlx-bun/inference 0.0.0-stage -> 1.0.0 diff on my.diffend.io.

Layouts here are the plain ones:
  codes   uint8  [B][H][R][D]         one code per byte
  scales  uint16 [B][H][R][D/64]      bf16 bit patterns
  biases  uint16 [B][H][R][D/64]
  a side of width 16 (an unquantized bf16 cache, the pages' bf16 sliding layers):
  vals    uint16 [B][H][R][D]         bf16 bit patterns, nearest-even rounding
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")
# An AddressSanitizer + UndefinedBehaviorSanitizer build of the same source, loaded
# instead when KVQO_SANITIZE=1 (the process must preload the sanitizer runtime).
_LIB_SAN = os.path.join(_HERE, "libkvq_oracle_san.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
GROUP = 64

_lib = None


class OracleError(RuntimeError):
    """A non-zero status from the oracle (1: invalid argument, 2: capacity)."""

    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


def _sanitized() -> bool:
    return os.environ.get("KVQO_SANITIZE") == "1"


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile kvq_oracle.c with gcc (IEEE fp32, no contraction, OpenMP); with
    sanitize=True the AddressSanitizer/UBSan build beside it."""
    lib = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
            "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
            *(_SAN_FLAGS if sanitize else []),
            _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        path = build(force=False, sanitize=_sanitized())
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.kvqo_quantize_group.argtypes = [P, i32, i32, P, P, P]
        lib.kvqo_quantize_group.restype = i32
        lib.kvqo_append.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, P]
        lib.kvqo_append.restype = i32
        lib.kvqo_pack_words.argtypes = [P, ctypes.c_int64, i32, i32, P]
        lib.kvqo_pack_words.restype = None
        lib.kvqo_dequant.argtypes = [P, P, P, ctypes.c_int64, i32, P]
        lib.kvqo_dequant.restype = None
        lib.kvqo_attend.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                    P, i32, i32, P, ctypes.c_double, P, i32]
        lib.kvqo_attend.restype = i32
        lib.kvqo_attend_any.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                        P, i32, i32, P, ctypes.c_double, P, i32]
        lib.kvqo_attend_any.restype = i32
        lib.kvqo_append_bf16.argtypes = [P, i32, i32, i32, i32, i32, P, P]
        lib.kvqo_append_bf16.restype = i32
        lib.kvqo_bf16.argtypes = [ctypes.c_float]
        lib.kvqo_bf16.restype = ctypes.c_uint16
        lib.kvqo_rms_factor.argtypes = [P, i32, ctypes.c_float]
        lib.kvqo_rms_factor.restype = ctypes.c_float
        lib.kvqo_norm_rows.argtypes = [P, ctypes.c_int64, i32, P, ctypes.c_float, P, P, i32, i32, P, P]
        lib.kvqo_norm_rows.restype = i32
        lib.kvqo_max_threads.argtypes = []
        lib.kvqo_max_threads.restype = i32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().kvqo_max_threads())


def quantize_group(x, bits: int):
    """Quantize one group (any length, normally 64) -> (codes uint8, scale_bits, bias_bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.size, np.uint8)
    s = np.zeros(1, np.uint16)
    b = np.zeros(1, np.uint16)
    st = _load().kvqo_quantize_group(_ptr(x), x.size, bits, _ptr(codes), _ptr(s), _ptr(b))
    if st:
        raise OracleError(st, "quantize_group")
    return codes, int(s[0]), int(b[0])


def bf16(x) -> int:
    """One fp32 value rounded to the nearest bf16, ties to even (bit pattern)."""
    h = int(_load().kvqo_bf16(float(np.float32(x))))
    if h == 0xFFFF:
        raise OracleError(1, "bf16")
    return h


class Cache:
    """A plain-layout cache for one layer, K and V each with its own width: 4 or 8
    (affine codes, scales, biases) or 16 (bf16 values, unquantized)."""

    def __init__(self, B: int, H: int, D: int, R: int, k_bits: int, v_bits: int, window: int = 0):
        if D % GROUP:
            raise ValueError("head_dim must be a multiple of 64")
        self.B, self.H, self.D, self.R = B, H, D, R
        self.k_bits, self.v_bits, self.window = k_bits, v_bits, window
        G = D // GROUP
        self.k_codes = np.zeros((B, H, R, D), np.uint8)
        self.v_codes = np.zeros((B, H, R, D), np.uint8)
        self.k_scales = np.zeros((B, H, R, G), np.uint16)
        self.k_biases = np.zeros((B, H, R, G), np.uint16)
        self.v_scales = np.zeros((B, H, R, G), np.uint16)
        self.v_biases = np.zeros((B, H, R, G), np.uint16)
        self.k_vals = np.zeros((B, H, R, D), np.uint16) if k_bits == 16 else None
        self.v_vals = np.zeros((B, H, R, D), np.uint16) if v_bits == 16 else None

    def append(self, k, v, pos0):
        """Quantize-and-append (or, for a 16-bit side, round-and-append) T tokens:
        k, v fp32 [B][H][T][D]; pos0 [B]."""
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        pos0 = np.ascontiguousarray(pos0, dtype=np.int32)
        B, H, T, D = k.shape
        assert (B, H, D) == (self.B, self.H, self.D) and v.shape == k.shape
        lib = _load()
        for x, bits, c, s, b, vals, what in (
                (k, self.k_bits, self.k_codes, self.k_scales, self.k_biases, self.k_vals, "K"),
                (v, self.v_bits, self.v_codes, self.v_scales, self.v_biases, self.v_vals, "V")):
            if bits == 16:
                st = lib.kvqo_append_bf16(_ptr(x), B, H, T, D, self.R, _ptr(pos0), _ptr(vals))
            else:
                st = lib.kvqo_append(_ptr(x), B, H, T, D, bits, self.R, _ptr(pos0), _ptr(c), _ptr(s), _ptr(b))
            if st:
                raise OracleError(st, f"append {what}")

    def packed_k(self):
        """K codes packed per row into uint32 words, [B][H][R][D*bits/32]."""
        return pack_words(self.k_codes, self.k_bits)

    def dequant_k(self):
        if self.k_vals is not None:
            return bf16_values(self.k_vals)
        return dequant(self.k_codes, self.k_scales, self.k_biases)

    def dequant_v(self):
        if self.v_vals is not None:
            return bf16_values(self.v_vals)
        return dequant(self.v_codes, self.v_scales, self.v_biases)

    def attend(self, q_bits, len_, scale: float = 1.0, nthreads: int = 0):
        """fp64 attention of q (bf16 bit patterns, [B][Hq][C][D]) over this cache."""
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        len_ = np.ascontiguousarray(len_, dtype=np.int32)
        B, Hq, C, D = q_bits.shape
        assert B == self.B and D == self.D
        out = np.zeros((B, Hq, C, D), np.float64)
        kv = None if self.k_vals is None else _ptr(self.k_vals)
        vv = None if self.v_vals is None else _ptr(self.v_vals)
        st = _load().kvqo_attend_any(
            _ptr(self.k_codes), _ptr(self.k_scales), _ptr(self.k_biases), kv,
            _ptr(self.v_codes), _ptr(self.v_scales), _ptr(self.v_biases), vv,
            B, self.H, D, self.R, self.window, _ptr(q_bits), Hq, C, _ptr(len_),
            float(scale), _ptr(out), int(nthreads))
        if st:
            raise OracleError(st, "attend")
        return out


def pack_words(codes, bits: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    D = codes.shape[-1]
    rows = codes.size // D
    out = np.zeros(codes.shape[:-1] + (D * bits // 32,), np.uint32)
    _load().kvqo_pack_words(_ptr(codes), rows, D, bits, _ptr(out))
    return out


def dequant(codes, scales, biases):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    biases = np.ascontiguousarray(biases, dtype=np.uint16)
    D = codes.shape[-1]
    out = np.zeros(codes.shape, np.float64)
    _load().kvqo_dequant(_ptr(codes), _ptr(scales), _ptr(biases), codes.size // D, D, _ptr(out))
    return out


def bf16_values(vals):
    """bf16 bit patterns -> fp64 values (exact)."""
    vals = np.ascontiguousarray(vals, dtype=np.uint16)
    return (vals.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rms_factor(x, eps: float) -> float:
    """The RMS factor of one row: fp32(1 / sqrt(tree sum of squares / D + eps)) (kvq_oracle.c)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return float(_load().kvqo_rms_factor(_ptr(x), x.size, np.float32(eps)))


def norm_rows(x, w=None, eps: float = 1e-6, rope=None, pos=None):
    """Normalize rows of x (fp32 [..., D]) with the RMS norm (weight w [D] or none),
    then, with rope = (cos [P][n/2], sin [P][n/2]), rotate the first n columns of
    each row at its absolute position pos [...] (kvq_oracle.c kvqo_norm_rows)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    rows = x.size // D
    y = np.zeros_like(x)
    wp = None if w is None else np.ascontiguousarray(w, dtype=np.float32)
    if rope is not None:
        cos_t = np.ascontiguousarray(rope[0], dtype=np.float32)
        sin_t = np.ascontiguousarray(rope[1], dtype=np.float32)
        n_rot, n_pos = 2 * cos_t.shape[1], cos_t.shape[0]
        pos = np.ascontiguousarray(np.broadcast_to(pos, x.shape[:-1]), dtype=np.int32)
    else:
        cos_t = sin_t = None
        n_rot, n_pos = 0, 0
    st = _load().kvqo_norm_rows(_ptr(x), rows, D, None if wp is None else _ptr(wp), np.float32(eps),
                                None if cos_t is None else _ptr(cos_t), None if sin_t is None else _ptr(sin_t),
                                n_rot, n_pos, None if pos is None else _ptr(pos), _ptr(y))
    if st:
        raise OracleError(st, "norm_rows")
    return y


def append_normed(cache: "Cache", k, v, pos0, k_weight, eps: float, rope=None):
    """The fused step the library offers as kvq_append_norm_quantize: keys through
    the weighted RMS norm and the rotation, values through the un-scaled norm,
    then the append [p80 model.ts attentionTraining: kNorm, RoPE, vNorm, appendWindow]."""
    k = np.ascontiguousarray(k, dtype=np.float32)
    B, H, T, D = k.shape
    pos = (np.asarray(pos0, np.int64)[:, None, None] + np.arange(T)[None, None, :]) * np.ones((1, H, 1), np.int64)
    kn = norm_rows(k, k_weight, eps, rope, pos.astype(np.int32))
    vn = norm_rows(v, None, eps)
    cache.append(kn, vn, pos0)
    return kn, vn


def attend_shared(cache: Cache, q_layers, len_, scale: float = 1.0, nthreads: int = 0):
    """Several KV-sharing layers reading one donor cache [p80 model.ts header: KV-shared
    layers; p78 gemma4-e4b.ts Gemma4Layer.cache]: each layer's queries attend the same
    cache with the donor's positions and window, i.e. one attend() per layer."""
    return [cache.attend(q, len_, scale, nthreads) for q in q_layers]
