"""The oracle's pins again, with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, CPU only), and a check that the sanitizer is
live: a copy of the source with one out-of-bounds write planted must abort."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "..")
SRC = os.path.join(ROOT, "oracle", "kvq_oracle.c")


def _runtime_env():
    pre = []
    for name in ("libasan.so", "libubsan.so"):
        path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
        if not os.path.isabs(path) or not os.path.exists(path):
            pytest.skip(f"{name} not available")
        pre.append(path)
    env = dict(os.environ, KVQO_SANITIZE="1", LD_PRELOAD=" ".join(pre),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    return env


def test_pins_pass_under_sanitizers():
    oracle.build(force=True, sanitize=True)
    env = _runtime_env()
    probe = "import oracle; oracle._load(); assert oracle._lib._name.endswith('_san.so'), oracle._lib._name"
    subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, check=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_quant.py", "tests/test_oracle_attention.py",
                        "tests/test_oracle_bf16.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_sanitizer_catches_planted_overflow(tmp_path):
    with open(SRC) as f:
        text = f.read()
    site = "codes[i] = (uint8_t)r;"
    assert text.count(site) == 1
    text = text.replace(site, "codes[i + 1] = (uint8_t)r;")     # writes one byte past the group
    src = tmp_path / "planted.c"
    lib = tmp_path / "libplanted.so"
    src.write_text(text)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           *oracle._SAN_FLAGS, "-w", str(src), "-o", str(lib), "-lm"])
    call = ("import ctypes, numpy as np\n"
            f"so = ctypes.CDLL({str(lib)!r})\n"
            "x = np.linspace(-1, 1, 64).astype(np.float32)\n"
            "c = np.zeros(64, np.uint8); s = np.zeros(1, np.uint16); b = np.zeros(1, np.uint16)\n"
            "p = lambda a: a.ctypes.data_as(ctypes.c_void_p)\n"
            "so.kvqo_quantize_group(p(x), 64, 8, p(c), p(s), p(b))\n")
    r = subprocess.run([sys.executable, "-c", call], env=_runtime_env(), capture_output=True, text=True)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]
