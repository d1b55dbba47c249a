"""Build libkvq.so (the gfx950 kernels and the C ABI) in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["append.hip", "append_norm.hip", "attn.hip", "attn_step.hip", "prefill.hip", "prefill_q.hip", "prefill_codes.hip", "bf16_cache.hip",
           "kvq_api.hip"]
# measurement probes (include/kvq_probes.h), a library of their own
PROBE_LIB = os.path.join(HERE, "libkvq_probes.so")
PROBE_SOURCES = ["probes.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden",
    # fused multiply-add wherever the source allows it, except where a pragma
    # asks for one IEEE rounding per operation (the quantizer, the norms)
    "-ffp-contract=fast-honor-pragmas",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the softmax and the scale folds read
    # them, and AGPR copies would cost a VALU move each
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def _link(sources, lib, verbose):
    """Compile the sources in parallel (one hipcc per file), then link them."""
    procs, objs = [], []
    for src in sources:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
        objs.append(obj)
    for cmd, p in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(p.returncode, cmd)
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _link(PROBE_SOURCES, PROBE_LIB, verbose)
    return _link(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
