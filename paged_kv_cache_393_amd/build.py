"""Build step of the HIP library (hipcc, gfx950), run from the repository root.

    python -m paged_kv_cache_393_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
# (sources, output) of every HIP library: the paged KV cache library (decode,
# the KV write path, PagedEviction, chunked prefill) and the bench's
# measurement kernels.
LIBS = [
    ([os.path.join(_HERE, "csrc", "paged_attn.hip"), os.path.join(_HERE, "csrc", "kv_write.hip"),
      os.path.join(_HERE, "csrc", "kv_evict.hip"), os.path.join(_HERE, "csrc", "paged_prefill.hip"),
      os.path.join(_HERE, "csrc", "kv_compress.hip"), os.path.join(_HERE, "csrc", "check_tables.hip")],
     os.path.join(_HERE, "libpagedattn.so")),
    ([os.path.join(_HERE, "csrc", "pa_probe.hip")], os.path.join(_HERE, "libpaprobe.so")),
]
LIB_PATH = LIBS[0][1]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(sources: list, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + list(sources) + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}) on {sources}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP library for gfx950; returns the decode library's path."""
    for sources, out in LIBS:
        _compile(sources, out, verbose)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
