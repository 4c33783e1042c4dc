"""Build libsinkattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and
the benchmark's streaming-read reference libhbmprobe.so (not part of the library)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsinkattn.so")
SOURCES = ["api.cpp", "prefill.hip", "decode.hip", "kv_append.hip"]
PROBE_LIB = os.path.join(PKG, "libhbmprobe.so")
PROBE_SOURCES = ["hbm_read_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsinkattn.so)")


def command(out: str, sources=SOURCES) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU ops are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result",
            f"-I{INCLUDE}", f"-I{CSRC}", "-o", out] + [os.path.join(CSRC, s) for s in sources]


def build(verbose: bool = False) -> str:
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return _compile(LIB, SOURCES, verbose)


def _compile(lib: str, sources, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = command(tmp, sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    noise = "is not a recognized feature for this target"
    msg = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
