"""Build the gfx950 HIP libraries in-tree with hipcc.

libw4a16.so        the matmul path (repack, GEMV and MFMA kernels, C ABI)
libw4a16_probe.so  a plain streaming-read kernel, used only by bench.py to
                   measure the read bandwidth the box reaches at a byte count
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libw4a16.so")
SOURCES = [os.path.join(PKG, "csrc", "w4a16.hip")]
PROBE_LIB = os.path.join(PKG, "libw4a16_probe.so")
PROBE_SOURCES = [os.path.join(PKG, "csrc", "probe_stream.hip")]
DEPENDS = SOURCES + [os.path.join(PKG, "csrc", "w4a16_kernels.hpp"),
                     os.path.join(ROOT, "include", "w4a16.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(out: str, sources: list, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
           # packed fp32 VALU forms stay off: plain fp32 ops only
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-o", tmp] + sources
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, out)
    return out


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libw4a16.so and libw4a16_probe.so for gfx950 (always, unless
    force=False and they exist).  Returns the path of libw4a16.so."""
    if force or not os.path.exists(PROBE_LIB):
        _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    if not force and os.path.exists(LIB):
        return LIB
    return _compile(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
