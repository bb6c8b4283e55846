"""Build the gfx950 HIP libraries in-tree with hipcc.

libw4a16.so        the matmul path (repack, GEMV and MFMA kernels, C ABI)
libw4a16_probe.so  a plain streaming-read kernel, used only by bench.py to
                   measure the read bandwidth the GPU reaches at a byte count
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libw4a16.so")
# compiled separately (in parallel) and linked into one library: the host
# code, the GPTQ matmul kernels (plain and with epilogue modes, each in three
# compile-time-row units and one run-time-row unit) and the NVFP4 ones (GEMV
# and matrix-core units, plain and with epilogue modes)
UNITS = ("w4a16.hip",
         "variants_plain_gemv.hip", "variants_plain_mfma12.hip", "variants_plain_mfma34.hip", "variants_plain_rt.hip",
         "variants_epi_gemv.hip", "variants_epi_mfma12.hip", "variants_epi_mfma34.hip", "variants_epi_rt.hip",
         "variants_nvfp4_gemv.hip", "variants_nvfp4_mfma.hip", "variants_nvfp4_epi_gemv.hip",
         "variants_nvfp4_epi_mfma.hip")
SOURCES = [os.path.join(PKG, "csrc", f) for f in UNITS]
# Matrix-core results in ordinary VGPRs rather than accumulation registers:
# the kernels that read every product back with VALU instructions (the
# NVFP4 block scales; the run-time-row shapes) otherwise copy each result out
# of the accumulation registers first.  Measured per unit: the GEMV and
# compile-time-row kernels are as fast or faster without it.
SOURCE_FLAGS = {name: ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
                for name in ("variants_plain_rt.hip", "variants_epi_rt.hip", "variants_nvfp4_gemv.hip",
                             "variants_nvfp4_mfma.hip", "variants_nvfp4_epi_gemv.hip", "variants_nvfp4_epi_mfma.hip")}
PROBE_LIB = os.path.join(PKG, "libw4a16_probe.so")
PROBE_SOURCES = [os.path.join(PKG, "csrc", "probe_stream.hip")]
DEPENDS = SOURCES + [os.path.join(PKG, "csrc", "w4a16_kernels.hpp"), os.path.join(PKG, "csrc", "w4a16_variants.hpp"),
                     os.path.join(ROOT, "include", "w4a16.h")]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
         # packed fp32 VALU forms stay off: plain fp32 ops only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, what):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (res.stderr or "").splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({res.returncode}):\n{err}")
    return err


CACHE = os.path.join(ROOT, "_build")


def _key(src: str, cmd: list) -> str:
    """Hash of a translation unit's text, every header it may include and its command."""
    import hashlib
    h = hashlib.sha256(" ".join(cmd[1:]).encode())
    for path in [src] + [d for d in DEPENDS if not d.endswith(".hip")]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:20]


def _compile(out: str, sources: list, verbose: bool, reuse: bool = False) -> str:
    """Compile each source to an object in parallel, then link the shared library.

    reuse=True keeps objects in _build/ keyed by a hash of their inputs and
    recompiles only the units whose inputs changed (development builds).
    """
    objs = [out + "." + os.path.basename(src) + ".o" for src in sources]
    procs = []
    for src, obj in zip(sources, objs):
        cmd = ([hipcc()] + FLAGS + SOURCE_FLAGS.get(os.path.basename(src), []) +
               ["-I", os.path.join(ROOT, "include"), "-c", "-o", obj, src])
        if reuse:
            os.makedirs(CACHE, exist_ok=True)
            cached = os.path.join(CACHE, os.path.basename(src) + "." + _key(src, cmd) + ".o")
            if os.path.exists(cached):
                shutil.copyfile(cached, obj)
                continue
            cmd[cmd.index("-o") + 1] = cached
            import shlex
            cmd = ["bash", "-c", shlex.join(cmd) + " && cp " + shlex.quote(cached) + " " + shlex.quote(obj)]
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), src))
    errs = []
    for proc, src in procs:
        _, err = proc.communicate()
        err = "\n".join(l for l in (err or "").splitlines() if NOISE not in l)
        if proc.returncode != 0:
            errs.append(f"hipcc failed on {os.path.basename(src)} ({proc.returncode}):\n{err}")
        elif verbose and err.strip():
            print(err)
    if errs:
        raise RuntimeError("\n".join(errs))
    if reuse:                       # keep the three newest cached objects of each unit
        for src in sources:
            unit = os.path.basename(src) + "."
            cached = sorted((os.path.join(CACHE, f) for f in os.listdir(CACHE)
                             if f.startswith(unit) and f.endswith(".o")), key=os.path.getmtime)
            for old in cached[:-3]:
                os.remove(old)
    tmp = out + ".tmp"
    _run([hipcc()] + FLAGS + ["-shared", "-o", tmp] + objs, "link")
    os.replace(tmp, out)
    for obj in objs:
        os.remove(obj)
    return out


def build(force: bool = True, verbose: bool = False, reuse: bool = False) -> str:
    """Compile libw4a16.so and libw4a16_probe.so for gfx950 (always, unless
    force=False and they exist; reuse=True recompiles only changed units).
    Returns the path of libw4a16.so."""
    if force or not os.path.exists(PROBE_LIB):
        _compile(PROBE_LIB, PROBE_SOURCES, verbose, reuse)
    if not force and os.path.exists(LIB):
        return LIB
    return _compile(LIB, SOURCES, verbose, reuse)


if __name__ == "__main__":
    import sys
    print(build(verbose=True, reuse="--reuse" in sys.argv))
