"""AddressSanitizer / UndefinedBehaviorSanitizer runs of host code (no GPU).

* The CPU oracle (oracle/oracle.c, oracle/nvfp4.c) built with gcc under both
  sanitizers, driven by tests/sanitize/oracle_check.c.
* The library's host side (planning, plan checks, workspace sizes, the
  argument checks of every entry point) built from its own sources with a
  subset of the kernel shapes, the sanitizers on host code only, driven by
  tests/sanitize/host_check.cpp.  Its calls never reach a device.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "weight_only_int4_gptq_amd", "csrc")
HIP_UNITS = ["w4a16.hip",
             "variants_plain_gemv.hip", "variants_plain_mfma12.hip", "variants_plain_mfma34.hip",
             "variants_plain_rt.hip", "variants_epi_gemv.hip", "variants_epi_mfma12.hip",
             "variants_epi_mfma34.hip", "variants_epi_rt.hip", "variants_nvfp4_gemv.hip",
             "variants_nvfp4_mfma.hip", "variants_nvfp4_epi_gemv.hip", "variants_nvfp4_epi_mfma.hip"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({res.returncode}):\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_address_and_undefined_behaviour_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_check")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-fopenmp", "-std=c99",
          os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "oracle", "nvfp4.c"), "-lm", "-o", exe])
    res = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", OMP_NUM_THREADS="2"),
               timeout=300)
    assert "oracle sanitizer check: ok" in res.stdout


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_library_host_side_under_address_and_undefined_behaviour_sanitizers():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the argument checks would reach it")
    os.makedirs(OUT, exist_ok=True)
    # the sanitizers apply to host code only (each after -Xarch_host)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++20", "-DW4A16_VARIANT_SUBSET",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = [os.path.join(CSRC, u) for u in HIP_UNITS] + [os.path.join(ROOT, "tests", "sanitize", "host_check.cpp")]
    objs = [os.path.join(OUT, os.path.basename(s) + ".o") for s in srcs]
    procs = [subprocess.Popen([_hipcc()] + flags + ["-c", "-o", o, s], stdout=subprocess.PIPE,
                              stderr=subprocess.PIPE, text=True) for s, o in zip(srcs, objs)]
    for p, s in zip(procs, srcs):
        _, err = p.communicate()
        assert p.returncode == 0, f"{s}: {err[-3000:]}"
    exe = os.path.join(OUT, "host_check")
    _run([_hipcc()] + flags + objs + ["-o", exe])
    res = _run([exe], env=ENV, timeout=600)
    assert "host sanitizer check: ok" in res.stdout
