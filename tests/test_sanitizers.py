"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU needed).

* The CPU oracle (plain C) built with gcc and both sanitizers, driven over every entry point on
  small inputs that reach its edge cases (tests/sanitize/oracle_driver.c).
* The HIP library's host code -- the C ABI's validation and the GEMM planner's workspace arithmetic
  -- built from the library's sources with the sanitizers on host code only (device code is
  compiled as usual), driven through the C ABI with fake device pointers and extreme sizes
  (tests/sanitize/abi_driver.c); without a GPU every call stops at validation or at the device
  check.

The two drivers link nothing of each other: the oracle and the library stay independent.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "nvfp4_quantized_gemm_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...: rc {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert "oracle driver ok" in r.stdout
    assert "runtime error" not in r.stderr


SOURCES = ["quantize.hip", "dequantize.hip", "prepack.hip", "gemm.hip", "gemm_skinny.hip", "mxfp4.hip", "debug_check.hip", "nvfp4_api.cpp"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    # sanitizers on the host side only: each -fsanitize= follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    common = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-ffp-contract=off",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include")]
    objs = []
    procs = []
    for src in SOURCES:
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC] + common + san + ["-c"] + (["-x", "hip"] if src.endswith(".cpp") else []) + \
            [os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for src, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"{src}: {err[-4000:]}"
    drv = str(tmp_path / "abi_driver.o")
    _run([HIPCC] + ["-O1", "-g", "-I" + os.path.join(ROOT, "include")] + san +
         ["-x", "c", "-c", os.path.join(HERE, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950"] + san + [drv] + objs + ["-o", exe])
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert "abi driver ok" in r.stdout
    assert "runtime error" not in r.stderr
