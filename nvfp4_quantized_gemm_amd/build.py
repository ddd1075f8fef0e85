"""Build libnvfp4.so (HIP, gfx950) in-tree with hipcc."""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "nvfp4")
LIB = os.path.join(PKG, "libnvfp4.so")

SOURCES = ["quantize.hip", "dequantize.hip", "prepack.hip", "gemm.hip", "gemm_skinny.hip", "mxfp4.hip", "debug_check.hip", "nvfp4_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c"]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += [os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    warn = [l for l in r.stderr.splitlines() if "warning" in l and "packed-fp32-ops" not in l]
    if warn:
        sys.stderr.write("\n".join(warn) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
