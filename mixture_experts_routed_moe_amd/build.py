"""Build libmoe_routed.so (HIP for gfx950) in-tree.

Every .hip source is compiled with hipcc for gfx950 only; the C-ABI layer
(api.cpp) is host C++ linked into the same shared library. Objects go to
_build/ next to this file; the library lands beside the Python binding.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_routed.so")
DRIVER = os.path.join(HERE, "moe_bench_driver")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 instructions stay off in every device compile.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-Wall"]
KERNEL_SOURCES = ["gate.hip", "dispatch.hip", "grouped_gemm.hip", "grouped_gemm_tile.hip",
                  "grouped_gemm_w8.hip", "grouped_gemm_w8a8.hip", "grouped_gemm_fused.hip",
                  "grouped_gemm_f32.hip", "quant.hip", "reduce.hip", "w4a8.hip", "mx.hip",
                  "noalloc.hip"]
HOST_SOURCES = ["api.cpp"]


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", "--offload-arch=" + ARCH] + DEVICE_FLAGS + COMMON
    else:
        cmd = [HIPCC] + COMMON + ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if l.strip() and noise not in l]
    if msgs and verbose:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = KERNEL_SOURCES + HOST_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(sources), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    # The C++ driver of the C ABI (profiler passes without Python in the process).
    dtmp = DRIVER + ".tmp"
    cmd = [HIPCC, "-x", "hip", "--offload-arch=" + ARCH] + DEVICE_FLAGS + COMMON + [
        os.path.join(CSRC, "bench_driver.hip"), "-o", dtmp, "-L" + HERE, "-lmoe_routed",
        "-Wl,-rpath,$ORIGIN"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("driver build failed:\n%s%s" % (res.stdout, res.stderr))
    os.replace(dtmp, DRIVER)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
