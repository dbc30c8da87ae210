"""Build libblake3_gpu.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every call recompiles. Objects go to blake3_merkle_tree_amd/_build/, the library to
blake3_merkle_tree_amd/libblake3_gpu.so.
"""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libblake3_gpu.so")
ARCH = os.environ.get("BLAKE3_GPU_ARCH", "gfx950")

HIP_SOURCES = ["b3_kernels.hip", "b3_api.hip"]
CXX_SOURCES = ["b3_plan.cpp"]

# hipcc flags for device code: gfx950 only; packed-FP32 instruction selection is switched
# off for every HIP translation unit (integer-only code, and a known-safe default).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, extra_hip_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([hipcc, *HIP_FLAGS, *extra_hip_flags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
