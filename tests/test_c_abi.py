"""The C ABI used from C: include/blake3_gpu.h compiles as strict C99 and C11, and a C
program (tests/c_abi/abi_check.c) built against libblake3_gpu.so and the HIP runtime calls
every hashing entry point on a stream of its own, comparing with the CPU oracle."""
import os
import shutil
import subprocess

import pytest

import blake3_merkle_tree_amd as b3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


def _build(tmp_path):
    lib_dir = os.path.dirname(b3.library_path())
    exe = str(tmp_path / "abi_check")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi", "abi_check.c"), os.path.join(ROOT, "oracle", "blake3_oracle.c"),
           "-L", lib_dir, "-lblake3_gpu", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-pthread",
           f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.mark.parametrize("std", ["c99", "c11"])
def test_header_is_plain_c(tmp_path, std):
    src = tmp_path / "hdr.c"
    src.write_text('#include "blake3_gpu.h"\nint main(void) { return blake3_gpu_version() > 0 ? 0 : 1; }\n')
    r = subprocess.run(["gcc", f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                        os.path.join(ROOT, "include"), "-c", str(src), "-o", str(tmp_path / "hdr.o")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


def test_c_program_builds_and_links(tmp_path):
    # every symbol the C program uses resolves against the built library (no GPU needed)
    assert os.path.exists(_build(tmp_path))


@pytest.mark.gpu
def test_c_program_matches_oracle(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "every result matches the oracle" in r.stdout
