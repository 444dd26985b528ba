"""The library driven from C alone (tests/c_abi_check.c): no Python or
PyTorch between the caller and the ABI. The program compares one gated
delta-rule call with the fp64 oracle and checks a host-side rejection."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi_check")


def test_c_program_is_built():
    assert os.path.exists(EXE), "run __graft_entry__.build() first"


@pytest.mark.gpu
def test_c_program_matches_oracle():
    print("\n[gpu-test] c_abi_check", flush=True)
    proc = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(proc.stdout, proc.stderr, flush=True)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    assert proc.stdout.strip().splitlines()[-1] == "ok"


@pytest.mark.skipif(shutil.which("cmake") is None, reason="cmake not found")
def test_cmake_project_configures(tmp_path):
    """CMakeLists.txt (the library for C/C++ projects) configures for
    gfx950 with the same source, flags and public header."""
    proc = subprocess.run(
        ["cmake", "-S", ROOT, "-B", str(tmp_path),
         "-DCMAKE_HIP_COMPILER=/opt/rocm/llvm/bin/clang++"],
        capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    cache = (tmp_path / "CMakeCache.txt").read_text()
    assert "CMAKE_HIP_ARCHITECTURES:STRING=gfx950" in cache
