"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the host side of the C ABI (tplinear.cpp: the placement -> view map and every
argument check, linked against launchers that abort) and the CPU oracle
(oracle.c), each driven by a small program in tests/host/.  No GPU code is
built here; the sanitizers instrument the host compilers' output only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_abi_host_code_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "tensor_linear_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    obj = str(tmp_path / "tplinear.o")
    _run(["g++", "-std=c++17", "-O1", "-c", os.path.join(ROOT, "tensor_linear_amd", "csrc", "tplinear.cpp"),
          "-o", obj] + SAN + inc, tmp_path)
    exe = str(tmp_path / "abi_driver")
    _run(["g++", "-std=c++17", "-O1", os.path.join(HOST, "abi_driver.cpp"), obj, "-o", exe] + SAN + inc,
         tmp_path)
    r = _run([exe], tmp_path)
    assert "abi driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_launch_offsets_follow_layout(tmp_path):
    """One placement map: the shard offsets each entry point passes to its
    kernels (recorded by stub launchers) equal tp_shard_layout's views of the
    layer's placements, for every mode (tests/host/launch_map_driver.cpp)."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "tensor_linear_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    obj = str(tmp_path / "tplinear.o")
    _run(["g++", "-std=c++17", "-O1", "-c", os.path.join(ROOT, "tensor_linear_amd", "csrc", "tplinear.cpp"),
          "-o", obj] + SAN + inc, tmp_path)
    exe = str(tmp_path / "launch_map_driver")
    _run(["g++", "-std=c++17", "-O1", os.path.join(HOST, "launch_map_driver.cpp"), obj, "-o", exe] + SAN + inc,
         tmp_path)
    r = _run([exe], tmp_path)
    assert "launch map driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_row_fold_routing(tmp_path):
    """Which kernel a column layer takes (skinny, narrow or tile), and which
    way TP_ROW_FUSED / TP_ROW_SCATTER fold (inside the GEMM or partials +
    fold, the same bits either way), for a GPU of 256 CUs, with the
    library's own choice, TPLINEAR_ROW_FOLD=gemm, and a workspace the
    partials would not fit (tests/host/route_driver.cpp)."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "tensor_linear_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    obj = str(tmp_path / "tplinear.o")
    _run(["g++", "-std=c++17", "-O1", "-c", os.path.join(ROOT, "tensor_linear_amd", "csrc", "tplinear.cpp"),
          "-o", obj] + SAN + inc, tmp_path)
    exe = str(tmp_path / "route_driver")
    _run(["g++", "-std=c++17", "-O1", os.path.join(HOST, "route_driver.cpp"), obj, "-o", exe] + SAN + inc,
         tmp_path)
    r = _run([exe], tmp_path)
    assert "route driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-O1", "-fopenmp", "-ffp-contract=off",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HOST, "oracle_driver.c"), "-o", exe] + SAN,
         tmp_path)
    r = _run([exe], tmp_path)
    assert "oracle driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
