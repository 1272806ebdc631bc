"""include/int8mm.h is a C header: a plain-C99 program includes it, links
libint8mm.so and gets the documented status codes from every entry point's
host-side checks (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

from int8_quantized_matmul_col_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def c_program(tmp_path_factory):
    if shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("gcc or the ROCm headers are missing")
    if not os.path.exists(binding.LIB_PATH):
        from int8_quantized_matmul_col_amd import build
        build.build()
    out = str(tmp_path_factory.mktemp("c_abi") / "c_abi_check")
    libdir = os.path.dirname(binding.LIB_PATH)
    # the HIP runtime headers name the platform when compiled as plain C
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-Wno-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", libdir, "-lint8mm",
           "-Wl,-rpath," + libdir, "-lm", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def test_c_client_gets_documented_statuses(c_program):
    r = subprocess.run([c_program], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert got["ld"] == "128"
    assert got["bytes"] == str(512 * 128)  # N = 300 padded to 512 rows
    assert got["ws_ok"] == "1" and got["ws_bad"] == "0"
    assert int(got["prepare"]) == binding.INT8MM_EINVAL
    assert int(got["matmul"]) == binding.INT8MM_EINVAL      # NaN threshold
    assert int(got["linear"]) == binding.INT8MM_ESHAPE      # negative M
    assert int(got["stages"]) == binding.INT8MM_EWORKSPACE  # no workspace
    assert int(got["profiled"]) == binding.INT8MM_EINVAL    # negative threshold
    assert int(got["colmax"]) == binding.INT8MM_EINVAL      # no output
    assert int(got["counts"]) == binding.INT8MM_EINVAL      # NaN threshold
    assert int(got["empty"]) == binding.INT8MM_OK           # M == 0
    assert got["strerror"].startswith("workspace")
    assert got["hiperr"] == "[]"
