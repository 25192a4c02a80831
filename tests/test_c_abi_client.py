"""The C ABI from plain C: tests/c_abi_client.c, built with gcc against
include/gemm_epi.h, libgemm_epi.so and the HIP runtime's C API, checks two
fused GEMMs with closed-form results (A = I) element by element."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "beta_epilogue_amd")
ROCM = "/opt/rocm"


def _build(tmp_path):
    if not shutil.which("gcc") or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("gcc or the HIP runtime library is not available")
    if not os.path.exists(os.path.join(PKG, "libgemm_epi.so")):
        pytest.skip("libgemm_epi.so is not built")
    exe = str(tmp_path / "c_abi_client")
    cmd = ["gcc", "-O1", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "c_abi_client.c"), "-o", exe,
           "-L", PKG, "-lgemm_epi", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + PKG + ":" + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_client_builds_and_runs_without_a_gpu(tmp_path):
    """Compiles with no warnings' errors and, with no usable GPU, says so
    (exit 77); with one, passes its checks (exit 0)."""
    exe = _build(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode in (0, 77), r.stdout + r.stderr


@pytest.mark.gpu
def test_c_client_on_the_gpu(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi client: ok" in r.stdout
