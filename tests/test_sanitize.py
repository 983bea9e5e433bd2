"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the CPU oracle and
of the C ABI's host-side validation (CPU only; no GPU code is built).

* The oracle (oracle/mala_oracle.c) is linked with tests/sanitize/
  oracle_driver.c, which calls every oracle entry point on small seeded
  problems (all rounding flags, decision tiles, selections, splits).
* The API source (its host validation and workspace arithmetic) is compiled
  as plain C++ against the HIP headers, with stub kernel launches, and
  driven by tests/sanitize/abi_driver.c through every error path and a
  seeded sweep of extreme shapes and configs.
Any sanitizer report aborts the driver, and the test fails."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", OMP_NUM_THREADS="4")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-Wall", "-fopenmp", *SAN, "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "mala_oracle.c"), "-lm"], tmp_path)
    assert "oracle driver ok" in _run([exe], tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip"),
                    reason="g++ or the HIP headers not found")
def test_abi_validation_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "adaptive_softmax_attention_amd", "csrc")
    inc = ["-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + csrc]
    # the API source is host code apart from its declarations; compile a copy
    # as C++ for the host compiler
    api = tmp_path / "api_host.cpp"
    shutil.copy(os.path.join(csrc, "mala_api.hip"), api)
    # (HIP_SYMBOL comes from the device-compiler headers; on the host it is
    # the identity, as there)
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-DHIP_SYMBOL(X)=X", *inc, *SAN, "-c",
          str(api), "-o", "api.o"], tmp_path)
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *inc, *SAN, "-c",
          os.path.join(ROOT, "tests", "sanitize", "stub_launch.cpp"), "-o", "stub.o"], tmp_path)
    _run(["gcc", "-std=c11", "-Wall", *SAN, "-I" + os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), "-o", "drv.o"], tmp_path)
    exe = str(tmp_path / "abi_driver")
    _run(["g++", *SAN, "drv.o", "api.o", "stub.o", "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe], tmp_path)
    assert "abi driver ok" in _run([exe], tmp_path)
