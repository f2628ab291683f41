"""The host C ABI (csrc/api.cpp, with stand-ins for the device launchers) and
the C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer, and
driven through every host-side path (tests/sanitize/): a memory error or
undefined behaviour aborts the driver and fails the test.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "multiresolution_hash_grid_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, cwd, env=None):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fopenmp", os.path.join(ROOT, "oracle", "hashgrid_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
          "-lm", "-o", exe], ROOT)
    r = _run([exe], ROOT, ENV)
    assert "all checks passed" in r.stdout


def test_host_abi_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_driver")
    # host-only compilation: the sanitizers apply to host code (-Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(SAN, "stubs.cpp"), os.path.join(SAN, "abi_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "-x", "hip", "--offload-host-only", "-std=c++20", "-O1", "-g", *san, *inc, "-c", src,
              "-o", obj], ROOT)
        objs.append(obj)
    _run([HIPCC, *san, *objs, "-o", exe], ROOT)
    r = _run([exe], ROOT, ENV)
    assert "all host-side checks passed" in r.stdout
