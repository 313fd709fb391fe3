"""The C ABI's host code (csrc/api.cpp: validation, device checks, dispatch,
status mapping, workspace rules) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven on the CPU by tests/host/abi_driver.cpp.

The driver replaces the HIP runtime calls api.cpp makes (device query,
properties, error strings, the scratch symbol lookup) and the kernel
launchers with host stubs, so a failing launch, a failing runtime query and a
device that is not gfx950 are forced from the host and the mapped status
(TWL_EHIP, TWL_EDEVICE) and message are checked, together with every shape,
null, alignment and workspace rule.  No GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ternary_weight_linear_block_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host", "abi_driver.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"

# sanitizers on the host side of a host-only HIP compile (no device code)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(_hipcc()) or not os.path.exists(CLANG):
        pytest.skip("ROCm compilers not available")
    d = tmp_path_factory.mktemp("san")
    objs = []
    # api.cpp as the library builds it (its device side holds only the
    # no-allocation scratch array); the driver as host code only
    for src, mode in ((os.path.join(CSRC, "api.cpp"), ["--offload-arch=gfx950"]),
                      (DRIVER, ["--cuda-host-only"])):
        obj = str(d / (os.path.basename(src) + ".o"))
        cmd = [_hipcc(), "-x", "hip"] + mode + ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"] + SAN + [
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        objs.append(obj)
    exe = str(d / "abi_driver")
    # the HIP runtime is linked for the code-object registration only: every
    # runtime call api.cpp makes resolves to the driver's stubs
    link = [CLANG, "-fsanitize=address,undefined"] + objs + [
        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    res = subprocess.run(link, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return exe


def test_driver_is_sanitized(driver):
    out = subprocess.run(["nm", driver], capture_output=True, text=True).stdout
    assert "__asan_init" in out and "__ubsan_handle" in out


def test_abi_host_code_under_asan_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "all checks passed" in res.stdout
    assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr
