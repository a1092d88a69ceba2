"""The oracle and the C ABI's host-side argument checks under AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only).

Two builds with -fsanitize=address,undefined (no recovery): the oracle
(oracle/qdiff_oracle.c, gcc) and the C ABI (capi.cpp and the host-side tile
choice, g++) linked against host stand-ins of the kernel launchers
(tests/sanitize/launch_stubs.cpp), so that every argument check runs without
a GPU.  A child pytest process loads them (the ASan runtime preloaded first)
and runs the ABI tests and the oracle pins against them; any sanitizer report
aborts it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_diffusion_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.fixture(scope="module")
def sanitized_libs(tmp_path_factory):
    import shutil
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc / g++ not available")
    d = tmp_path_factory.mktemp("san")
    oracle_so = str(d / "liboracle_san.so")
    _run(["gcc", *SAN, "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          os.path.join(ROOT, "oracle", "qdiff_oracle.c"), "-o", oracle_so, "-lm"])
    abi_so = str(d / "libqdiff_hostcheck_san.so")
    _run(["g++", *SAN, "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          os.path.join(CSRC, "capi.cpp"), os.path.join(CSRC, "gemm_policy.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", abi_so])
    return oracle_so, abi_so


def test_abi_and_oracle_pins_under_asan_ubsan(sanitized_libs):
    oracle_so, abi_so = sanitized_libs
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": " ".join(p for p in (asan, ubsan, env.get("LD_PRELOAD", "")) if p),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "QD_SANITIZED_LIB": abi_so,
        "ORACLE_SANITIZED_LIB": oracle_so,
        "PYTHONPATH": os.pathsep.join([ROOT, os.path.join(ROOT, "tests"), os.path.join(ROOT, "tests", "sanitize")]),
        "OMP_NUM_THREADS": "4",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "plugin", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_fp6_format.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=1800)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
