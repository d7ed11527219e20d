"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU.

1. The fp64 oracle (oracle/oracle.c, test infrastructure) with every entry point
   exercised on small and degenerate shapes (tests/sanitize/oracle_driver.c).
2. The C ABI's argument validation and planning (the host code of
   efficient_transformer_amd/csrc/la_api.hip, rebuilt with the sanitizers on the
   host side only) driven through calls that return before any HIP runtime call
   (tests/sanitize/abi_driver.c); the library's other objects are linked as built.

Both drivers exit non-zero on a sanitizer report or a failed check."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, f"{os.path.basename(exe)} failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", *SAN, "-o", exe, os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    assert "oracle sanitizer run ok" in _run(exe)


def test_abi_validation_under_sanitizers(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hipcc = os.path.join(rocm, "bin", "hipcc")
    build = os.path.join(ROOT, "efficient_transformer_amd", "_build")
    objs = [o for o in sorted(glob.glob(os.path.join(build, "*.o"))) if os.path.basename(o) != "la_api.o"]
    if not os.path.exists(hipcc) or not objs:
        pytest.skip("hipcc or the library's objects are not available (build the library first)")
    api = str(tmp_path / "la_api_san.o")
    host_san = [x for s in SAN for x in ("-Xarch_host", s)]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
                    *host_san, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "efficient_transformer_amd", "csrc", "la_api.hip"), "-o", api],
                   check=True, capture_output=True)
    drv = str(tmp_path / "abi_driver.o")
    subprocess.run(["gcc", "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(HERE, "abi_driver.c"), "-o", drv], check=True)
    exe = str(tmp_path / "abi_driver")
    subprocess.run(["g++", *SAN, "-o", exe, drv, api, *objs, "-L" + os.path.join(rocm, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(rocm, "lib")], check=True)
    assert "abi sanitizer run ok" in _run(exe)
