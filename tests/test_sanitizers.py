"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the host-side code (no GPU).

* The fp64 oracle, built with gcc and both sanitizers (leak detection on), runs every one of
  its functions on small and edge-case shapes (tests/sanitize/oracle_driver.c).
* The library, built with the sanitizers on its host code only (the device code is compiled
  as usual; GPU code cannot be sanitized here), runs argument validation of every entry
  point, the workspace-size functions over the extremes of every limit and the status
  strings (tests/sanitize/abi_driver.c) -- every path that returns before the device is
  touched.
Any sanitizer report aborts the driver with a non-zero status.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "draft_verify_sampling_step_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
ENV = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, env=None, timeout=600):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    out = res.stdout + res.stderr
    assert res.returncode == 0, f"{' '.join(cmd[:3])}... failed ({res.returncode}):\n{out[-4000:]}"
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-o", exe, os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "dspark_oracle.c"), "-lm"])
    out = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "every function ran" in out


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("gcc") is None,
                    reason="hipcc or gcc not available")
def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    inc = "-I" + os.path.join(ROOT, "include")

    def compile_one(f):
        obj = str(tmp_path / (f + ".o"))
        # sanitizers on the host code only: each -fsanitize= is preceded by -Xarch_host
        _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", inc, "-c", os.path.join(CSRC, f),
              "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "abi_driver.o")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", inc, "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-o", exe, drv] + objs)
    # the HIP runtime's own allocations are not this library's: leaks are not checked here
    out = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0"))
    assert "0 failures" in out
